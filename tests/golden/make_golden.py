"""Writes the expected values of tests/golden/*.json from the oracle only.

Inputs are the numbers the pages print; expected values come from
``oracle.accounting``.  Run from the repository root:
``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def paging_example():
    # explore.n1n.ai, "vLLM 深度解析：PagedAttention 如何让大模型推理更快、更省钱":
    # the fragmentation section's example of a request that produced 100 tokens
    # while 2048 positions were reserved, and the 映射机制详解 section's example
    # page size of 16 tokens (only the last page of a sequence can hold waste).
    tokens, reserved, page = 100, 2048, 16
    blocks = -(-tokens // page)
    return {
        "source": "explore.n1n.ai, 'vLLM 深度解析：PagedAttention 如何让大模型推理更快、"
                  "更省钱', KV-cache fragmentation section (100 of 2048 reserved) and "
                  "映射机制详解 (16-token pages, waste only in the last page)",
        "inputs": {"tokens": tokens, "reserved": reserved, "page_tokens": page},
        "expected": {
            "contiguous_utilisation": oracle.contiguous_utilisation([tokens], reserved),
            "paged_blocks": blocks,
            "paged_slots": blocks * page,
            "paged_waste_slots": blocks * page - tokens,
            "paged_utilisation": oracle.paged_utilisation([tokens]),
        },
    }


def kv_size_example():
    # gheillcoat.github.io, "概念-vLLM", 核心概念：KV Cache 与显存效率: size =
    # batch x seq_len x layers x hidden x 2 (K+V) x 2 bytes (FP16).  The page's
    # own 70B example number does not follow from its formula for any standard
    # 70B shape, so only the formula is used: here for one 8-KV-head layer of
    # the 70B-class long-context workload (8 x 32768 tokens, 8 x 128 wide).
    return {
        "source": "gheillcoat.github.io, '概念-vLLM', 核心概念：KV Cache 与显存效率 (formula)",
        "inputs": {"batch": 8, "seq_len": 32768, "layers": 1, "width": 1024, "elem_bytes": 2},
        "expected": {"bytes": oracle.kv_cache_bytes(8, 32768, 1, 1024, 2)},
    }


if __name__ == "__main__":
    for name, fn in [("paging_example", paging_example), ("kv_size_example", kv_size_example)]:
        with open(os.path.join(HERE, name + ".json"), "w", encoding="utf-8") as f:
            json.dump(fn(), f, ensure_ascii=False, indent=1)
            f.write("\n")
