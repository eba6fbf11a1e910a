#!/usr/bin/env python3
"""Throughput of the paged decode path on one MI355X.

Workload: a Llama-3-8B-shaped GQA attention layer at decode time -- batch
256, 32 query heads over 8 KV heads, head_dim 128, bf16 KV in 16-token
blocks shuffled through a pool, context lengths lognormal (median 512,
sigma 0.8) clipped to [16, 4096] (seeded, ``workloads.config3``).

One step is one decode iteration of a stack of ``--layers`` attention layers
(default 4), each with its own K/V cache; the block table is shared by the
layers, as in a decoder:

  1. host block manager: append one token to each of the 256 sequences
     (slot mapping, new blocks) and pack the tables -- pa_bm_append_batch,
     pa_bm_pack, into pinned buffers;
  2. one async upload of the slot mapping, the context lengths and the block-table
     entries of blocks opened this step, scattered into the device-resident tables;
  3. per layer: pa_write_kv of the new token's K/V rows, then pa_decode.

With 4 layers of 0.75 GB each, a layer's KV has been pushed out of the
256 MB last-level cache by the other layers' reads before it is read again,
so every decode streams its KV from HBM.  ``value`` is decoded sequences per
second per attention layer: 256 * layers * steps / wall time of the timed
steps.  Inputs (caches, new K/V rows, queries) are resident in HBM before the
timed region starts.

The JSON line also carries
  * ``roofline``: pa_decode's algorithmic KV bytes per call (sum over
    sequences of L * Hkv * D * 2 bytes * 2 for K and V) over its mean
    duration, taken with HIP events on one pa_decode of every timed step
    (layer step mod layers, so each layer in turn), against the 8 TB/s HBM
    peak.  For single-token steps the events are recorded by the decode's own
    kernel dispatch on its stream (pa_time_next_call: hipExtLaunchKernel with
    start and stop events), so no marker packet sits between pa_write_kv and
    the decode; chunks (--chunk) record them as markers around the call.
    They are created without the system-scope fence (the path exchanges
    nothing with the host);
    ``traffic`` is the HBM bytes per call from the committed rocprofv3
    counter summary, when that was taken on the current kernel source;
  * ``cpu_baseline``: the CPU float64 oracle's decode of the same batch on the
    host, single-threaded;
  * ``path_steps``: the other steps of the path, each timed on its own -- the
    host block manager's time per step (append + pack), pa_write_kv of the
    whole cache's rows (the bulk fill of one layer) and of one step's rows,
    and pa_copy_blocks of 1024 whole-block pairs, with their rates (bytes
    read plus written) against the HBM peak;
  * ``stream_read_probe``: context for the roofline fraction -- the rate
    pa_read_probe streams a 4 GiB buffer at with the decode kernel's load
    form, in address order and in 4 KiB chunks visited in a seeded random
    order (the paged pattern), and decode's fraction of the latter.

With ``--chunk T`` (T = 2..16) each step brings T new tokens per sequence
instead of one -- a draft-verification or chunked-prefill step: T appends per
sequence, pa_write_kv of B*T rows, then pa_decode_chunk with q [B, T, Hq, D]
(causal inside the chunk).  ``value`` is then query tokens per second per
layer, and the roofline is pa_decode_chunk's.  The default (T = 1) is the
decode step above.

With ``--swap`` the step is a swap-out and swap-in of 64 of the 256
sequences of one layer's cache (block manager pa_bm_swap_out / _in, then
pa_swap_blocks between the device cache and a pinned host pool); ``value``
is the bytes moved per second over both directions, and the roofline is
the host link (PCIe 5.0 x16, 63 GB/s per direction).  A plain contiguous
copy of the same bytes (the DMA engines, hipMemcpyAsync) is timed beside it
as context.

With ``--prefix`` the batch is 256 requests sharing a 2048-token system
prompt, each with its own 64..512-token question, built with prefix
caching (the prompt's blocks are stored once and shared); the step is the
decode step above, with the block manager's shared-prefix groups and
pa_decode_shared_prefix (one launch: per KV head, row groups of 4 requests
each attend the prompt from L2, then their own blocks) unless
``--prefix-path plain``
asks for pa_decode over every whole context.  The roofline takes the unique
KV bytes a call reads (shared blocks once) over the whole call; the logical
bytes (every sequence's whole context) are reported beside them, with the
other path's time on the final batch, the block manager's hit rate and that
of a simulated multi-turn chat.

With ``--config N`` (2, 4 or 5) the step is pa_decode alone on another of
the seeded decode configurations, once per layer, lengths fixed: 2 is a
13B-shaped MHA layer (batch 64, 40 heads, lengths U[128, 2048]), 4 a
70B-shaped long-context GQA layer (batch 8, 64 query / 8 KV heads, 32768
tokens each: 64 pieces of 512 tokens per sequence), 5 parallel sampling on
an fp8-e4m3 cache (64 prompts of 1024 + r tokens, each forked into 4
samples with copy-on-write of the shared partial block, suffixes U[1, 256]).
The roofline takes the distinct KV bytes a call reads; for config 5 the
logical bytes (each sample's whole context, the shared prompt blocks once per
sample) are reported beside them.

With ``--window W`` the decode (or chunk) step attends only the last W
positions of each context (pa_decode_window); the roofline's algorithmic
bytes are then the positions the window keeps, min(L, W + T - 1) per
sequence.

With ``--block-size BS`` (8, 32 or 64) the caches use BS-token blocks (the
pool re-sized for them, with its own seeded free order); the JSON line adds
the paged utilisation and the simulated chat's block-cache hit rate at that
block size.  Blocks of 32 and 64 stream as 2 and 4 tiles; 8-token blocks
take the partition path.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers N]
                      [--chunk T | --swap | --prefix] [--window W]
                      [--block-size BS] [--kv-dtype bf16|fp8] [--no-cpu-baseline]
                      [--copy-calibration MIB] [--probe-calibration MIB]

--copy-calibration MIB ends the run with plain device copies of MIB MiB (the
reference a hardware-counter run scales WRITE_SIZE by); --probe-calibration
MIB with pa_read_probe passes over MIB MiB, read with the decode kernel's own
load form (the reference FETCH_SIZE is scaled by).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded input generators; no method arithmetic)

METRIC = "paged decode attention: KV-cache GB/s vs HBM peak; decoded seqs/sec"
METRIC_CHUNK = ("paged chunk attention (T new tokens per sequence, causal): KV-cache GB/s "
                "vs HBM peak; query tokens/sec")
HBM_PEAK_GBPS = 8000.0
PCIE5_X16_GBPS = 63.0        # 32 GT/s x 16 lanes x 128/130 / 8, per direction
METRIC_PREFIX = ("paged decode with prefix caching: unique KV GB/s vs HBM peak; decoded "
                 "seqs/sec; block-cache hit rate")
METRIC_SWAP = "paged KV swap: device<->pinned host block copy GB/s vs host link peak"
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_421_amd", "csrc", "decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_gqa8b_b256.txt")
TRAFFIC_FILE_FP8 = os.path.join(ROOT, "profiles", "decode_traffic_gqa8b_fp8_b256.txt")
TRAFFIC_FILE_CHUNK = os.path.join(ROOT, "profiles", "chunk_traffic_gqa8b_b256_t{T}.txt")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _kv_bytes(lens, hkv, d, elem):
    return int(np.asarray(lens, dtype=np.int64).sum()) * hkv * d * elem * 2


class HipEvent:
    """A HIP timing event recorded on an explicit stream (ctypes on the HIP
    runtime that torch has loaded).  hipEventDisableSystemFence: recording it
    does not flush caches to system scope."""
    _hip = None
    FLAGS = 0x20000000          # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self._c = ctypes
        self.h = ctypes.c_void_p()
        self._check(HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h),
                                                          ctypes.c_uint(self.FLAGS)), "create")

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"hipEvent{what} failed with HIP error {rc}")

    def record(self, stream):
        self._check(HipEvent._hip.hipEventRecord(self.h, self._c.c_void_p(stream.cuda_stream)),
                    "Record")

    def elapsed_ms(self, end):
        ms = self._c.c_float()
        self._check(HipEvent._hip.hipEventSynchronize(end.h), "Synchronize")
        self._check(HipEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.h, end.h),
                    "ElapsedTime")
        return ms.value

    def destroy(self):
        if self.h:
            self._check(HipEvent._hip.hipEventDestroy(self.h), "Destroy")
            self.h = self._c.c_void_p()


def kernel_source_sha256():
    """Hash of the decode kernel's device code: the text from the kernel's
    signature line to the end of its body in decode.hip."""
    text = open(DECODE_SRC).read()
    a = text.index("decode_stream_kernel(StreamArgs a")
    b = text.index("// Zero-fill of a decode workspace.")
    return hashlib.sha256(text[a:b].encode()).hexdigest()


def _traffic_per_call(kv_bytes, T=1, kv_dtype="bf16"):
    """HBM bytes of one pa_decode (pa_decode_chunk for T > 1) call reading
    ``kv_bytes`` algorithmic KV bytes, from the committed rocprofv3 counter
    summary (bytes read per algorithmic byte, bytes written per call), if that
    summary was taken on the current kernel source; else None."""
    if kv_dtype == "fp8":
        path = TRAFFIC_FILE_FP8 if T == 1 else None
    else:
        path = TRAFFIC_FILE if T == 1 else TRAFFIC_FILE_CHUNK.format(T=T)
    if path is None:
        return None
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_r = re.search(r"fetch_bytes_per_algorithmic_byte:\s*([0-9.eE+]+)", text)
    m_w = re.search(r"write_bytes_per_call:\s*([0-9.eE+]+)", text)
    if not (m_src and m_r and m_w) or m_src.group(1) != kernel_source_sha256():
        return None
    return float(m_r.group(1)) * kv_bytes + float(m_w.group(1))


def opened_table_entries(lens, slots, block_size):
    """Table entries of the blocks a step opened.  lens: context lengths
    before the step [B]; slots: the slots the manager gave the step's new
    tokens [B, T] (token t of sequence s at position lens[s] + t).  A token
    whose position is a multiple of the block size opens a block, whose id
    is its slot // block_size.  Returns (rows, cols, blocks)."""
    T = slots.shape[1]
    pos = lens[:, None] + np.arange(T)
    opened = pos % block_size == 0
    return np.nonzero(opened)[0], pos[opened] // block_size, slots[opened] // block_size


def stream_read_probe(dev, stream, gib=4, reps=3):
    """GB/s of pa_read_probe over a ``gib`` GiB buffer: (in order, random 4 KiB)."""
    import torch
    import paged_kv_cache_421_amd as pk
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    order = torch.randperm(n // 4096, device=dev, generator=g).to(torch.int32)
    sink = pk.read_probe(buf, stream=stream)
    out = []
    for o in (None, order):
        pk.read_probe(buf, o, sink, stream=stream)             # warm
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for _ in range(reps):
            pk.read_probe(buf, o, sink, stream=stream)
        e1.record(stream)
        out.append(round(reps * n / (e0.elapsed_ms(e1) / 1e3) / 1e9, 1))
        e0.destroy()
        e1.destroy()
    del buf, order, sink
    return out[0], out[1]


def cpu_baseline(w, budget_s=10.0, T=1, fmt="bf16", k_scale=1.0, v_scale=1.0):
    """The oracle's decode (gather blocks, textbook fp64 softmax attention) of
    the whole batch at its initial lengths, repeated until ``budget_s``
    seconds have passed (at least 3 runs); median run time.  With T > 1, the
    oracle's chunk attention, the last T positions of each context being the
    chunk.  ``fmt`` is the cache format (fp8: the bf16 rows quantised with
    the given scales, as pa_write_kv stores them).  The BLAS library may use
    one thread per host core the process may run on; the same batch on one
    thread is reported beside it."""
    import oracle
    from threadpoolctl import threadpool_limits

    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    per = {}
    for s in range(w.B):
        bm.add_seq(s)
        per[s], _ = bm.append_tokens(s, int(w.lens[s]))
    starts = np.concatenate([[0], np.cumsum(w.lens)[:-1]]).astype(np.int64)
    slots = np.concatenate([per[s] for s in range(w.B)])
    assert len(slots) == len(w.row_seq) and np.all(w.row_pos == np.arange(len(slots)) -
                                                  np.repeat(starts, w.lens))
    shape = (w.num_blocks, w.Hkv, 16, w.D)
    store = np.uint8 if fmt == "fp8" else np.uint16
    kc, vc = oracle.write_kv(np.zeros(shape, store), np.zeros(shape, store),
                             w.k_rows, w.v_rows, slots, "bf16", fmt, k_scale, v_scale)
    cap = max(-(-int(L) // 16) for L in w.lens)
    bt, cl = bm.pack(list(range(w.B)), cap)
    qc = None
    if T > 1:
        qc = workloads.chunk_queries(np.random.default_rng(1004), w.B, T, w.Hq, w.D, "bf16")

    def median_run(threads, budget):
        times = []
        with threadpool_limits(limits=threads):
            t_all = time.perf_counter()
            while len(times) < 3 or time.perf_counter() - t_all < budget:
                t0 = time.perf_counter()
                if T == 1:
                    oracle.decode(w.q, "bf16", kc, vc, fmt, bt, cl, w.scale, k_scale, v_scale)
                else:
                    oracle.decode_chunk(qc, "bf16", kc, vc, fmt, bt, cl, w.scale, k_scale,
                                        v_scale)
                times.append(time.perf_counter() - t0)
        return statistics.median(times), len(times)

    cores = len(os.sched_getaffinity(0))
    t, runs = median_run(cores, budget_s)
    t1, runs1 = median_run(1, budget_s / 2)
    e = 1 if fmt == "fp8" else 2
    what = "256 seqs x 32 heads" if T == 1 else f"256 seqs x {T} chunk tokens x 32 heads"
    return {"value": round(w.B * T / t, 2), "unit": "seqs/s" if T == 1 else "tokens/s",
            "cores": cores, "kind": "oracle",
            "kv_gbps": round(_kv_bytes(cl, w.Hkv, w.D, e) / t / 1e9, 4),
            "host_cores_visible": cores,
            "value_1_thread": round(w.B * T / t1, 2),
            "sample": (f"whole batch ({what}, {fmt} cache, sum L {int(cl.sum())}, initial "
                       f"lengths), {runs} runs, median {t:.3f} s; numpy float64 with BLAS "
                       f"limited to {cores} threads (the host cores visible); on 1 thread "
                       f"{runs1} runs, median {t1:.3f} s")}


def swap_cpu_baseline(kc, vc, pairs, budget_s=10.0):
    """The oracle's swap_blocks (numpy whole-block copies) over the same
    pairs, on host arrays, until ``budget_s`` seconds have passed."""
    import oracle
    hk = np.zeros((int(pairs[:, 1].max()) + 1,) + kc.shape[1:], kc.dtype)
    hv = np.zeros_like(hk)
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_all < budget_s:
        t0 = time.perf_counter()
        oracle.swap_blocks(kc, vc, hk, hv, pairs)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    nbytes = len(pairs) * 2 * kc[0].nbytes
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"{len(pairs)} block pairs ({nbytes / 1e6:.0f} MB, K and V) between numpy "
                       f"arrays in host memory, {len(times)} runs, median {t:.3f} s")}


def run_swap(args):
    """Swap 64 of the 256 sequences of the GQA batch-256 cache out to a
    pinned host pool and back, ``steps`` times."""
    import torch
    import paged_kv_cache_421_amd as pk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    steps = args.steps or 20
    warm = args.warmup if args.warmup is not None else 3
    w = workloads.config3(rows=False)
    B, Hkv, D = w.B, w.Hkv, w.D
    group = np.arange(0, B, 4, dtype=np.int64)           # 64 sequences, every 4th
    need = int(sum(-(-int(w.lens[s]) // 16) for s in group))
    H = need + 16
    desc = pk.CacheDesc(w.num_blocks, Hkv, D, "bf16")
    bm = pk.BlockManager(w.num_blocks, free_order=w.free_order, num_host_blocks=H)
    for s in range(B):
        bm.add_seq(s)
        bm.append_tokens(s, int(w.lens[s]))
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    kc = torch.randn(desc.shape, device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn(desc.shape, device=dev, generator=g).to(torch.bfloat16)
    hk = torch.empty((H,) + tuple(desc.shape[1:]), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    block_bytes = Hkv * 16 * D * 2
    pairs_dev = torch.empty((max(H, w.num_blocks), 2), dtype=torch.int32, device=dev)
    _log(f"bench: swap {len(group)} sequences = {need} blocks = {need * 2 * block_bytes / 1e6:.0f} MB "
         f"each way, {steps} steps")

    def one(out, evs):
        pairs = bm.swap_out(group) if out else bm.swap_in(group)
        n = len(pairs)
        pairs_dev[:n].copy_(torch.from_numpy(pairs), non_blocking=False)
        if evs is not None:
            evs[0].record(stream)
        if out:
            pk.swap_blocks(desc, kc, vc, hk, hv, pairs_dev[:n], stream=stream)
        else:
            pk.swap_blocks(desc, hk, hv, kc, vc, pairs_dev[:n], stream=stream)
        if evs is not None:
            evs[1].record(stream)
        return n * 2 * block_bytes

    for _ in range(warm):
        one(True, None)
        one(False, None)
    torch.cuda.synchronize()
    ev_out = [(HipEvent(), HipEvent()) for _ in range(steps)]
    ev_in = [(HipEvent(), HipEvent()) for _ in range(steps)]
    moved = 0
    t0 = time.perf_counter()
    for i in range(steps):
        moved += one(True, ev_out[i])
        moved += one(False, ev_in[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_out = statistics.mean(a.elapsed_ms(b) for a, b in ev_out) / 1e3
    t_in = statistics.mean(a.elapsed_ms(b) for a, b in ev_in) / 1e3
    for a, b in ev_out + ev_in:
        a.destroy()
        b.destroy()
    per_dir = need * 2 * block_bytes
    gbps_out, gbps_in = per_dir / t_out / 1e9, per_dir / t_in / 1e9
    # context: the DMA engines on one contiguous buffer of the same size
    src = torch.empty(per_dir // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty(per_dir // 2, dtype=torch.bfloat16, pin_memory=True)
    dma = {}
    for name, (a, b) in (("d2h", (dst, src)), ("h2d", (src, dst))):
        a.copy_(b, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for _ in range(5):
            a.copy_(b, non_blocking=True)
        e1.record(stream)
        dma[name] = round(5 * per_dir / (e0.elapsed_ms(e1) / 1e3) / 1e9, 2)
        e0.destroy()
        e1.destroy()
    _log(f"bench: swap out {t_out * 1e6:.0f} us ({gbps_out:.1f} GB/s), in {t_in * 1e6:.0f} us "
         f"({gbps_in:.1f} GB/s); DMA contiguous copy d2h {dma['d2h']} h2d {dma['h2d']} GB/s")
    mean_gbps = 2 * per_dir / (t_out + t_in) / 1e9
    res = {
        "metric": METRIC_SWAP,
        "value": round(moved / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("gqa8b-bf16-b256 cache (Llama-3-8B-shaped layer, 8 KV heads, "
                                "head_dim 128, 16-token shuffled blocks): swap out and back in "
                                f"{len(group)} of 256 sequences ({need} blocks, "
                                f"{per_dir / 1e6:.0f} MB K+V each way) to a pinned host pool"),
                   "step": "pa_bm_swap_out + pa_swap_blocks (device->host), pa_bm_swap_in + "
                           "pa_swap_blocks (host->device)",
                   "value_is": "bytes moved per second over the timed steps, both directions, "
                               "host bookkeeping and pair uploads included",
                   "parallelism": "single GPU"},
        "swap_out_gbps": round(gbps_out, 2), "swap_in_gbps": round(gbps_in, 2),
        "dma_contiguous_gbps": dma,
        "roofline": {"kernel": "copy_blocks_kernel (pa_swap_blocks)", "bound": "pcie",
                     "achieved": round(mean_gbps, 2), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                     "frac": round(mean_gbps / PCIE5_X16_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        _log("bench: timing the CPU oracle")
        nb = 512
        rng = np.random.default_rng(5)
        kh = rng.integers(0, 2**16, (nb,) + tuple(desc.shape[1:]), dtype=np.uint16)
        vh = rng.integers(0, 2**16, (nb,) + tuple(desc.shape[1:]), dtype=np.uint16)
        pr = np.stack([rng.permutation(nb), rng.permutation(nb)], 1).astype(np.int64)
        res["cpu_baseline"] = swap_cpu_baseline(kh, vh, pr)
    print(json.dumps(res), flush=True)


def chat_hit_rate(seed=11, conversations=64, turns=8, block_size=16):
    """Host-only: multi-turn chats through the library's block manager with
    prefix caching.  Turn k's prompt is the whole conversation so far plus a
    new user message (64..256 tokens); the answer (128..512 tokens) is
    appended with its ids; the request then ends and its blocks become
    evictable.  Returns (hit rate, queried blocks, microseconds per prompt
    lookup)."""
    import paged_kv_cache_421_amd as pk
    rng = np.random.default_rng(seed)
    bm = pk.BlockManager((1 << 20) // block_size, block_size=block_size)
    bm.enable_prefix_caching()
    hist = [np.zeros(0, np.int32) for _ in range(conversations)]
    sid, t_lookup, n_lookup = 0, 0.0, 0
    for _ in range(turns):
        for c in range(conversations):
            prompt = np.concatenate([hist[c], rng.integers(0, 32000, int(rng.integers(64, 257)))])
            t0 = time.perf_counter()
            bm.add_seq_prompt(sid, prompt)
            t_lookup += time.perf_counter() - t0
            n_lookup += 1
            ans = rng.integers(0, 32000, int(rng.integers(128, 513)))
            bm.append_token_ids(sid, ans)
            bm.free_seq(sid)
            hist[c] = np.concatenate([prompt, ans]).astype(np.int32)
            sid += 1
    q, h, _, _ = bm.cache_stats()
    return h / q, q, t_lookup / n_lookup * 1e6


def run_config(args):
    """pa_decode on decode configuration 2, 4 or 5 (lengths fixed); configuration 5
    through pa_decode_shared_prefix unless --prefix-path plain."""
    import torch
    import paged_kv_cache_421_amd as pk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    steps = args.steps or 50
    warm = args.warmup if args.warmup is not None else 5
    NL = args.layers
    n = args.config
    w = workloads.CONFIGS[n](rows=False)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    fmt = "fp8" if n == 5 else "bf16"
    elem = 1 if fmt == "fp8" else 2
    g = torch.Generator(device=dev)
    g.manual_seed(n)
    bm = pk.BlockManager(w.num_blocks, free_order=w.free_order)
    pairs = []
    if n == 5:                       # prompt, 3 forks, then each sample's suffix
        for grp in w.groups:
            s0 = grp["seqs"][0]
            bm.add_seq(s0)
            bm.append_tokens(s0, grp["prompt"])
            for sid in grp["seqs"][1:]:
                bm.fork(s0, sid)
            for sid, sl in zip(grp["seqs"], grp["suffix"]):
                _, pr = bm.append_tokens(sid, sl)
                if pr is not None:
                    pairs.append(pr)
    else:
        for s in range(B):
            bm.add_seq(s)
            bm.append_tokens(s, int(w.lens[s]))
    cap = int(-(-int(w.lens.max()) // 16))
    bt, cl = bm.pack(np.arange(B), cap)
    used = np.unique(bt[bt >= 0])
    # caches: random rows in every slot of every block a table names (the
    # contents do not change the work); fp8 codes from N(0, 1) rows at scale
    # max|x| / 448
    rows = int(len(used)) * 16
    slots = torch.from_numpy((used.astype(np.int64)[:, None] * 16 + np.arange(16)).reshape(-1)).to(dev)
    k_rows = torch.randn((rows, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    v_rows = torch.randn((rows, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    ks = float(k_rows.float().abs().max()) / 448.0 if fmt == "fp8" else 1.0
    vs = float(v_rows.float().abs().max()) / 448.0 if fmt == "fp8" else 1.0
    desc = pk.CacheDesc(w.num_blocks, Hkv, D, fmt, ks, vs)
    tdt = torch.uint8 if fmt == "fp8" else torch.bfloat16
    kc = [torch.zeros(desc.shape, dtype=tdt, device=dev) for _ in range(NL)]
    vc = [torch.zeros(desc.shape, dtype=tdt, device=dev) for _ in range(NL)]
    pk.write_kv(desc, kc[0], vc[0], k_rows, v_rows, slots, stream=stream)
    for l in range(1, NL):
        kc[l].view(torch.uint8).copy_(kc[0].view(torch.uint8))
        vc[l].view(torch.uint8).copy_(vc[0].view(torch.uint8))
    del k_rows, v_rows, slots
    q = [torch.randn((B, Hq, D), device=dev, generator=g).to(torch.bfloat16) for _ in range(NL)]
    out = [torch.empty_like(q[0]) for _ in range(NL)]
    btd = torch.from_numpy(bt).to(dev)
    cld = torch.from_numpy(cl).to(dev)
    max_len = int(cl.max())
    workspace = pk.new_decode_workspace(desc, B, Hq, max_len, dev)
    logical = _kv_bytes(cl, Hkv, D, elem)
    # distinct bytes: every position of every sequence once, shared positions once
    seen = {}
    for s in range(B):
        L = int(cl[s])
        for j in range(-(-L // 16)):
            b = int(bt[s, j])
            seen[b] = max(seen.get(b, 0), min(16, L - 16 * j))
    unique = sum(seen.values()) * Hkv * D * elem * 2
    # configuration 5 goes through pa_decode_shared_prefix, which attends each
    # prompt's full blocks (shared by its 4 samples) once, and times pa_decode
    # beside it; --prefix-path plain swaps the two
    groups = bm.shared_prefix_groups(np.arange(B)) if n == 5 else np.zeros((0, 3), np.int32)
    cascade = len(groups) > 0 and args.prefix_path != "plain"
    sp_ws = (pk.new_shared_prefix_workspace(desc, B, Hq, bt.shape[1], max_len, dev)
             if len(groups) else None)
    torch.cuda.synchronize()

    def call(l, shared):
        if shared:
            pk.decode_shared_prefix(desc, kc[l], vc[l], q[l], out[l], btd, cld, max_len,
                                    float(w.scale), groups, sp_ws, stream=stream)
        else:
            pk.decode(desc, kc[l], vc[l], q[l], out[l], btd, cld, max_len, float(w.scale),
                      workspace, stream=stream)

    def timed(shared, nsteps):
        """nsteps steps of NL calls, HIP events around every call.  (With an
        event pair around one call per step only, nothing paces the host
        between back-to-back launches; a run then showed one stall of about
        35 ms inside an event pair, so every call keeps its pair here.)"""
        for i in range(warm * NL):
            call(i % NL, shared)
        torch.cuda.synchronize()
        evs = [(HipEvent(), HipEvent()) for _ in range(nsteps * NL)]
        t0 = time.perf_counter()
        for i in range(nsteps * NL):
            evs[i][0].record(stream)
            call(i % NL, shared)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us = [a.elapsed_ms(b) * 1e3 for a, b in evs]
        for a, b in evs:
            a.destroy()
            b.destroy()
        return wall, us

    wall, dec_us = timed(cascade, steps)
    mean_s = statistics.mean(dec_us) / 1e6
    other = None
    if len(groups):
        # the other path on the same batch, and how far its output lies from this one's
        res_this = [o.float().clone() for o in out]
        _, other_us = timed(not cascade, max(steps // 2, 1))
        diff = max(float((o.float() - r).abs().max()) for o, r in zip(out, res_this))
        other = {"path": "pa_decode" if cascade else "pa_decode_shared_prefix",
                 "decode_us_mean": round(statistics.mean(other_us), 2),
                 "max_abs_diff_vs_this_path": round(diff, 5)}
        _log(f"bench: config {n}: {other['path']} mean {other['decode_us_mean']:.1f} us; "
             f"outputs differ by at most {diff:.4g}")
    ach = unique / mean_s / 1e9
    names = {2: "mha13b-bf16-b64: 13B-shaped MHA decode layer, batch 64, 40 heads, head_dim 128, "
                "bf16 KV in 16-token shuffled blocks, lengths U[128, 2048]",
             4: "gqa70b-bf16-32k: 70B-shaped long-context GQA decode layer, batch 8, 64 query / 8 KV "
                "heads, head_dim 128, bf16 KV, 32768 tokens per sequence in shuffled 16-token blocks",
             5: "cow-fp8-4x64: parallel sampling, 64 prompts of 1024 + U[1, 15] tokens forked into 4 "
                "samples each (copy-on-write of the shared partial block), suffixes U[1, 256]; "
                "32 query / 8 KV heads, head_dim 128, fp8-e4m3 KV with per-tensor scales"}
    _log(f"bench: config {n}: pa_decode mean {mean_s * 1e6:.1f} us (p10 "
         f"{np.percentile(dec_us, 10):.1f}, p90 {np.percentile(dec_us, 90):.1f}); distinct "
         f"{unique / 1e9:.4f} GB at {ach:.0f} GB/s, logical {logical / 1e9:.4f} GB")
    res = {
        "metric": METRIC,
        "value": round(B * steps * NL / wall, 1),
        "unit": "seqs/s",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": fmt, "data": "synthetic",
        "config": {"workload": names[n], "global_batch": B, "layers_per_step": NL,
                   "step": ("per layer pa_decode_shared_prefix (lengths fixed)" if cascade
                            else "per layer pa_decode (lengths fixed)"),
                   "value_is": "sequences decoded per second per attention layer",
                   "parallelism": "single GPU"},
        "decode_us_mean": round(mean_s * 1e6, 2),
        "decode_us_p10": round(float(np.percentile(dec_us, 10)), 2),
        "decode_us_p90": round(float(np.percentile(dec_us, 90)), 2),
        "distinct_kv_gb": round(unique / 1e9, 4), "logical_kv_gb": round(logical / 1e9, 4),
        "logical_kv_gbps": round(logical / mean_s / 1e9, 1),
        "copy_on_write_pairs": len(pairs),
        "shared_prefix_groups": len(groups),
        "other_path": other,
        "roofline": {"kernel": ("decode_stream_kernel in group mode "
                                "(pa_decode_shared_prefix, one launch)" if cascade else "decode_stream_kernel (pa_decode)" if n != 4 else
                                "decode_stream_kernel (pa_decode: long contexts split over waves)"),
                     "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def run_prefix(args):
    """256 requests sharing a 2048-token prompt, decoded step by step."""
    import torch
    import paged_kv_cache_421_amd as pk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    steps = args.steps or 100
    warm = args.warmup if args.warmup is not None else 10
    NL = args.layers
    P = 2048
    w = workloads.prefix_batch(9, 256, P, 64, 512, rows=False)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    nb = w.num_blocks + B * (-(-(steps + warm) // 16) + 1)
    desc = pk.CacheDesc(nb, Hkv, D, "bf16")
    bm = pk.BlockManager(nb, free_order=np.r_[w.free_order, np.arange(w.num_blocks, nb)])
    bm.enable_prefix_caching()
    kc = [torch.empty(desc.shape, dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    vc = [torch.empty(desc.shape, dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    written = 0
    for r in range(B):
        slots, nc = bm.add_seq_prompt(r, w.prompt(r))
        n = len(slots) - nc
        sm = torch.from_numpy(np.ascontiguousarray(slots[nc:], dtype=np.int64)).to(dev)
        for l in range(NL):
            k = torch.randn((n, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
            v = torch.randn((n, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
            pk.write_kv(desc, kc[l], vc[l], k, v, sm, stream=stream)
        written += n
    queried, hits, registered, _ = bm.cache_stats()
    lens = np.array([len(w.prompt(r)) for r in range(B)], dtype=np.int64)
    _log(f"bench: prefix batch: {B} requests, prompt {P} shared, hit rate {hits / queried:.4f}, "
         f"{written} of {int(lens.sum())} prompt rows written")
    rng = np.random.default_rng(1003)
    k_new, v_new, q = [], [], []
    for _ in range(NL):
        kn, vn, qq = workloads.config3_step(rng, B, Hq, Hkv, D)
        k_new.append(torch.from_numpy(kn.view(np.int16)).to(dev).view(torch.bfloat16))
        v_new.append(torch.from_numpy(vn.view(np.int16)).to(dev).view(torch.bfloat16))
        q.append(torch.from_numpy(qq.view(np.int16)).to(dev).view(torch.bfloat16))
    out = [torch.empty_like(q[0]) for _ in range(NL)]
    max_len_final = int(lens.max()) + steps + warm
    cap = -(-max_len_final // 16)
    cascade = args.prefix_path != "plain"
    workspace = pk.new_decode_workspace(desc, B, Hq, max_len_final, dev)
    sp_workspace = pk.new_shared_prefix_workspace(desc, B, Hq, cap, max_len_final, dev)
    # as in the decode step: device-resident tables patched with the entries
    # of opened blocks; slots, lengths and those entries staged in pinned
    # buffers, triple-buffered against the running GPU
    NBUF = 3
    h_i64 = [torch.empty(3 * B, dtype=torch.int64, pin_memory=True) for _ in range(NBUF)]
    h_i32 = [torch.empty(2 * B, dtype=torch.int32, pin_memory=True) for _ in range(NBUF)]
    buf_ev = [None] * NBUF
    d_i64 = torch.empty(3 * B, dtype=torch.int64, device=dev)
    d_i32 = torch.empty(2 * B, dtype=torch.int32, device=dev)
    d_slots = d_i64[:B]
    d_cl = d_i32[:B]
    ids = np.arange(B, dtype=np.int64)
    d_bt = torch.from_numpy(bm.pack(ids, cap)[0]).to(dev)
    nfull = P // 16

    def attend(l, groups, max_len):
        if groups is not None:
            pk.decode_shared_prefix(desc, kc[l], vc[l], q[l], out[l], d_bt, d_cl, max_len,
                                    float(w.scale), groups, sp_workspace, stream=stream)
        else:
            pk.decode(desc, kc[l], vc[l], q[l], out[l], d_bt, d_cl, max_len, float(w.scale),
                      workspace, stream=stream)

    def step(i, ev_pair):
        """One step; with ev_pair, HIP events around layer i mod layers."""
        b = i % NBUF
        if buf_ev[b] is not None:
            buf_ev[b].synchronize()          # the upload that last read buffer b is done
        hi, hj = h_i64[b].numpy(), h_i32[b].numpy()
        sl, pairs = bm.append_batch(ids, slots=hi[:B])
        assert len(pairs) == 0
        rows, cols, blocks = opened_table_entries(lens, hi[:B].reshape(B, 1), 16)
        n = len(rows)
        hi[B:B + n] = rows
        hi[2 * B:2 * B + n] = cols
        hj[B:B + n] = blocks
        lens[:] += 1
        hj[:B] = lens
        d_i64.copy_(h_i64[b], non_blocking=True)
        d_i32.copy_(h_i32[b], non_blocking=True)
        if n:
            d_bt[d_i64[B:B + n], d_i64[2 * B:2 * B + n]] = d_i32[B:B + n]
        ev = torch.cuda.Event()
        ev.record()
        buf_ev[b] = ev
        max_len = int(lens.max())
        groups = bm.shared_prefix_groups(ids) if cascade else None
        for l in range(NL):
            pk.write_kv(desc, kc[l], vc[l], k_new[l], v_new[l], d_slots, stream=stream)
            timed_here = ev_pair is not None and l == i % NL
            if timed_here:
                ev_pair[0].record(stream)
            attend(l, groups, max_len)
            if timed_here:
                ev_pair[1].record(stream)
        logical = int(lens.sum()) * Hkv * D * 4
        unique = (16 * nfull + int((lens - 16 * nfull).sum())) * Hkv * D * 4
        return logical, unique

    for i in range(warm):
        step(i, None)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    per = []
    t0 = time.perf_counter()
    for i in range(steps):
        per.append(step(warm + i, evs[i]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bt_ref, cl_ref = bm.pack(ids, cap)
    assert np.array_equal(d_bt.cpu().numpy(), bt_ref), "device block tables drifted"
    assert np.array_equal(d_cl.cpu().numpy(), cl_ref), "device lengths drifted"
    dec_ms = [a.elapsed_ms(b) for (a, b) in evs]
    for a, b in evs:
        a.destroy()
        b.destroy()
    mean_s = statistics.mean(dec_ms) / 1e3
    logical = statistics.mean(p[0] for p in per)
    unique = statistics.mean(p[1] for p in per)
    ach = unique / mean_s / 1e9
    # the other path on the final batch, for comparison (not the timed value)
    final_groups = bm.shared_prefix_groups(ids)
    other = []
    for _ in range(3):
        for l in range(NL):
            a, b = HipEvent(), HipEvent()
            a.record(stream)
            attend(l, None if cascade else final_groups, int(lens.max()))
            b.record(stream)
            other.append((a, b))
    torch.cuda.synchronize()
    other_us = statistics.mean(a.elapsed_ms(b) for a, b in other[NL:]) * 1e3
    for a, b in other:
        a.destroy()
        b.destroy()
    name = "pa_decode_shared_prefix" if cascade else "pa_decode"
    other_name = "pa_decode" if cascade else "pa_decode_shared_prefix"
    chat_rate, chat_q, lookup_us = chat_hit_rate()
    _log(f"bench: {name} mean {mean_s * 1e6:.1f} us: unique {unique / 1e9:.3f} GB "
         f"({ach:.0f} GB/s), logical {logical / 1e9:.3f} GB ({logical / mean_s / 1e9:.0f} GB/s); "
         f"{other_name} on the final batch {other_us:.1f} us; chat hit rate {chat_rate:.4f}")
    res = {
        "metric": METRIC_PREFIX,
        "value": round(B * NL * steps / wall, 1),
        "unit": "seqs/s",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("prefix-shared GQA batch: Llama-3-8B-shaped layer (32 query / 8 KV "
                                "heads, head_dim 128, bf16), 256 requests sharing a 2048-token "
                                "system prompt plus their own 64..512-token questions, built "
                                "through prefix caching"),
                   "layers_per_step": NL,
                   "step": ("block-manager append + table upload" +
                            (" + shared-prefix groups" if cascade else "") +
                            f" + per layer pa_write_kv and {name}"),
                   "value_is": "sequences decoded per second per attention layer",
                   "parallelism": "single GPU"},
        "block_cache_hit_rate": round(hits / queried, 4),
        "prompt_rows_written": written, "prompt_rows_total": int(lens.sum() - B * (steps + warm)),
        "unique_kv_gb": round(unique / 1e9, 4), "logical_kv_gb": round(logical / 1e9, 4),
        "logical_kv_gbps": round(logical / mean_s / 1e9, 1),
        "decode_us_mean": round(mean_s * 1e6, 2),
        "decode_path": name,
        "other_path": {"name": other_name, "us_on_final_batch": round(other_us, 2)},
        "chat_sim": {"hit_rate": round(chat_rate, 4), "queried_blocks": chat_q,
                     "conversations": 64, "turns": 8,
                     "us_per_prompt_lookup": round(lookup_us, 2)},
        "roofline": {"kernel": ("decode_stream_kernel in group mode, KV head by KV head "
                               "(pa_decode_shared_prefix, whole call)"
                               if cascade else
                               "decode_stream_kernel (pa_decode over shared prompt blocks)"),
                     "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="default 100 (50 with --chunk)")
    ap.add_argument("--warmup", type=int, default=None, help="default 10 (5 with --chunk)")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--chunk", type=int, default=1, metavar="T",
                    help="new tokens per sequence per step (1 = decode)")
    ap.add_argument("--swap", action="store_true",
                    help="measure swapping sequences out to pinned host memory and back")
    ap.add_argument("--block-size", type=int, default=16, metavar="BS",
                    help="tokens per cache block: 8, 16, 32 or 64")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="sliding window of W positions (0: none)")
    ap.add_argument("--prefix", action="store_true",
                    help="decode a batch that shares a system prompt through prefix caching")
    ap.add_argument("--prefix-path", choices=("cascade", "plain"), default=None,
                    help="with --prefix or --config 5: pa_decode_shared_prefix (cascade, the "
                         "default) or pa_decode (plain)")
    ap.add_argument("--config", type=int, default=0, choices=(0, 2, 4, 5),
                    help="pa_decode alone on decode configuration 2, 4 or 5")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="cache format of the decode step (fp8: E4M3 with one scale per "
                         "cache, written from the same bf16 rows by pa_write_kv)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--probe-calibration", type=int, default=0, metavar="MIB",
                    help="end with 3 pa_read_probe passes over MIB MiB in address order: a "
                         "known byte count read with the decode kernel's load form, the "
                         "reference FETCH_SIZE is scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the decode path "
              f"has no cross-GPU step in this library", file=sys.stderr)
        sys.exit(2)
    if args.swap:
        return run_swap(args)
    if args.prefix:
        return run_prefix(args)
    if args.config:
        return run_config(args)
    T = args.chunk
    if not 1 <= T <= 16:
        sys.exit("--chunk must be in 1..16")
    if args.steps is None:
        args.steps = 100 if T == 1 else 50
    if args.warmup is None:
        args.warmup = 10 if T == 1 else 5
    if T * (args.steps + args.warmup) > workloads.CONFIG3_MAX_APPEND:
        sys.exit(f"chunk * (steps + warmup) must be <= {workloads.CONFIG3_MAX_APPEND} "
                 f"(pool headroom for appended tokens)")

    import torch
    import paged_kv_cache_421_amd as pk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    NL = args.layers

    _log("bench: generating the GQA batch-256 workload")
    w = workloads.config3()
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    bs = args.block_size
    if bs == 16:
        n_blocks, order = w.num_blocks, w.free_order
    else:        # the same token capacity in bs-token blocks, one more per sequence
        n_blocks = -(-w.num_blocks * 16 // bs) + B
        order = np.random.default_rng(3000 + bs).permutation(n_blocks).astype(np.int32)
    kvd = args.kv_dtype
    ks = vs = 1.0
    if kvd == "fp8":
        # one scale per cache: the largest magnitude of the rows written, / 448
        ks = float(np.float32(np.abs(workloads.bf16_bits_to_f32(w.k_rows)).max() / np.float32(448)))
        vs = float(np.float32(np.abs(workloads.bf16_bits_to_f32(w.v_rows)).max() / np.float32(448)))
    elem = 1 if kvd == "fp8" else 2
    desc = pk.CacheDesc(n_blocks, Hkv, D, kvd, ks, vs, block_size=bs)

    # ---- caches of layer 0 through the library's own write path; the other
    # layers get copies (distinct HBM, same contents)
    bm = pk.BlockManager(n_blocks, free_order=order, block_size=bs)
    per = []
    for s in range(B):
        bm.add_seq(s)
        sl, pair = bm.append_tokens(s, int(w.lens[s]))
        assert pair is None
        per.append(sl)
    slots = torch.from_numpy(np.concatenate(per)).to(dev)
    kc = [torch.zeros(desc.shape, dtype=desc.torch_dtype, device=dev) for _ in range(NL)]
    vc = [torch.zeros(desc.shape, dtype=desc.torch_dtype, device=dev) for _ in range(NL)]
    k_rows = torch.from_numpy(w.k_rows.view(np.int16)).to(dev).view(torch.bfloat16)
    v_rows = torch.from_numpy(w.v_rows.view(np.int16)).to(dev).view(torch.bfloat16)
    pk.write_kv(desc, kc[0], vc[0], k_rows, v_rows, slots)
    # the same rows into layer 1, 5 times back to back between one event
    # pair: the bulk rate of pa_write_kv
    torch.cuda.synchronize()
    bulk_ev = (HipEvent(), HipEvent())
    bulk_ev[0].record(stream)
    for _ in range(5):
        pk.write_kv(desc, kc[1 % NL], vc[1 % NL], k_rows, v_rows, slots, stream=stream)
    bulk_ev[1].record(stream)
    bulk_us = bulk_ev[0].elapsed_ms(bulk_ev[1]) * 1e3 / 5
    bulk_ev[0].destroy()
    bulk_ev[1].destroy()
    bulk_rows = int(slots.numel())
    for l in range(2, NL):
        kc[l].copy_(kc[0])
        vc[l].copy_(vc[0])
    del k_rows, v_rows, slots

    # ---- per-layer step inputs, resident in HBM: the new tokens' K/V rows
    # [B*T, Hkv, D] (sequence-major) and their queries
    rng = np.random.default_rng(1003)
    k_new, v_new, q = [], [], []
    for _ in range(NL):
        if T == 1:
            kn, vn, qq = workloads.config3_step(rng, B, Hq, Hkv, D)
        else:
            kn, vn, qq = workloads.config3_chunk_step(rng, T, B, Hq, Hkv, D)
            kn, vn = kn.reshape(B * T, Hkv, D), vn.reshape(B * T, Hkv, D)
        k_new.append(torch.from_numpy(kn.view(np.int16)).to(dev).view(torch.bfloat16))
        v_new.append(torch.from_numpy(vn.view(np.int16)).to(dev).view(torch.bfloat16))
        q.append(torch.from_numpy(qq.view(np.int16)).to(dev).view(torch.bfloat16))
    out = [torch.empty_like(q[0]) for _ in range(NL)]

    total = args.steps + args.warmup
    max_len_final = int(w.lens.max()) + T * total
    cap = -(-max_len_final // bs)
    workspace = pk.new_chunk_workspace(desc, B, Hq, T, max_len_final, dev)

    # ---- pinned host staging, triple-buffered against the running GPU
    # The block tables stay on the device; a step uploads the slot mapping,
    # the lengths and only the table entries of blocks it opened (a block
    # opens where a new token's position is a multiple of the block size),
    # as (row, column, block) triples that one scatter writes in place.
    NBUF = 3
    nmax = B * T
    h_i64 = [torch.empty(3 * nmax, dtype=torch.int64, pin_memory=True)      # slots | rows | cols
             for _ in range(NBUF)]
    h_i32 = [torch.empty(B + nmax, dtype=torch.int32, pin_memory=True)      # lens | blocks
             for _ in range(NBUF)]
    buf_ev = [None] * NBUF
    d_i64 = torch.empty(3 * nmax, dtype=torch.int64, device=dev)
    d_i32 = torch.empty(B + nmax, dtype=torch.int32, device=dev)
    d_slots = d_i64[:nmax]
    d_cl = d_i32[:B]
    slots_tb = np.empty((T, B), dtype=np.int64)
    ids = np.arange(B, dtype=np.int64)
    lens = w.lens.astype(np.int64).copy()
    d_bt = torch.from_numpy(bm.pack(ids, cap)[0]).to(dev)

    host_bm_s = []                           # block manager + table packing, per step

    def step(i, ev_pair):
        """One step; with ev_pair, HIP events around the decode of layer i mod
        layers (one timed decode per step, the layers in turn: each event
        delays the next dispatch by a few microseconds, so timing every call
        would slow the step it measures)."""
        b = i % NBUF
        if buf_ev[b] is not None:
            buf_ev[b].synchronize()          # the upload that last read buffer b is done
        th = time.perf_counter()
        hi, hj = h_i64[b].numpy(), h_i32[b].numpy()
        if T == 1:
            sl, pairs = bm.append_batch(ids, slots=hi[:nmax])
            assert len(pairs) == 0
        else:
            for t in range(T):                   # token t of every sequence
                sl, pairs = bm.append_batch(ids, slots=slots_tb[t])
                assert len(pairs) == 0
            hi[:nmax].reshape(B, T)[:] = slots_tb.T
        rows, cols, blocks = opened_table_entries(lens, hi[:nmax].reshape(B, T), bs)
        n = len(rows)
        hi[nmax:nmax + n] = rows
        hi[2 * nmax:2 * nmax + n] = cols
        hj[B:B + n] = blocks
        lens[:] += T
        hj[:B] = lens
        host_bm_s.append(time.perf_counter() - th)
        d_i64.copy_(h_i64[b], non_blocking=True)
        d_i32.copy_(h_i32[b], non_blocking=True)
        if n:
            d_bt[d_i64[nmax:nmax + n], d_i64[2 * nmax:2 * nmax + n]] = d_i32[B:B + n]
        ev = torch.cuda.Event()
        ev.record()
        buf_ev[b] = ev
        max_len = int(lens.max())
        for l in range(NL):
            pk.write_kv(desc, kc[l], vc[l], k_new[l], v_new[l], d_slots, stream=stream)
            timed_here = ev_pair is not None and l == i % NL
            if timed_here and T == 1:
                # the decode's own dispatch records the pair (no marker packet
                # between pa_write_kv and the decode)
                pk.time_next_call(ev_pair[0].h, ev_pair[1].h)
            elif timed_here:
                # chunks: markers around the call (launching them with
                # dispatch-recorded events slowed the whole chunk step)
                ev_pair[0].record(stream)
            if T == 1 and not args.window:
                pk.decode(desc, kc[l], vc[l], q[l], out[l], d_bt, d_cl, max_len,
                          float(w.scale), workspace, stream=stream)
            else:
                qq = q[l] if T > 1 else q[l].view(B, 1, Hq, D)
                oo = out[l] if T > 1 else out[l].view(B, 1, Hq, D)
                pk.decode_chunk(desc, kc[l], vc[l], qq, oo, d_bt, d_cl, max_len,
                                float(w.scale), workspace, stream=stream, window=args.window)
            if timed_here and T > 1:
                ev_pair[1].record(stream)
        if args.window:
            return _kv_bytes(np.minimum(lens, args.window + T - 1), Hkv, D, elem)
        return _kv_bytes(lens, Hkv, D, elem)

    _log(f"bench: {NL} layers x {n_blocks} blocks of {bs}, warmup {args.warmup}, steps {args.steps}")
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()

    evs = [(HipEvent(), HipEvent()) for _ in range(args.steps)]
    kv_per_call = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        kv_per_call.append(step(args.warmup + i, evs[i]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    assert torch.isfinite(out[0].float()).all(), "non-finite decode output"
    # the patched device tables and lengths are the manager's, entry for entry
    bt_ref, cl_ref = bm.pack(ids, cap)
    assert np.array_equal(d_bt.cpu().numpy(), bt_ref), "device block tables drifted"
    assert np.array_equal(d_cl.cpu().numpy(), cl_ref), "device lengths drifted"
    host_bm_us = statistics.mean(host_bm_s[args.warmup:]) * 1e6

    # ---- the other device steps of the path, each timed on its own after the
    # timed steps (back to back, one event pair around n calls): pa_write_kv of
    # one step's B*T rows, and pa_copy_blocks of 1024 pairs from blocks in use
    # into free ones (whole blocks of both caches) on the last layer's cache
    def timed_calls(fn, n=50):
        e0, e1 = HipEvent(), HipEvent()
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        us = e0.elapsed_ms(e1) * 1e3 / n
        e0.destroy()
        e1.destroy()
        return us

    step_us = timed_calls(lambda: pk.write_kv(desc, kc[0], vc[0], k_new[0], v_new[0], d_slots,
                                              stream=stream))
    bt_now, _ = bm.pack(ids, cap)
    used_blocks = np.unique(bt_now[bt_now >= 0])
    free_blocks = np.setdiff1d(np.arange(n_blocks), used_blocks)
    prng = np.random.default_rng(77)
    n_pairs = int(min(1024, len(free_blocks), len(used_blocks)))
    cp_pairs = torch.from_numpy(np.stack([prng.choice(used_blocks, n_pairs, replace=False),
                                          prng.choice(free_blocks, n_pairs, replace=False)],
                                         axis=1).astype(np.int32)).to(dev)
    copy_us = timed_calls(lambda: pk.copy_blocks(desc, kc[NL - 1], vc[NL - 1], cp_pairs,
                                                 stream=stream))
    blk_bytes = bs * Hkv * D * elem                    # one block of one cache
    row_bytes = Hkv * D * 2                            # one bf16 source row of K (or V)
    row_out = Hkv * D * elem                           # the same row in the cache
    bulk_b = 2 * bulk_rows * (row_bytes + row_out)     # K and V rows read, then written
    step_b = 2 * B * T * (row_bytes + row_out)
    copy_b = 2 * 2 * n_pairs * blk_bytes               # both caches, read and written
    path_steps = {
        "block_manager_host_us_per_step": round(host_bm_us, 1),
        "pa_write_kv_bulk": {"rows": bulk_rows, "us": round(bulk_us, 1),
                             "gbps": round(bulk_b / bulk_us / 1e3, 1),
                             "frac": round(bulk_b / bulk_us / 1e3 / HBM_PEAK_GBPS, 4)},
        "pa_write_kv_step": {"rows": B * T, "us": round(step_us, 2),
                             "gbps": round(step_b / step_us / 1e3, 1)},
        "pa_copy_blocks": {"pairs": n_pairs, "us": round(copy_us, 2),
                           "gbps": round(copy_b / copy_us / 1e3, 1),
                           "frac": round(copy_b / copy_us / 1e3 / HBM_PEAK_GBPS, 4)},
    }
    _log(f"bench: block manager {host_bm_us:.0f} us/step (host); pa_write_kv bulk "
         f"{bulk_rows} rows {bulk_us:.1f} us ({bulk_b / bulk_us / 1e3:.0f} GB/s), "
         f"{B * T} rows {step_us:.2f} us; pa_copy_blocks {n_pairs} pairs {copy_us:.2f} us "
         f"({copy_b / copy_us / 1e3:.0f} GB/s)")

    dec_ms = [a.elapsed_ms(b) for (a, b) in evs]
    for a, b in evs:
        a.destroy()
        b.destroy()
    mean_dec_s = statistics.mean(dec_ms) / 1e3
    mean_kv = statistics.mean(kv_per_call)
    achieved = mean_kv / mean_dec_s / 1e9
    steps_s = wall / args.steps
    traffic = None if (args.window or bs != 16) else _traffic_per_call(mean_kv, T, kvd)
    _log(f"bench: {'pa_decode' if T == 1 else 'pa_decode_chunk'} mean {mean_dec_s * 1e6:.1f} us "
         f"(median {np.median(dec_ms) * 1e3:.1f}, p10 "
         f"{np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f}), "
         f"{achieved:.0f} GB/s; step {steps_s * 1e3:.3f} ms")

    workload = ("gqa8b-bf16-b256: Llama-3-8B-shaped GQA decode layer, batch 256, "
                "32 query / 8 KV heads, head_dim 128, bf16 KV in 16-token shuffled "
                "blocks, lognormal context (median 512, sigma 0.8, [16, 4096])")
    if T > 1:
        workload = workload.replace("GQA decode layer", f"GQA layer, {T}-token chunk per sequence")
    if args.window:
        workload += f", sliding window of {args.window} positions"
    if bs != 16:
        workload = workload.replace("16-token shuffled blocks", f"{bs}-token shuffled blocks")
    if kvd == "fp8":
        workload = workload.replace("gqa8b-bf16-b256", "gqa8b-fp8-b256").replace(
            "bf16 KV", "fp8-e4m3 KV (one scale per cache; bf16 q and output)")
    res = {
        "metric": METRIC if T == 1 else METRIC_CHUNK,
        "value": round(B * T * NL * args.steps / wall, 1),
        "unit": "seqs/s" if T == 1 else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(steps_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kvd == "bf16" else "fp8-e4m3 KV, bf16 q/out, fp32 accumulation",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "global_batch": B,
            "chunk_tokens": T,
            "layers_per_step": NL,
            "step": ("block-manager append + upload of slots, lengths and opened table entries + "
                     "per layer pa_write_kv and " +
                     ("pa_decode" if T == 1 else "pa_decode_chunk")),
            "value_is": ("sequences decoded per second per attention layer" if T == 1 else
                         "query tokens per second per attention layer"),
            "mean_context_len": round(float(lens.mean()) - T * args.steps / 2, 1),
            "parallelism": "single GPU",
        },
        "kv_gbps_step": round(mean_kv * NL / steps_s / 1e9, 1),
        "path_steps": path_steps,
        "block_size": bs,
        "paged_utilisation": round(float(lens.sum()) / (bs * float(np.sum(-(-lens // bs)))), 4),
        "decode_us_mean": round(mean_dec_s * 1e6, 2),
        "decode_us_median": round(float(np.median(dec_ms)) * 1e3, 2),
        "decode_us_p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
        "decode_us_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
        "roofline": {
            "kernel": ("decode_stream_kernel (pa_decode_window)" if args.window else
                       "decode_stream_kernel (pa_decode: one persistent kernel)" if T == 1 else
                       "decode_stream_kernel (pa_decode_chunk: one persistent kernel per "
                       f"{16 // (Hq // Hkv)}-token pass)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else round(traffic / mean_dec_s / 1e9, 1),
        },
    }
    if T == 1 and not args.window and bs == 16 and kvd == "bf16":
        seq_gbps, rnd_gbps = stream_read_probe(dev, stream)
        res["stream_read_probe"] = {"in_order_gbps": seq_gbps, "random_4k_gbps": rnd_gbps,
                                    "decode_frac_of_random_4k": round(achieved / rnd_gbps, 4)}
        _log(f"bench: read probe {seq_gbps} GB/s in order, {rnd_gbps} GB/s random 4 KiB chunks")
    if args.probe_calibration > 0:
        n = args.probe_calibration << 20
        buf = torch.ones(n, dtype=torch.uint8, device=dev)
        sink = pk.read_probe(buf, stream=stream)
        for _ in range(3):
            pk.read_probe(buf, None, sink, stream=stream)
        torch.cuda.synchronize()
        del buf, sink
        _log(f"bench: probe calibration {n} bytes x 3 (+1 warm)")
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        _log(f"bench: copy calibration {n} bytes x 3")
    if bs != 16:
        rate, _, _ = chat_hit_rate(block_size=bs)
        res["chat_sim_hit_rate"] = round(rate, 4)
    if not args.no_cpu_baseline and not args.window and bs == 16:
        _log("bench: timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(w, T=T, fmt=kvd, k_scale=ks, v_scale=vs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
