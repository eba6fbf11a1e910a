"""Torch-facing wrappers of the C ABI: argument marshalling only.

Device tensors must be contiguous and on the current HIP device; calls are
asynchronous on the current torch stream unless ``stream`` is given.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib as _libmod
from ._lib import CacheDescC, PagedKVError, check, lib

BLOCK_SIZE = 16
PARTITION_TOKENS = 512
MAX_CHUNK = 16

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3,
           torch.float8_e4m3fn: PA_FP8_E4M3}
_NAMES = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}


def dtype_code(x) -> int:
    """pa_dtype of a torch dtype or of "f32" / "bf16" / "fp8"."""
    if isinstance(x, str):
        return _NAMES[x]
    return _DTYPES[x]


class CacheDesc:
    """pa_cache_desc: shape and format of a pair of K/V caches, each
    ``[num_blocks, num_kv_heads, block_size, head_dim]`` (block_size 8, 16,
    32 or 64; 16 by default)."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype,
                 k_scale: float = 1.0, v_scale: float = 1.0, block_size: int = BLOCK_SIZE):
        self.c = CacheDescC(int(num_blocks), int(block_size), int(num_kv_heads), int(head_dim),
                            dtype_code(dtype), float(k_scale), float(v_scale))

    @property
    def block_size(self) -> int:
        return int(self.c.block_size)

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        """Shape of each of the K and V caches."""
        return (self.c.num_blocks, self.c.num_kv_heads, self.c.block_size, self.c.head_dim)

    @property
    def torch_dtype(self):
        return {PA_F32: torch.float32, PA_BF16: torch.bfloat16,
                PA_FP8_E4M3: torch.uint8}[self.c.cache_dtype]

    def cache_bytes(self) -> int:
        return int(lib.pa_cache_bytes(ctypes.byref(self.c)))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str) -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_CACHE_DTYPES = {PA_F32: (torch.float32, torch.int32), PA_BF16: (torch.bfloat16, torch.int16),
                 PA_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}


def _caches(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor):
    """Pointers of a K and a V cache that have the dtype and byte size
    ``desc`` describes, so the kernels' addresses stay inside them.  Both are
    checked before the device test, so a mismatch is reported without
    touching the GPU."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype not in _CACHE_DTYPES[desc.c.cache_dtype]:
            raise ValueError(f"{name}: dtype {t.dtype} does not match the descriptor's cache "
                             f"format {desc.torch_dtype}")
        nbytes = t.numel() * t.element_size()
        if nbytes != desc.cache_bytes():
            raise ValueError(f"{name}: {nbytes} bytes, the descriptor describes "
                             f"{desc.cache_bytes()} ({desc.shape})")
    return _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache")


def _queries(desc: CacheDesc, q: torch.Tensor, out: torch.Tensor, ndim: int) -> None:
    """q and out: [B, Hq, D] (decode) or [B, T, Hq, D] (chunks), D = the
    cache's head_dim, Hq a multiple of its KV heads."""
    if q.dim() != ndim:
        raise ValueError(f"q must have {ndim} dimensions, got {tuple(q.shape)}")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if q.shape[-1] != desc.c.head_dim:
        raise ValueError(f"q head_dim {q.shape[-1]} != the cache's {desc.c.head_dim}")
    if q.shape[-2] % desc.c.num_kv_heads != 0:
        raise ValueError(f"{q.shape[-2]} query heads are not a multiple of "
                         f"{desc.c.num_kv_heads} KV heads")


def _tables(block_tables: torch.Tensor, context_lens: torch.Tensor, B: int) -> None:
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")


def _call_workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A zero-filled workspace for one call on ``stream``: allocated from
    that stream's pool of the caching allocator and filled on that stream, so
    the fill is ordered before the call, and the memory, released when the
    tensor dies, is handed out again only to work ordered after the call."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    with torch.cuda.stream(s):
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    decode_workspace_init(ws, stream=s)
    return ws


def write_kv(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
             k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
             stream=None) -> None:
    """pa_write_kv: rows k[i], v[i] ([Hkv, D]) into slot slot_mapping[i]."""
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must match")
    T = k.shape[0]
    if tuple(k.shape[1:]) != (desc.c.num_kv_heads, desc.c.head_dim) or slot_mapping.numel() != T:
        raise ValueError("k/v must be [T, Hkv, D] and slot_mapping [T]")
    kc, vc = _caches(desc, k_cache, v_cache)
    check(lib.pa_write_kv(ctypes.byref(desc.c), kc, vc, _dev(k, "k"), _dev(v, "v"),
                          dtype_code(k.dtype), _dev(slot_mapping, "slot_mapping"), T,
                          _stream(stream)))


def copy_blocks(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                pairs: torch.Tensor, stream=None) -> None:
    """pa_copy_blocks: pairs int32 [n, 2] of (src, dst) blocks."""
    if pairs.dtype != torch.int32:
        raise ValueError("pairs must be int32")
    kc, vc = _caches(desc, k_cache, v_cache)
    n = pairs.numel() // 2
    if n == 0:
        return
    check(lib.pa_copy_blocks(ctypes.byref(desc.c), kc, vc, _dev(pairs, "pairs"), n,
                             _stream(stream)))


def decode_workspace_bytes(desc: CacheDesc, num_seqs: int, num_q_heads: int,
                           max_context_len: int) -> int:
    """pa_decode_workspace_bytes: scratch bytes pa_decode needs for this shape."""
    return int(lib.pa_decode_workspace_bytes(ctypes.byref(desc.c), int(num_seqs),
                                             int(num_q_heads), int(max_context_len)))


def decode_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """pa_decode_workspace_init: zero-fill a workspace before its first use."""
    check(lib.pa_decode_workspace_init(_dev(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def new_decode_workspace(desc: CacheDesc, num_seqs: int, num_q_heads: int,
                         max_context_len: int, device=None, stream=None) -> torch.Tensor:
    """A uint8 device tensor of pa_decode_workspace_bytes bytes (at least one
    byte), zero-filled on ``stream`` (default: the current stream), ready for
    pa_decode on that stream."""
    n = decode_workspace_bytes(desc, num_seqs, num_q_heads, max_context_len)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device or "cuda")
    decode_workspace_init(ws, stream=stream)
    return ws


def decode(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
           out: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
           max_context_len: int, scale: float, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """pa_decode: out[s, h] = softmax(scale q[s,h] K_s^T) V_s through block tables.

    ``workspace`` is a zero-filled device buffer of at least
    ``decode_workspace_bytes`` bytes (``new_decode_workspace``), reusable by
    later calls on the same stream; if None, one is made for this call on
    ``stream``."""
    _queries(desc, q, out, 3)
    B, Hq, D = q.shape
    _tables(block_tables, context_lens, B)
    kc, vc = _caches(desc, k_cache, v_cache)
    if workspace is None:
        workspace = _call_workspace(decode_workspace_bytes(desc, B, Hq, max_context_len),
                                    q.device, stream)
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.pa_decode(ctypes.byref(desc.c), kc, vc,
                        _dev(q, "q"), dtype_code(q.dtype), _dev(out, "out"),
                        _dev(block_tables, "block_tables"), block_tables.shape[1],
                        _dev(context_lens, "context_lens"), int(max_context_len), B, Hq,
                        float(scale), ws_ptr, ws_bytes, _stream(stream)))
    return out


def decode_noalloc(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, max_context_len: int, scale: float,
                   stream=None) -> torch.Tensor:
    """pa_decode_noalloc: pa_decode with the library's static per-GPU scratch
    instead of a workspace (nothing is allocated; calls that may overlap on
    one GPU race)."""
    _queries(desc, q, out, 3)
    B, Hq, D = q.shape
    _tables(block_tables, context_lens, B)
    kc, vc = _caches(desc, k_cache, v_cache)
    check(lib.pa_decode_noalloc(ctypes.byref(desc.c), kc, vc, _dev(q, "q"), dtype_code(q.dtype),
                                _dev(out, "out"), _dev(block_tables, "block_tables"),
                                block_tables.shape[1], _dev(context_lens, "context_lens"),
                                int(max_context_len), B, Hq, float(scale), _stream(stream)))
    return out


def chunk_workspace_bytes(desc: CacheDesc, num_seqs: int, num_q_heads: int, chunk_len: int,
                          max_context_len: int) -> int:
    """pa_decode_chunk_workspace_bytes: scratch bytes pa_decode_chunk needs."""
    return int(lib.pa_decode_chunk_workspace_bytes(ctypes.byref(desc.c), int(num_seqs),
                                                   int(num_q_heads), int(chunk_len),
                                                   int(max_context_len)))


def new_chunk_workspace(desc: CacheDesc, num_seqs: int, num_q_heads: int, chunk_len: int,
                        max_context_len: int, device=None, stream=None) -> torch.Tensor:
    """A uint8 device tensor sized for pa_decode_chunk, zero-filled on
    ``stream`` (default: the current stream)."""
    n = chunk_workspace_bytes(desc, num_seqs, num_q_heads, chunk_len, max_context_len)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device or "cuda")
    decode_workspace_init(ws, stream=stream)
    return ws


def decode_chunk(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, max_context_len: int, scale: float,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 window: int = 0) -> torch.Tensor:
    """pa_decode_chunk (pa_decode_window when ``window`` > 0): attention of
    T = q.shape[1] new tokens per sequence, causal inside the chunk; q and
    out are [B, T, Hq, D]."""
    _queries(desc, q, out, 4)
    B, T, Hq, D = q.shape
    _tables(block_tables, context_lens, B)
    kc, vc = _caches(desc, k_cache, v_cache)
    if workspace is None:
        workspace = _call_workspace(chunk_workspace_bytes(desc, B, Hq, T, max_context_len),
                                    q.device, stream)
    if window:
        check(lib.pa_decode_window(ctypes.byref(desc.c), kc, vc, _dev(q, "q"), dtype_code(q.dtype),
                                   _dev(out, "out"), T, int(window),
                                   _dev(block_tables, "block_tables"), block_tables.shape[1],
                                   _dev(context_lens, "context_lens"), int(max_context_len), B,
                                   Hq, float(scale), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
        return out
    check(lib.pa_decode_chunk(ctypes.byref(desc.c), kc, vc, _dev(q, "q"), dtype_code(q.dtype),
                              _dev(out, "out"), T, _dev(block_tables, "block_tables"),
                              block_tables.shape[1], _dev(context_lens, "context_lens"),
                              int(max_context_len), B, Hq, float(scale),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def shared_prefix_workspace_bytes(desc: CacheDesc, num_seqs: int, num_q_heads: int,
                                  max_blocks_per_seq: int, max_context_len: int) -> int:
    return int(lib.pa_decode_shared_prefix_workspace_bytes(
        ctypes.byref(desc.c), int(num_seqs), int(num_q_heads), int(max_blocks_per_seq),
        int(max_context_len)))


def new_shared_prefix_workspace(desc: CacheDesc, num_seqs: int, num_q_heads: int,
                                max_blocks_per_seq: int, max_context_len: int,
                                device=None, stream=None) -> torch.Tensor:
    """A uint8 device tensor sized for pa_decode_shared_prefix, zero-filled on
    ``stream`` (default: the current stream)."""
    n = shared_prefix_workspace_bytes(desc, num_seqs, num_q_heads, max_blocks_per_seq,
                                      max_context_len)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device or "cuda")
    decode_workspace_init(ws, stream=stream)
    return ws


def decode_shared_prefix(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, max_context_len: int, scale: float,
                         groups, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """pa_decode_shared_prefix: pa_decode, with the shared prefix of each
    group (host int32 [k, 3] of (first, count, shared blocks)) attended once."""
    _queries(desc, q, out, 3)
    B, Hq, D = q.shape
    _tables(block_tables, context_lens, B)
    kc, vc = _caches(desc, k_cache, v_cache)
    grp = np.ascontiguousarray(groups, dtype=np.int32).reshape(-1, 3)
    if workspace is None:
        workspace = _call_workspace(
            shared_prefix_workspace_bytes(desc, B, Hq, block_tables.shape[1], max_context_len),
            q.device, stream)
    check(lib.pa_decode_shared_prefix(
        ctypes.byref(desc.c), kc, vc, _dev(q, "q"),
        dtype_code(q.dtype), _dev(out, "out"), _dev(block_tables, "block_tables"),
        block_tables.shape[1], _dev(context_lens, "context_lens"), int(max_context_len), B, Hq,
        float(scale), _ptr(grp), len(grp), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def time_next_call(start_event, stop_event) -> None:
    """pa_time_next_call: the next decode call on this thread records these
    HIP events (raw hipEvent_t handles, or None) from its own kernel
    dispatches."""
    check(lib.pa_time_next_call(start_event, stop_event))


def read_probe(buf: torch.Tensor, chunk_order: Optional[torch.Tensor] = None,
               sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_read_probe: stream ``buf`` (device) in 4 KiB chunks, in order or in
    ``chunk_order`` (int32 device tensor).  Returns the sink tensor."""
    cus = torch.cuda.get_device_properties(buf.device).multi_processor_count
    if sink is None:
        sink = torch.empty(lib.pa_read_probe_sink_bytes(cus) // 4, dtype=torch.int32,
                           device=buf.device)
    order = ctypes.c_void_p(0) if chunk_order is None else _dev(chunk_order, "chunk_order")
    check(lib.pa_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(), order,
                            _dev(sink, "sink"), cus, _stream(stream)))
    return sink


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _pool(t: torch.Tensor, name: str) -> ctypes.c_void_p:
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def swap_blocks(desc: CacheDesc, src_k: torch.Tensor, src_v: torch.Tensor,
                dst_k: torch.Tensor, dst_v: torch.Tensor, pairs: torch.Tensor,
                stream=None) -> None:
    """pa_swap_blocks: whole-block copies dst[d] = src[s] for each (s, d) of
    ``pairs`` (int32 [n, 2]); pools and pairs are device tensors or pinned
    host tensors (``pin_memory=True``)."""
    if pairs.dtype != torch.int32:
        raise ValueError("pairs must be int32")
    n = pairs.numel() // 2
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape:
        raise ValueError("K and V pools must have the same shape")
    for name, t in (("src", src_k), ("dst", dst_k)):
        if t.dtype not in _CACHE_DTYPES[desc.c.cache_dtype] or t.dim() != 4 or \
                tuple(t.shape[1:]) != desc.shape[1:]:
            raise ValueError(f"{name} pools must be [blocks, {desc.shape[1]}, {desc.shape[2]}, "
                             f"{desc.shape[3]}] of the descriptor's cache format")
    check(lib.pa_swap_blocks(ctypes.byref(desc.c), _pool(src_k, "src_k"), _pool(src_v, "src_v"),
                             _pool(dst_k, "dst_k"), _pool(dst_v, "dst_v"),
                             _pool(pairs, "pairs"), n, _stream(stream)))


class BlockManager:
    """Host block manager (pa_bm_*): FIFO free pools (device, and host for
    swapping), refcounts, copy-on-write."""

    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None,
                 num_host_blocks: int = 0, host_free_order: Optional[Sequence[int]] = None,
                 block_size: int = BLOCK_SIZE):
        self._lib = _libmod.host_lib   # kept alive for __del__ at interpreter exit
        self._order = self._horder = None
        ptr = hptr = ctypes.c_void_p(0)
        if free_order is not None:
            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            ptr = _ptr(self._order)
        if host_free_order is not None:
            self._horder = np.ascontiguousarray(host_free_order, dtype=np.int32)
            hptr = _ptr(self._horder)
        h = self._lib.pa_bm_create_ex(int(num_blocks), int(block_size), ptr, int(num_host_blocks), hptr)
        if not h:
            raise PagedKVError(-1, self._lib.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.num_host_blocks = int(num_host_blocks)
        self.block_size = int(block_size)

    def _check(self, status: int) -> None:
        check(status, self._lib)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def _move(self, fn, seq_ids, cap: int) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        pairs = np.empty((max(cap, 1), 2), dtype=np.int32)
        n = ctypes.c_int32()
        self._check(fn(self._h, _ptr(ids), len(ids), _ptr(pairs), cap, ctypes.byref(n)))
        return pairs[:n.value].copy()

    def swap_out(self, seq_ids) -> np.ndarray:
        """pa_bm_swap_out: (device block, host block) pairs, int32 [k, 2]."""
        return self._move(self._lib.pa_bm_swap_out, seq_ids, self.num_host_blocks)

    def swap_in(self, seq_ids) -> np.ndarray:
        """pa_bm_swap_in: (host block, device block) pairs, int32 [k, 2]."""
        return self._move(self._lib.pa_bm_swap_in, seq_ids, self.num_blocks)

    def enable_prefix_caching(self) -> None:
        self._check(self._lib.pa_bm_enable_prefix_caching(self._h))

    def add_seq_prompt(self, seq: int, tokens):
        """pa_bm_add_seq_prompt: (slots int64 [n], num_cached)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(len(toks), 1), dtype=np.int64)
        nc = ctypes.c_int32()
        self._check(self._lib.pa_bm_add_seq_prompt(self._h, int(seq), _ptr(toks), len(toks), _ptr(slots),
                                       ctypes.byref(nc)))
        return slots[:len(toks)], nc.value

    def append_token_ids(self, seq: int, tokens):
        """pa_bm_append_token_ids: (slots, copy pair or None)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(len(toks), 1), dtype=np.int64)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_append_token_ids(self._h, int(seq), _ptr(toks), len(toks), _ptr(slots),
                                         ctypes.byref(src), ctypes.byref(dst)))
        return slots[:len(toks)], (None if src.value < 0 else (src.value, dst.value))

    def cache_stats(self):
        """(queried blocks, hit blocks, registered blocks, evictable blocks)."""
        q, h = ctypes.c_int64(), ctypes.c_int64()
        r, e = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_cache_stats(self._h, ctypes.byref(q), ctypes.byref(h), ctypes.byref(r),
                                    ctypes.byref(e)))
        return q.value, h.value, r.value, e.value

    def shared_prefix_groups(self, seq_ids) -> np.ndarray:
        """pa_bm_shared_prefix_groups: int32 [k, 3] of (first index, count, shared blocks)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        cap = max(len(ids) // 2, 1)
        out = np.empty((cap, 3), dtype=np.int32)
        n = ctypes.c_int32()
        self._check(self._lib.pa_bm_shared_prefix_groups(self._h, _ptr(ids), len(ids), _ptr(out), cap,
                                             ctypes.byref(n)))
        return out[:n.value].copy()

    def num_free_host(self) -> int:
        return int(self._lib.pa_bm_num_free_host(self._h))

    def host_refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_host_refcount(self._h, int(block)))

    def is_swapped(self, seq: int) -> bool:
        v = ctypes.c_int32()
        self._check(self._lib.pa_bm_is_swapped(self._h, int(seq), ctypes.byref(v)))
        return bool(v.value)

    def add_seq(self, seq: int) -> None:
        self._check(self._lib.pa_bm_add_seq(self._h, int(seq)))

    def fork(self, parent: int, child: int) -> None:
        self._check(self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def append_slot(self, seq: int):
        slot = ctypes.c_int64()
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_append_slot(self._h, int(seq), ctypes.byref(slot), ctypes.byref(src),
                                    ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_tokens(self, seq: int, n: int):
        slots = np.empty(max(int(n), 1), dtype=np.int64)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_append_tokens(self._h, int(seq), int(n), _ptr(slots), ctypes.byref(src),
                                      ctypes.byref(dst)))
        return slots[:int(n)], (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seq_ids: np.ndarray, slots: Optional[np.ndarray] = None,
                     pairs: Optional[np.ndarray] = None):
        """One token for each sequence; returns (slots int64 [n], pairs int32 [k, 2]).
        ``slots``/``pairs`` may be preallocated (e.g. pinned) host arrays."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        if slots is None:
            slots = np.empty(n, dtype=np.int64)
        if pairs is None:
            pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32()
        self._check(self._lib.pa_bm_append_batch(self._h, _ptr(ids), n, _ptr(slots), _ptr(pairs),
                                     ctypes.byref(npairs)))
        return slots[:n], pairs[:npairs.value]

    def free_seq(self, seq: int) -> None:
        self._check(self._lib.pa_bm_free_seq(self._h, int(seq)))

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, int(block)))

    def length(self, seq: int) -> int:
        n = ctypes.c_int32()
        self._check(self._lib.pa_bm_length(self._h, int(seq), ctypes.byref(n)))
        return n.value

    def pack(self, seq_ids, cap: int, block_tables: Optional[np.ndarray] = None,
             context_lens: Optional[np.ndarray] = None):
        """block_tables int32 [n, cap] (pad -1), context_lens int32 [n]."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        if block_tables is None:
            block_tables = np.empty((n, cap), dtype=np.int32)
        if context_lens is None:
            context_lens = np.empty(n, dtype=np.int32)
        self._check(self._lib.pa_bm_pack(self._h, _ptr(ids), n, _ptr(block_tables), int(cap),
                             _ptr(context_lens)))
        return block_tables, context_lens
