"""pa_decode_noalloc (the decode entry point that allocates nothing: its
scratch is a static per-GPU array inside the library) against pa_decode
through the C ABI: bit-identical outputs on two calls in a row, the second
with a smaller batch, for the bf16 GQA path, an fp8 batch and the fp32
partition path, plus the host-side rejection of batches beyond the static
scratch (nothing is launched for those)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests._gpu_setup import GpuView, fill_sequential, to_device_rows

pk = pytest.importorskip("paged_kv_cache_421_amd")

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(seed, fmt, lens, Hq, Hkv, D):
    w = workloads.small_random(seed, len(lens), Hq, Hkv, D, fmt, 0,
                               lens=np.asarray(lens, np.int32))
    view = GpuView(w)
    fill_sequential(view)
    view.tables()
    return w, view


def _both(w, view):
    """pa_decode with its own workspace, then pa_decode_noalloc on the same
    inputs (through the C ABI); returns both outputs."""
    q = to_device_rows(w.q, w.q_fmt)
    ref = view.decode()
    out = torch.full_like(q, float("nan"))
    ml = int(max(1, int(view.cl_host.max())))
    st = pk.lib.pa_decode_noalloc(ctypes.byref(view.desc.c), ctypes.c_void_p(view.kc.data_ptr()),
                                  ctypes.c_void_p(view.vc.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                  pk.dtype_code(q.dtype), ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(view.bt.data_ptr()), view.bt.shape[1],
                                  ctypes.c_void_p(view.cl.data_ptr()), ml, w.B, w.Hq,
                                  float(w.scale),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, pk.lib.pa_last_error()
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("fmt,G,D", [("bf16", 4, 128), ("fp8", 8, 64), ("bf16", 16, 128),
                                     ("f32", 2, 64), ("bf16", 32, 64)])
def test_noalloc_matches_decode_on_two_calls_second_smaller(fmt, G, D):
    Hkv = 4 if fmt != "f32" else 2
    big = [0, 1, 17, 300, 2100, 5000, 640, 33, 1200, 16, 9000, 700] * 3
    small = [5, 0, 260, 1800, 31]
    for seed, lens in ((1400 + G, big), (1500 + G, small)):
        w, view = _case(seed, fmt, lens, G * Hkv, Hkv, D)
        _say(f"noalloc {fmt} G={G} D={D} B={w.B} max_len={max(lens)}")
        ref, out = _both(w, view)
        if fmt == "f32":
            assert torch.equal(ref.view(torch.int32), out.view(torch.int32))
        else:
            assert torch.equal(ref.view(torch.int16), out.view(torch.int16))


def test_noalloc_gqa_batch256_then_a_smaller_batch():
    """The decode benchmark's batch (the arrival counters of 2048 segments,
    pieces merged across waves), then 40 sequences: the counters the first
    call used are zero again, and the second call's output is pa_decode's."""
    w = workloads.config3()
    view = GpuView(w)
    fill_sequential(view)
    view.tables()
    _say("noalloc config 3")
    ref, out = _both(w, view)
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    lens = np.random.default_rng(1601).integers(1, 3000, 40)
    w2, view2 = _case(1602, "bf16", lens, 32, 8, 128)
    _say("noalloc 40 sequences")
    ref2, out2 = _both(w2, view2)
    assert torch.equal(ref2.view(torch.int16), out2.view(torch.int16))


def test_noalloc_rejects_batches_beyond_the_static_scratch():
    """Host-side checks only: no kernel is launched for these."""
    d = pk.CacheDesc(4, 8, 128, "bf16")
    one, al = ctypes.c_void_p(256), ctypes.c_void_p(256)
    # 10000 sequences x 8 KV heads > 65536 counters
    st = pk.lib.pa_decode_noalloc(ctypes.byref(d.c), one, one, al, 1, al, one, 4, one, 64,
                                  10000, 32, 1.0, None)
    assert st == -6 and b"counters" in pk.lib.pa_last_error()
    # fp32 partition path: 4096 x 32 heads x 8 partitions x 130 floats > 24 MiB
    d32 = pk.CacheDesc(4, 8, 128, "f32")
    st = pk.lib.pa_decode_noalloc(ctypes.byref(d32.c), one, one, al, 0, al, one, 256, one, 4096,
                                  4096, 32, 1.0, None)
    assert st == -6 and b"static scratch" in pk.lib.pa_last_error()
