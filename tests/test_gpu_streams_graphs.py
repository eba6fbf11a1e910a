"""The path on a stream other than the default one, and captured in a HIP
graph.  The library launches only kernels on the stream it is given (no
allocation, no memset, no synchronisation) and leaves the decode workspace's
arrival counters at zero after every call, so a captured pa_write_kv +
pa_decode replays correctly.  Each replay is checked against the eager result
on the same inputs, with eager work (new queries written into the captured
buffer) between the replays."""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu_setup import GpuView, fill_sequential, to_device_rows

pk = pytest.importorskip("paged_kv_cache_421_amd")

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _view(seed):
    lens = np.array([1, 17, 300, 640, 33, 2100, 900, 5], dtype=np.int32)
    w = workloads.small_random(seed, len(lens), 16, 4, 128, "bf16", 0, lens=lens)
    view = GpuView(w)
    fill_sequential(view)
    view.tables(cap=int(lens.max()) // 16 + 2)
    return w, view


def test_decode_on_a_side_stream_matches_default_stream():
    w, view = _view(1200)
    _say("side stream: decode on the default stream, then on a new stream")
    a = view.decode().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b = view.decode()
    side.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_on_an_explicit_stream_without_a_workspace():
    """stream= given, no workspace, and that stream not current: the call's
    workspace is made and zero-filled on that stream, so the fill precedes the
    kernel there and the memory is not reused by the current stream while the
    kernel may still run.  The current stream is kept busy with unrelated work
    meanwhile; the output equals the default-stream result bit for bit."""
    w, view = _view(1203)
    a = view.decode().clone()
    torch.cuda.synchronize()
    qd = to_device_rows(w.q, w.q_fmt)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        out = torch.empty_like(qd)
        # memory freed on the current stream, so a workspace allocated there
        # would likely be this block, still being written below
        junk = torch.full((1 << 22,), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
        del junk
        busy = torch.full((1 << 22,), 0x01010101, dtype=torch.int32, device="cuda")
        pk.decode(view.desc, view.kc, view.vc, qd, out, view.bt, view.cl,
                  int(view.cl_host.max()), float(w.scale), stream=side)
        busy.add_(1)
        outs.append(out)
    side.synchronize()
    torch.cuda.synchronize()
    for b in outs:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.skipif(
    pytest.importorskip("paged_kv_cache_421_amd._lib").LIB_PATH.endswith("_debug.so"),
    reason="the PA_DEBUG library copies device arrays back before each launch (a synchronising "
           "copy), which graph capture does not allow")
def test_write_and_decode_replay_from_a_captured_graph():
    w, view = _view(1201)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    rng = np.random.default_rng(1202)
    max_len = int(view.cl_host.max()) + 1
    # one new token per sequence: its slot from the manager, its rows drawn here
    slots = np.array([view.bm.append_slot(s)[0] for s in range(B)], dtype=np.int64)
    view.tables(cap=view.bt_host.shape[1])
    k_new = to_device_rows(workloads.f32_to_bf16_bits(
        rng.standard_normal((B, Hkv, D)).astype(np.float32)), "bf16")
    v_new = to_device_rows(workloads.f32_to_bf16_bits(
        rng.standard_normal((B, Hkv, D)).astype(np.float32)), "bf16")
    d_slots = torch.from_numpy(slots).cuda()
    q = to_device_rows(w.q, w.q_fmt)
    out = torch.empty_like(q)
    ws = pk.new_decode_workspace(view.desc, B, Hq, max_len)

    def step(stream=None):
        pk.write_kv(view.desc, view.kc, view.vc, k_new, v_new, d_slots, stream=stream)
        pk.decode(view.desc, view.kc, view.vc, q, out, view.bt, view.cl, max_len,
                  float(w.scale), ws, stream=stream)

    _say("graph: warm-up on a side stream, capture, then 3 replays against eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        q.copy_(to_device_rows(workloads.f32_to_bf16_bits(
            rng.standard_normal((B, Hq, D)).astype(np.float32)), "bf16"))
        step()                                   # eager, on the current stream
        torch.cuda.synchronize()
        eager = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert int(ws[:B * Hkv * 4].count_nonzero()) == 0, "arrival counters not reset"
        _say(f"  replay {i}: bit-identical to eager")


class _Ev:
    """A raw HIP event on the runtime torch loaded (ctypes)."""
    _hip = None

    def __init__(self):
        import ctypes
        if _Ev._hip is None:
            _Ev._hip = ctypes.CDLL("libamdhip64.so.7")
        self._c = ctypes
        self.h = ctypes.c_void_p()
        assert _Ev._hip.hipEventCreate(ctypes.byref(self.h)) == 0

    def ms_to(self, other):
        ms = self._c.c_float()
        assert _Ev._hip.hipEventSynchronize(other.h) == 0
        assert _Ev._hip.hipEventElapsedTime(self._c.byref(ms), self.h, other.h) == 0
        return ms.value

    def destroy(self):
        assert _Ev._hip.hipEventDestroy(self.h) == 0


@pytest.mark.parametrize("T,window", [(1, 0), (4, 0), (1, 200)])
def test_time_next_call_records_the_decode_kernels(T, window):
    """pa_time_next_call: the next decode call's own dispatches record the
    events; the output is the untimed call's, bit for bit; the request is
    used once (a later call leaves the events as they were)."""
    w, view = _view(1203 + T)
    q = workloads.chunk_queries(np.random.default_rng(7), w.B, T, w.Hq, w.D, "bf16")
    untimed = view.decode_chunk(q, window=window).clone()
    e0, e1 = _Ev(), _Ev()
    pk.time_next_call(e0.h, e1.h)
    timed = view.decode_chunk(q, window=window).clone()
    ms = e0.ms_to(e1)
    again = view.decode_chunk(q, window=window)
    torch.cuda.synchronize()
    _say(f"time_next_call T={T} W={window}: {ms * 1e3:.1f} us")
    assert 0.0 < ms < 1000.0
    assert e0.ms_to(e1) == ms                      # the later call did not touch them
    assert torch.equal(timed.view(torch.int16), untimed.view(torch.int16))
    assert torch.equal(again.view(torch.int16), untimed.view(torch.int16))
    e0.destroy()
    e1.destroy()
