"""Layers recorded in one HIP graph give bitwise the eager results.

* A stack of layers of the 30-layer decode shape (RMSNorm before the router,
  residual after the combine) recorded as one graph and replayed, with the
  program's own eager work between replays: every replay equals the eager
  layer-by-layer run bitwise (the routing is on the device, so the graph
  holds no host step).
* The large-batch path runs the MFMA segments on a second stream forked from
  the caller's: recorded in a graph it still equals the eager run, and the
  eager run equals the in-order run (stage events requested) bitwise, since
  the two streams write disjoint routes.
"""
import numpy as np
import pytest
import torch

import mixture_experts_decode_gemv_amd as moe
import workload as wl
from gpu_util import dev, make_device_layer, note

pytestmark = pytest.mark.gpu

STACK_LAYERS = 3
STACK_SPEC = wl.STACK
MIXED = wl.LayerSpec(E=8, top_k=2, H=384, I=384)


def _eager(layers, x, T, flags, ws, stream):
    h = x.clone()
    with torch.cuda.stream(stream):
        for L in layers:
            moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
    stream.synchronize()
    return h.cpu().numpy()


def _graph_check(layers, x0, T, flags, replays=3):
    stream = torch.cuda.Stream(dev())
    ws = layers[0].workspace(T, stream)
    ref = _eager(layers, x0, T, flags, ws, stream)
    h = x0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for L in layers:  # warm-up outside the capture
            moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
    stream.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for L in layers:
            moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
    for i in range(replays):
        note("graph replay %d, T=%d, flags=%d" % (i, T, flags))
        with torch.cuda.stream(stream):
            h.copy_(x0)
            graph.replay()
        stream.synchronize()
        got = h.cpu().numpy()
        assert np.array_equal(got, ref), "replay %d differs from the eager run" % i
        # eager work of the program between replays
        again = _eager(layers, x0, T, flags, ws, stream)
        assert np.array_equal(again, ref)
    return ref


@pytest.fixture(scope="module")
def stack_layers():
    note("generating %d stack layers" % STACK_LAYERS)
    return [moe.DeviceLayer(wl.make_layer(STACK_SPEC, layer=l), device=dev()) for l in range(STACK_LAYERS)]


@pytest.mark.parametrize("T", [1, 4])
def test_stack_graph_equals_eager_bitwise(stack_layers, T):
    note("stack graph T=%d" % T)
    x0 = torch.from_numpy(wl.make_x(T, STACK_SPEC.H, draw=21)).to(dev())
    out = _graph_check(stack_layers, x0, T, moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("T", [64, 300], ids=["in_order", "forked"])
def test_mfma_layer_graph_equals_eager_bitwise(T):
    note("mfma layer graph T=%d" % T)
    bias = np.zeros(MIXED.E, np.float32)
    bias[:3] = 2.0  # hot experts: segments well above the MFMA threshold
    w, layer, olayer = make_device_layer(MIXED, bias)
    x0 = torch.from_numpy(wl.make_x(T, MIXED.H, draw=22)).to(dev())
    ref = _graph_check([layer], x0, T, 0)
    # in-order run (stage events requested) equals the default run bitwise
    stream = torch.cuda.Stream(dev())
    ws = layer.workspace(T, stream)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_N_STAGES + 1)]
    for e in evs:
        e.record(stream)
    out = torch.empty_like(x0)
    with torch.cuda.stream(stream):
        moe.moe_layer_fwd_events(layer.struct, x0, T, out, 0, ws, ws.numel(), stream, [e.cuda_event for e in evs])
    stream.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_forked_calls_from_two_threads_on_two_streams():
    """Two host threads, each on its own stream and workspace, call the
    large-batch path (MFMA segments on a side stream forked from the caller's)
    many times at once, one of them also while capturing a graph: every
    output equals the in-order run bitwise.  Each caller stream has its own
    side stream and events, and one call's fork/join sequence is enqueued
    without interleaving with the other thread's."""
    import threading

    T = 300
    bias = np.zeros(MIXED.E, np.float32)
    bias[:3] = 2.0
    w, layer, olayer = make_device_layer(MIXED, bias)
    xs = [torch.from_numpy(wl.make_x(T, MIXED.H, draw=40 + i)).to(dev()) for i in range(2)]
    refs = []
    for i in range(2):  # in-order reference (stage events requested)
        s = torch.cuda.Stream(dev())
        ws = layer.workspace(T, s)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_N_STAGES + 1)]
        for e in evs:
            e.record(s)
        out = torch.empty_like(xs[i])
        with torch.cuda.stream(s):
            moe.moe_layer_fwd_events(layer.struct, xs[i], T, out, 0, ws, ws.numel(), s, [e.cuda_event for e in evs])
        s.synchronize()
        refs.append(out.cpu().numpy())
    note("two threads, T=%d" % T)
    streams = [torch.cuda.Stream(dev()) for _ in range(2)]
    wss = [layer.workspace(T, s) for s in streams]
    outs = [[torch.empty_like(xs[i]) for _ in range(8)] for i in range(2)]
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(2)

    def worker(i):
        try:
            torch.cuda.set_device(dev())
            s = streams[i]
            barrier.wait()
            with torch.cuda.stream(s):
                for o in outs[i]:
                    moe.moe_layer_fwd(layer.struct, xs[i], T, o, 0, wss[i], wss[i].numel(), s)
            s.synchronize()
        except Exception as exc:  # noqa: BLE001 - reported below
            errors.append(exc)

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for i in range(2):
        for o in outs[i]:
            assert np.array_equal(o.cpu().numpy(), refs[i])
