"""Expert-usage telemetry (moe_expert_usage): per-expert route counts added
into caller-owned uint64 counters, exactly, across layer steps, inside a
recorded graph, and not at all for a routing the sort rejected."""
import numpy as np
import pytest
import torch

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl
from gpu_util import dev, gpu_layer_fwd, make_device_layer, note, stream, to_dev

pytestmark = pytest.mark.gpu


def test_usage_accumulates_the_counts_of_every_step():
    w, layer, olayer = make_device_layer(wl.SWEEP)
    T = 64
    ws = layer.workspace(T)
    r = moe.moe_layer_routing(layer.struct, T, ws, ws.numel())
    hist = torch.zeros(wl.SWEEP.E, dtype=torch.int64, device=dev())
    expect = np.zeros(wl.SWEEP.E, np.int64)
    for d in range(5):
        note("usage step %d" % d)
        xd = to_dev(wl.make_x(T, wl.SWEEP.H, draw=900 + d).astype(np.float32))
        out = torch.empty_like(xd)
        moe.moe_layer_fwd(layer.struct, xd, T, out, 0, ws, ws.numel(), stream())
        moe.moe_expert_usage(r["counts"], r["n_uniq"], wl.SWEEP.E, hist, stream())
        torch.cuda.synchronize()
        ids = ws[r["topk_ids"] - ws.data_ptr():r["topk_ids"] - ws.data_ptr() + T * wl.SWEEP.top_k * 4]
        ids = ids.view(torch.int32).cpu().numpy()
        expect += oracle.sort(ids.reshape(T, wl.SWEEP.top_k), wl.SWEEP.E)["counts"]
        assert np.array_equal(hist.cpu().numpy(), expect), "step %d" % d
    assert int(expect.sum()) == 5 * T * wl.SWEEP.top_k


def test_usage_in_a_graph_and_rejected_routing():
    spec = wl.TINY
    w, layer, olayer = make_device_layer(spec)
    T = 4
    s = torch.cuda.Stream(dev())
    ws = layer.workspace(T, s)
    r = moe.moe_layer_routing(layer.struct, T, ws, ws.numel())
    x = to_dev(wl.make_x(T, spec.H, draw=3).astype(np.float32))
    out = torch.empty_like(x)
    hist = torch.zeros(spec.E, dtype=torch.int64, device=dev())
    with torch.cuda.stream(s):  # warm-up outside the capture
        moe.moe_layer_fwd(layer.struct, x, T, out, 0, ws, ws.numel(), s)
    s.synchronize()
    counts = ws[r["counts"] - ws.data_ptr():r["counts"] - ws.data_ptr() + spec.E * 4].view(torch.int32).cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_layer_fwd(layer.struct, x, T, out, 0, ws, ws.numel(), s)
        moe.moe_expert_usage(r["counts"], r["n_uniq"], spec.E, hist, s)
    for i in range(3):
        note("usage graph replay %d" % i)
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert np.array_equal(hist.cpu().numpy(), (i + 1) * counts.astype(np.int64))
    # a routing with an id out of range: the sort reports n_uniq = -1 and
    # nothing is added
    bad = to_dev(np.array([[0, 9]], np.int32))
    c = torch.zeros(spec.E, dtype=torch.int32, device=dev())
    o = torch.zeros(spec.E + 1, dtype=torch.int32, device=dev())
    sr = torch.zeros(2, dtype=torch.int32, device=dev())
    u = torch.zeros(spec.E, dtype=torch.int32, device=dev())
    n = torch.zeros(1, dtype=torch.int32, device=dev())
    moe.moe_sort(bad, 1, 2, spec.E, c, o, sr, u, n, stream())
    before = hist.clone()
    moe.moe_expert_usage(c, n, spec.E, hist, stream())
    torch.cuda.synchronize()
    assert int(n.item()) == -1
    assert torch.equal(hist, before)
