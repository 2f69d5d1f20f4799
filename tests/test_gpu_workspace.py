"""One workspace serves every batch size it holds: calls of different
sizes in any order give bitwise the results of a fresh workspace, and the
synchronisation words at its front are zero again after each call.

The synchronisation words (the routing kernel's arrival counters) sit in a
front of fixed size and place, so no call's logits or routing arrays ever
land on them, whatever batch, layer shape or byte size the calls on one
workspace pass.
"""
import numpy as np
import pytest
import torch

import mixture_experts_decode_gemv_amd as moe
import workload as wl
from gpu_util import make_device_layer, note, stream, to_dev

pytestmark = pytest.mark.gpu


def _run(layer, x, T, flags, ws):
    xd = to_dev(x.astype(np.float32))
    out = torch.full_like(xd, float("nan"))
    moe.moe_layer_fwd(layer.struct, xd, T, out, flags, ws, ws.numel(), stream())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _front_is_clear(layer, T, ws):
    """Every word between the statistics block and the logits is zero."""
    s = layer.spec
    r = moe.moe_layer_routing(layer.struct, T, ws, ws.numel())
    logits_off = r["topk_ids"] - ws.data_ptr() - ((T * s.E * 4 + 255) // 256) * 256
    front = ws[256:logits_off].view(torch.int32).cpu().numpy()
    assert front.size > 0 and not front.any(), "%d synchronisation words left nonzero" % int((front != 0).sum())


@pytest.mark.parametrize("spec,flags,sizes", [
    (wl.SWEEP, 0, (64, 3, 64, 17, 1, 3, 64, 9)),
    (wl.STACK, moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL, (4, 1, 4, 2, 1)),
    (wl.TINY, 0, (37, 4, 1, 37, 12)),
], ids=["sweep", "stack", "tiny"])
def test_batch_sizes_interleaved_on_one_workspace(spec, flags, sizes):
    w, layer, olayer = make_device_layer(spec)
    cap = max(sizes)
    xs = {T: wl.make_x(T, spec.H, draw=700 + T) for T in sizes}
    ref = {}
    for T in xs:
        note("fresh workspace T=%d" % T)
        ref[T] = _run(layer, xs[T], T, flags, layer.workspace(T))
    ws = layer.workspace(cap)
    for T in sizes:
        note("shared workspace T=%d" % T)
        assert np.array_equal(_run(layer, xs[T], T, flags, ws), ref[T]), "T=%d" % T
        _front_is_clear(layer, T, ws)


def test_byte_sizes_and_layer_shapes_alternate_on_one_buffer():
    """One buffer, passed with its full size and with the smaller sizes two
    other batches need, and shared by layers of two shapes: every call equals
    a fresh workspace bitwise, and the front is clear after each."""
    wa, la, _ = make_device_layer(wl.SWEEP)
    wb, lb, _ = make_device_layer(wl.TINY)
    xa = {T: wl.make_x(T, wl.SWEEP.H, draw=720 + T) for T in (8, 2)}
    xb = {T: wl.make_x(T, wl.TINY.H, draw=730 + T) for T in (5,)}
    ref = {("a", T): _run(la, xa[T], T, 0, la.workspace(T)) for T in xa}
    ref[("b", 5)] = _run(lb, xb[5], 5, 0, lb.workspace(5))
    ws = la.workspace(8)
    plan = [("a", 8, ws.numel()), ("a", 2, moe.moe_workspace_bytes(la.struct, 2)),
            ("b", 5, moe.moe_workspace_bytes(lb.struct, 5)), ("a", 8, ws.numel()),
            ("b", 5, ws.numel()), ("a", 2, moe.moe_workspace_bytes(la.struct, 2)), ("a", 8, ws.numel())]
    for name, T, nbytes in plan:
        note("shared buffer: layer %s T=%d ws_bytes=%d" % (name, T, nbytes))
        layer, x = (la, xa[T]) if name == "a" else (lb, xb[T])
        xd = to_dev(x.astype(np.float32))
        out = torch.full_like(xd, float("nan"))
        moe.moe_layer_fwd(layer.struct, xd, T, out, 0, ws, nbytes, stream())
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref[(name, T)]), (name, T, nbytes)
        _front_is_clear(layer, T, ws)


def test_larger_workspace_than_needed():
    """A workspace bigger than moe_workspace_bytes(T) gives the same bits."""
    w, layer, olayer = make_device_layer(wl.SWEEP)
    x = wl.make_x(8, wl.SWEEP.H, draw=990)
    a = _run(layer, x, 8, 0, layer.workspace(8))
    b = _run(layer, x, 8, 0, layer.workspace(200))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("spec,flags", [
    (wl.TINY, 0),
    (wl.LayerSpec(E=16, top_k=4, H=512, I=256), 0),
    (wl.STACK, moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL),
], ids=["tiny", "bf16-small", "stack"])
def test_small_batch_calls_repeat_on_one_workspace(spec, flags):
    """Calls that alternate two inputs on one workspace, at the batch sizes
    whose pass 2 and combine run as one launch, give bitwise the results of
    fresh workspaces every time: nothing a call leaves in the workspace (its
    counters, its activation rows) reaches the next call's results."""
    w, layer, olayer = make_device_layer(spec)
    for T in (1, 2, 4):
        xs = [wl.make_x(T, spec.H, draw=900 + 10 * T + i) for i in range(2)]
        ref = [_run(layer, x, T, flags, layer.workspace(T)) for x in xs]
        ws = layer.workspace(T)
        for rep in range(6):
            note("repeat %d on one workspace, T=%d" % (rep, T))
            assert np.array_equal(_run(layer, xs[rep % 2], T, flags, ws), ref[rep % 2]), "T=%d call %d" % (T, rep)
            _front_is_clear(layer, T, ws)
