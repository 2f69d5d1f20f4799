"""moe_stack_fwd: a stack of layers (RMSNorm before the router, residual
after the combine) in which each layer's combine runs inside the next
layer's routing launch.  Its output must equal, bit for bit, the same layers
run one moe_layer_fwd call at a time with MOE_RMSNORM_IN |
MOE_ACCUM_RESIDUAL (whose parity with the oracle the other tests check):
the fused rows are formed with the combine kernel's arithmetic in the same
order.  Covered: the 30-layer stack's layer shape, several token tiles, an
odd top_k (a route group of one), segments on the matrix cores (narrow
tiles, and the wide tiles on the second stream), every walk arm, an output
that aliases the input, and graph replays."""
import numpy as np
import pytest
import torch

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl
from gpu_util import (ambiguous_tokens, dev, gpu_layer_fwd, max_rel, note, oracle_for_gpu_selection)

pytestmark = pytest.mark.gpu

NORM_RES = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
SMALL = wl.LayerSpec(E=16, top_k=5, H=512, I=256)  # 8 tokens per routing tile


def _layers(spec, n, bias=None):
    return [moe.DeviceLayer(wl.make_layer(spec, layer=l), bias, device=dev()) for l in range(n)]


def _sequential(layers, x0, T, flags):
    stream = torch.cuda.Stream(dev())
    ws = layers[0].workspace(T, stream)
    h = x0.clone()
    with torch.cuda.stream(stream):
        for L in layers:
            moe.moe_layer_fwd(L.struct, h, T, h, flags | NORM_RES, ws, ws.numel(), stream)
    stream.synchronize()
    return h.cpu().numpy()


def _stack_ws(layers, T, stream):
    n = moe.moe_stack_workspace_bytes(layers[0].struct, T)
    ws = torch.empty(n, dtype=torch.uint8, device=dev())
    moe.moe_stack_workspace_init(layers[0].struct, T, ws, n, stream)
    return ws


def _fused(layers, x0, T, flags, in_place=False):
    stream = torch.cuda.Stream(dev())
    ws = _stack_ws(layers, T, stream)
    out = x0.clone() if in_place else torch.full_like(x0, float("nan"))
    src = out if in_place else x0
    with torch.cuda.stream(stream):
        moe.moe_stack_fwd([L.struct for L in layers], src, T, out, flags, ws, ws.numel(), stream)
    stream.synchronize()
    return out.cpu().numpy()


@pytest.fixture(scope="module")
def stack3():
    note("generating 3 layers of the stack shape")
    return _layers(wl.STACK, 3)


@pytest.mark.parametrize("T", [1, 4, 5])
def test_stack_fused_equals_layer_calls_stack_shape(stack3, T):
    note("fused stack, stack shape, T=%d" % T)
    x0 = torch.from_numpy(wl.make_x(T, wl.STACK.H, draw=31 + T)).to(dev())
    ref = _sequential(stack3, x0, T, 0)
    assert np.isfinite(ref).all()
    assert np.array_equal(_fused(stack3, x0, T, 0), ref)
    assert np.array_equal(_fused(stack3, x0, T, 0, in_place=True), ref)


@pytest.mark.parametrize("T", [1, 4])
def test_stack_fused_against_oracle(stack3, T):
    """moe_stack_fwd against the oracle, layer by layer and teacher-forced:
    the fused stacks of the first l and l + 1 layers give the GPU's h_l and
    h_{l+1}; the oracle layer (RMSNorm, router, top-k, experts, combine,
    residual) applied to h_l must give h_{l+1}.  A token whose oracle logits
    have a near tie may be routed either way; it is compared against the
    oracle rerun with the GPU's ids for that layer (from a layer call on the
    same h_l, which routes bitwise as the stack does)."""
    x0 = torch.from_numpy(wl.make_x(T, wl.STACK.H, draw=131 + T)).to(dev())
    hs = [x0.cpu().numpy()]
    for n in range(1, len(stack3) + 1):
        note("fused stack prefix of %d layers, T=%d" % (n, T))
        hs.append(_fused(stack3[:n], x0, T, 0))
    for l in range(len(stack3)):
        note("oracle check of stack layer %d, T=%d" % (l, T))
        olayer = oracle.Layer(wl.make_layer(wl.STACK, layer=l))
        h_in, h_out = hs[l], hs[l + 1]
        ref = oracle.moe_layer(olayer, h_in, rmsnorm_in=True, residual=True)
        ids = gpu_layer_fwd(stack3[l], h_in, NORM_RES, full=True)["ids"]
        amb = ambiguous_tokens(ref["logits"], wl.STACK.top_k)
        same = (ids == ref["ids"]).all(1)
        assert (same | amb).all(), "layer %d: selection differs on tokens with a clear gap" % l
        expect = ref["out"].copy()
        if (~same).any():
            alt = oracle_for_gpu_selection(olayer, h_in, ref["logits"], ids, rmsnorm_in=True, residual=True)
            expect[~same] = alt[~same]
        assert np.isfinite(h_out).all()
        assert max_rel(h_out, expect) <= 1e-4, "layer %d" % l
        # the MoE part alone (the residual removed on both sides)
        moe_gpu = h_out.astype(np.float64) - h_in
        moe_ref = expect - h_in.astype(np.float64)
        assert max_rel(moe_gpu, moe_ref) <= 1e-4, "layer %d (MoE part)" % l


@pytest.mark.parametrize("T", [1, 9, 40, 130])
@pytest.mark.parametrize("flags", [0, moe.MOE_WALK_PER_ROUTE, moe.MOE_WALK_DEDUP_PASS1, moe.MOE_NO_MFMA],
                         ids=["dedup", "per_route", "dedup_pass1", "no_mfma"])
def test_stack_fused_equals_layer_calls(T, flags):
    note("fused stack, E=16 k=5 H=512 I=256, T=%d flags=%d" % (T, flags))
    bias = np.zeros(SMALL.E, np.float32)
    bias[:2] = 3.0  # two hot experts: segments on the matrix cores from T = 16
    layers = _layers(SMALL, 4, bias)
    x0 = torch.from_numpy(wl.make_x(T, SMALL.H, draw=41 + T)).to(dev())
    ref = _sequential(layers, x0, T, flags)
    assert np.isfinite(ref).all()
    assert np.array_equal(_fused(layers, x0, T, flags), ref)


@pytest.mark.parametrize("dtype", [wl.FP8, wl.MXFP4, wl.Q4_0], ids=["fp8", "mxfp4", "q4_0"])
@pytest.mark.parametrize("T", [3, 40, 130])
def test_stack_fused_equals_layer_calls_quantised(dtype, T):
    """fp8 (128x128 block scales), MXFP4 and q4_0 experts, below and above
    the MFMA threshold, on narrow and wide tiles; MXFP4 and q4_0 down rows of
    8 chunks (I = 256) take pass 2 without the combine at any batch, so the
    next layer's routing launch forms the combine."""
    spec = wl.LayerSpec(E=16, top_k=5, H=512, I=256, expert_dtype=dtype, router_dtype=wl.BF16)
    note("fused stack, %s, T=%d" % (wl.DTYPE_NAMES[dtype], T))
    bias = np.zeros(spec.E, np.float32)
    bias[:2] = 3.0
    layers = _layers(spec, 3, bias)
    x0 = torch.from_numpy(wl.make_x(T, spec.H, draw=71 + T)).to(dev())
    ref = _sequential(layers, x0, T, 0)
    assert np.isfinite(ref).all()
    assert np.array_equal(_fused(layers, x0, T, 0), ref)


def test_stack_fused_wide_router_rows():
    """H = 4096 with a bf16 router: 8 router chunks per lane held in registers
    beside the fused staging (the largest routing instantiation)."""
    spec = wl.LayerSpec(E=8, top_k=2, H=4096, I=128)
    note("fused stack, H=4096")
    layers = _layers(spec, 3)
    for T in (1, 3):
        x0 = torch.from_numpy(wl.make_x(T, spec.H, draw=81 + T)).to(dev())
        assert np.array_equal(_fused(layers, x0, T, 0), _sequential(layers, x0, T, 0))


def test_stack_workspace_serves_smaller_batches():
    """One stack workspace sized for 8 tokens, used at 3, 8 and 1 tokens in
    turn: every call equals the layer calls (the synchronisation words sit
    where the workspace's byte size puts them, whatever the batch)."""
    layers = _layers(SMALL, 2)
    stream = torch.cuda.Stream(dev())
    ws = _stack_ws(layers, 8, stream)
    structs = [L.struct for L in layers]
    for T in (3, 8, 1, 3):
        note("stack workspace for 8 tokens, T=%d" % T)
        x0 = torch.from_numpy(wl.make_x(T, SMALL.H, draw=91 + T)).to(dev())
        out = torch.full_like(x0, float("nan"))
        with torch.cuda.stream(stream):
            moe.moe_stack_fwd(structs, x0, T, out, 0, ws, ws.numel(), stream)
        stream.synchronize()
        assert np.array_equal(out.cpu().numpy(), _sequential(layers, x0, T, 0))


def test_stack_fused_single_layer():
    note("fused stack of one layer")
    layers = _layers(SMALL, 1)
    x0 = torch.from_numpy(wl.make_x(3, SMALL.H, draw=51)).to(dev())
    assert np.array_equal(_fused(layers, x0, 3, 0), _sequential(layers, x0, 3, 0))


def test_stack_fused_graph_replays(stack3):
    """Recorded in a HIP graph, with eager work of the program between the
    replays: every replay equals the layer-by-layer run."""
    T = 4
    x0 = torch.from_numpy(wl.make_x(T, wl.STACK.H, draw=61)).to(dev())
    ref = _sequential(stack3, x0, T, 0)
    stream = torch.cuda.Stream(dev())
    ws = _stack_ws(stack3, T, stream)
    structs = [L.struct for L in stack3]
    h = x0.clone()
    with torch.cuda.stream(stream):
        moe.moe_stack_fwd(structs, h, T, h, 0, ws, ws.numel(), stream)  # warm-up outside the capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        moe.moe_stack_fwd(structs, h, T, h, 0, ws, ws.numel(), stream)
    for i in range(3):
        note("fused stack graph replay %d" % i)
        with torch.cuda.stream(stream):
            h.copy_(x0)
            graph.replay()
        stream.synchronize()
        assert np.array_equal(h.cpu().numpy(), ref), "replay %d" % i
        assert np.array_equal(_sequential(stack3, x0, T, 0), ref)
