"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: bit-exact for expert ids, counts, offsets, sorted routes and uniq;
router logits within 1e-4 (max abs error over max |logit|); outputs within
the tolerance stated per test, never looser than 2e-2 (max abs error over
max |ref| per output tensor).  The tolerance 1e-4 used for fp32-accumulated
paths covers fp32 rounding over K <= 4096 terms (about sqrt(K) * 2^-24 per
dot product relative to the row norm, far below 1e-4) with margin.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import mixture_experts_decode_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
import workload as wl  # noqa: E402

from gpu_util import (BF16_OPERAND_TOL, call_tol, check_layer_against_oracle, gpu_expert_fwd,  # noqa: E402
                      gpu_layer_fwd, gpu_route, gpu_sort, make_device_layer, max_rel, note, dev)


def _routing_struct(E, k):
    return moe.moe_layer_t(E, k, 64, 32, moe.MOE_F32, moe.MOE_F32, None, None, None, None, None, None)


class _Shell:
    def __init__(self, E, k):
        self.spec = wl.LayerSpec(E=E, top_k=k, H=64, I=32, expert_dtype=wl.F32, router_dtype=wl.F32)
        self.struct = _routing_struct(E, k)

    def workspace(self, T):
        n = moe.moe_workspace_bytes(self.struct, T)
        ws = torch.empty(n, dtype=torch.uint8, device=dev())
        moe.moe_workspace_init(self.struct, T, ws, n, torch.cuda.current_stream())
        return ws


# ------------------------------------------------------------------ selection --

@pytest.mark.parametrize("E,k,T", [(8, 2, 4), (256, 8, 64), (256, 6, 37), (128, 2, 4), (1024, 32, 5), (100, 7, 33),
                                   (1, 1, 3), (16, 16, 9), (256, 8, 512)])
@pytest.mark.parametrize("mode", ["normal", "quarter", "equal", "zeros"])
def test_select_on_given_logits_bit_exact(E, k, T, mode):
    note("select E=%d k=%d T=%d mode=%s" % (E, k, T, mode))
    lg = wl.make_logits(T, E, draw=E + k + T)
    if mode == "quarter":
        lg = (np.round(lg * 4) / 4).astype(np.float32)
    elif mode == "equal":
        lg = np.full((T, E), 0.25, np.float32)
    elif mode == "zeros":
        lg = np.where(lg > 0, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    ids, w, lo = gpu_route(_Shell(E, k), logits_in=lg)
    rid, rw = oracle.select(lg.astype(np.float64), k)
    assert np.array_equal(ids, rid)
    assert np.abs(w - rw).max() <= 1e-5
    assert np.array_equal(lo, lg)
    assert np.allclose(w.sum(1), 1.0, atol=k * 2.0 ** -22)


@pytest.mark.parametrize("spec,T,bias", [(wl.TINY, 4, None), (wl.TINY, 4, "collision"), (wl.SWEEP, 1, None),
                                         (wl.SWEEP, 64, None), (wl.SKEWED, 37, "zipf"), (wl.STACK, 4, None)])
def test_router_logits_from_x(spec, T, bias):
    note("router %s T=%d bias=%s" % (spec, T, bias))
    b = {None: None, "collision": wl.collision_bias(spec.E), "zipf": wl.zipf_bias(spec.E)}[bias]
    w = wl.make_layer(spec, experts=False)
    w["w_gate_up"] = np.zeros(16, np.uint16 if spec.expert_dtype == wl.BF16 else np.float32)
    w["w_down"] = w["w_gate_up"]
    layer = moe.DeviceLayer(w, b, device=dev())
    x = wl.make_x(T, spec.H, draw=T)
    ids, gw, lo = gpu_route(layer, x=x)
    ref = oracle.router_logits(oracle.Layer(w, b), x)  # reads W_r and the bias only
    assert max_rel(lo, ref) <= 1e-4
    # selection on the GPU's own fp32 logits is exactly the oracle's on them
    rid, rw = oracle.select(lo.astype(np.float64), spec.top_k)
    assert np.array_equal(ids, rid)
    assert np.abs(gw - rw).max() <= 1e-5


# ----------------------------------------------------------------------- sort --

@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (4, 2, 8), (64, 8, 256), (37, 6, 100), (512, 8, 256), (300, 3, 1024),
                                   (1, 8, 256), (2048, 2, 128), (128, 8, 256), (205, 5, 64), (585, 7, 1000),
                                   (600, 8, 256), (32, 8, 256), (257, 1, 16), (258, 1, 1)])
@pytest.mark.parametrize("kind", ["distinct", "repeats", "collide"])
def test_sort_bit_exact(T, k, E, kind):
    note("sort T=%d k=%d E=%d %s" % (T, k, E, kind))
    rng = np.random.default_rng(T * 7 + k * 3 + E)
    if kind == "distinct":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    elif kind == "repeats":
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    else:
        ids = np.tile(np.arange(k, dtype=np.int32) % E, (T, 1))
    g = gpu_sort(ids, E)
    r = oracle.sort(ids, E)
    for key in ("counts", "offsets", "sorted_routes", "uniq"):
        assert np.array_equal(g[key], r[key]), key
    assert g["n_uniq"] == r["n_uniq"]


@pytest.mark.parametrize("T", [2, 50, 300, 700], ids=["one-wave", "four-waves-small", "four-waves", "workgroup"])
def test_sort_flags_bad_id(T):
    """An id out of range (8 for E = 8) in the last route, for each sort
    variant (up to 256, 4096 and more routes)."""
    note("sort bad id T=%d" % T)
    ids = np.tile(np.array([[0, 3, 2, 5, 1, 7]], np.int32), (T, 1))
    ids[-1, -1] = 8
    assert gpu_sort(ids, 8)["n_uniq"] == -1


# -------------------------------------------------------------------- experts --

@pytest.mark.parametrize("walk", [moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE, moe.MOE_WALK_DEDUP_PASS1])
@pytest.mark.parametrize("flags", [0, moe.MOE_ACCUM_RESIDUAL])
def test_expert_fwd_rejected_routing_leaves_out_untouched(walk, flags):
    """A routing that the sort rejects (an id outside [0, E): n_uniq = -1)
    runs no expert work, and the combine leaves out as it was."""
    note("expert_fwd rejected routing walk=%d flags=%d" % (walk, flags))
    w, layer, olayer = make_device_layer(wl.TINY)
    T, s = 4, wl.TINY
    ids = np.tile(np.array([[0, 3]], np.int32), (T, 1))
    ids[2, 1] = s.E  # out of range
    d_ids = torch.from_numpy(ids).to(dev())
    d_w = torch.full((T, s.top_k), 0.5, dtype=torch.float32, device=dev())
    counts = torch.empty(s.E, dtype=torch.int32, device=dev())
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device=dev())
    sorted_routes = torch.empty(T * s.top_k, dtype=torch.int32, device=dev())
    uniq = torch.empty(s.E, dtype=torch.int32, device=dev())
    n = torch.empty(1, dtype=torch.int32, device=dev())
    st = torch.cuda.current_stream()
    x = torch.from_numpy(wl.make_x(T, s.H, draw=5)).to(dev())
    out = torch.full((T, s.H), 7.25, dtype=torch.float32, device=dev())
    ws = layer.workspace(T)
    # a valid routing first, so the workspace's y rows and the routing
    # arrays hold plausible values
    good = torch.from_numpy(np.tile(np.array([[0, 3]], np.int32), (T, 1))).to(dev())
    moe.moe_sort(good, T, s.top_k, s.E, counts, offsets, sorted_routes, uniq, n, st)
    moe.moe_expert_fwd(layer.struct, x, T, good, d_w, counts, offsets, sorted_routes, uniq, n,
                       torch.empty_like(out), walk, ws, ws.numel(), st)
    moe.moe_sort(d_ids, T, s.top_k, s.E, counts, offsets, sorted_routes, uniq, n, st)
    moe.moe_expert_fwd(layer.struct, x, T, d_ids, d_w, counts, offsets, sorted_routes, uniq, n, out,
                       walk | flags, ws, ws.numel(), st)
    torch.cuda.synchronize()
    assert int(n.item()) == -1
    assert (out == 7.25).all()


def _oracle_routing(olayer, x):
    lg = oracle.router_logits(olayer, x)
    return oracle.select(lg, olayer.k)


@pytest.mark.parametrize("walk", [moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE, moe.MOE_WALK_DEDUP_PASS1])
def test_expert_fwd_tiny_fp32(walk):
    note("expert_fwd tiny walk=%d" % walk)
    w, layer, olayer = make_device_layer(wl.TINY)
    x = wl.make_x(4, wl.TINY.H)
    ids, rw = _oracle_routing(olayer, x)
    got = gpu_expert_fwd(layer, x, ids, rw, flags=walk)
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    assert max_rel(got, ref) <= 1e-5


RAGGED = wl.LayerSpec(E=64, top_k=4, H=1088, I=416)  # row chunks not a multiple of 64 lanes


@pytest.mark.parametrize("spec,T", [(RAGGED, 37), (RAGGED, 1), (wl.LayerSpec(E=10, top_k=3, H=72, I=24), 21)])
def test_expert_fwd_ragged_all_walks_bitwise(spec, T):
    note("expert_fwd ragged %s T=%d" % (spec, T))
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, spec.H, draw=2)
    ids, rw = _oracle_routing(olayer, x)
    outs = [gpu_expert_fwd(layer, x, ids, rw, flags=f)
            for f in (moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE, moe.MOE_WALK_DEDUP_PASS1)]
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    assert max_rel(outs[0], ref) <= 1e-4
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def _fp8_codes_layer():
    """Two fp8 experts, H = I = 128, whose gate rows carry every E4M3 code once:
    expert e, gate row i holds code 128*e + i in column 0 and zeros elsewhere;
    up rows are 1.0 everywhere, down is the identity, all scales 1 except the
    gate blocks (0.5).  For x = e_0 (one-hot) the output is
    out[h] = silu(0.5 * value(code 128e + h)) * 1."""
    E, H, I = 2, 128, 128
    one = wl.e4m3_encode(1.0)
    gu = np.zeros((E, 2 * I, H), np.uint8)
    for e in range(E):
        for i in range(I):
            c = 128 * e + i
            gu[e, i, 0] = c if c not in (0x7F, 0xFF) else 0  # skip the two NaN codes
        gu[e, I:, :] = one
    dn = np.zeros((E, H, I), np.uint8)
    for e in range(E):
        dn[e, np.arange(H), np.arange(I)] = one
    s_gu = np.ones((E, 2, 1), np.float32)
    s_gu[:, 0, 0] = 0.5
    s_dn = np.ones((E, 1, 1), np.float32)
    spec = wl.LayerSpec(E=E, top_k=1, H=H, I=I, expert_dtype=wl.FP8, router_dtype=wl.BF16)
    w = dict(spec=spec, w_router=np.zeros((E, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu, s_down=s_dn)
    return spec, w


def test_fp8_every_code_decodes_exactly():
    note("fp8 all codes")
    spec, w = _fp8_codes_layer()
    layer = moe.DeviceLayer(w, device=dev())
    olayer = oracle.Layer(w)
    x = np.zeros((2, 128), np.float32)
    x[:, 0] = 1.0
    ids = np.array([[0], [1]], np.int32)
    got = gpu_expert_fwd(layer, x, ids, np.ones((2, 1)))
    ref = oracle.expert_fwd(olayer, x, ids, np.ones((2, 1)))
    # silu in fp32 on exactly decoded inputs: a few ulp
    assert np.allclose(got, ref, rtol=4e-7, atol=1e-30)
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert not np.isnan(ref).any() and np.isfinite(vals[[1, 8, 0x7E]]).all()


@pytest.mark.parametrize("T", [1, 9, 40])
def test_fp8_random_layer(T):
    note("fp8 random T=%d" % T)
    spec = wl.LayerSpec(E=16, top_k=4, H=512, I=256, expert_dtype=wl.FP8, router_dtype=wl.BF16)
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, spec.H, draw=T)
    # experts with many routes run on the matrix cores (bf16 operands); the
    # GEMV path alone holds the fp32 bar
    check_layer_against_oracle(layer, olayer, x, tol=call_tol(layer, x))
    check_layer_against_oracle(layer, olayer, x, flags=moe.MOE_NO_MFMA, tol=1e-4)


# ---------------------------------------------------------------------- layer --

@pytest.mark.parametrize("bias", [None, "collision"])
def test_layer_tiny(bias):
    note("layer tiny bias=%s" % bias)
    b = None if bias is None else wl.collision_bias(wl.TINY.E)
    w, layer, olayer = make_device_layer(wl.TINY, b)
    x = wl.make_x(4, wl.TINY.H)
    err, _ = check_layer_against_oracle(layer, olayer, x, tol=1e-5)
    g = gpu_layer_fwd(layer, x, full=True)
    if bias is not None:
        assert set(np.unique(g["ids"])) == {0, 1}
        assert g["n_uniq"] == 2 and list(g["counts"][:2]) == [4, 4]


def test_layer_k_equals_E_and_single_expert():
    for spec in (wl.LayerSpec(E=8, top_k=8, H=64, I=32, expert_dtype=wl.F32, router_dtype=wl.F32),
                 wl.LayerSpec(E=1, top_k=1, H=64, I=32, expert_dtype=wl.F32, router_dtype=wl.F32)):
        note("layer %s" % (spec,))
        w, layer, olayer = make_device_layer(spec)
        x = wl.make_x(5, spec.H)
        check_layer_against_oracle(layer, olayer, x, tol=1e-5)


def test_layer_T0_is_noop():
    note("layer T=0")
    w, layer, _ = make_device_layer(wl.TINY)
    out = torch.full((1, wl.TINY.H), 3.0, device=dev())
    ws = layer.workspace(1)
    moe.moe_layer_fwd(layer.struct, out, 0, out, 0, ws, ws.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert (out == 3.0).all()


@pytest.fixture(scope="module")
def sweep_layer():
    w, layer, olayer = make_device_layer(wl.SWEEP)
    return w, layer, olayer


@pytest.mark.parametrize("T", [1, 4, 64])
def test_layer_sweep_shape(sweep_layer, T):
    note("layer E=256 k=8 H=2048 I=768 bf16 T=%d" % T)
    w, layer, olayer = sweep_layer
    x = wl.make_x(T, wl.SWEEP.H, draw=100 + T)
    err, napart = check_layer_against_oracle(layer, olayer, x, tol=call_tol(layer, x))
    g = gpu_layer_fwd(layer, x, full=True)
    assert g["stats"][0] == g["n_uniq"] == len(np.unique(g["ids"]))
    assert g["stats"][1] == T * wl.SWEEP.top_k
    assert g["stats"][2] == g["counts"].max()
    r = oracle.sort(g["ids"], wl.SWEEP.E)
    for key in ("counts", "offsets", "sorted_routes", "uniq"):
        assert np.array_equal(g[key], r[key]), key


def test_sweep_walks_bitwise_equal_and_deterministic(sweep_layer):
    note("walks bitwise T=64")
    w, layer, olayer = sweep_layer
    x = wl.make_x(64, wl.SWEEP.H, draw=7)
    # bitwise on GEMV segments (the per-route walk never takes the matrix cores)
    outs = [gpu_layer_fwd(layer, x, f | moe.MOE_NO_MFMA) for f in (moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE,
                                                                    moe.MOE_WALK_DEDUP_PASS1, moe.MOE_WALK_DEDUP)]
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


def test_sweep_token_permutation_bitwise(sweep_layer):
    note("token permutation T=32")
    w, layer, olayer = sweep_layer
    x = wl.make_x(32, wl.SWEEP.H, draw=9)
    perm = np.random.default_rng(0).permutation(32)
    a = gpu_layer_fwd(layer, x)
    b = gpu_layer_fwd(layer, x[perm])
    assert np.array_equal(a[perm], b)


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_layer_skewed(T):
    note("layer skewed k=6 T=%d" % T)
    bias = wl.zipf_bias(wl.SKEWED.E)
    w, layer, olayer = make_device_layer(wl.SKEWED, bias)
    x = wl.make_x(T, wl.SKEWED.H, draw=200 + T)
    # hot experts (moe_mfma_min_routes() routes or more) run on MFMA with bf16 operands
    check_layer_against_oracle(layer, olayer, x, tol=BF16_OPERAND_TOL if T >= 16 else 1e-4)
    check_layer_against_oracle(layer, olayer, x, flags=moe.MOE_NO_MFMA, tol=1e-4)
    g = gpu_layer_fwd(layer, x, full=True)
    if T == 64:
        assert g["counts"].max() >= 16  # skew produces hot experts (at least 16 routes)
        a = gpu_layer_fwd(layer, x, moe.MOE_WALK_PER_ROUTE)
        b = gpu_layer_fwd(layer, x, moe.MOE_NO_MFMA)
        assert np.array_equal(a, b)
        assert not np.array_equal(a, g["out"])


def test_stack_layers_rmsnorm_residual_teacher_forced():
    """Three layers of the stack shape, each fed the GPU output of the one
    before: RMSNorm before the router, residual after the combine."""
    T = 4
    h = wl.make_x(T, wl.STACK.H, draw=300)
    for l in range(3):
        note("stack layer %d" % l)
        w, layer, olayer = make_device_layer(wl.STACK, layer_idx=l)
        flags = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
        check_layer_against_oracle(layer, olayer, h, flags=flags, tol=1e-4, rmsnorm_in=True, residual=True)
        h = gpu_layer_fwd(layer, h, flags)
        del layer


def test_stack_shape_layer_bs1_rmsnorm_residual():
    """The 30-layer stack's layer shape (E=128, top_k=2, H=2048, I=1024) at
    one token, RMSNorm before the router and the residual after the combine,
    against the oracle (GEMV segments only at one token: fp32 bar)."""
    flags = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
    for l in (0, 7):
        note("stack-shape layer %d T=1" % l)
        w, layer, olayer = make_device_layer(wl.STACK, layer_idx=l)
        x = wl.make_x(1, wl.STACK.H, draw=310 + l)
        check_layer_against_oracle(layer, olayer, x, flags=flags, tol=1e-4, rmsnorm_in=True, residual=True)
        del layer


def test_out_may_alias_x():
    note("in-place residual")
    w, layer, olayer = make_device_layer(wl.TINY)
    x = wl.make_x(4, wl.TINY.H)
    xd = torch.from_numpy(x).to(dev())
    ref = gpu_layer_fwd(layer, x, moe.MOE_ACCUM_RESIDUAL)
    ws = layer.workspace(4)
    moe.moe_layer_fwd(layer.struct, xd, 4, xd, moe.MOE_ACCUM_RESIDUAL, ws, ws.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().numpy(), ref)


@pytest.mark.parametrize("flags", [0, moe.MOE_ACCUM_RESIDUAL])
def test_token_output_independent_of_batch_bitwise(sweep_layer, flags):
    """A token's expert rows and its combine do not depend on the rest of the
    batch (segment sizes, grid sizes, persistent-loop strides), so the first
    tokens of a 16-token batch come out bitwise as the same tokens alone."""
    note("batch independence, flags=%d" % flags)
    w, layer, olayer = sweep_layer
    x = wl.make_x(16, wl.SWEEP.H, draw=11)
    f = flags | moe.MOE_NO_MFMA
    full = gpu_layer_fwd(layer, x, f)
    for T in (1, 5, 15):
        part = gpu_layer_fwd(layer, x[:T], f)
        assert np.array_equal(part, full[:T]), T
    again = gpu_layer_fwd(layer, x[:5], f)
    assert np.array_equal(again, full[:5])
    # pass 2 with the combine in one launch (up to 64 tokens) against the
    # separate pass-2 and combine launches (above 64)
    x72 = wl.make_x(72, wl.SWEEP.H, draw=12)
    assert np.array_equal(gpu_layer_fwd(layer, x72[:64], f), gpu_layer_fwd(layer, x72, f)[:64])


def test_stack_layer_large_batch_rmsnorm():
    """The stack shape at 160 tokens: 64 KiB router tiles of 8 tokens,
    RMSNorm on the tile, several tiles with a ragged last one, the workgroup
    sort (R = 320 > one tile); GEMV segments only, so the fp32 bar holds."""
    note("stack layer T=160")
    T = 160
    w, layer, olayer = make_device_layer(wl.STACK, layer_idx=4)
    h = wl.make_x(T, wl.STACK.H, draw=301)
    flags = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL | moe.MOE_NO_MFMA
    check_layer_against_oracle(layer, olayer, h, flags=flags, tol=1e-4, rmsnorm_in=True, residual=True)
