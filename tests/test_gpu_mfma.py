"""Parity of the MFMA segment path (experts that hold moe_mfma_min_routes()
routes or more: 8 below 128 tokens, 4 from 128) with the CPU oracle, through
the C ABI.

The MFMA path rounds both operands of each product to bf16 and accumulates
in fp32: the activations x (pass 1) and a (pass 2), and, for fp8 weights, the
decoded code times its block scale (for MXFP4 weights, code times its E8M0
scale, which is exact in bf16).  Its bar is the 2e-2 max relative error
(max abs error over max |ref|) stated for bf16 weights with fp32
accumulation.  Segments below the threshold stay on the GEMV path, whose
results must not change bit for bit when other segments of the same call
take the MFMA path.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import mixture_experts_decode_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
import workload as wl  # noqa: E402

from gpu_util import (check_layer_against_oracle, check_layer_sampled, dev, gpu_expert_fwd,  # noqa: E402
                      gpu_layer_fwd, make_device_layer, max_rel, note, oracle_weights_for)

BF16_OPERAND_TOL = 2e-2  # bar for paths with bf16 operands: max abs error over max |ref|
MFMA_TOKENS = 16  # MFMA launches from this many tokens


def _min_routes(layer, T, flags=0):
    """Routes per expert from which a segment of a T-token call runs on MFMA."""
    return moe.moe_mfma_min_routes(layer.struct, T, flags)

# H = I = 384: 3 K-stages of 128 in both passes (an odd count), 6 pass-1 row
# blocks of 64 gate/up pairs, 3 pass-2 row blocks of 128 down rows
MIXED = wl.LayerSpec(E=8, top_k=2, H=384, I=384)
MIXED_FP8 = wl.LayerSpec(E=8, top_k=2, H=384, I=256, expert_dtype=wl.FP8)
MIXED_FP4 = wl.LayerSpec(E=8, top_k=2, H=384, I=256, expert_dtype=wl.MXFP4)


def _oracle_routing(olayer, x):
    logits = oracle.router_logits(olayer, x)
    ids, _ = oracle.select(logits, olayer.k)
    return ids, oracle_weights_for(logits, ids)


def _routing(kind, olayer, x, thr=8):
    T = x.shape[0]
    if kind == "router":
        return _oracle_routing(olayer, x)
    rng = np.random.default_rng(T)
    rw = rng.uniform(0.1, 1.0, size=(T, 2))
    rw /= rw.sum(1, keepdims=True)
    if kind == "collide":  # every token on experts 0 and 1: T routes each
        return np.tile(np.array([[0, 1]], np.int32), (T, 1)), rw
    # "edge": thr tokens on {0, 1} (exactly the threshold), thr - 1 on {2, 3}
    # (one short of it), the rest on {4, 5}
    ids = np.tile(np.array([[4, 5]], np.int32), (T, 1))
    ids[:thr] = [0, 1]
    ids[thr:2 * thr - 1] = [2, 3]
    return ids, rw


@pytest.mark.parametrize("spec", [MIXED, MIXED_FP8, MIXED_FP4], ids=["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("T,kind", [(16, "collide"), (31, "edge"), (45, "router"), (300, "router"),
                                    (300, "collide")])
def test_mfma_expert_fwd(spec, T, kind):
    note("mfma expert_fwd %s T=%d %s" % (wl.DTYPE_NAMES[spec.expert_dtype], T, kind))
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, spec.H, draw=T)
    thr = _min_routes(layer, T)
    ids, rw = _routing(kind, olayer, x, thr)
    counts = np.bincount(ids.ravel(), minlength=spec.E)
    big = counts >= thr
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    gemv = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA)
    err = max_rel(got, ref)
    note("  max rel err %.3g (GEMV path %.3g), %d of %d experts on MFMA" %
         (err, max_rel(gemv, ref), big.sum(), (counts > 0).sum()))
    assert err <= BF16_OPERAND_TOL
    assert max_rel(gemv, ref) <= 1e-4
    assert big.any()
    assert not np.array_equal(got, gemv), "no segment took the MFMA path"
    small_only = ~big[ids].any(axis=1)
    assert np.array_equal(got[small_only], gemv[small_only])
    # MFMA pass 1 feeding the per-route GEMV pass 2
    p1 = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_WALK_DEDUP_PASS1)
    assert max_rel(p1, ref) <= BF16_OPERAND_TOL
    assert np.array_equal(p1[small_only], gemv[small_only])
    # the per-route walk never takes the MFMA path
    pr = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_WALK_PER_ROUTE)
    assert np.array_equal(pr, gemv)


@pytest.mark.parametrize("T,spec", [(64, MIXED), (300, MIXED), (64, MIXED_FP4), (300, MIXED_FP4)],
                         ids=["narrow", "wide", "mxfp4-64", "mxfp4-300"])
def test_mfma_deterministic_and_token_permutation(T, spec):
    note("mfma determinism and token permutation, T=%d %s" % (T, wl.DTYPE_NAMES[spec.expert_dtype]))
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, spec.H, draw=5)
    ids, rw = _oracle_routing(olayer, x)
    a = gpu_expert_fwd(layer, x, ids, rw)
    b = gpu_expert_fwd(layer, x, ids, rw)
    assert np.array_equal(a, b)
    perm = np.random.default_rng(1).permutation(T)
    c = gpu_expert_fwd(layer, x[perm], ids[perm], rw[perm])
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    assert max_rel(c[np.argsort(perm)], ref) <= BF16_OPERAND_TOL


@pytest.mark.parametrize("spec", [MIXED, MIXED_FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("cold", [0, 4], ids=["hot-only", "hot-and-cold"])
def test_pass2_with_combine_equals_separate_launches(spec, cold):
    """Up to 64 tokens pass 2 runs with the combine in one launch, which reads
    the y rows of the routes on the matrix cores from memory (pass 2 on the
    MFMA kernel runs first); above 64 tokens pass 2 and the combine are
    separate launches.  64 tokens (64 - cold on experts 0 and 1, on MFMA;
    cold on experts 2 and 3, below the threshold of 5 so on the GEMV kernels)
    alone and followed by 8 tokens on experts 4 and 5 give bitwise the same
    rows, and the rows follow the oracle."""
    note("pass 2 with the combine vs separate launches, %s, %d cold tokens" %
         (wl.DTYPE_NAMES[spec.expert_dtype], cold))
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(72, spec.H, draw=60 + cold)
    ids = np.tile(np.array([[0, 1]], np.int32), (72, 1))
    ids[64 - cold:64] = [2, 3]
    ids[64:] = [4, 5]
    rw = np.random.default_rng(60).uniform(0.1, 1.0, size=(72, 2)).astype(np.float32)
    rw /= rw.sum(1, keepdims=True)
    thr = _min_routes(layer, 64)
    assert thr > 0 and thr == _min_routes(layer, 72) and cold < thr
    full = gpu_expert_fwd(layer, x, ids, rw)
    part = gpu_expert_fwd(layer, x[:64], ids[:64], rw[:64])
    assert np.array_equal(part, full[:64])
    ref = oracle.expert_fwd(olayer, x[:64], ids[:64], rw[:64])
    assert max_rel(part, ref) <= BF16_OPERAND_TOL
    if cold:
        gemv = gpu_expert_fwd(layer, x[:64], ids[:64], rw[:64], flags=moe.MOE_NO_MFMA)
        assert np.array_equal(part[64 - cold:], gemv[64 - cold:])  # cold tokens: GEMV rows only


# A long K: pass 1 runs 20 stages of 128 through the narrow kernel's LDS
# ring (its steady state, not only the prologue), pass 2 runs 5, fewer than
# the fp8 and MXFP4 rings hold
LONG_K = wl.LayerSpec(E=8, top_k=2, H=2560, I=640)
LONG_K_FP8 = wl.LayerSpec(E=8, top_k=2, H=2560, I=640, expert_dtype=wl.FP8)
LONG_K_FP4 = wl.LayerSpec(E=8, top_k=2, H=2560, I=640, expert_dtype=wl.MXFP4)


@pytest.mark.parametrize("spec", [LONG_K, LONG_K_FP8, LONG_K_FP4], ids=["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("T", [16, 31, 45, 64, 100])
def test_mfma_narrow_long_k(spec, T):
    """Narrow items over a long K, every token on experts 0 and 1, so each
    of them holds T routes: one to four token blocks, the last one ragged.
    Within the bar of the oracle, deterministic, and bitwise unchanged when
    the tokens are permuted (a route's arithmetic does not depend on its
    place in the token block)."""
    note("mfma narrow long K, %s T=%d" % (wl.DTYPE_NAMES[spec.expert_dtype], T))
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, spec.H, draw=40 + T)
    ids, rw = _routing("collide", olayer, x)
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    note("  max rel err %.3g" % max_rel(got, ref))
    assert max_rel(got, ref) <= BF16_OPERAND_TOL
    assert np.array_equal(gpu_expert_fwd(layer, x, ids, rw), got)
    perm = np.random.default_rng(T).permutation(T)
    c = gpu_expert_fwd(layer, x[perm], ids[perm], rw[perm])
    assert np.array_equal(c[np.argsort(perm)], got)


def _fp8_codes_layer():
    """Two fp8 experts, H = I = 128, whose gate rows carry every E4M3 code
    once (expert e, gate row i: code 128*e + i in column 0, zeros elsewhere;
    the two NaN codes replaced by 0); up rows are 1.0, down is the identity,
    scales 1 except the gate blocks (0.5).  For a one-hot x = e_0 the output
    is out[h] = silu(0.5 * value(code 128e + h))."""
    E, H, I = 2, 128, 128
    one = wl.e4m3_encode(1.0)
    gu = np.zeros((E, 2 * I, H), np.uint8)
    for e in range(E):
        for i in range(I):
            c = 128 * e + i
            gu[e, i, 0] = c if c not in (0x7F, 0xFF) else 0
        gu[e, I:, :] = one
    dn = np.zeros((E, H, I), np.uint8)
    for e in range(E):
        dn[e, np.arange(H), np.arange(I)] = one
    s_gu = np.ones((E, 2, 1), np.float32)
    s_gu[:, 0, 0] = 0.5
    s_dn = np.ones((E, 1, 1), np.float32)
    spec = wl.LayerSpec(E=E, top_k=1, H=H, I=I, expert_dtype=wl.FP8, router_dtype=wl.BF16)
    return dict(spec=spec, w_router=np.zeros((E, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu,
                s_down=s_dn)


@pytest.mark.parametrize("T", [2 * MFMA_TOKENS, 256], ids=["narrow", "wide"])
def test_mfma_fp8_every_code(T):
    """Every E4M3 code through the MFMA decode: code * 0.5 is exact in bf16,
    so the only rounding is that of the activation to bf16 before the down
    projection (at most 2^-8 relative)."""
    note("mfma fp8 all codes, T=%d" % T)
    w = _fp8_codes_layer()
    layer = moe.DeviceLayer(w, device=dev())
    olayer = oracle.Layer(w)
    x = np.zeros((T, 128), np.float32)
    x[:, 0] = 1.0
    ids = np.repeat(np.array([[0], [1]], np.int32), T // 2, axis=0)
    got = gpu_expert_fwd(layer, x, ids, np.ones((T, 1)))
    ref = oracle.expert_fwd(olayer, x, ids, np.ones((T, 1)))
    assert np.allclose(got, ref, rtol=2.0 ** -8 * 1.01, atol=1e-30)
    gemv = gpu_expert_fwd(layer, x, ids, np.ones((T, 1)), flags=moe.MOE_NO_MFMA)
    assert not np.array_equal(got, gemv)


def _pack_fp4(codes):
    """[..., cols] E2M1 codes to [..., cols / 2] bytes, even element in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _fp4_codes_layer():
    """One MXFP4 expert, H = I = 128 (4 scale blocks per row).  Gate row i,
    column p holds code (i + p) % 16 with scale 2^((i + p // 32) % 5 - 2);
    up rows hold 1.0 (scale 1); down is the identity with scale
    2^((3 h + h // 32) % 4 - 1) on row h.  For x = e_p:
    out[h] = silu(value((h + p) % 16) * 2^((h + p // 32) % 5 - 2)) * 2^((3 h + h // 32) % 4 - 1)."""
    H = I = 128
    one = wl.e2m1_encode(1.0)
    gate = np.array([[(i + p) % 16 for p in range(H)] for i in range(I)])
    up = np.full((I, H), one)
    gu = _pack_fp4(np.concatenate([gate, up]))[None]
    s_gu = np.full((1, 2 * I, H // 32), 127, np.uint8)
    for i in range(I):
        for b in range(H // 32):
            s_gu[0, i, b] = 127 + (i + b) % 5 - 2
    dn = _pack_fp4(np.where(np.eye(H, I, dtype=bool), one, 0))[None]
    s_dn = np.full((1, H, I // 32), 127, np.uint8)
    for h in range(H):
        s_dn[0, h, :] = 127 + (3 * h + h // 32) % 4 - 1
    spec = wl.LayerSpec(E=1, top_k=1, H=H, I=I, expert_dtype=wl.MXFP4, router_dtype=wl.BF16)
    return dict(spec=spec, w_router=np.zeros((1, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu,
                s_down=s_dn)


@pytest.mark.parametrize("T", [127, 128], ids=["narrow", "wide"])
def test_mfma_mxfp4_every_code_every_position(T):
    """Every E2M1 code at every column of a gate row (columns 0..T-1), with a
    scale per (row, block of 32), through the MFMA decode: code * scale is
    exact in bf16, so the only rounding is that of the activation to bf16
    before the down projection (at most 2^-8 relative).  A swapped nibble,
    byte or scale block, or a wrong row's scale, fails it."""
    note("mfma mxfp4 all codes, T=%d" % T)
    w = _fp4_codes_layer()
    layer = moe.DeviceLayer(w, device=dev())
    olayer = oracle.Layer(w)
    x = np.eye(T, 128, dtype=np.float32)
    ids = np.zeros((T, 1), np.int32)
    got = gpu_expert_fwd(layer, x, ids, np.ones((T, 1)))
    ref = oracle.expert_fwd(olayer, x, ids, np.ones((T, 1)))
    assert np.allclose(got, ref, rtol=2.0 ** -8 * 1.01, atol=1e-30)
    gemv = gpu_expert_fwd(layer, x, ids, np.ones((T, 1)), flags=moe.MOE_NO_MFMA)
    assert not np.array_equal(got, gemv)
    assert np.allclose(gemv, ref, rtol=4e-7, atol=1e-30)


def test_mxfp4_unaligned_scales_stay_on_gemv():
    """MXFP4 scale arrays that are not 4-byte aligned cannot be copied a word
    at a time, so every segment stays on the GEMV kernels: the output equals
    the MOE_NO_MFMA output of the aligned layer bit for bit."""
    import torch

    note("mxfp4 unaligned scales")
    spec = MIXED_FP4
    w, layer, olayer = make_device_layer(spec)
    T = 64
    x = wl.make_x(T, spec.H, draw=11)
    ids, rw = _routing("collide", olayer, x)
    shifted = layer.with_bias(None)
    for n in ("s_gate_up", "s_down"):
        src = layer.tensors[n].reshape(-1)
        buf = torch.zeros(src.numel() + 16, dtype=torch.uint8, device=src.device)
        buf[1:1 + src.numel()] = src
        shifted.tensors[n + "_buf"] = buf
    t = shifted.tensors
    shifted.struct = moe.moe_layer_t(spec.E, spec.top_k, spec.H, spec.I, spec.router_dtype, spec.expert_dtype,
                                     t["w_router"].data_ptr(), t["w_gate_up"].data_ptr(), t["w_down"].data_ptr(),
                                     t["s_gate_up_buf"].data_ptr() + 1, t["s_down_buf"].data_ptr() + 1, None)
    got = gpu_expert_fwd(shifted, x, ids, rw)
    gemv = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA)
    mfma = gpu_expert_fwd(layer, x, ids, rw)
    assert np.array_equal(got, gemv)
    assert not np.array_equal(mfma, gemv), "the aligned layer takes the MFMA path"
    assert max_rel(got, oracle.expert_fwd(olayer, x, ids, rw)) <= 1e-4


# ---------------------------------------------------------------------------
# The large-batch regime at its full size: E=256, top_k=8, H=4096, I=1536,
# Zipf(1.1)-skewed routing, bf16, fp8 e4m3 with 128x128 block scales, MXFP4, q4_0.
# Every token's routing is checked; outputs on sampled tokens.

def _sample(g, T, thr, n_random=6):
    """Random tokens plus the last route of the hottest expert (the ragged
    end of its last token block) and a route of the coldest MFMA expert."""
    rng = np.random.default_rng(T)
    pick = set(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    counts, offsets, srt = g["counts"], g["offsets"], g["sorted_routes"]
    k = g["ids"].shape[1]
    hot = int(np.argmax(counts))
    pick.add(int(srt[offsets[hot + 1] - 1]) // k)
    mf = np.where(counts >= thr)[0]
    if len(mf):
        cold = int(mf[np.argmin(counts[mf])])
        pick.add(int(srt[offsets[cold]]) // k)
    return np.array(sorted(pick))


def _large(spec):
    bias = wl.zipf_bias(spec.E)
    return make_device_layer(spec, bias)


@pytest.fixture(scope="module")
def large_bf16():
    note("generating the E=256 H=4096 I=1536 bf16 layer")
    yield _large(wl.LARGE)


@pytest.fixture(scope="module")
def large_fp8():
    note("generating the E=256 H=4096 I=1536 fp8 layer")
    yield _large(wl.LARGE_FP8)


def _run_large(fixture, T):
    w, layer, olayer = fixture
    x = wl.make_x(T, layer.spec.H, draw=500 + T)
    thr = _min_routes(layer, T)
    g0 = check_layer_sampled(layer, olayer, x, [0])[1]
    sample = _sample(g0, T, thr)
    err, g = check_layer_sampled(layer, olayer, x, sample)
    c = g["counts"]
    note("  T=%d: %d unique, max count %d, %d experts on MFMA, sampled %d tokens, max rel err %.3g" %
         (T, g["n_uniq"], c.max(), (c >= thr).sum(), len(sample), err))
    assert thr > 0 and (c >= thr).any()


@pytest.mark.parametrize("T", [128, 256, 512])
def test_large_bf16_sampled(large_bf16, T):
    note("large bf16 T=%d" % T)
    _run_large(large_bf16, T)


@pytest.mark.parametrize("T", [128, 256, 512])
def test_large_fp8_sampled(large_fp8, T):
    note("large fp8 T=%d" % T)
    _run_large(large_fp8, T)


@pytest.fixture(scope="module")
def large_mxfp4():
    note("generating the E=256 H=4096 I=1536 MXFP4 layer")
    yield _large(wl.LARGE_MXFP4)


@pytest.mark.parametrize("T", [128, 512])
def test_large_mxfp4_sampled(large_mxfp4, T):
    note("large mxfp4 T=%d" % T)
    _run_large(large_mxfp4, T)


@pytest.fixture(scope="module")
def large_q4_0():
    note("generating the E=256 H=4096 I=1536 q4_0 layer")
    yield _large(wl.LARGE_Q4_0)


@pytest.mark.parametrize("T", [64, 128])
def test_large_q4_0_sampled(large_q4_0, T):
    """q4_0 at the large layer's size: narrow tiles (exact operands, sums
    scaled per k-step) at 64 tokens, wide tiles ((code - 8) * scale rounded
    to bf16) at 128."""
    note("large q4_0 T=%d" % T)
    _run_large(large_q4_0, T)


def test_mfma_narrow_many_experts():
    """E = 1024 (the largest the library takes: 8 KiB of expert tables in the
    narrow kernel's LDS), K = 128 (one stage), four hot experts on MFMA."""
    note("mfma narrow E=1024")
    spec = wl.LayerSpec(E=1024, top_k=2, H=128, I=128)
    bias = np.zeros(spec.E, np.float32)
    bias[[3, 500, 777, 1023]] = 6.0
    w, layer, olayer = make_device_layer(spec, bias)
    T = 64
    x = wl.make_x(T, spec.H, draw=7)
    err, apart = check_layer_against_oracle(layer, olayer, x, tol=BF16_OPERAND_TOL)
    g = gpu_layer_fwd(layer, x, 0, full=True)
    assert g["counts"].max() >= _min_routes(layer, T)
    gemv = gpu_layer_fwd(layer, x, moe.MOE_NO_MFMA)
    assert max_rel(g["out"], gemv) <= BF16_OPERAND_TOL


# ---------------------------------------------------------------------------
# moe_layer_fwd below 128 tokens: experts of moe_mfma_min_routes() routes or
# more take the MFMA path only when the call's largest expert holds
# moe_mfma_hot_routes() or more.  The router picks each token's expert
# exactly: token t is one-hot at column t, and router row e holds 1.0 at the
# columns of the tokens assigned to e (top_k = 1).

ONE_HOT = wl.LayerSpec(E=8, top_k=1, H=128, I=128, router_dtype=wl.BF16)


def _assigned_layer(assign):
    w = wl.make_layer(ONE_HOT)
    wr = np.zeros((ONE_HOT.E, ONE_HOT.H), np.uint16)
    for t, e in enumerate(assign):
        wr[e, t] = 0x3F80  # bf16 1.0
    w["w_router"] = wr
    return w, moe.DeviceLayer(w, device=dev()), oracle.Layer(w)


@pytest.mark.parametrize("largest", [6, 10], ids=["below-hot", "hot"])
def test_layer_mfma_only_with_a_hot_expert(largest):
    """32 tokens: `largest` on expert 0, 6 on expert 1, the rest at most 4 per
    expert.  With the largest expert below moe_mfma_hot_routes() every row is
    the GEMV path's, bitwise; with it at or above, experts 0 and 1 (both at
    or above moe_mfma_min_routes()) run on the matrix cores and the other
    rows stay the GEMV path's.  Both within the bar of the oracle."""
    T = 32
    L = _assigned_layer([0])[1]
    thr, hot = moe.moe_mfma_min_routes(L.struct, T), moe.moe_mfma_hot_routes(L.struct, T)
    assert thr <= 6 < hot <= largest or largest < hot
    rest = [2 + i % 6 for i in range(T - largest - 6)]
    assign = [0] * largest + [1] * 6 + rest
    assert max(np.bincount(rest)) < thr
    note("layer MFMA rule: largest %d, thr %d, hot %d" % (largest, thr, hot))
    w, layer, olayer = _assigned_layer(assign)
    x = np.eye(T, ONE_HOT.H, dtype=np.float32)
    g = gpu_layer_fwd(layer, x, full=True)
    assert np.array_equal(g["ids"][:, 0], np.array(assign, np.int32))
    got = g["out"]
    gemv = gpu_layer_fwd(layer, x, flags=moe.MOE_NO_MFMA)
    ref = oracle.moe_layer(olayer, x)["out"]
    mf = np.array(assign) < 2
    if largest < hot:
        assert np.array_equal(got, gemv)
        assert max_rel(got, ref) <= 1e-4
    else:
        assert np.array_equal(got[~mf], gemv[~mf])
        assert not np.array_equal(got[mf], gemv[mf])
        assert max_rel(got, ref) <= BF16_OPERAND_TOL


@pytest.mark.parametrize("dtype", [wl.BF16, wl.FP8, wl.MXFP4, wl.Q4_0], ids=["bf16", "fp8", "mxfp4", "q4_0"])
def test_mfma_narrow_many_items_per_workgroup(dtype):
    """Eight hot experts of 100 routes each on the narrow tiles (H = 2048,
    I = 768): 1536 pass-1 and 2048 pass-2 items, 3 and 4 per workgroup of the
    512-workgroup grid, so each workgroup takes its next item's route ids,
    scales and first stages while it finishes the current one.  Against the
    oracle at the bf16-operand bar, deterministic, and bitwise stable under
    token permutation."""
    note("mfma narrow many items per workgroup %s" % wl.DTYPE_NAMES[dtype])
    spec = wl.LayerSpec(E=16, top_k=8, H=2048, I=768, expert_dtype=dtype, router_dtype=wl.BF16)
    w, layer, olayer = make_device_layer(spec)
    T = 100
    x = wl.make_x(T, spec.H, draw=90)
    ids = np.tile(np.arange(8, dtype=np.int32), (T, 1))
    rw = np.random.default_rng(90).uniform(0.1, 1.0, size=(T, 8))
    rw /= rw.sum(1, keepdims=True)
    assert _min_routes(layer, T) > 0
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    note("  max rel err %.3g" % max_rel(got, ref))
    assert max_rel(got, ref) <= BF16_OPERAND_TOL
    assert not np.array_equal(got, gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA))
    assert np.array_equal(gpu_expert_fwd(layer, x, ids, rw), got)
    perm = np.random.default_rng(91).permutation(T)
    c = gpu_expert_fwd(layer, x[perm], ids[perm], rw[perm])
    assert np.array_equal(c[np.argsort(perm)], got)
