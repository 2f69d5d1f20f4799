"""q4_0 expert weights (blocks of 32 elements along a row with one binary16
scale d, 4-bit codes q, value (q - 8) * d; element j of a block in the low
nibble of byte j, element j + 16 in its high nibble) on the GEMV path,
against the oracle.

The GPU converts each code to the exact fp32 value q - 8, sums a chunk's
products in fp32 and applies the chunk's scale to the sum; every weight is
exact in fp32, so the outputs follow the oracle to fp32 rounding (bar 1e-4,
as for the other GEMV paths).  The per-code test places every code at every
element position of a block, so a swapped nibble half or code offset fails
it.  Segments at the matrix-core threshold run on the MFMA kernels (narrow
tiles below 128 tokens, wide from 128), tested against the oracle at the
bf16-operand bar, 2e-2.

Also here: down rows whose chunks would exceed a lane's largest instance at
32 or 16 lanes per row (bf16 I = 2304, MXFP4 I = 7680), which take 64 lanes."""
import numpy as np
import pytest

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl
from gpu_util import call_tol, check_layer_against_oracle, dev, gpu_expert_fwd, gpu_layer_fwd, make_device_layer, note

pytestmark = pytest.mark.gpu


def _pack(codes):
    """[rows, cols] codes (0..15) to [rows, cols/2] bytes: per block of 32,
    element j in the low nibble of byte j, element j + 16 in its high nibble."""
    c = np.asarray(codes, np.uint8)
    b = c.reshape(c.shape[0], -1, 32)
    return (b[..., :16] | (b[..., 16:] << 4)).astype(np.uint8).reshape(c.shape[0], -1)


def _f16(v):
    return np.asarray(v, np.float16).view(np.uint16)


def _codes_layer():
    """One expert, H = I = 32.  Gate row i, column p holds code (i + p) % 16
    (every code at every position) with scale 2^(i % 5 - 2); up rows hold the
    value 1 everywhere (code 9, scale 1); down is the identity (code 9 on the
    diagonal, 8 elsewhere).  With x = e_p, out[h] = silu(((h + p) % 16 - 8)
    * 2^(h % 5 - 2))."""
    H = I = 32
    gate = np.array([[(i + p) % 16 for p in range(H)] for i in range(I)])
    up = np.full((I, H), 9)
    gu = _pack(np.concatenate([gate, up]))[None]
    s_gu = _f16(np.ones((1, 2 * I, 1)))
    s_gu[0, :I, 0] = _f16([2.0 ** (i % 5 - 2) for i in range(I)])
    dn = _pack(np.where(np.eye(H, I, dtype=bool), 9, 8))[None]
    s_dn = _f16(np.ones((1, H, 1)))
    spec = wl.LayerSpec(E=1, top_k=1, H=H, I=I, expert_dtype=wl.Q4_0, router_dtype=wl.BF16)
    w = dict(spec=spec, w_router=np.zeros((1, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu, s_down=s_dn)
    return spec, w


def test_q4_0_every_code_at_every_position_decodes_exactly():
    note("q4_0 all codes")
    spec, w = _codes_layer()
    layer = moe.DeviceLayer(w, device=dev())
    olayer = oracle.Layer(w)
    x = np.eye(32, dtype=np.float32)
    ids = np.zeros((32, 1), np.int32)
    got = gpu_expert_fwd(layer, x, ids, np.ones((32, 1)))
    ref = oracle.expert_fwd(olayer, x, ids, np.ones((32, 1)))
    assert np.allclose(got, ref, rtol=4e-7, atol=1e-30)
    want = np.array([[((h + p) % 16 - 8) * 2.0 ** (h % 5 - 2) for h in range(32)] for p in range(32)])
    assert np.allclose(got, want / (1.0 + np.exp(-want)), rtol=4e-7, atol=1e-30)


@pytest.mark.parametrize("shape,T", [((16, 4, 512, 256), 1), ((16, 4, 512, 256), 9), ((16, 4, 512, 512), 40),
                                     ((16, 4, 512, 256), 72), ((8, 2, 2048, 1536), 9), ((64, 8, 2048, 768), 24),
                                     ((8, 2, 256, 8192), 3)],
                         ids=["I256-T1", "I256-T9", "I512-T40", "I256-T72", "H2048-I1536-T9", "H2048-I768-T24",
                              "I8192-T3"])
def test_q4_0_layer_against_oracle(shape, T):
    """Down rows of 8, 16, 48, 24 and 256 chunks: 8, 16 or 64 lanes per row in
    pass 2; up to 64 tokens pass 2 carries the combine, from 65 it does not."""
    E, k, H, I = shape
    note("q4_0 layer E=%d k=%d H=%d I=%d T=%d" % (E, k, H, I, T))
    spec = wl.LayerSpec(E=E, top_k=k, H=H, I=I, expert_dtype=wl.Q4_0, router_dtype=wl.BF16)
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, H, draw=50 + T)
    check_layer_against_oracle(layer, olayer, x, tol=call_tol(layer, x))
    check_layer_against_oracle(layer, olayer, x, flags=moe.MOE_NO_MFMA, tol=1e-4)
    outs = [gpu_layer_fwd(layer, x, f | moe.MOE_NO_MFMA) for f in (moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE,
                                                                    moe.MOE_WALK_DEDUP_PASS1)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert (moe.moe_mfma_min_routes(layer.struct, T, 0) > 0) == (T >= 16)


@pytest.mark.parametrize("dtype,I", [(wl.BF16, 2304), (wl.MXFP4, 7680)], ids=["bf16-I2304", "mxfp4-I7680"])
@pytest.mark.parametrize("T", [3, 70])
def test_down_rows_beyond_eight_chunks_at_fewer_lanes(dtype, I, T):
    """288 bf16 chunks (a multiple of 32, not of 64) and 240 MXFP4 chunks (of
    16, not of 32) per down row: at 32 / 16 lanes a lane would hold 9 / 15
    chunks, more than the largest kernel instance; such rows take 64 lanes."""
    E, k, H = 4, 2, 256
    note("wide down rows dtype=%d I=%d T=%d" % (dtype, I, T))
    spec = wl.LayerSpec(E=E, top_k=k, H=H, I=I, expert_dtype=dtype, router_dtype=wl.BF16)
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, H, draw=60 + T)
    check_layer_against_oracle(layer, olayer, x, flags=moe.MOE_NO_MFMA, tol=1e-4)


# ---------------------------------------------------------------------------
# q4_0 segments on the matrix cores.  Narrow tiles (below 128 tokens): codes
# minus 8 as exact bf16 operands, each k-step (one block per row) summed fresh
# and scaled by the rows' binary16 scales.  Wide tiles: (code - 8) * scale
# rounded to bf16 once.

MIXED_Q4 = wl.LayerSpec(E=8, top_k=2, H=384, I=256, expert_dtype=wl.Q4_0)
LONG_K_Q4 = wl.LayerSpec(E=8, top_k=2, H=2560, I=640, expert_dtype=wl.Q4_0)
BF16_OPERAND_TOL = 2e-2


def _max_rel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _routing(kind, T, thr):
    rng = np.random.default_rng(T)
    rw = rng.uniform(0.1, 1.0, size=(T, 2))
    rw /= rw.sum(1, keepdims=True)
    if kind == "collide":  # every token on experts 0 and 1
        return np.tile(np.array([[0, 1]], np.int32), (T, 1)), rw
    ids = np.tile(np.array([[4, 5]], np.int32), (T, 1))  # edge: thr on {0, 1}, thr - 1 on {2, 3}
    ids[:thr] = [0, 1]
    ids[thr:2 * thr - 1] = [2, 3]
    return ids, rw


@pytest.mark.parametrize("T,kind", [(16, "collide"), (31, "edge"), (45, "collide"), (100, "collide")])
def test_q4_0_mfma_expert_fwd(T, kind):
    note("q4_0 mfma expert_fwd T=%d %s" % (T, kind))
    w, layer, olayer = make_device_layer(MIXED_Q4)
    x = wl.make_x(T, MIXED_Q4.H, draw=T)
    thr = moe.moe_mfma_min_routes(layer.struct, T, 0)
    assert thr > 0
    ids, rw = _routing(kind, T, thr)
    big = np.bincount(ids.ravel(), minlength=MIXED_Q4.E) >= thr
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    gemv = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA)
    note("  max rel err %.3g (GEMV path %.3g)" % (_max_rel(got, ref), _max_rel(gemv, ref)))
    assert _max_rel(got, ref) <= BF16_OPERAND_TOL
    assert _max_rel(gemv, ref) <= 1e-4
    assert not np.array_equal(got, gemv), "no segment took the MFMA path"
    small_only = ~big[ids].any(axis=1)
    assert np.array_equal(got[small_only], gemv[small_only])
    p1 = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_WALK_DEDUP_PASS1)
    assert _max_rel(p1, ref) <= BF16_OPERAND_TOL
    assert np.array_equal(gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_WALK_PER_ROUTE), gemv)
    assert np.array_equal(gpu_expert_fwd(layer, x, ids, rw), got)


@pytest.mark.parametrize("T", [128, 300])
def test_q4_0_wide_tiles(T):
    """From 128 tokens q4_0 segments run on the wide tiles, whose operands are
    (code - 8) * scale rounded to bf16 once: within the bf16-operand bar,
    deterministic, stable under token permutation, GEMV-only rows unchanged."""
    note("q4_0 wide tiles T=%d" % T)
    w, layer, olayer = make_device_layer(MIXED_Q4)
    x = wl.make_x(T, MIXED_Q4.H, draw=7)
    thr = moe.moe_mfma_min_routes(layer.struct, T, 0)
    assert thr > 0
    ids, rw = _routing("edge", T, thr)
    big = np.bincount(ids.ravel(), minlength=MIXED_Q4.E) >= thr
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    gemv = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA)
    note("  max rel err %.3g" % _max_rel(got, ref))
    assert _max_rel(got, ref) <= BF16_OPERAND_TOL
    assert not np.array_equal(got, gemv)
    small_only = ~big[ids].any(axis=1)
    assert np.array_equal(got[small_only], gemv[small_only])
    assert np.array_equal(gpu_expert_fwd(layer, x, ids, rw), got)
    perm = np.random.default_rng(T).permutation(T)
    c = gpu_expert_fwd(layer, x[perm], ids[perm], rw[perm])
    assert np.array_equal(c[np.argsort(perm)], got)


@pytest.mark.parametrize("T", [16, 45, 100])
def test_q4_0_mfma_narrow_long_k(T):
    """Pass 1 over 20 stages of 128 (the ring's steady state), pass 2 over 5;
    one to four token blocks; bitwise unchanged under token permutation."""
    note("q4_0 mfma long K T=%d" % T)
    w, layer, olayer = make_device_layer(LONG_K_Q4)
    x = wl.make_x(T, LONG_K_Q4.H, draw=40 + T)
    ids, rw = _routing("collide", T, 0)
    ref = oracle.expert_fwd(olayer, x, ids, rw)
    got = gpu_expert_fwd(layer, x, ids, rw)
    note("  max rel err %.3g" % _max_rel(got, ref))
    assert _max_rel(got, ref) <= BF16_OPERAND_TOL
    perm = np.random.default_rng(T).permutation(T)
    c = gpu_expert_fwd(layer, x[perm], ids[perm], rw[perm])
    assert np.array_equal(c[np.argsort(perm)], got)


def _q4_codes_layer_128():
    """One q4_0 expert, H = I = 128 (4 blocks per row).  Gate row i, column p
    holds code (i + p) % 16 with scale 2^((i + p // 32) % 5 - 2); up rows hold
    the value 1 (code 9, scale 1); down is the identity (code 9 on the
    diagonal, 8 elsewhere) with scale 2^((3 h + h // 32) % 4 - 1) on row h."""
    H = I = 128
    gate = np.array([[(i + p) % 16 for p in range(H)] for i in range(I)])
    up = np.full((I, H), 9)
    gu = _pack(np.concatenate([gate, up]))[None]
    s_gu = _f16(np.ones((1, 2 * I, H // 32)))
    for i in range(I):
        s_gu[0, i, :] = _f16([2.0 ** ((i + b) % 5 - 2) for b in range(H // 32)])
    dn = _pack(np.where(np.eye(H, I, dtype=bool), 9, 8))[None]
    s_dn = _f16(np.ones((1, H, I // 32)))
    for h in range(H):
        s_dn[0, h, :] = _f16(2.0 ** ((3 * h + h // 32) % 4 - 1))
    spec = wl.LayerSpec(E=1, top_k=1, H=H, I=I, expert_dtype=wl.Q4_0, router_dtype=wl.BF16)
    return dict(spec=spec, w_router=np.zeros((1, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu,
                s_down=s_dn)


@pytest.mark.parametrize("T", [127, 128], ids=["narrow", "wide"])
def test_q4_0_mfma_every_code_every_position(T):
    """Every q4_0 code at every column of a gate row, a power-of-two scale per
    (row, block), through the MFMA path (narrow and wide tiles): (code - 8) *
    scale is exact, so the only rounding is the activation's to bf16 before
    the down projection (at most 2^-8 relative).  A swapped nibble half,
    word or block, or a wrong row's scale, fails it."""
    note("q4_0 mfma all codes T=%d" % T)
    w = _q4_codes_layer_128()
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


def test_q4_0_scales_off_4_byte_alignment_stay_on_gemv():
    """q4_0 scale arrays 2-byte but not 4-byte aligned are accepted, and every
    segment stays on the GEMV kernels (the MFMA kernels copy scale words)."""
    import torch

    note("q4_0 2-byte aligned scales")
    w, layer, olayer = make_device_layer(MIXED_Q4)
    T = 64
    x = wl.make_x(T, MIXED_Q4.H, draw=11)
    ids, rw = _routing("collide", T, 0)
    shifted = layer.with_bias(None)
    for n in ("s_gate_up", "s_down"):
        src = layer.tensors[n].reshape(-1).view(torch.uint8)
        buf = torch.zeros(src.numel() + 16, dtype=torch.uint8, device=src.device)
        buf[2:2 + src.numel()] = src
        shifted.tensors[n + "_buf"] = buf
    t = shifted.tensors
    s = MIXED_Q4
    shifted.struct = moe.moe_layer_t(s.E, s.top_k, s.H, s.I, s.router_dtype, s.expert_dtype,
                                     t["w_router"].data_ptr(), t["w_gate_up"].data_ptr(), t["w_down"].data_ptr(),
                                     t["s_gate_up_buf"].data_ptr() + 2, t["s_down_buf"].data_ptr() + 2, None)
    got = gpu_expert_fwd(shifted, x, ids, rw)
    gemv = gpu_expert_fwd(layer, x, ids, rw, flags=moe.MOE_NO_MFMA)
    assert np.array_equal(got, gemv)
    assert not np.array_equal(gpu_expert_fwd(layer, x, ids, rw), gemv), "the aligned layer takes the MFMA path"
