"""q4_0 expert weights (blocks of 32 elements along a row with one binary16
scale d, 4-bit codes q, value (q - 8) * d; element j of a block in the low
nibble of byte j, element j + 16 in its high nibble) on the GEMV path,
against the oracle.

The GPU converts each code to the exact fp32 value q - 8, sums a chunk's
products in fp32 and applies the chunk's scale to the sum; every weight is
exact in fp32, so the outputs follow the oracle to fp32 rounding (bar 1e-4,
as for the other GEMV paths).  The per-code test places every code at every
element position of a block, so a swapped nibble half or code offset fails
it.  q4_0 experts never run on the matrix cores.

Also here: down rows whose chunks would exceed a lane's largest instance at
32 or 16 lanes per row (bf16 I = 2304, MXFP4 I = 7680), which take 64 lanes."""
import numpy as np
import pytest

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl
from gpu_util import check_layer_against_oracle, dev, gpu_expert_fwd, gpu_layer_fwd, make_device_layer, note

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
    check_layer_against_oracle(layer, olayer, x, tol=1e-4)
    outs = [gpu_layer_fwd(layer, x, f) for f in (moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE,
                                                  moe.MOE_WALK_DEDUP_PASS1, moe.MOE_NO_MFMA)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert moe.moe_mfma_min_routes(layer.struct, T, 0) == 0


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
