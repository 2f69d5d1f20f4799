"""MXFP4 expert weights (OCP microscaling: E2M1 codes two per byte, one E8M0
scale per 32 elements of a row) on the GEMV path (MOE_NO_MFMA: segments with
moe_mfma_min_routes() routes or more would otherwise run on the matrix
cores, tested with the other MFMA paths), against the oracle.

The GPU converts codes with the hardware E2M1 conversion and applies each
chunk's scale to the chunk's fp32 sum; every weight is exact in fp32, so the
outputs follow the oracle to fp32 rounding (bar 1e-4, as for the other GEMV
paths).  The per-code test places every code at every element position of a
32-element block, so a swapped nibble or byte order fails it."""
import numpy as np
import pytest

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl
from gpu_util import check_layer_against_oracle, dev, gpu_expert_fwd, gpu_layer_fwd, make_device_layer, note

pytestmark = pytest.mark.gpu


def _pack(codes):
    """[rows, cols] codes (0..15) to [rows, cols/2] bytes, even element low."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _codes_layer():
    """One expert, H = I = 32.  Gate row i, column p holds code (i + p) % 16
    (every code at every position) with scale 2^(i % 5 - 2); up rows hold
    1.0 everywhere; down is the identity.  With x = e_p, out[h] =
    silu(value((h + p) % 16) * 2^(h % 5 - 2)) * 1."""
    H = I = 32
    one = wl.e2m1_encode(1.0)
    gate = np.array([[(i + p) % 16 for p in range(H)] for i in range(I)])
    up = np.full((I, H), one)
    gu = _pack(np.concatenate([gate, up]))[None]
    s_gu = np.full((1, 2 * I, 1), 127, np.uint8)
    s_gu[0, :I, 0] = [127 + i % 5 - 2 for i in range(I)]
    dn = _pack(np.where(np.eye(H, I, dtype=bool), one, 0))[None]
    s_dn = np.full((1, H, 1), 127, np.uint8)
    spec = wl.LayerSpec(E=1, top_k=1, H=H, I=I, expert_dtype=wl.MXFP4, router_dtype=wl.BF16)
    w = dict(spec=spec, w_router=np.zeros((1, H), np.uint16), w_gate_up=gu, w_down=dn, s_gate_up=s_gu, s_down=s_dn)
    return spec, w


def test_mxfp4_every_code_at_every_position_decodes_exactly():
    note("mxfp4 all codes")
    spec, w = _codes_layer()
    layer = moe.DeviceLayer(w, device=dev())
    olayer = oracle.Layer(w)
    x = np.eye(32, dtype=np.float32)
    ids = np.zeros((32, 1), np.int32)
    got = gpu_expert_fwd(layer, x, ids, np.ones((32, 1)))
    ref = oracle.expert_fwd(olayer, x, ids, np.ones((32, 1)))
    assert np.allclose(got, ref, rtol=4e-7, atol=1e-30)
    vals = {oracle.e2m1_value(c) for c in range(16)}
    assert len(vals) == 15  # +0 and -0 compare equal


@pytest.mark.parametrize("shape,T", [((16, 4, 512, 256), 1), ((16, 4, 512, 256), 9), ((16, 4, 512, 512), 40),
                                     ((8, 2, 2048, 1536), 9), ((64, 8, 2048, 768), 24)],
                         ids=["I256-T1", "I256-T9", "I512-T40", "H2048-I1536-T9", "H2048-I768-T24"])
def test_mxfp4_layer_against_oracle(shape, T):
    """Down rows of 8, 16, 48 and 24 chunks: 8 or 16 lanes per row in pass 2."""
    E, k, H, I = shape
    note("mxfp4 layer E=%d k=%d H=%d I=%d T=%d" % (E, k, H, I, T))
    spec = wl.LayerSpec(E=E, top_k=k, H=H, I=I, expert_dtype=wl.MXFP4, router_dtype=wl.BF16)
    w, layer, olayer = make_device_layer(spec)
    x = wl.make_x(T, H, draw=40 + T)
    check_layer_against_oracle(layer, olayer, x, flags=moe.MOE_NO_MFMA, tol=1e-4)
    outs = [gpu_layer_fwd(layer, x, f | moe.MOE_NO_MFMA) for f in (moe.MOE_WALK_DEDUP, moe.MOE_WALK_PER_ROUTE,
                                                                    moe.MOE_WALK_DEDUP_PASS1)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
