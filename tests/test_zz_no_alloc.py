"""moe_layer_fwd_static, the entry point for callers that cannot allocate:
the layer with its scratch in the library's own device array.  Its output
must equal moe_layer_fwd's bitwise (the same kernels on the same inputs), on
calls in a row whose second is smaller, with layers of other shapes and
flags sharing the array in between, with matrix-core segments in order and
(from 128 tokens) where moe_layer_fwd would fork them onto a side stream.
A batch that needs more than the array holds is refused before any work is
enqueued."""
import numpy as np
import pytest
import torch

import mixture_experts_decode_gemv_amd as moe
import workload as wl
from gpu_util import gpu_layer_fwd, make_device_layer, note, stream, to_dev

pytestmark = pytest.mark.gpu


def _static(layer, x, flags=0):
    xd = to_dev(x.astype(np.float32))
    out = torch.full_like(xd, float("nan"))
    moe.moe_layer_fwd_static(layer.struct, xd, x.shape[0], out, flags, stream())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_static_scratch_two_calls_second_smaller():
    w, layer, olayer = make_device_layer(wl.SWEEP)
    for T in (64, 8):
        note("static scratch, sweep layer, T=%d" % T)
        x = wl.make_x(T, wl.SWEEP.H, draw=1100 + T)
        got = _static(layer, x)
        assert np.isfinite(got).all()
        assert np.array_equal(got, gpu_layer_fwd(layer, x))


def test_static_scratch_shared_by_shapes_and_flags():
    norm_res = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
    ws_, stack_layer, _ = make_device_layer(wl.STACK)
    wt, tiny, _ = make_device_layer(wl.TINY)
    wk, skew, _ = make_device_layer(wl.SKEWED, wl.zipf_bias(wl.SKEWED.E))
    plan = [(stack_layer, wl.STACK, 4, norm_res), (tiny, wl.TINY, 4, 0), (skew, wl.SKEWED, 150, 0),
            (skew, wl.SKEWED, 64, 0), (stack_layer, wl.STACK, 1, norm_res), (tiny, wl.TINY, 3, 0)]
    for i, (layer, spec, T, flags) in enumerate(plan):
        note("static scratch, call %d: E=%d H=%d T=%d flags=%d" % (i, spec.E, spec.H, T, flags))
        x = wl.make_x(T, spec.H, draw=1200 + i)
        got = _static(layer, x, flags)
        assert np.isfinite(got).all()
        assert np.array_equal(got, gpu_layer_fwd(layer, x, flags)), "call %d" % i


def test_static_scratch_refuses_a_batch_it_cannot_hold():
    w, layer, olayer = make_device_layer(wl.TINY)
    spec = wl.SWEEP
    big = moe.moe_layer_t(spec.E, spec.top_k, spec.H, spec.I, spec.router_dtype, spec.expert_dtype,
                          layer.struct.w_router, layer.struct.w_gate_up, layer.struct.w_down, None, None, None)
    T = 160  # needs more than MOE_STATIC_SCRATCH_BYTES at this shape
    assert moe.moe_workspace_bytes(big, T) > moe.MOE_STATIC_SCRATCH_BYTES >= moe.moe_workspace_bytes(big, T - 1)
    x = torch.zeros((T, spec.H), dtype=torch.float32, device="cuda:0")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_fwd_static(big, x, T, x, 0, stream())
    assert e.value.status == 4


@pytest.mark.parametrize("dtype", [wl.FP8, wl.MXFP4, wl.Q4_0], ids=["fp8", "mxfp4", "q4_0"])
def test_static_scratch_weight_formats(dtype):
    """The skewed layer shape with fp8, MXFP4 and q4_0 experts: 150 tokens
    (wide tiles), 64 (narrow MFMA items: some expert holds 8 or more routes)
    and 8 (GEMV kernels only), in that order on the one array."""
    spec = wl.LayerSpec(E=256, top_k=6, H=2048, I=768, expert_dtype=dtype)
    w, layer, _ = make_device_layer(spec, wl.zipf_bias(spec.E))
    for T in (150, 64, 8):
        note("static scratch, skewed shape, expert dtype %d, T=%d" % (dtype, T))
        assert moe.moe_workspace_bytes(layer.struct, T) <= moe.MOE_STATIC_SCRATCH_BYTES
        x = wl.make_x(T, spec.H, draw=1300 + T)
        got = _static(layer, x)
        assert np.isfinite(got).all()
        assert np.array_equal(got, gpu_layer_fwd(layer, x))
