"""The C-ABI library loads, exports what include/moe.h declares, and
validates arguments on the host (no GPU work is launched here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_decode_gemv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert sorted(moe.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def _layer(**kw):
    d = dict(E=8, top_k=2, H=64, I=32, router_dtype=moe.MOE_F32, expert_dtype=moe.MOE_F32,
             w_router=0x1000, w_gate_up=0x2000, w_down=0x3000, s_gate_up=None, s_down=None, router_bias=None)
    d.update(kw)
    return moe.moe_layer_t(*[d[f] for f, _ in moe.moe_layer_t._fields_])


def test_workspace_bytes():
    n = moe.moe_workspace_bytes(_layer(), 4)
    assert n > 4 * 2 * (64 + 32) * 4
    assert moe.moe_workspace_bytes(_layer(), 0) > 0
    assert moe.moe_workspace_bytes(_layer(top_k=9), 4) == 0
    assert moe.moe_workspace_bytes(_layer(), -1) == 0
    assert moe.moe_workspace_bytes(_layer(), 64) > moe.moe_workspace_bytes(_layer(), 4)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), 1), (dict(top_k=9), 1), (dict(E=2000, top_k=2), 2), (dict(top_k=33, E=64), 2),
    (dict(H=66), 2), (dict(expert_dtype=7), 3), (dict(router_dtype=moe.MOE_FP8_E4M3), 3),
    (dict(expert_dtype=moe.MOE_FP8_E4M3, H=64), 2), (dict(expert_dtype=moe.MOE_BF16, I=36), 2),
    (dict(expert_dtype=moe.MOE_BF16, H=8192, router_dtype=moe.MOE_BF16), 2),
])
def test_layer_validation(kw, status):
    L = _layer(**kw)
    st = moe.lib().moe_layer_fwd(ctypes.byref(L), 0x4000, 4, 0x5000, 0, 0x6000, 1 << 30, None)
    assert st == status


def test_argument_errors_return_before_any_launch():
    L = _layer()
    lib = moe.lib()
    # NULL x / out
    assert lib.moe_layer_fwd(ctypes.byref(L), None, 4, 0x5000, 0, 0x6000, 1 << 30, None) == 1
    # workspace too small
    assert lib.moe_layer_fwd(ctypes.byref(L), 0x4000, 4, 0x5000, 0, 0x6000, 16, None) == 4
    # misaligned activations
    assert lib.moe_layer_fwd(ctypes.byref(L), 0x4004, 4, 0x5000, 0, 0x6000, 1 << 30, None) == 7
    # misaligned weights
    assert lib.moe_layer_fwd(ctypes.byref(_layer(w_gate_up=0x2008)), 0x4000, 4, 0x5000, 0, 0x6000, 1 << 30,
                             None) == 7
    # unknown walk
    assert lib.moe_layer_fwd(ctypes.byref(L), 0x4000, 4, 0x5000, 5, 0x6000, 1 << 30, None) == 1
    # T == 0 is a no-op
    assert lib.moe_layer_fwd(ctypes.byref(L), 0x4000, 0, 0x5000, 0, 0x6000, 1 << 30, None) == 0
    # route needs x or logits
    assert lib.moe_route(ctypes.byref(L), None, None, 4, None, 0x100, 0x200, None, 0, None) == 1
    # sort argument checks
    assert lib.moe_sort(0x100, 4, 3, 2, 0x1, 0x2, 0x3, 0x4, 0x5, None) == 1
    assert lib.moe_sort(0x100, 4, 2, 2000, 0x1, 0x2, 0x3, 0x4, 0x5, None) == 2
    assert lib.moe_sort(None, 4, 2, 8, 0x1, 0x2, 0x3, 0x4, 0x5, None) == 1
    assert lib.moe_sort(0x100, 0, 2, 8, 0x1, 0x2, 0x3, 0x4, 0x5, None) == 0
    # fp8 without scales
    L8 = _layer(expert_dtype=moe.MOE_FP8_E4M3, H=128, I=128)
    assert lib.moe_layer_fwd(ctypes.byref(L8), 0x4000, 4, 0x5000, 0, 0x6000, 1 << 30, None) == 1


def test_status_strings():
    for st in range(8):
        assert moe.moe_status_str(st) and moe.moe_status_str(st) != "unknown status"
    assert moe.moe_status_str(99) == "unknown status"


def test_routing_accessor_points_into_the_workspace():
    L = _layer()
    n = moe.moe_workspace_bytes(L, 4)
    r = moe.moe_layer_routing(L, 4, 0x10000, n)
    for v in r.values():
        assert 0x10000 <= v < 0x10000 + n
    with pytest.raises(moe.MoeError):
        moe.moe_layer_routing(L, 4, 0x10000, 8)


def test_workspace_front_is_fixed():
    """The synchronisation words sit in a front of fixed size at the start of
    every workspace, whatever the batch, the layer shape or the byte size the
    call passes: the data region (logits first) starts at the same offset
    for all of them.  A batch larger than ws_bytes holds, or above 65536
    tokens, is refused."""
    starts = set()
    for L in (_layer(), _layer(E=256, top_k=8, H=2048, I=768, expert_dtype=moe.MOE_BF16,
                               router_dtype=moe.MOE_BF16)):
        for cap in (64, 300):
            n = moe.moe_workspace_bytes(L, cap)
            for T in (1, 3, 17, 64):
                r = moe.moe_layer_routing(L, T, 0x10000, n)
                starts.add(r["topk_ids"] - 0x10000 - ((T * L.E * 4 + 255) // 256) * 256)
            with pytest.raises(moe.MoeError):
                moe.moe_layer_routing(L, cap + 1, 0x10000, n)
    assert len(starts) == 1 and starts.pop() >= 65537 * 4
    L = _layer()
    assert moe.moe_workspace_bytes(L, 65536) > 0
    assert moe.moe_workspace_bytes(L, 65537) == 0
    assert moe.moe_stack_workspace_bytes(L, 65537) == 0


def test_expert_usage_argument_errors():
    lib = moe.lib()
    assert lib.moe_expert_usage(None, 0x200, 8, 0x300, None) == 1
    assert lib.moe_expert_usage(0x100, None, 8, 0x300, None) == 1
    assert lib.moe_expert_usage(0x100, 0x200, 8, None, None) == 1
    assert lib.moe_expert_usage(0x100, 0x200, 0, 0x300, None) == 1
    assert lib.moe_expert_usage(0x100, 0x200, 2000, 0x300, None) == 2
    assert lib.moe_expert_usage(0x100, 0x200, 8, 0x304, None) == 7


def test_mxfp4_layer_validation():
    lib = moe.lib()
    ok = dict(expert_dtype=moe.MOE_MXFP4, H=64, I=64, s_gate_up=0x7000, s_down=0x8000)
    args = (0x4000, 4, 0x5000, 0, 0x6000, 1 << 30, None)
    # H, I multiples of 32
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, H=48))), *args) == 2
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, I=80))), *args) == 2
    # scales required
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, s_down=None))), *args) == 1
    # at most 512 chunks of 32 codes per row
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, H=32 * 513, router_dtype=moe.MOE_BF16))), *args) == 2



def test_q4_0_layer_validation():
    lib = moe.lib()
    ok = dict(expert_dtype=moe.MOE_Q4_0, H=64, I=64, s_gate_up=0x7000, s_down=0x8000)
    args = (0x4000, 4, 0x5000, 0, 0x6000, 1 << 30, None)
    # H, I multiples of 32
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, H=48))), *args) == 2
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, I=80))), *args) == 2
    # scales required, 2-byte aligned
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, s_gate_up=None))), *args) == 1
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, s_down=0x8001))), *args) == 7
    # at most 256 blocks of 32 codes per row (4 chunks per lane)
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, I=32 * 257))), *args) == 2
    # an unknown expert dtype
    assert lib.moe_layer_fwd(ctypes.byref(_layer(**dict(ok, expert_dtype=5))), *args) == 3

def test_stack_workspace_and_argument_errors():
    """Stack workspace size and the host-side checks of moe_stack_fwd."""
    L = _layer()
    n = moe.moe_stack_workspace_bytes(L, 4)
    assert n >= 2 * moe.moe_workspace_bytes(L, 4) + 2 * 4 * 64 * 4
    assert moe.moe_stack_workspace_bytes(_layer(top_k=9), 4) == 0
    x = out = ws = 0x10000

    def status(layers, T=4, ws_bytes=n, flags=0, xp=x, wsp=ws):
        try:
            moe.moe_stack_fwd(layers, xp, T, out, flags, wsp, ws_bytes)
        except moe.MoeError as e:
            return e.status
        return 0

    assert status(None) == 1                                  # no layers
    assert status([]) == 1                                    # n_layers = 0
    assert status([L, _layer(I=64)]) == 2                     # shapes differ
    assert status([L, _layer(expert_dtype=moe.MOE_BF16)]) == 2
    assert status([L, L], xp=None) == 1
    assert status([L, L], flags=3) == 1                       # no such walk
    assert status([L, L], xp=0x10004) == 7                    # misaligned x
    assert status([L, L], ws_bytes=n - 1) == 4                # workspace too small for T = 4
    assert status([L, L], wsp=None) == 4
    assert status([L, L], T=0) == 0                           # no-op
    for bad in (None, 0x10008):
        try:
            moe.moe_stack_workspace_init(L, 4, bad, n)
            st = 0
        except moe.MoeError as e:
            st = e.status
        assert st == (1 if bad is None else 7)


def test_static_entry_point_validation():
    """moe_layer_fwd_static refuses bad arguments and a batch that needs more
    than its 16 MiB of scratch on the host, before anything is enqueued."""
    lib = moe.lib()
    L = _layer(E=256, top_k=8, H=2048, I=768, expert_dtype=moe.MOE_BF16, router_dtype=moe.MOE_BF16)
    x = out = 0x10000
    assert moe.MOE_STATIC_SCRATCH_BYTES == 16 << 20
    assert moe.moe_workspace_bytes(L, 159) <= moe.MOE_STATIC_SCRATCH_BYTES < moe.moe_workspace_bytes(L, 160)
    assert lib.moe_layer_fwd_static(ctypes.byref(L), x, 160, out, 0, None) == 4   # scratch too small
    assert lib.moe_layer_fwd_static(ctypes.byref(L), x, 70000, out, 0, None) == 2  # above 65536 tokens
    assert lib.moe_layer_fwd_static(ctypes.byref(L), None, 4, out, 0, None) == 1
    assert lib.moe_layer_fwd_static(ctypes.byref(L), x, -1, out, 0, None) == 1
    assert lib.moe_layer_fwd_static(ctypes.byref(L), x, 4, out, 3, None) == 1     # no such walk
    assert lib.moe_layer_fwd_static(ctypes.byref(L), 0x10004, 4, out, 0, None) == 7
    assert lib.moe_layer_fwd_static(ctypes.byref(L), x, 0, out, 0, None) == 0     # no-op
    assert lib.moe_layer_fwd_static(ctypes.byref(_layer(top_k=9)), x, 4, out, 0, None) == 1


def test_mfma_min_routes():
    """The matrix-core thresholds a call applies (host only): experts of 5
    routes or more below 128 tokens when the largest holds 8 or more, 4 from
    128, none below 16 tokens, for fp32 experts, for H or I not a multiple of
    128, with MOE_NO_MFMA or the per-route walk, or for activation rows of
    2 GiB or more."""
    L = _layer(H=256, I=128, expert_dtype=moe.MOE_BF16)
    assert moe.moe_mfma_min_routes(L, 15) == 0 and moe.moe_mfma_hot_routes(L, 15) == 0
    assert moe.moe_mfma_min_routes(L, 16) == 5 and moe.moe_mfma_hot_routes(L, 16) == 8
    assert moe.moe_mfma_min_routes(L, 127) == 5 and moe.moe_mfma_hot_routes(L, 127) == 8
    assert moe.moe_mfma_min_routes(L, 128) == 4 and moe.moe_mfma_hot_routes(L, 128) == 4
    assert moe.moe_mfma_min_routes(L, 4096) == 4 and moe.moe_mfma_hot_routes(L, 4096) == 4
    assert moe.moe_mfma_min_routes(L, 64, moe.MOE_WALK_DEDUP_PASS1) == 5
    assert moe.moe_mfma_min_routes(L, 64, moe.MOE_NO_MFMA) == 0 and moe.moe_mfma_hot_routes(L, 64, moe.MOE_NO_MFMA) == 0
    assert moe.moe_mfma_min_routes(L, 64, moe.MOE_WALK_PER_ROUTE) == 0
    assert moe.moe_mfma_min_routes(_layer(H=256, I=128, expert_dtype=moe.MOE_FP8_E4M3, s_gate_up=0x4000,
                                          s_down=0x5000), 64) == 5
    assert moe.moe_mfma_min_routes(_layer(H=256, I=128), 64) == 0  # fp32 experts
    assert moe.moe_mfma_min_routes(_layer(H=192, I=128, expert_dtype=moe.MOE_BF16), 64) == 0
    # activation rows of 2 GiB or more (R x I x 4 bytes) stay on the GEMV kernels
    Lw = _layer(H=256, I=4096, expert_dtype=moe.MOE_BF16)
    assert moe.moe_mfma_min_routes(Lw, 65535) == 4
    assert moe.moe_mfma_min_routes(Lw, 65536) == 0 and moe.moe_mfma_hot_routes(Lw, 65536) == 0
    assert moe.moe_mfma_min_routes(L, -1) == -1 and moe.moe_mfma_hot_routes(L, -1) == -1
    assert moe.moe_mfma_min_routes(_layer(top_k=9), 64) == -1
    assert moe.moe_mfma_min_routes(L, 64, 7) == -1  # unknown walk
