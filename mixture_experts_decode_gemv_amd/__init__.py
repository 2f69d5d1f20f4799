"""MI355X (gfx950) sparse-MoE decode layer: thin ctypes binding over the C ABI.

The binding only marshals arguments: every step of the layer runs in the HIP
kernels of ``libmoe_gfx950.so`` (built in-tree by ``build.py``).  PyTorch is
used for device memory and streams.  There is no fallback: if the library is
missing or fails to load, importing the functions raises.

Entry points (same names as ``include/moe.h``): ``moe_workspace_bytes``,
``moe_workspace_init``, ``moe_route``, ``moe_sort``, ``moe_expert_fwd``,
``moe_layer_fwd``, ``moe_layer_fwd_static``, ``moe_layer_fwd_events``, ``moe_layer_routing``,
``moe_expert_usage``, ``moe_stack_workspace_bytes``,
``moe_stack_workspace_init``, ``moe_stack_fwd``, ``moe_mfma_min_routes``, ``moe_mfma_hot_routes``,
``moe_status_str``.  Tensor arguments may be torch
tensors (their ``data_ptr()`` is passed), raw integer device addresses or
None (NULL).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_Q4_0 = 0, 1, 2, 3, 4
MOE_WALK_DEDUP, MOE_WALK_PER_ROUTE, MOE_WALK_DEDUP_PASS1 = 0, 1, 2
MOE_ACCUM_RESIDUAL = 1 << 4
MOE_RMSNORM_IN = 1 << 6
MOE_NO_MFMA = 1 << 7

STATUS = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE", 4: "MOE_ERR_WORKSPACE",
          5: "MOE_ERR_HIP", 6: "MOE_ERR_UNSUPPORTED", 7: "MOE_ERR_ALIGN"}

EXPORTS = ("moe_workspace_bytes", "moe_workspace_init", "moe_route", "moe_sort", "moe_expert_fwd", "moe_layer_fwd",
           "moe_layer_fwd_static", "moe_layer_fwd_events", "moe_layer_routing", "moe_expert_usage", "moe_stack_workspace_bytes",
           "moe_stack_workspace_init", "moe_stack_fwd", "moe_mfma_min_routes", "moe_mfma_hot_routes",
           "moe_status_str")

MOE_N_STAGES = 6
MOE_STATIC_SCRATCH_BYTES = 16 << 20
STAGES = ("routing", "pass1_gemv", "pass1_mfma", "pass2_mfma", "pass2_gemv", "combine")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), _str(status)))


class moe_layer_t(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p), ("router_bias", ctypes.c_void_p)]


_lib = None


def lib():
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_gfx950.so is not built; run mixture_experts_decode_gemv_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        P = ctypes.POINTER(moe_layer_t)
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [P, i32]
        L.moe_mfma_min_routes.restype = i32
        L.moe_mfma_min_routes.argtypes = [P, i32, u32]
        L.moe_mfma_hot_routes.restype = i32
        L.moe_mfma_hot_routes.argtypes = [P, i32, u32]
        L.moe_workspace_init.restype = ctypes.c_int
        L.moe_workspace_init.argtypes = [P, i32, vp, sz, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [P, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_sort.restype = ctypes.c_int
        L.moe_sort.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.moe_expert_fwd.restype = ctypes.c_int
        L.moe_expert_fwd.argtypes = [P, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, sz, vp]
        L.moe_layer_fwd.restype = ctypes.c_int
        L.moe_layer_fwd.argtypes = [P, vp, i32, vp, u32, vp, sz, vp]
        L.moe_layer_fwd_static.restype = ctypes.c_int
        L.moe_layer_fwd_static.argtypes = [P, vp, i32, vp, u32, vp]
        L.moe_layer_fwd_events.restype = ctypes.c_int
        L.moe_layer_fwd_events.argtypes = [P, vp, i32, vp, u32, vp, sz, vp, ctypes.POINTER(ctypes.c_void_p)]
        pp = ctypes.POINTER(ctypes.c_void_p)
        L.moe_layer_routing.restype = ctypes.c_int
        L.moe_layer_routing.argtypes = [P, i32, vp, sz, pp, pp, pp, pp, pp, pp, pp]
        L.moe_expert_usage.restype = ctypes.c_int
        L.moe_expert_usage.argtypes = [vp, vp, i32, vp, vp]
        L.moe_stack_workspace_bytes.restype = sz
        L.moe_stack_workspace_bytes.argtypes = [P, i32]
        L.moe_stack_workspace_init.restype = ctypes.c_int
        L.moe_stack_workspace_init.argtypes = [P, i32, vp, sz, vp]
        L.moe_stack_fwd.restype = ctypes.c_int
        L.moe_stack_fwd.argtypes = [P, i32, vp, i32, vp, u32, vp, sz, vp]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _str(status):
    try:
        return lib().moe_status_str(int(status)).decode()
    except Exception:  # noqa: BLE001 - message only
        return "?"


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != 0:
        raise MoeError(fn, st)


def moe_status_str(status: int) -> str:
    return _str(status)


def moe_workspace_bytes(layer: moe_layer_t, max_tokens: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(layer), int(max_tokens)))


def moe_mfma_min_routes(layer: moe_layer_t, T: int, flags: int = 0) -> int:
    """Routes an expert needs in a call of T tokens for its segment to run on
    the matrix cores; 0 when no segment of such a call does, -1 on bad
    arguments."""
    return int(lib().moe_mfma_min_routes(ctypes.byref(layer), int(T), int(flags)))


def moe_mfma_hot_routes(layer: moe_layer_t, T: int, flags: int = 0) -> int:
    """Routes the largest expert of a moe_layer_fwd / moe_stack_fwd call must
    hold for any segment to take the MFMA path (0: never; -1: invalid)."""
    return int(lib().moe_mfma_hot_routes(ctypes.byref(layer), int(T), int(flags)))


def moe_workspace_init(layer, max_tokens, ws, ws_bytes, stream=None):
    _check("moe_workspace_init", lib().moe_workspace_init(ctypes.byref(layer), int(max_tokens), _p(ws),
                                                          int(ws_bytes), _s(stream)))


def moe_route(layer, x, logits_in, T, logits_out, topk_ids, topk_w, ws=None, ws_bytes=0, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(layer), _p(x), _p(logits_in), int(T), _p(logits_out),
                                        _p(topk_ids), _p(topk_w), _p(ws), int(ws_bytes), _s(stream)))


def moe_sort(topk_ids, T, k, E, counts, offsets, sorted_routes, uniq, n_uniq, stream=None):
    _check("moe_sort", lib().moe_sort(_p(topk_ids), int(T), int(k), int(E), _p(counts), _p(offsets),
                                      _p(sorted_routes), _p(uniq), _p(n_uniq), _s(stream)))


def moe_expert_fwd(layer, x, T, topk_ids, topk_w, counts, offsets, sorted_routes, uniq, n_uniq, out, flags=0,
                   ws=None, ws_bytes=0, stream=None):
    _check("moe_expert_fwd",
           lib().moe_expert_fwd(ctypes.byref(layer), _p(x), int(T), _p(topk_ids), _p(topk_w), _p(counts),
                                _p(offsets), _p(sorted_routes), _p(uniq), _p(n_uniq), _p(out), int(flags), _p(ws),
                                int(ws_bytes), _s(stream)))


def moe_layer_fwd(layer, x, T, out, flags=0, ws=None, ws_bytes=0, stream=None):
    _check("moe_layer_fwd", lib().moe_layer_fwd(ctypes.byref(layer), _p(x), int(T), _p(out), int(flags), _p(ws),
                                                int(ws_bytes), _s(stream)))


def moe_layer_fwd_static(layer, x, T, out, flags=0, stream=None):
    """moe_layer_fwd with the library's own device scratch (no workspace)."""
    _check("moe_layer_fwd_static", lib().moe_layer_fwd_static(ctypes.byref(layer), _p(x), int(T), _p(out),
                                                              int(flags), _s(stream)))


def moe_layer_fwd_events(layer, x, T, out, flags=0, ws=None, ws_bytes=0, stream=None, events=None):
    """``events``: MOE_N_STAGES + 1 raw hipEvent_t handles (ints), or None."""
    arr = None
    if events is not None:
        if len(events) != MOE_N_STAGES + 1:
            raise ValueError("moe_layer_fwd_events needs %d events" % (MOE_N_STAGES + 1))
        arr = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
    _check("moe_layer_fwd_events", lib().moe_layer_fwd_events(ctypes.byref(layer), _p(x), int(T), _p(out),
                                                              int(flags), _p(ws), int(ws_bytes), _s(stream), arr))


ROUTING_FIELDS = ("topk_ids", "topk_w", "counts", "offsets", "sorted_routes", "uniq", "n_uniq")


def moe_layer_routing(layer, T, ws, ws_bytes) -> dict:
    """Device addresses (ints) of the routing a moe_layer_fwd call left in ws."""
    ptrs = [ctypes.c_void_p() for _ in ROUTING_FIELDS]
    _check("moe_layer_routing", lib().moe_layer_routing(ctypes.byref(layer), int(T), _p(ws), int(ws_bytes),
                                                        *[ctypes.byref(p) for p in ptrs]))
    return {n: p.value for n, p in zip(ROUTING_FIELDS, ptrs)}


def moe_expert_usage(counts, n_uniq, E, hist, stream=None):
    """hist[e] += counts[e] (uint64 device counters), skipped when *n_uniq < 0."""
    _check("moe_expert_usage", lib().moe_expert_usage(_p(counts), _p(n_uniq), int(E), _p(hist), _s(stream)))


def moe_stack_workspace_bytes(layer: moe_layer_t, max_tokens: int) -> int:
    return int(lib().moe_stack_workspace_bytes(ctypes.byref(layer), int(max_tokens)))


def moe_stack_workspace_init(layer, max_tokens, ws, ws_bytes, stream=None):
    _check("moe_stack_workspace_init", lib().moe_stack_workspace_init(ctypes.byref(layer), int(max_tokens), _p(ws),
                                                                      int(ws_bytes), _s(stream)))


def moe_stack_fwd(layers, x, T, out, flags=0, ws=None, ws_bytes=0, stream=None):
    """``layers``: a sequence of moe_layer_t (or None: NULL, for the error tests)."""
    arr = None
    n = 0
    if layers is not None:
        n = len(layers)
        arr = (moe_layer_t * max(n, 1))(*layers)
    _check("moe_stack_fwd", lib().moe_stack_fwd(arr, int(n), _p(x), int(T), _p(out), int(flags), _p(ws),
                                                int(ws_bytes), _s(stream)))


class DeviceLayer:
    """One layer's weights resident on the GPU plus its ``moe_layer_t``.

    ``w`` is a host dict with ``spec`` (E, top_k, H, I, expert_dtype,
    router_dtype) and arrays ``w_router``, ``w_gate_up``, ``w_down`` (fp32,
    bf16 bit patterns as uint16 or E4M3 codes as uint8), ``s_gate_up``,
    ``s_down`` (fp8 block scales) and optionally ``router_bias``.
    """

    def __init__(self, w: dict, router_bias=None, device="cuda"):
        import numpy as np
        import torch

        spec = w["spec"]
        self.spec = spec
        self.tensors = {}
        for n in ("w_router", "w_gate_up", "w_down", "s_gate_up", "s_down"):
            a = w.get(n)
            if a is None:
                self.tensors[n] = None
                continue
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            self.tensors[n] = torch.from_numpy(a).to(device)
        self.tensors["router_bias"] = (None if router_bias is None else
                                       torch.from_numpy(np.ascontiguousarray(router_bias, np.float32)).to(device))
        self.struct = self._struct(self.tensors["router_bias"])

    def _struct(self, bias):
        t = self.tensors
        s = self.spec
        return moe_layer_t(s.E, s.top_k, s.H, s.I, s.router_dtype, s.expert_dtype, _p(t["w_router"]),
                           _p(t["w_gate_up"]), _p(t["w_down"]), _p(t["s_gate_up"]), _p(t["s_down"]), _p(bias))

    def with_bias(self, router_bias, top_k=None):
        """Same weights, another router bias and optionally another top_k (a
        shallow view sharing memory)."""
        import dataclasses

        import numpy as np
        import torch

        other = DeviceLayer.__new__(DeviceLayer)
        other.spec = self.spec if top_k is None else dataclasses.replace(self.spec, top_k=top_k)
        other.tensors = dict(self.tensors)
        other.tensors["router_bias"] = (None if router_bias is None else torch.from_numpy(
            np.ascontiguousarray(router_bias, np.float32)).to(self.tensors["w_router"].device))
        other.struct = other._struct(other.tensors["router_bias"])
        return other

    def workspace(self, max_tokens: int, stream=None):
        """A workspace for up to max_tokens tokens, initialised on `stream`
        (torch's current stream if None)."""
        import torch

        n = moe_workspace_bytes(self.struct, max_tokens)
        if n == 0:
            raise MoeError("moe_workspace_bytes", 1)
        dev = self.tensors["w_router"].device
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        moe_workspace_init(self.struct, max_tokens, ws, n, stream if stream is not None else torch.cuda.current_stream(dev))
        return ws
