"""CPU oracle of the sparse-MoE decode layer (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the GPU library or its binding.  It
shares no code with the GPU path.  See ``moe_oracle.c`` for what each step
computes and which page passage it follows; everything is accumulated in
double and returned as float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, FP8 = 0, 1, 2
RMSNORM, RESIDUAL = 1, 2
WALK_PER_ROUTE, WALK_GROUPED = 0, 1
RMS_EPS = 1e-6


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OracleLayer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p), ("router_bias", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        P = ctypes.POINTER(OracleLayer)
        L.oracle_bf16_value.restype = dbl
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_value.restype = dbl
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_value.restype = dbl
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_value.restype = dbl
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_f16_value.restype = dbl
        L.oracle_f16_value.argtypes = [ctypes.c_uint16]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [i32, i32, vp, dbl, vp]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [P, i32, vp, vp]
        L.oracle_select.restype = None
        L.oracle_select.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_sort.restype = i32
        L.oracle_sort.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_walk_per_route.restype = None
        L.oracle_walk_per_route.argtypes = [P, i32, vp, vp, vp, i32]
        L.oracle_walk_grouped.restype = None
        L.oracle_walk_grouped.argtypes = [P, i32, vp, vp, vp]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_expert_fwd.restype = i32
        L.oracle_expert_fwd.argtypes = [P, i32, vp, vp, vp, i32, vp, i32]
        L.oracle_moe_layer.restype = i32
        L.oracle_moe_layer.argtypes = [P, i32, vp, vp, i32, dbl, i32, vp, vp, vp, vp, i32]
        L.oracle_check_layer.restype = i32
        L.oracle_check_layer.argtypes = [P]
        _lib = L
    return _lib


def _threads(n):
    return n if n else max(1, min(os.cpu_count() or 1, 16))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Layer:
    """Weights of one layer, as host arrays, bound into the C struct.

    ``w`` holds ``w_router``, ``w_gate_up``, ``w_down`` (fp32 arrays, bf16 as
    uint16 bit patterns, E4M3 codes as uint8, or MXFP4 / q4_0 codes packed
    two per byte) and ``s_gate_up``/``s_down`` (fp8 block scales, MXFP4 E8M0
    scale bytes, or q4_0 binary16 scales as uint16 bit patterns) plus ``spec`` (E, top_k, H, I, expert_dtype, router_dtype).
    """

    def __init__(self, w: dict, router_bias=None):
        spec = w["spec"]
        self.E, self.k, self.H, self.I = spec.E, spec.top_k, spec.H, spec.I
        self.keep = {}
        for n in ("w_router", "w_gate_up", "w_down", "s_gate_up", "s_down"):
            a = w.get(n)
            self.keep[n] = None if a is None else np.ascontiguousarray(a)
        self.keep["router_bias"] = None if router_bias is None else _c(router_bias, np.float32)

        def p(n):
            a = self.keep[n]
            return None if a is None else a.ctypes.data

        self.s = OracleLayer(spec.E, spec.top_k, spec.H, spec.I, spec.router_dtype, spec.expert_dtype,
                             p("w_router"), p("w_gate_up"), p("w_down"), p("s_gate_up"), p("s_down"),
                             p("router_bias"))
        if lib().oracle_check_layer(ctypes.byref(self.s)):
            raise ValueError("bad oracle layer")


def bf16_value(b: int) -> float:
    return lib().oracle_bf16_value(int(b))


def e4m3_value(c: int) -> float:
    return lib().oracle_e4m3_value(int(c))


def e2m1_value(c: int) -> float:
    return lib().oracle_e2m1_value(int(c))


def e8m0_value(s: int) -> float:
    return lib().oracle_e8m0_value(int(s))


def f16_value(h: int) -> float:
    return lib().oracle_f16_value(int(h))


def rmsnorm(x, eps=RMS_EPS):
    x = _c(x, np.float64)
    T, H = x.shape
    out = np.empty_like(x)
    lib().oracle_rmsnorm(T, H, x.ctypes.data, eps, out.ctypes.data)
    return out


def router_logits(layer: Layer, x):
    x = _c(x, np.float64)
    T = x.shape[0]
    out = np.empty((T, layer.E), dtype=np.float64)
    lib().oracle_router_logits(ctypes.byref(layer.s), T, x.ctypes.data, out.ctypes.data)
    return out


def select(logits, k: int):
    lg = _c(logits, np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_select(T, E, k, lg.ctypes.data, ids.ctypes.data, w.ctypes.data)
    return ids, w


def sort(ids, E: int):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    R = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_routes = np.empty(max(R, 1), np.int32)
    uniq = np.empty(E, np.int32)
    n = np.zeros(1, np.int32)
    rc = lib().oracle_sort(T, k, E, ids.ctypes.data, counts.ctypes.data, offsets.ctypes.data,
                           sorted_routes.ctypes.data, uniq.ctypes.data, n.ctypes.data)
    if rc:
        raise ValueError("expert id out of range")
    return dict(counts=counts, offsets=offsets, sorted_routes=sorted_routes[:R], uniq=uniq[: int(n[0])],
                n_uniq=int(n[0]))


def walk(layer: Layer, x, ids, kind=WALK_PER_ROUTE, nthreads=None):
    """y[R, H] per route r = t*k + j."""
    x = _c(x, np.float64)
    ids = _c(ids, np.int32)
    T = x.shape[0]
    y = np.empty((T * layer.k, layer.H), dtype=np.float64)
    if kind == WALK_GROUPED:
        lib().oracle_walk_grouped(ctypes.byref(layer.s), T, x.ctypes.data, ids.ctypes.data, y.ctypes.data)
    else:
        lib().oracle_walk_per_route(ctypes.byref(layer.s), T, x.ctypes.data, ids.ctypes.data, y.ctypes.data,
                                    _threads(nthreads))
    return y


def combine(w, y, H: int):
    w = _c(w, np.float64)
    y = _c(y, np.float64)
    T, k = w.shape
    out = np.empty((T, H), dtype=np.float64)
    lib().oracle_combine(T, k, H, w.ctypes.data, y.ctypes.data, out.ctypes.data)
    return out


def expert_fwd(layer: Layer, x, ids, w, kind=WALK_PER_ROUTE, nthreads=None):
    x = _c(x, np.float64)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T = x.shape[0]
    out = np.zeros((T, layer.H), dtype=np.float64)
    rc = lib().oracle_expert_fwd(ctypes.byref(layer.s), T, x.ctypes.data, ids.ctypes.data, w.ctypes.data, kind,
                                 out.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_expert_fwd: bad arguments")
    return out


def moe_layer(layer: Layer, x, logits_in=None, rmsnorm_in=False, residual=False, eps=RMS_EPS,
              kind=WALK_PER_ROUTE, nthreads=None):
    """The whole layer.  Returns dict(out, logits, ids, w)."""
    x = _c(x, np.float32)
    T = x.shape[0]
    out = np.zeros((T, layer.H), dtype=np.float64)
    logits = np.zeros((T, layer.E), dtype=np.float64)
    ids = np.zeros((T, layer.k), dtype=np.int32)
    w = np.zeros((T, layer.k), dtype=np.float64)
    li = None if logits_in is None else _c(logits_in, np.float64)
    flags = (RMSNORM if rmsnorm_in else 0) | (RESIDUAL if residual else 0)
    rc = lib().oracle_moe_layer(ctypes.byref(layer.s), T, x.ctypes.data, None if li is None else li.ctypes.data,
                                flags, eps, kind, logits.ctypes.data, ids.ctypes.data, w.ctypes.data,
                                out.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_moe_layer: bad arguments")
    return dict(out=out, logits=logits, ids=ids, w=w)
