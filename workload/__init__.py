"""Seeded synthetic inputs for the MoE decode layer (inputs only, no layer math).

Both the CPU oracle and the GPU harness take their inputs from here, so the two
sides always see the same bytes.  Every tensor is counter-based (see
``moegen.c``): element ``i`` of tensor ``(seed, layer, tensor)`` depends on
those four integers only, so one expert's slice can be regenerated without the
rest of the layer.

Workload recipe (the shapes and distributions follow the pages' workloads):

* expert weights ``gate_up[e] : [2I, H]`` (rows ``[0, I)`` gate, ``[I, 2I)``
  up) and ``down[e] : [H, I]``, drawn N(0, sigma) with sigma = 1/sqrt(fan_in),
  fan_in = H for ``gate_up`` and the router, I for ``down``;
* router ``W_r : [E, H]`` with the same recipe;
* activations ``x : [T, H]`` ~ N(0, 1) fp32;
* skewed routing: per-expert bias ``-s * ln(rank(e))`` over a seeded
  permutation of the experts (Zipf(s) popularity), added to the logits;
* forced collision: bias +64 on experts 0 and 1, so every token picks them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moegen.c")
_LIB = os.path.join(_HERE, "libmoegen.so")

# tensor ids inside one (seed, layer) stream family
T_ROUTER, T_GATE_UP, T_DOWN, T_X, T_PERM, T_LOGITS = 0, 1, 2, 3, 4, 5

SEED_WEIGHTS = 0
SEED_X = 1          # + draw index
SEED_ZIPF_PERM = 2
SEED_LOGITS = 3     # + draw index (selection fed straight from i.i.d. N(0,1) logits)

F32, BF16, FP8, MXFP4, Q4_0 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3", MXFP4: "mxfp4", Q4_0: "q4_0"}


def build(force: bool = False) -> str:
    """Compile ``libmoegen.so`` with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, u32, i32, dbl, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.moegen_key.restype = u64
        L.moegen_key.argtypes = [u64, u32, u32]
        L.moegen_normal_f32.restype = None
        L.moegen_normal_f32.argtypes = [u64, u64, u64, dbl, vp, i32]
        L.moegen_normal_bf16.restype = None
        L.moegen_normal_bf16.argtypes = [u64, u64, u64, dbl, vp, i32]
        L.moegen_fp8_matrix.restype = i32
        L.moegen_fp8_matrix.argtypes = [u64, u64, i32, i32, dbl, vp, vp, i32]
        L.moegen_mxfp4_matrix.restype = i32
        L.moegen_mxfp4_matrix.argtypes = [u64, u64, i32, i32, dbl, vp, vp, i32]
        L.moegen_e2m1_encode.restype = ctypes.c_uint8
        L.moegen_e2m1_encode.argtypes = [dbl]
        L.moegen_q4_0_matrix.restype = i32
        L.moegen_q4_0_matrix.argtypes = [u64, u64, i32, i32, dbl, vp, vp, i32]
        L.moegen_f16_encode.restype = ctypes.c_uint16
        L.moegen_f16_encode.argtypes = [dbl]
        L.moegen_permutation.restype = None
        L.moegen_permutation.argtypes = [u64, i32, vp]
        L.moegen_normal_one.restype = dbl
        L.moegen_normal_one.argtypes = [u64, u64]
        L.moegen_e4m3_encode.restype = ctypes.c_uint8
        L.moegen_e4m3_encode.argtypes = [dbl]
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def key(seed: int, layer: int, tensor: int) -> int:
    return lib().moegen_key(seed, layer, tensor)


def normal_f32(k: int, n: int, sigma: float, start: int = 0, nthreads: int | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().moegen_normal_f32(k, start, n, sigma, out.ctypes.data, nthreads or default_threads())
    return out


def normal_bf16(k: int, n: int, sigma: float, start: int = 0, nthreads: int | None = None) -> np.ndarray:
    """bf16 bit patterns as uint16."""
    out = np.empty(n, dtype=np.uint16)
    lib().moegen_normal_bf16(k, start, n, sigma, out.ctypes.data, nthreads or default_threads())
    return out


def fp8_matrices(k: int, count: int, rows: int, cols: int, sigma: float, nthreads: int | None = None):
    """``count`` consecutive [rows, cols] matrices of one stream as (codes uint8, scales f32)."""
    q = np.empty((count, rows, cols), dtype=np.uint8)
    s = np.empty((count, rows // 128, cols // 128), dtype=np.float32)
    for c in range(count):
        rc = lib().moegen_fp8_matrix(k, c * rows * cols, rows, cols, sigma, q[c].ctypes.data, s[c].ctypes.data,
                                     nthreads or default_threads())
        if rc != 0:
            raise ValueError("fp8 matrices need rows and cols that are multiples of 128")
    return q, s


def mxfp4_matrices(k: int, count: int, rows: int, cols: int, sigma: float, nthreads: int | None = None):
    """``count`` consecutive [rows, cols] matrices of one stream as MXFP4:
    (codes uint8 [count, rows, cols/2], two per byte with the even element in
    the low nibble; E8M0 scale bytes uint8 [count, rows, cols/32])."""
    q = np.empty((count, rows, cols // 2), dtype=np.uint8)
    s = np.empty((count, rows, cols // 32), dtype=np.uint8)
    for c in range(count):
        rc = lib().moegen_mxfp4_matrix(k, c * rows * cols, rows, cols, sigma, q[c].ctypes.data, s[c].ctypes.data,
                                       nthreads or default_threads())
        if rc != 0:
            raise ValueError("mxfp4 matrices need cols that are a multiple of 32")
    return q, s


def q4_0_matrices(k: int, count: int, rows: int, cols: int, sigma: float, nthreads: int | None = None):
    """``count`` consecutive [rows, cols] matrices of one stream as q4_0:
    (codes uint8 [count, rows, cols/2], per block of 32 elements along a row
    16 bytes with element j in the low nibble of byte j and element j + 16 in
    its high nibble; binary16 scales as uint16 bit patterns
    [count, rows, cols/32])."""
    q = np.empty((count, rows, cols // 2), dtype=np.uint8)
    s = np.empty((count, rows, cols // 32), dtype=np.uint16)
    for c in range(count):
        rc = lib().moegen_q4_0_matrix(k, c * rows * cols, rows, cols, sigma, q[c].ctypes.data, s[c].ctypes.data,
                                      nthreads or default_threads())
        if rc != 0:
            raise ValueError("q4_0 matrices need cols that are a multiple of 32")
    return q, s


def f16_encode(v: float) -> int:
    return int(lib().moegen_f16_encode(float(v)))


def e2m1_encode(v: float) -> int:
    return int(lib().moegen_e2m1_encode(float(v)))


def e4m3_encode(v: float) -> int:
    return int(lib().moegen_e4m3_encode(float(v)))


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().moegen_permutation(k, n, out.ctypes.data)
    return out


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    E: int
    top_k: int
    H: int
    I: int
    expert_dtype: int = BF16
    router_dtype: int = BF16


def _dt_array(k, n, sigma, dtype, nthreads):
    if dtype == F32:
        return normal_f32(k, n, sigma, nthreads=nthreads)
    if dtype == BF16:
        return normal_bf16(k, n, sigma, nthreads=nthreads)
    raise ValueError("dtype")


def make_layer(spec: LayerSpec, layer: int = 0, seed: int = SEED_WEIGHTS, nthreads: int | None = None,
               experts: bool = True) -> dict:
    """Weights of one layer as host arrays (bf16 as uint16 bit patterns, fp8 as uint8 codes, MXFP4 as packed
    uint8 codes with E8M0 scale bytes)."""
    E, H, I = spec.E, spec.H, spec.I
    sh, si = 1.0 / math.sqrt(H), 1.0 / math.sqrt(I)
    out = {"spec": spec}
    out["w_router"] = _dt_array(key(seed, layer, T_ROUTER), E * H, sh, spec.router_dtype, nthreads).reshape(E, H)
    if not experts:
        return out
    if spec.expert_dtype in (FP8, MXFP4, Q4_0):
        mats = {FP8: fp8_matrices, MXFP4: mxfp4_matrices, Q4_0: q4_0_matrices}[spec.expert_dtype]
        q, s = mats(key(seed, layer, T_GATE_UP), E, 2 * I, H, sh, nthreads)
        out["w_gate_up"], out["s_gate_up"] = q, s
        q, s = mats(key(seed, layer, T_DOWN), E, H, I, si, nthreads)
        out["w_down"], out["s_down"] = q, s
    else:
        out["w_gate_up"] = _dt_array(key(seed, layer, T_GATE_UP), E * 2 * I * H, sh, spec.expert_dtype,
                                     nthreads).reshape(E, 2 * I, H)
        out["w_down"] = _dt_array(key(seed, layer, T_DOWN), E * H * I, si, spec.expert_dtype,
                                  nthreads).reshape(E, H, I)
        out["s_gate_up"] = out["s_down"] = None
    return out


def make_x(T: int, H: int, draw: int = 0, layer: int = 0) -> np.ndarray:
    return normal_f32(key(SEED_X + draw, layer, T_X), T * H, 1.0).reshape(T, H)


def make_logits(T: int, E: int, draw: int = 0) -> np.ndarray:
    """i.i.d. N(0, 1) fp32 router logits, for selection fed straight from the harness."""
    return normal_f32(key(SEED_LOGITS + draw, 0, T_LOGITS), T * E, 1.0).reshape(T, E)


def zipf_bias(E: int, s: float = 1.1, layer: int = 0) -> np.ndarray:
    """bias[e] = -s * ln(rank(e)), ranks 1..E over a seeded expert permutation."""
    perm = permutation(key(SEED_ZIPF_PERM, layer, T_PERM), E)
    bias = np.empty(E, dtype=np.float64)
    for r, e in enumerate(perm):
        bias[e] = -s * math.log(r + 1)
    return bias.astype(np.float32)


def collision_bias(E: int) -> np.ndarray:
    """+64 on experts 0 and 1: every token routes to {0, 1}."""
    b = np.zeros(E, dtype=np.float32)
    b[:2] = 64.0
    return b


# The workloads: one tiny fp32 parity layer, the uniform bf16 batch sweep, the
# skewed sweep, the 30-layer stack and the large-batch grouped-GEMM regime.
TINY = LayerSpec(E=8, top_k=2, H=64, I=32, expert_dtype=F32, router_dtype=F32)
SWEEP = LayerSpec(E=256, top_k=8, H=2048, I=768)
SKEWED = LayerSpec(E=256, top_k=6, H=2048, I=768)
STACK = LayerSpec(E=128, top_k=2, H=2048, I=1024)
LARGE = LayerSpec(E=256, top_k=8, H=4096, I=1536)
LARGE_FP8 = LayerSpec(E=256, top_k=8, H=4096, I=1536, expert_dtype=FP8)
LARGE_MXFP4 = LayerSpec(E=256, top_k=8, H=4096, I=1536, expert_dtype=MXFP4)
LARGE_Q4_0 = LayerSpec(E=256, top_k=8, H=4096, I=1536, expert_dtype=Q4_0)
SWEEP_MXFP4 = LayerSpec(E=256, top_k=8, H=2048, I=768, expert_dtype=MXFP4)
SWEEP_Q4_0 = LayerSpec(E=256, top_k=8, H=2048, I=768, expert_dtype=Q4_0)

SWEEP_BS = (1, 4, 8, 16, 32, 64)
SKEWED_BS = (1, 8, 32, 64)
STACK_BS = (1, 4)
STACK_LAYERS = 30
LARGE_BS = (128, 256, 512)

