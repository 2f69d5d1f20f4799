// Internal header of the gfx950 MoE decode library: device helpers shared by
// the kernels, launcher declarations and the workspace layout.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 waves per workgroup everywhere
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxChunksPerLane = 8;  // 16-byte chunks per lane per weight row
// q4_0 rows stop at 4 chunks per lane (K <= 8192): with 8, its decode made
// the compiler call the route loop out of line (scratch and calls).
__host__ __device__ constexpr int max_chunks_per_lane(int dtype) { return dtype == MOE_Q4_0 ? 4 : kMaxChunksPerLane; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Elements held by one 16-byte chunk of a weight row.
template <int WDT> struct WT;
template <> struct WT<MOE_F32> { static constexpr int kEpc = 4; static constexpr int kBytes = 4; };
template <> struct WT<MOE_BF16> { static constexpr int kEpc = 8; static constexpr int kBytes = 2; };
template <> struct WT<MOE_FP8_E4M3> { static constexpr int kEpc = 16; static constexpr int kBytes = 1; };
// MXFP4: 32 E2M1 codes per chunk, one E8M0 scale block (kBytes is not used:
// row bytes are chunks x 16 for every dtype).
template <> struct WT<MOE_MXFP4> { static constexpr int kEpc = 32; static constexpr int kBytes = 0; };
// q4_0: 32 codes per chunk, one block with one binary16 scale.
template <> struct WT<MOE_Q4_0> { static constexpr int kEpc = 32; static constexpr int kBytes = 0; };

__host__ __device__ constexpr int elems_per_chunk(int dtype) {
    return dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 8 : dtype == MOE_FP8_E4M3 ? 16 : 32;
}

// Two fp32 -> packed bf16 pair (element 0 in the low half), round to nearest even.
__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// bf16 halves of a packed 32-bit word (element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// OCP E4M3 codes are converted by the hardware (v_cvt_pk_f32_fp8 reads the
// OCP format on gfx950): two codes of a 16-bit half of a word to two exact
// fp32 values, subnormals included (the NaN code is never produced by the
// encoder).  Products with activations of ordinary magnitude stay far from
// the fp32 subnormal range (the smallest code is 2^-9).

// acc + sum_e w[e] * xs[e] over the elements of one 16-byte weight chunk,
// in element order.
template <int WDT>
__device__ __forceinline__ float chunk_dot(const u32x4 w, const float *xs, float acc);

template <>
__device__ __forceinline__ float chunk_dot<MOE_F32>(const u32x4 w, const float *xs, float acc) {
    acc = fmaf(__uint_as_float(w.x), xs[0], acc);
    acc = fmaf(__uint_as_float(w.y), xs[1], acc);
    acc = fmaf(__uint_as_float(w.z), xs[2], acc);
    acc = fmaf(__uint_as_float(w.w), xs[3], acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_BF16>(const u32x4 w, const float *xs, float acc) {
    acc = fmaf(bf16_lo(w.x), xs[0], acc);
    acc = fmaf(bf16_hi(w.x), xs[1], acc);
    acc = fmaf(bf16_lo(w.y), xs[2], acc);
    acc = fmaf(bf16_hi(w.y), xs[3], acc);
    acc = fmaf(bf16_lo(w.z), xs[4], acc);
    acc = fmaf(bf16_hi(w.z), xs[5], acc);
    acc = fmaf(bf16_lo(w.w), xs[6], acc);
    acc = fmaf(bf16_hi(w.w), xs[7], acc);
    return acc;
}

// fp8: the sum of code values times x; callers multiply by the block scale.
template <>
__device__ __forceinline__ float chunk_dot<MOE_FP8_E4M3>(const u32x4 w, const float *xs, float acc) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], true);
        acc = fmaf(lo[0], xs[4 * q], acc);
        acc = fmaf(lo[1], xs[4 * q + 1], acc);
        acc = fmaf(hi[0], xs[4 * q + 2], acc);
        acc = fmaf(hi[1], xs[4 * q + 3], acc);
    }
    return acc;
}

// 8 E2M1 codes of a 32-bit word (element 2b in the low nibble of byte b) to
// 8 exact fp32 values in element order, without their E8M0 scale, by the
// hardware conversion (OCP E2M1 on gfx950).
__device__ __forceinline__ void e2m1x8_decode(uint32_t v, float *f) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)v, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)v, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)v, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)v, 1.0f, 3);
    f[0] = p0[0]; f[1] = p0[1];
    f[2] = p1[0]; f[3] = p1[1];
    f[4] = p2[0]; f[5] = p2[1];
    f[6] = p3[0]; f[7] = p3[1];
}

// 8 q4_0 codes of a 32-bit word (bytes b0..b3 of a block's word v) as the
// exact fp32 values (code - 8) / 16: f[0..3] the low nibbles (elements
// 4v .. 4v + 3 of the block), f[4..7] the high nibbles (elements 16 + 4v ..
// 16 + 4v + 3); callers fold the 16 into the block's scale, which leaves every
// sum the one of code - 8 times x, scaled by a power of two.  With every
// nibble's top bit flipped, a nibble read as a signed 4-bit field is
// code - 8, which v_cvt_off_f32_i4 converts (divided by 16) from the low 4
// bits of the byte its SDWA operand selects: one instruction per element.
__device__ __forceinline__ void q4x8_decode16(uint32_t v, float *f) {
    const uint32_t lo = v ^ 0x88888888u, hi = lo >> 4;
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(f[0]) : "v"(lo));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f[1]) : "v"(lo));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f[2]) : "v"(lo));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f[3]) : "v"(lo));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(f[4]) : "v"(hi));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f[5]) : "v"(hi));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f[6]) : "v"(hi));
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f[7]) : "v"(hi));
}

// 8 q4_0 codes of a word (bytes b0..b3 of a block's word g) as 8 bf16 values
// (code - 8) * scale: the low nibbles (block elements 4g .. 4g + 3), then the
// high nibbles (16 + 4g .. 16 + 4g + 3).  Exact for scale 1 (and any power
// of two); otherwise each product is rounded to bf16 once.  A nibble with
// its top bit flipped, read as a signed 4-bit field, is code - 8.
__device__ __forceinline__ u32x4 q4x8_to_bf16(unsigned w, float scale = 1.f) {
    const int s = (int)(w ^ 0x88888888u);
    float v[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        v[b] = (float)((s << (28 - 8 * b)) >> 28) * scale;
        v[4 + b] = (float)((s << (24 - 8 * b)) >> 28) * scale;
    }
    return u32x4{bf16_pair_rne(v[0], v[1]), bf16_pair_rne(v[2], v[3]), bf16_pair_rne(v[4], v[5]),
                 bf16_pair_rne(v[6], v[7])};
}

// IEEE binary16 bit pattern to fp32 (exact).
__device__ __forceinline__ float f16_value(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// E8M0 scale byte to fp32: 2^(s - 127) (s = 0 is the subnormal 2^-127; 255,
// NaN in the format, is never produced by the encoder).
__device__ __forceinline__ float e8m0_value(uint32_t s) { return __uint_as_float(s ? s << 23 : 0x00400000u); }

// A chunk decoded to fp32 (exact): EPC values in memory order.  fp8 codes
// are decoded without their block scale.
template <int WDT>
__device__ __forceinline__ void chunk_decode(const u32x4 w, float *f);

template <>
__device__ __forceinline__ void chunk_decode<MOE_F32>(const u32x4 w, float *f) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
}

template <>
__device__ __forceinline__ void chunk_decode<MOE_BF16>(const u32x4 w, float *f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

template <>
__device__ __forceinline__ void chunk_decode<MOE_FP8_E4M3>(const u32x4 w, float *f) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], true);
        f[4 * q] = lo[0];
        f[4 * q + 1] = lo[1];
        f[4 * q + 2] = hi[0];
        f[4 * q + 3] = hi[1];
    }
}

// Sum over the 64 lanes; every lane receives the same value (each butterfly
// step adds the same two operands in both partner lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Value of a butterfly partner of this lane at level `mask` (a power of two
// below 64), without going through the LDS crossbar: the partner differs
// from the lane in bit `mask` and in no bit above it.  32 and 16: the
// partner is lane ^ mask (v_permlane32_swap / v_permlane16_swap, which
// exchange the two halves of the wave / the rows of 16 lanes pairwise);
// 8 and 4: lane ^ 15 and lane ^ 7 (DPP row_mirror, row_half_mirror); 2 and
// 1: lane ^ 2, lane ^ 1 (DPP quad_perm).  Pairing lane with lane ^ (2 mask
// - 1) instead of lane ^ mask still adds disjoint lane sets at every level
// of a reduction that runs the masks from high to low.
__device__ __forceinline__ float xor_partner(float v, int mask, int lane) {
    const unsigned u = __float_as_uint(v);
    switch (mask) {
        case 32: {
            const auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            return __uint_as_float((lane & 32) ? q[0] : q[1]);
        }
        case 16: {
            const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            return __uint_as_float((lane & 16) ? r[0] : r[1]);
        }
        case 8: return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));
        case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
    }
}

// Reduce-scatter of NS slots of NW lane partials over the G lanes of a row:
// level s (mask G/2 >> s) halves the live slots, each lane keeping the half
// its lane bit selects and adding its partner's copy of that half; after
// log2(NS) levels a lane holds slot (l % G) >> (log2 G - log2 NS), and a
// butterfly over the remaining masks completes that slot's sum in every lane
// of its group (partners from xor_partner).  The order of the additions
// depends only on lane positions.
template <int NS, int NW, int G>
__device__ __forceinline__ void reduce_slots(float (&p)[NS][NW], int lane) {
    constexpr int LOG = ilog2(NS);
    static_assert((1 << LOG) == NS, "slots must be a power of two");
    static_assert(NS <= G, "more slots than lanes");
#pragma unroll
    for (int s = 0; s < LOG; ++s) {
        const int mask = (G / 2) >> s;
        const int half = NS >> (s + 1);
        const bool upper = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i)
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                // the empty asm makes lo and hi plain values: otherwise the
                // selects below fold into a select of array addresses, which
                // puts p in scratch memory (and its loads wait for every
                // outstanding global load)
                float lo = p[i][v], hi = p[half + i][v];
                asm("" : "+v"(lo), "+v"(hi));
                const float keep = upper ? hi : lo;
                const float give = upper ? lo : hi;
                p[i][v] = keep + xor_partner(give, mask, lane);
            }
    }
#pragma unroll
    for (int mask = (G / 2) >> LOG; mask >= 1; mask >>= 1)
#pragma unroll
        for (int v = 0; v < NW; ++v) p[0][v] += xor_partner(p[0][v], mask, lane);
}

// Slot held by this lane after reduce_slots, and whether it writes it.
template <int NS, int G>
__device__ __forceinline__ int reduced_slot(int lane) { return (lane & (G - 1)) >> (ilog2(G) - ilog2(NS)); }
template <int NS, int G>
__device__ __forceinline__ bool slot_leader(int lane) { return (lane & ((G / NS) - 1)) == 0; }

// ---- data shared between workgroups of one launch ---------------------------
// The XCDs have separate L2 caches.  Rows written by one workgroup and read by
// another in the same launch are stored and loaded with device-scope atomic
// accesses, which are coherent across the L2s; a producer wave runs
// wait_vm_stores() before the workgroup barrier that precedes its counter
// update, and a consumer loads only after it has seen the counter.  This
// avoids device-scope fences, which write back or invalidate a whole L2.

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt bits [3:0] and [15:14] = 0, expcnt
// [6:4] = 7 and lgkmcnt [11:8] = 15 unconstrained).  The workgroup barrier
// alone does not wait for stores.
__device__ __forceinline__ void wait_vm_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename V>
__device__ __forceinline__ void store_shared(V *p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V load_shared(const V *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Streaming 16-byte weight load (weights are read once per step).
__device__ __forceinline__ u32x4 load_weight_chunk(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// Rows held by one wave for a given number of chunks per lane.
__host__ __device__ constexpr int rows_per_wave(int nc) { return nc <= 2 ? 8 : nc <= 4 ? 4 : 2; }

// ---- workspace layout (all offsets 256-byte aligned) ----------------------
// A workspace starts with a front of fixed size: the statistics words and the
// routing kernel's arrival counters, which must be zero when a call starts
// and are zero again when it ends.  Their place and extent depend on nothing
// (not on the batch, the layer shape or the workspace's byte size), so no
// data array of any call ever lands on them, whatever sizes the calls on one
// workspace pass.  The data arrays follow, laid out for the call's batch.
constexpr int kMaxTokens = 65536;                  // tokens per call
constexpr int kArriveWords = kMaxTokens + 1;       // per token tile (<= T) + 1
inline constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr size_t kWsStats = 0;                     // 4 int32
constexpr size_t kWsArrive = 256;
constexpr size_t kWsFrontBytes = kWsArrive + align256((size_t)kArriveWords * 4);

struct WsLayout {
    size_t stats, arrive, logits, ids, w, counts, offsets, sorted, uniq, nuniq, xn, xb, act, y, total;
};

// T tokens: the front at `front`, the data arrays from `data` on.
inline WsLayout ws_layout_at(const moe_layer_t &L, int64_t T, size_t front, size_t data) {
    WsLayout s;
    const int64_t R = T * L.top_k;
    s.stats = front + kWsStats;
    s.arrive = front + kWsArrive;
    size_t o = data;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    s.logits = take((size_t)T * L.E * 4);
    s.ids = take((size_t)R * 4);
    s.w = take((size_t)R * 4);
    s.counts = take((size_t)L.E * 4);
    s.offsets = take((size_t)(L.E + 1) * 4);
    s.sorted = take((size_t)R * 4);
    s.uniq = take((size_t)L.E * 4);
    s.nuniq = take(4);
    s.xn = take((size_t)T * L.H * 4);
    s.xb = take((size_t)T * L.H * 2);
    s.act = take((size_t)R * L.I * 4);
    s.y = take((size_t)R * L.H * 4);
    s.total = o;
    return s;
}

inline size_t ws_data_bytes(const moe_layer_t &L, int64_t T) { return ws_layout_at(L, T, 0, 0).total; }

// A layer workspace: the front, then the data arrays.
inline WsLayout ws_layout(const moe_layer_t &L, int64_t T) { return ws_layout_at(L, T, 0, kWsFrontBytes); }

// Bytes of a layer workspace for up to T tokens.
inline size_t ws_bytes_for(const moe_layer_t &L, int64_t T) { return kWsFrontBytes + ws_data_bytes(L, T); }

// ---- launchers (return hipSuccess or the launch error) -----------------------
int num_cus();

// The previous layer of a stack, combined inside the next routing launch:
// rows h_out[t] = h[t] + sum_j w[t, j] * y[t * k + j] (j ascending), which
// are then that layer's input.
struct PrevCombine {
    const float *y;  // [T * k, H]
    const float *w;  // [T, k]
    const float *h;  // [T, H] residual
    float *h_out;    // [T, H]
    int k;
};

// Routing: router GEMV (unless logits_in), selection and, if counts is not
// null, the sort; xn non-null with rmsnorm writes the normalised rows.  With
// prev, the input rows are prev's combine (x is not read).
hipError_t launch_route(const moe_layer_t &L, const float *x, const float *logits_in, int T, float *xn,
                        float *logits, int32_t *ids, float *w, int32_t *counts, int32_t *offsets, int32_t *sorted,
                        int32_t *uniq, int32_t *n_uniq, int32_t *stats, unsigned *arrive, bool rmsnorm,
                        unsigned *zero, int n_zero, hipStream_t st, const PrevCombine *prev = nullptr,
                        uint32_t *xb = nullptr);
hipError_t launch_sort(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                       int32_t *uniq, int32_t *n_uniq, hipStream_t st);
hipError_t launch_zero(unsigned *p, int n, hipStream_t st);
hipError_t launch_usage(const int32_t *counts, const int32_t *n_uniq, int E, unsigned long long *hist,
                        hipStream_t st);

struct Routing {
    const int32_t *ids, *counts, *offsets, *sorted, *uniq, *n_uniq;
    const float *w;
    const int32_t *max_count;  // largest count of one expert (from the sort), or null
    // a caller-supplied routing's n_uniq (null for the library's own): when
    // negative (rejected by the sort) the combine leaves out untouched
    const int32_t *reject;
    // the routing launch wrote the bf16 copy of x into xb
    bool xb_ready = false;
};
// ev (optional): events recorded after pass 1 GEMV, pass 1 MFMA, pass 2 GEMV,
// pass 2 MFMA and the combine (ev[0..4]); a stage that does not run records
// its event right after the previous one.
// xb: scratch for a bf16 copy of x [T, H] (used when segments take the MFMA path).
// out null: no combine (y and rt.w are left for the next layer of a stack).
// Whether launch_experts runs pass 2 and the combine as one launch for T
// tokens (small batches): then it needs out, and writes no y rows.
bool fused_combine(const moe_layer_t &L, int T);
// Routes an expert needs in a call of T tokens for its segment to run on the
// MFMA kernels, or 0 when no segment of such a call does.
int mfma_min_routes(const moe_layer_t &L, int T, uint32_t flags);
// The largest segment's routes from which any segment of the call takes the
// MFMA path (0: never).
int mfma_hot_routes(const moe_layer_t &L, int T, uint32_t flags);
// may_fork false: the MFMA segments of large batches stay on st (no side
// stream is created or used).
hipError_t launch_experts(const moe_layer_t &L, const float *x, const float *xres, int T, const Routing &rt,
                          void *xb, float *act, float *y, float *out, uint32_t flags, hipStream_t st,
                          const hipEvent_t *ev = nullptr, bool may_fork = true);

}  // namespace moe
