// Templates of the grouped-GEMV expert passes, instantiated once per weight
// dtype in experts_<dtype>.hip.  See experts.hip for what the passes compute.
//
// Layout of a wave's work: a wave holds NS "slots" of weight rows in
// registers as raw 16-byte chunks.  G lanes share one row (G = 64 or 32), so
// a slot covers 64/G rows at once; lane l works on row half = l / G of the
// slot and on chunks (l % G) + G*c, c < NC.  The weights are loaded once per
// work item with streaming loads; then every route of the segment is applied
// to them: one lane partial per slot (chunks in order), then a reduce-scatter
// across the G lanes of each row (see reduce_slots).  The arithmetic of one
// (row, route) pair depends only on lane positions, never on the segment, so
// every walk gives bitwise the same result.
#pragma once

#include <limits.h>

#include <type_traits>

#include "common.h"

namespace moe {

struct SegArgs {
    const int32_t *ids, *counts, *offsets, *sorted, *uniq, *n_uniq;
    int grouped;  // 1: segment = unique expert, 0: segment = one route
    int R;        // routes
    int E;        // experts (ids outside [0, E) make an empty segment)
    int gemv_below;  // segments with this many routes or more are left to the MFMA kernels,
    // but only if the largest segment (*max_count, when set) holds at least
    // hot routes; otherwise every segment stays here.  Kernels resolve this
    // once, at their start, into gemv_below.
    const int32_t *max_count;
    int hot;
};

// A wave-uniform int32 read through the scalar cache (s_load_dword), waited
// for on the LDS/scalar counter: it never waits behind the wave's
// outstanding vector loads, as a vector load would (those complete in
// order).  The routing arrays were written by an earlier launch.
__device__ __forceinline__ int load_uniform(const int32_t *p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(v) : "s"(p) : "memory");
    return v;
}

// Two / three / four wave-uniform int32 reads issued together, with one wait.
__device__ __forceinline__ void load_uniform2(const int32_t *p0, const int32_t *p1, int &v0, int &v1) {
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(v0), "=&s"(v1)
                 : "s"(p0), "s"(p1)
                 : "memory");
}
__device__ __forceinline__ void load_uniform3(const int32_t *p0, const int32_t *p1, const int32_t *p2, int &v0,
                                              int &v1, int &v2) {
    asm volatile(
        "s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %4, 0x0\n\ts_load_dword %2, %5, 0x0\n\ts_waitcnt lgkmcnt(0)"
        : "=&s"(v0), "=&s"(v1), "=&s"(v2)
        : "s"(p0), "s"(p1), "s"(p2)
        : "memory");
}
__device__ __forceinline__ void load_uniform4(const int32_t *p0, const int32_t *p1, const int32_t *p2,
                                              const int32_t *p3, int &v0, int &v1, int &v2, int &v3) {
    asm volatile(
        "s_load_dword %0, %4, 0x0\n\ts_load_dword %1, %5, 0x0\n\ts_load_dword %2, %6, 0x0\n\t"
        "s_load_dword %3, %7, 0x0\n\ts_waitcnt lgkmcnt(0)"
        : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3)
        : "s"(p0), "s"(p1), "s"(p2), "s"(p3)
        : "memory");
}

// Expert, first sorted slot and route count of segment s (s uniform).
__device__ __forceinline__ void segment(const SegArgs &sa, int s, int &e, int &first, int &n) {
    first = 0;
    n = 0;
    if (sa.grouped) {
        e = load_uniform(sa.uniq + s);
        if (e >= 0 && e < sa.E) {
            first = load_uniform(sa.offsets + e);
            n = load_uniform(sa.counts + e);
        }
    } else {
        e = load_uniform(sa.ids + s);
        first = s;
        n = 1;
    }
    if (e < 0 || e >= sa.E) {
        e = 0;
        n = 0;
    }
    if (n >= sa.gemv_below) n = 0;
}

__device__ __forceinline__ int segment_route(const SegArgs &sa, int first, int i) {
    return sa.grouped ? sa.sorted[first + i] : first + i;
}

// The same for a wave-uniform i, through the scalar cache.
__device__ __forceinline__ int segment_route_uniform(const SegArgs &sa, int first, int i) {
    return sa.grouped ? load_uniform(sa.sorted + first + i) : first + i;
}

__device__ __forceinline__ int segment_count(const SegArgs &sa) {
    const int n = sa.grouped ? *sa.n_uniq : sa.R;
    return n > 0 ? n : 0;
}

// The segment count and segment s for a workgroup's first item, with as few
// dependent scalar round trips as possible before its weight loads can be
// issued: n_uniq and uniq[s] are read together.  When no segment is left to
// the MFMA kernels (every unique expert has at least one route here), the
// expert alone addresses the weights: late is set, n is 1 for now, and the
// caller reads first and n with segment_rest() once the loads are in flight.
__device__ __forceinline__ int first_segment(SegArgs &sa, int s, int &e, int &first, int &n, bool &late) {
    late = false;
    first = 0;
    n = 0;
    e = 0;
    if (!sa.grouped) {
        if (s < sa.R) segment(sa, s, e, first, n);
        return sa.R;
    }
    int nu, ev;
    if (sa.gemv_below != INT_MAX && sa.max_count) {  // the threshold too, in the same round trip
        int mx;
        asm volatile(
            "s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %4, 0x0\n\ts_load_dword %2, %5, 0x0\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&s"(nu), "=&s"(ev), "=&s"(mx)
            : "s"(sa.n_uniq), "s"(sa.uniq + min(s, sa.E - 1)), "s"(sa.max_count)
            : "memory");
        if (mx < sa.hot) sa.gemv_below = INT_MAX;
    } else {
        asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                     : "=&s"(nu), "=&s"(ev)
                     : "s"(sa.n_uniq), "s"(sa.uniq + min(s, sa.E - 1))
                     : "memory");
    }
    const int nseg = nu > 0 ? nu : 0;
    if (s < nseg && ev >= 0 && ev < sa.E) {
        e = ev;
        if (sa.gemv_below == INT_MAX) {
            late = true;
            n = 1;
        } else {
            first = load_uniform(sa.offsets + e);
            n = load_uniform(sa.counts + e);
            if (n >= sa.gemv_below) n = 0;
        }
    }
    return nseg;
}

// first and n of a unique expert's segment (after first_segment set late).
__device__ __forceinline__ void segment_rest(const SegArgs &sa, int e, int &first, int &n) {
    first = load_uniform(sa.offsets + e);
    n = load_uniform(sa.counts + e);
}

// Loads chunk c of slot rows rows[s] (byte pointers of this lane's row), zero
// where invalid.
template <int NC, int NS, int G>
__device__ __forceinline__ void load_rows(u32x4 (&w)[NS][NC], const char *const (&rows)[NS], const bool (&ok)[NS],
                                          int nq, int lane) {
    const int sub = lane & (G - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = sub + G * c;
            w[s][c] = (ok[s] && q < nq) ? load_weight_chunk(reinterpret_cast<const u32x4 *>(rows[s]) + q)
                                        : u32x4{0u, 0u, 0u, 0u};
        }
}

// ---- activation rows in LDS ---------------------------------------------------
// The four waves of a workgroup work on the same segment, so the activation
// rows of its routes (x[t] in pass 1, a[r] in pass 2, fp32, K elements) are
// staged once into LDS with direct global->LDS loads and read by every wave;
// with the rows fetched by each wave itself, several routes per segment
// carry more x than weight traffic through the CU's vector memory path and
// the weight stream slows down.

// Threads per workgroup of the GEMV passes.
constexpr int kGemvBlock = 256;

// Issue the loads of rows m = 0..mb-1 (global rows src(m) of q4 float4s)
// into LDS rows of q4 float4s at xl; the caller waits (vmcnt(0)) and syncs.
template <typename RowOf>
__device__ __forceinline__ void stage_rows_lds(float4 *xl, int mb, int q4, RowOf row_of) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    for (int m = 0; m < mb; ++m) {
        const float4 *src = row_of(m);  // m is uniform: route lookups may shuffle
        for (int u0 = wv * kWave; u0 < q4; u0 += kGemvBlock)
            if (u0 + lane < q4)
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(src + u0 + lane),
                                                 (__attribute__((address_space(3))) void *)(xl + m * q4 + u0), 16, 0,
                                                 0);
    }
}

// Workgroup barrier after this wave's LDS reads have completed; unlike
// __syncthreads it does not wait for outstanding global loads (the weights).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait for this wave's loads (weights and staged rows), then for the
// workgroup: the staged rows of every wave are in LDS after it.
__device__ __forceinline__ void wait_loads_and_sync() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc[r][s] = this lane's partial of slot s . x_r for RB routes, chunks in
// order, with the x rows read from LDS; fp8 chunks are scaled by their block
// scale.  Each weight chunk is decoded once for all RB routes; a route's
// arithmetic (fp32 FMAs in element order per chunk, chunks in order) is the
// same for any RB, so pairing routes changes no result bit.  The weights
// stay packed in registers across the route loop: the empty asm makes them
// opaque on every call, so the compiler cannot hoist their decode out of the
// loop (which would double their register footprint and halve the waves in
// flight).
template <int WDT, int NC, int NS, int G, int RB>
__device__ __forceinline__ void dot_rows(u32x4 (&w)[NS][NC], const float (&sc)[NS][NC],
                                         const float4 *const (&xl)[RB], int nq, int lane, float (&acc)[RB][NS]) {
    constexpr int EPC = WT<WDT>::kEpc;
    const int sub = lane & (G - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(w[s][c]));
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[r][s] = 0.f;
    if constexpr (WDT == MOE_MXFP4 || WDT == MOE_Q4_0) {
        // 32 codes per chunk, taken a 32-bit word (8 elements) at a time:
        // per (route, slot) one fp32 chain over the chunk's elements, then
        // scaled by the chunk's scale (E8M0, or q4_0's binary16).  MXFP4
        // word v holds elements 8v .. 8v + 7; q4_0 word v elements
        // 4v .. 4v + 3 (low nibbles) and 16 + 4v .. 16 + 4v + 3 (high).
        // Each element's value is exact in fp32 (q4_0: (code - 8) / 16, the
        // 16 folded into the scale; taking the offset out of the sums instead,
        // as sum q x - 8 sum x, loses the low bits of a small sum to
        // cancellation).
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = sub + G * c;
            if (q < nq) {
                float t[RB][NS];
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int s = 0; s < NS; ++s) t[r][s] = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float xs[RB][8];
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        const float4 f0 = WDT == MOE_Q4_0 ? xl[r][q * 8 + v] : xl[r][q * 8 + 2 * v];
                        const float4 f1 = WDT == MOE_Q4_0 ? xl[r][q * 8 + 4 + v] : xl[r][q * 8 + 2 * v + 1];
                        xs[r][0] = f0.x; xs[r][1] = f0.y; xs[r][2] = f0.z; xs[r][3] = f0.w;
                        xs[r][4] = f1.x; xs[r][5] = f1.y; xs[r][6] = f1.z; xs[r][7] = f1.w;
                    }
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const uint32_t word = v == 0 ? w[s][c].x : v == 1 ? w[s][c].y : v == 2 ? w[s][c].z : w[s][c].w;
                        float wf[8];
                        if constexpr (WDT == MOE_Q4_0) q4x8_decode16(word, wf);
                        else e2m1x8_decode(word, wf);
#pragma unroll
                        for (int r = 0; r < RB; ++r)
#pragma unroll
                            for (int i = 0; i < 8; ++i) t[r][s] = fmaf(wf[i], xs[r][i], t[r][s]);
                    }
                }
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int s = 0; s < NS; ++s) acc[r][s] = fmaf(sc[s][c], t[r][s], acc[r][s]);
            }
        }
        return;
    }
    if constexpr (WDT != MOE_MXFP4 && WDT != MOE_Q4_0) {  // 4 to 16 elements per chunk
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = sub + G * c;
            if (q < nq) {
                float xs[RB][EPC];
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int v = 0; v < EPC / 4; ++v) {
                        const float4 f = xl[r][q * (EPC / 4) + v];
                        xs[r][4 * v] = f.x; xs[r][4 * v + 1] = f.y; xs[r][4 * v + 2] = f.z; xs[r][4 * v + 3] = f.w;
                    }
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    float wf[EPC];
                    chunk_decode<WDT>(w[s][c], wf);
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        float t = WDT == MOE_FP8_E4M3 ? 0.f : acc[r][s];
#pragma unroll
                        for (int i = 0; i < EPC; ++i) t = fmaf(wf[i], xs[r][i], t);
                        acc[r][s] = WDT == MOE_FP8_E4M3 ? fmaf(sc[s][c], t, acc[r][s]) : t;
                    }
                }
            }
        }
    }
}

// Slots per wave for NC chunks per lane: 32 to 64 VGPRs of weights.
__host__ __device__ constexpr int slots_for(int nc) { return nc <= 2 ? 8 : 4; }

// Routes staged per LDS batch for rows of K floats: 32 KiB of LDS per 4
// waves of a workgroup, at most 16 rows.
inline int lds_batch_rows(int K) {
    const int nb = (32 * 1024 * (kGemvBlock / 256)) / (K * 4);
    return nb < 1 ? 1 : nb > 16 ? 16 : nb;
}

// ---- pass 1: gate/up row pairs and the activation ------------------------
// G = 64; slots 2p and 2p+1 hold gate row i0+p and up row I+i0+p, so one
// reduce_slots leaves a pair's two sums in the same lane group.  A
// workgroup item is one segment and 4 * P consecutive pairs (P per wave).
struct Pass1Args {
    const void *gate_up;
    const void *s_gate_up;  // fp8: float block scales; MXFP4: E8M0 bytes
    const float *x;
    float *act;
    int H, I, k;
    SegArgs sa;
    uint32_t *xb;  // if set: bf16 copy of x [T, H] for the MFMA segments, written first
    int nb;        // routes per LDS batch
};

template <int WDT, int NC>
__global__ __launch_bounds__(kGemvBlock) void pass1_kernel(Pass1Args a) {
    extern __shared__ float4 xl[];  // nb rows of H floats
    constexpr int G = kWave;
    constexpr int NS = slots_for(NC);
    constexpr int P = NS / 2;  // gate/up pairs per wave
    constexpr int EPC = WT<WDT>::kEpc;
    constexpr int WPB = kGemvBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int H = a.H, I = a.I, nq = H / EPC;
    const int items_per_seg = (I + P * WPB - 1) / (P * WPB);
    const size_t row_bytes = (size_t)nq * 16;

    if (a.xb) {  // the MFMA pass 1, launched after this kernel, reads x as bf16
        const int npairs = a.sa.R / a.k * H / 2;
        // stored as float-typed words: no store of this kernel may alias the
        // int32 routing arrays, whose wave-uniform loads can then be scalar
        float *xb = reinterpret_cast<float *>(a.xb);
        for (int i = blockIdx.x * kGemvBlock + threadIdx.x; i < npairs; i += gridDim.x * kGemvBlock) {
            const float2 v = reinterpret_cast<const float2 *>(a.x)[i];
            xb[i] = __uint_as_float(bf16_pair_rne(v.x, v.y));
        }
    }

    // Items are strided over the workgroups, so at any time the grid streams
    // one narrow window of the weights.  The segment of the next item is
    // fetched while the current one is processed.
    int e_nx = 0, first_nx = 0, n_nx = 0;
    bool late;
    const int n_items = first_segment(a.sa, blockIdx.x / items_per_seg, e_nx, first_nx, n_nx, late) * items_per_seg;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int blk = item % items_per_seg;
        const int e = e_nx;
        int first = first_nx, n = n_nx;
        const int i0 = (blk * WPB + wv) * P;
        const char *rows[NS];
        bool ok[NS];
        float sc[NS][NC];
        const char *base = static_cast<const char *>(a.gate_up) + (size_t)e * 2 * I * row_bytes;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p;
            ok[2 * p] = ok[2 * p + 1] = i < I && n > 0;
            rows[2 * p] = base + (size_t)i * row_bytes;
            rows[2 * p + 1] = base + (size_t)(I + i) * row_bytes;
        }
#pragma unroll
        for (int r = 0; r < NS; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) sc[r][c] = 1.f;
        if (WDT == MOE_Q4_0) {  // one binary16 scale per chunk of 32: [E, 2I, H/32]
            const uint16_t *sg = reinterpret_cast<const uint16_t *>(a.s_gate_up);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int i = min(i0 + p, I - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int q = min(lane + G * c, nq - 1);
                    sc[2 * p][c] = 16.f * f16_value(sg[((size_t)e * 2 * I + i) * nq + q]);  // decode's 1/16
                    sc[2 * p + 1][c] = 16.f * f16_value(sg[((size_t)e * 2 * I + I + i) * nq + q]);
                }
            }
        }
        if (WDT == MOE_MXFP4) {  // one E8M0 byte per chunk of 32: [E, 2I, H/32]
            const uint8_t *sg = reinterpret_cast<const uint8_t *>(a.s_gate_up);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int i = min(i0 + p, I - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int q = min(lane + G * c, nq - 1);
                    sc[2 * p][c] = e8m0_value(sg[((size_t)e * 2 * I + i) * nq + q]);
                    sc[2 * p + 1][c] = e8m0_value(sg[((size_t)e * 2 * I + I + i) * nq + q]);
                }
            }
        }
        if (WDT == MOE_FP8_E4M3) {
            const int nbh = H / 128;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int i = min(i0 + p, I - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int hb = min((lane + G * c) * EPC / 128, nbh - 1);
                    sc[2 * p][c] = static_cast<const float *>(a.s_gate_up)[((size_t)e * (2 * I / 128) + i / 128) * nbh + hb];
                    sc[2 * p + 1][c] =
                        static_cast<const float *>(a.s_gate_up)[((size_t)e * (2 * I / 128) + (I + i) / 128) * nbh + hb];
                }
            }
        }
        u32x4 w[NS][NC];
        load_rows<NC, NS, G>(w, rows, ok, nq, lane);
        if (late) {
            segment_rest(a.sa, e, first, n);
            late = false;
        }
        if (item + gridDim.x < n_items) segment(a.sa, (item + gridDim.x) / items_per_seg, e_nx, first_nx, n_nx);
        // one batch of routes: rows into LDS, then every route of the batch
        // against the wave's rows.  The first batch (the whole segment when
        // it fits) is peeled off the loop so the compiler's wait counts stay
        // exact and the staging does not wait for the weights.
        auto batch = [&](int m0, int mb) {
            lds_sync();  // every wave is done reading the rows in LDS
            // route ids are wave-uniform (scalar loads): the staging does not
            // wait behind the weight loads
            stage_rows_lds(xl, mb, H / 4, [&](int m) {
                const int r = segment_route_uniform(a.sa, first, m0 + m);
                return reinterpret_cast<const float4 *>(a.x + (size_t)(r / a.k) * H);
            });
            wait_loads_and_sync();
            // routes in pairs (one weight decode for both), then a single one
            auto routes = [&](auto rb_tag, int m) {
                constexpr int RB = decltype(rb_tag)::value;
                const float4 *x[RB];
                int r[RB];
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    r[j] = segment_route_uniform(a.sa, first, m0 + m + j);
                    x[j] = xl + (size_t)(m + j) * (H / 4);
                }
                float acc[RB][NS];
                dot_rows<WDT, NC, NS, G, RB>(w, sc, x, nq, lane, acc);
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    float gu[P][2];
#pragma unroll
                    for (int p = 0; p < P; ++p) { gu[p][0] = acc[j][2 * p]; gu[p][1] = acc[j][2 * p + 1]; }
                    reduce_slots<P, 2, G>(gu, lane);
                    const int p = reduced_slot<P, G>(lane);
                    if (slot_leader<P, G>(lane) && i0 + p < I)
                        a.act[(size_t)r[j] * I + i0 + p] = silu(gu[0][0]) * gu[0][1];
                }
            };
            int m = 0;
            for (; m + 1 < mb; m += 2) routes(std::integral_constant<int, 2>{}, m);
            if (m < mb) routes(std::integral_constant<int, 1>{}, m);
        };
        if (n > 0) batch(0, min(a.nb, n));
        for (int m0 = a.nb; m0 < n; m0 += a.nb) batch(m0, min(a.nb, n - m0));
    }
}

// ---- pass 2: down rows -------------------------------------------------------
// Slot j of a wave whose first row is h0 holds row h0 + j * RPS + half for
// the lane's half (RPS = 64 / G rows per slot): its byte pointer in expert
// e, whether it exists (and live), and the block scales of the lane's chunks.
template <int WDT, int NC, int NS, int G>
__device__ __forceinline__ void down_rows(const void *down, const void *s_down, int e, int h0, int H, int I,
                                          bool live, int lane, const char *(&rows)[NS], bool (&ok)[NS],
                                          float (&sc)[NS][NC]) {
    constexpr int RPS = kWave / G;
    constexpr int EPC = WT<WDT>::kEpc;
    const int half = lane / G, nq = I / EPC;
    const size_t row_bytes = (size_t)nq * 16;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int h = h0 + j * RPS + half;
        ok[j] = h < H && live;
        rows[j] = static_cast<const char *>(down) + ((size_t)e * H + min(h, H - 1)) * row_bytes;
#pragma unroll
        for (int c = 0; c < NC; ++c) sc[j][c] = 1.f;
    }
    if (WDT == MOE_Q4_0) {  // one binary16 scale per chunk of 32: [E, H, I/32]
        const uint16_t *sd = reinterpret_cast<const uint16_t *>(s_down);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int h = min(h0 + j * RPS + half, H - 1);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int q = min((lane & (G - 1)) + G * c, nq - 1);
                sc[j][c] = 16.f * f16_value(sd[((size_t)e * H + h) * nq + q]);  // decode's 1/16
            }
        }
    }
    if (WDT == MOE_MXFP4) {  // one E8M0 byte per chunk of 32: [E, H, I/32]
        const uint8_t *sd = reinterpret_cast<const uint8_t *>(s_down);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int h = min(h0 + j * RPS + half, H - 1);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int q = min((lane & (G - 1)) + G * c, nq - 1);
                sc[j][c] = e8m0_value(sd[((size_t)e * H + h) * nq + q]);
            }
        }
    }
    if (WDT == MOE_FP8_E4M3) {
        const int nbi = I / 128;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int h = min(h0 + j * RPS + half, H - 1);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ib = min(((lane & (G - 1)) + G * c) * EPC / 128, nbi - 1);
                sc[j][c] = static_cast<const float *>(s_down)[((size_t)e * (H / 128) + h / 128) * nbi + ib];
            }
        }
    }
}

// A workgroup item is one segment and 4 * NR consecutive down rows.
struct Pass2Args {
    const void *down;
    const void *s_down;  // fp8: float block scales; MXFP4: E8M0 bytes
    const float *act;
    float *y;
    int H, I;
    SegArgs sa;
    int nb;  // routes per LDS batch
};

template <int WDT, int NC, int G>
__global__ __launch_bounds__(kGemvBlock) void pass2_kernel(Pass2Args a) {
    extern __shared__ float4 xl[];  // nb rows of I floats
    constexpr int NS = slots_for(NC);
    constexpr int RPS = kWave / G;  // rows per slot
    constexpr int NR = NS * RPS;    // rows per wave
    constexpr int EPC = WT<WDT>::kEpc;
    constexpr int WPB = kGemvBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1), half = lane / G, wv = threadIdx.x / kWave;
    const int H = a.H, I = a.I, nq = I / EPC;
    const int items_per_seg = (H + NR * WPB - 1) / (NR * WPB);

    int e_nx = 0, first_nx = 0, n_nx = 0;
    bool late;
    const int n_items = first_segment(a.sa, blockIdx.x / items_per_seg, e_nx, first_nx, n_nx, late) * items_per_seg;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int blk = item % items_per_seg;
        const int e = e_nx;
        int first = first_nx, n = n_nx;
        const int h0 = (blk * WPB + wv) * NR;
        const char *rows[NS];
        bool ok[NS];
        float sc[NS][NC];
        down_rows<WDT, NC, NS, G>(a.down, a.s_down, e, h0, H, I, n > 0, lane, rows, ok, sc);
        u32x4 w[NS][NC];
        load_rows<NC, NS, G>(w, rows, ok, nq, lane);
        if (late) {
            segment_rest(a.sa, e, first, n);
            late = false;
        }
        if (item + gridDim.x < n_items) segment(a.sa, (item + gridDim.x) / items_per_seg, e_nx, first_nx, n_nx);
        auto batch = [&](int m0, int mb) {
            lds_sync();  // every wave is done reading the rows in LDS
            stage_rows_lds(xl, mb, I / 4, [&](int m) {
                const int r = segment_route_uniform(a.sa, first, m0 + m);
                return reinterpret_cast<const float4 *>(a.act + (size_t)r * I);
            });
            wait_loads_and_sync();
            // routes in pairs (one weight decode for both), then a single one
            auto routes = [&](auto rb_tag, int m) {
                constexpr int RB = decltype(rb_tag)::value;
                const float4 *x[RB];
                int r[RB];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    r[i] = segment_route_uniform(a.sa, first, m0 + m + i);
                    x[i] = xl + (size_t)(m + i) * (I / 4);
                }
                float acc[RB][NS];
                dot_rows<WDT, NC, NS, G, RB>(w, sc, x, nq, lane, acc);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    float v[NS][1];
#pragma unroll
                    for (int j = 0; j < NS; ++j) v[j][0] = acc[i][j];
                    reduce_slots<NS, 1, G>(v, lane);
                    const int j = reduced_slot<NS, G>(lane);
                    const int h = h0 + j * RPS + half;
                    if (slot_leader<NS, G>(lane) && h < H) a.y[(size_t)r[i] * H + h] = v[0][0];
                }
            };
            int m = 0;
            for (; m + 1 < mb; m += 2) routes(std::integral_constant<int, 2>{}, m);
            if (m < mb) routes(std::integral_constant<int, 1>{}, m);
        };
        if (n > 0) batch(0, min(a.nb, n));
        for (int m0 = a.nb; m0 < n; m0 += a.nb) batch(m0, min(a.nb, n - m0));
    }
}

// ---- pass 2 with the combine, for small batches ------------------------------
// The same per-(row, route) arithmetic as pass2_kernel (a wave's NR down rows
// in NS slots of G lanes, the same rows per slot, lane -> chunk assignment and
// reduce-scatter, so every y value is bitwise the one pass2_kernel writes), in
// another order: a workgroup owns one NR-row block of down for every segment.
// Its waves (16, four per SIMD, so that one wave's memory latency is hidden
// by the others; fewer where the weights take more registers) take the
// segments in turn, QS at a time with the
// weight loads of all QS in flight at once, and read the activation rows
// straight from memory (a few per segment at small batches).  The y values of the
// block stay in LDS ([R][NR]); after a barrier the workgroup forms
// out[t, h] = sum_j w[t, j] y[t * k + j, h] (+ x[t, h]) for its rows with the
// combine kernel's arithmetic (FMAs in slot order from zero, then the
// residual).  So there is no y in memory and no combine launch.  Segments on
// the matrix cores (gemv_below) are skipped here; pass 2 on the MFMA kernel
// runs before this launch and writes their y rows to memory (y), from where
// the combine reads them.  A byte per route in LDS, set by the wave that
// computes the route, tells the combine which routes are in LDS, so it reads
// no routing arrays (two dependent round trips per output).
constexpr int kPass2cSegs = 1;   // segments per wave with their loads in flight together
constexpr int kPass2cMaxT = 64;  // batches up to this size take this kernel

// Waves per pass2c workgroup for NC chunks per lane and G lanes per row: as
// many as the weight registers of one wave allow without spilling (fp8 and
// MXFP4 decode into more temporaries).
__host__ __device__ constexpr int pass2c_waves(int WDT, int NC, int G) {
    return (WDT == MOE_FP8_E4M3 || WDT == MOE_MXFP4 || WDT == MOE_Q4_0) ? (NC >= 8 ? 4 : 8)
                                                                        : (NC == 8 || (NC == 2 && G < 64) ? 8 : 16);
}

struct Pass2cArgs {
    const void *down;
    const void *s_down;     // fp8: float block scales; MXFP4: E8M0 bytes
    const float *act;       // [R, I] fp32
    const float *w;         // [T, k] combine weights
    const float *xres;      // [T, H] residual or null
    float *out;             // [T, H]; may alias xres (same element, same thread)
    const int32_t *reject;  // a caller-supplied routing's n_uniq, or null: out untouched when negative
    const float *y;         // [R, H] rows of the routes on the matrix cores, or null (none)
    int H, I, k, T;
    SegArgs sa;
};

template <int WDT, int NC, int G, int QS>
__global__ __launch_bounds__(pass2c_waves(WDT, NC, G) * kWave) void pass2c_kernel(Pass2cArgs a) {
    static_assert(QS == 1 || QS == 2, "segments are fetched one or two at a time");
    extern __shared__ float yl[];  // [R][NR], then a byte per route: its y values are in yl
    constexpr int NS = slots_for(NC);
    constexpr int RPS = kWave / G;
    constexpr int NR = NS * RPS;
    constexpr int EPC = WT<WDT>::kEpc;
    constexpr int WPB = pass2c_waves(WDT, NC, G);
    unsigned char *in_yl = reinterpret_cast<unsigned char *>(yl + a.T * a.k * NR);
    for (int r = threadIdx.x; r < a.T * a.k; r += WPB * kWave) in_yl[r] = 0;
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1), half = lane / G;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int H = a.H, I = a.I, nq = I / EPC;
    const int h0 = blockIdx.x * NR;
    SegArgs sa = a.sa;
    const int nu = a.reject ? __builtin_nontemporal_load(a.reject) : 0;
    // The experts of a wave's QS segments come in one scalar round trip
    // (with the segment count, for the first ones); the weight loads are
    // issued with the experts alone, and the segments' first slots and counts
    // are read while they are in flight.  ids / uniq indices are clamped: an
    // entry past the segment count is read but not used.
    const int lim = sa.grouped ? sa.E - 1 : sa.R - 1;
    const int32_t *elist = sa.grouped ? sa.uniq : sa.ids;
    int s0 = wv * QS, nseg, ev[2];
    if (sa.grouped) {
        if (sa.gemv_below != INT_MAX && sa.max_count) {  // the threshold too, in the same round trip
            int mx;
            load_uniform4(sa.n_uniq, elist + min(s0, lim), elist + min(s0 + 1, lim), sa.max_count, nseg, ev[0],
                          ev[1], mx);
            if (mx < sa.hot) sa.gemv_below = INT_MAX;
        } else {
            load_uniform3(sa.n_uniq, elist + min(s0, lim), elist + min(s0 + 1, lim), nseg, ev[0], ev[1]);
        }
        nseg = nseg > 0 ? nseg : 0;
    } else {
        nseg = sa.R;
        load_uniform2(elist + min(s0, lim), elist + min(s0 + 1, lim), ev[0], ev[1]);
    }
    for (; s0 < nseg; s0 += WPB * QS) {
        int e[QS], first[QS], n[QS];
        bool live[QS];
#pragma unroll
        for (int q = 0; q < QS; ++q) {
            live[q] = s0 + q < nseg && ev[q] >= 0 && ev[q] < sa.E;
            e[q] = live[q] ? ev[q] : 0;
        }
        u32x4 w[QS][NS][NC];
        float sc[QS][NS][NC];
#pragma unroll
        for (int q = 0; q < QS; ++q) {
            const char *rows[NS];
            bool ok[NS];
            down_rows<WDT, NC, NS, G>(a.down, a.s_down, e[q], h0, H, I, live[q], lane, rows, ok, sc[q]);
            load_rows<NC, NS, G>(w[q], rows, ok, nq, lane);
        }
        if (sa.grouped) {
            if constexpr (QS == 2)
                load_uniform4(sa.offsets + e[0], sa.counts + e[0], sa.offsets + e[1], sa.counts + e[1], first[0],
                              n[0], first[1], n[1]);
            else
                load_uniform2(sa.offsets + e[0], sa.counts + e[0], first[0], n[0]);
        } else {
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                first[q] = s0 + q;
                n[q] = 1;
            }
        }
#pragma unroll
        for (int q = 0; q < QS; ++q)
            if (!live[q] || n[q] >= sa.gemv_below) n[q] = 0;
        // the next pair's experts, while this pair's weights are in flight
        const int s1 = s0 + WPB * QS;
        if (s1 < nseg) load_uniform2(elist + min(s1, lim), elist + min(s1 + 1, lim), ev[0], ev[1]);
#pragma unroll
        for (int q = 0; q < QS; ++q) {
            // routes in pairs (one weight decode for both), then a single one
            auto routes = [&](auto rb_tag, int m) {
                constexpr int RB = decltype(rb_tag)::value;
                const float4 *x[RB];
                int r[RB];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    r[i] = segment_route_uniform(sa, first[q], m + i);
                    x[i] = reinterpret_cast<const float4 *>(a.act + (size_t)r[i] * I);
                }
                float acc[RB][NS];
                dot_rows<WDT, NC, NS, G, RB>(w[q], sc[q], x, nq, lane, acc);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    float v[NS][1];
#pragma unroll
                    for (int j = 0; j < NS; ++j) v[j][0] = acc[i][j];
                    reduce_slots<NS, 1, G>(v, lane);
                    const int j = reduced_slot<NS, G>(lane);
                    if (slot_leader<NS, G>(lane)) yl[r[i] * NR + j * RPS + half] = v[0][0];
                    if (lane == 0) in_yl[r[i]] = 1;
                }
            };
            int m = 0;
            for (; m + 1 < n[q]; m += 2) routes(std::integral_constant<int, 2>{}, m);
            if (m < n[q]) routes(std::integral_constant<int, 1>{}, m);
        }
    }
    __syncthreads();
    if (nu < 0) return;
    const int T = a.T, k = a.k;
    for (int idx = threadIdx.x; idx < T * NR; idx += WPB * kWave) {
        const int t = idx / NR, i = idx - t * NR, h = h0 + i;
        if (h >= H) continue;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int r = t * k + j;
            // a route of an expert on the matrix cores: its y row is in memory
            const bool mf = a.y && !in_yl[r];
            acc = fmaf(a.w[r], mf ? a.y[(size_t)r * H + h] : yl[r * NR + i], acc);
        }
        if (a.xres) acc += a.xres[(size_t)t * H + h];
        a.out[(size_t)t * H + h] = acc;
    }
}

// Chunks per lane are instantiated for 1, 2, 3, 4 and 8; other counts run on
// the next larger instance (chunks past the row end are masked).
__host__ __device__ constexpr int nc_instance(int nc) { return nc <= 4 ? nc : 8; }

// Lanes per down row: 32 when a row's 16-byte chunks are a multiple of 32 but
// not of 64 (e.g. 768 bf16), so no lane idles; otherwise 64.  MXFP4 and q4_0
// rows are short (I/32 chunks): 16 or 8 lanes per row when the chunks divide so.
// Fewer lanes than 64 only while a lane's chunks stay within the kernels'
// largest instance (8 chunks, 4 for q4_0): 288 bf16 chunks (I = 2304) take
// 64 lanes of 5 chunks, not 32 of 9.
inline int pass2_lanes(int nq, int dtype) {
    const int max_nc = max_chunks_per_lane(dtype);
    if (nq % 64 == 0) return 64;
    if (nq % 32 == 0 && nq / 32 <= max_nc) return 32;
    if (dtype == MOE_MXFP4 || dtype == MOE_Q4_0) {
        if (nq % 16 == 0 && nq / 16 <= max_nc) return 16;
        if (nq % 8 == 0 && nq / 8 <= max_nc) return 8;
    }
    return 64;
}

template <int WDT>
hipError_t launch_pass1(int nc, int grid, hipStream_t st, const Pass1Args &a) {
    const size_t lds = (size_t)a.nb * a.H * 4;
#define MOE_P1(N) hipLaunchKernelGGL((pass1_kernel<WDT, N>), dim3(grid), dim3(kGemvBlock), lds, st, a)
    switch (nc_instance(nc)) {
        case 1: MOE_P1(1); break;
        case 2: MOE_P1(2); break;
        case 3: MOE_P1(3); break;
        case 4: MOE_P1(4); break;
        case 8:
            if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
            else MOE_P1(8);
            break;
        default: return hipErrorInvalidValue;
    }
#undef MOE_P1
    return hipGetLastError();
}

template <int WDT>
hipError_t launch_pass2(int nc, int lanes, int grid, hipStream_t st, const Pass2Args &a) {
    const size_t lds = (size_t)a.nb * a.I * 4;
#define MOE_P2(N, L) hipLaunchKernelGGL((pass2_kernel<WDT, N, L>), dim3(grid), dim3(kGemvBlock), lds, st, a)
    if constexpr (WDT == MOE_MXFP4 || WDT == MOE_Q4_0) {
        if (lanes == 16 || lanes == 8) {
            switch (nc_instance(nc) * 100 + lanes) {
                case 116: MOE_P2(1, 16); break;
                case 216: MOE_P2(2, 16); break;
                case 316: MOE_P2(3, 16); break;
                case 416: MOE_P2(4, 16); break;
                case 816:
                    if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
                    else MOE_P2(8, 16);
                    break;
                case 108: MOE_P2(1, 8); break;
                case 208: MOE_P2(2, 8); break;
                case 308: MOE_P2(3, 8); break;
                case 408: MOE_P2(4, 8); break;
                case 808:
                    if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
                    else MOE_P2(8, 8);
                    break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    if (lanes == 32) {
        switch (nc_instance(nc)) {
            case 1: MOE_P2(1, 32); break;
            case 2: MOE_P2(2, 32); break;
            case 3: MOE_P2(3, 32); break;
            case 4: MOE_P2(4, 32); break;
            case 8:
                if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
                else MOE_P2(8, 32);
                break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (nc_instance(nc)) {
            case 1: MOE_P2(1, 64); break;
            case 2: MOE_P2(2, 64); break;
            case 3: MOE_P2(3, 64); break;
            case 4: MOE_P2(4, 64); break;
            case 8:
                if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
                else MOE_P2(8, 64);
                break;
            default: return hipErrorInvalidValue;
        }
    }
#undef MOE_P2
    return hipGetLastError();
}

// Rows of down per pass2c workgroup (one wave's NR) for chunks-per-lane
// instance nc and lanes per row.
inline int pass2c_rows(int nc, int lanes) { return slots_for(nc) * (kWave / lanes); }

template <int WDT>
hipError_t launch_pass2c(int nc, int lanes, hipStream_t st, const Pass2cArgs &a) {
    const int nr = pass2c_rows(nc_instance(nc), lanes);
    const dim3 grid((a.H + nr - 1) / nr);
    const size_t lds = (size_t)a.T * a.k * (nr * 4 + 1);
#define MOE_P2C(N, L) \
    hipLaunchKernelGGL((pass2c_kernel<WDT, N, L, kPass2cSegs>), grid, dim3(pass2c_waves(WDT, N, L) * kWave), lds, st, a)
    switch (nc_instance(nc) * 100 + lanes) {
        case 164: MOE_P2C(1, 64); break;
        case 264: MOE_P2C(2, 64); break;
        case 364: MOE_P2C(3, 64); break;
        case 464: MOE_P2C(4, 64); break;
        case 864:
            if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
            else MOE_P2C(8, 64);
            break;
        case 132: MOE_P2C(1, 32); break;
        case 232: MOE_P2C(2, 32); break;
        case 332: MOE_P2C(3, 32); break;
        case 432: MOE_P2C(4, 32); break;
        case 832:
            if constexpr (WDT == MOE_Q4_0) return hipErrorInvalidValue;
            else MOE_P2C(8, 32);
            break;
        default:  // 16 or 8 lanes per row take pass2_kernel and the combine launch
            return hipErrorInvalidValue;
    }
#undef MOE_P2C
    return hipGetLastError();
}

// ---- MFMA segments ------------------------------------------------------------
// Segments with at least kMfmaMinRoutes routes (kMfmaMinRoutesWide from
// kMfmaWideTokens tokens) run on the matrix cores (see experts_mfma.hip and
// experts_mfma_wide.hip), in token blocks of kMfmaNarrowTokens (narrow tiles)
// or kMfmaTokens (wide tiles) routes; below kMfmaWideTokens tokens, only
// when the call's largest segment holds kMfmaHotRoutes or more (decided on
// the device from the sort's statistics).  Measured on the large Zipf layer,
// the skewed sweep and the uniform sweep (graph replays): from 5 routes an
// expert's GEMV walk is bound by its fp32 FMAs rather than by HBM, so the
// matrix cores pay from there, but below 128 tokens an MFMA launch that
// holds only a few such experts costs more than it saves (uniform bs=32/64
// +4/+3 us with the threshold at 5 for every call, skewed bs=16/64 -5/-4 us).
constexpr int kMfmaMinRoutes = 5;
constexpr int kMfmaHotRoutes = 8;
constexpr int kMfmaMinRoutesWide = 4;
// MFMA launches are made from this many tokens on.
constexpr int kMfmaMinTokens = 16;
constexpr int kMfmaTokens = 64;
// Token blocks of the narrow tiles (batches below kMfmaWideTokens): half
// the activation rows per LDS stage leave room for a deeper weight ring.
constexpr int kMfmaNarrowTokens = 32;

struct MfmaArgs {
    const void *w;        // pass 1: gate_up [E, 2I, H]; pass 2: down [E, H, I]
    const void *scales;   // fp8: float block scales of w; MXFP4: E8M0 bytes; else null
    const void *src;      // bf16 rows: pass 1 x [T, H]; pass 2 a[r] in the first half of fp32 row r of act
    float *dst;           // pass 1: act [R, I]; pass 2: y [R, H]
    int H, I, k;
    int min_n;            // segments with at least min_n routes (if the largest holds hot or more)
    int hot;
    int act_bf16;         // pass 1: write a[r] as bf16 (for the MFMA pass 2) instead of fp32
    SegArgs sa;           // grouped segments
    const int32_t *max_count;  // if set: largest segment; below min_n the launch has no work
};

// Narrow tiles (experts_mfma.hip): 32 weight rows per item, the 4 waves
// split K.  Wide tiles (experts_mfma_wide.hip): 128 weight rows per item,
// for batches of at least kMfmaWideTokens tokens.
constexpr int kMfmaWideTokens = 128;
template <int WDT>
hipError_t launch_mfma(int pass, int grid, hipStream_t st, const MfmaArgs &a);
extern template hipError_t launch_mfma<MOE_BF16>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma<MOE_FP8_E4M3>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma<MOE_MXFP4>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma<MOE_Q4_0>(int, int, hipStream_t, const MfmaArgs &);
template <int WDT>
hipError_t launch_mfma_wide(int pass, int grid, hipStream_t st, const MfmaArgs &a);
extern template hipError_t launch_mfma_wide<MOE_BF16>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma_wide<MOE_FP8_E4M3>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma_wide<MOE_MXFP4>(int, int, hipStream_t, const MfmaArgs &);
extern template hipError_t launch_mfma_wide<MOE_Q4_0>(int, int, hipStream_t, const MfmaArgs &);

// Defined in experts_<dtype>.hip.
extern template hipError_t launch_pass1<MOE_F32>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass1<MOE_BF16>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass1<MOE_FP8_E4M3>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass2<MOE_F32>(int, int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2<MOE_BF16>(int, int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2<MOE_FP8_E4M3>(int, int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass1<MOE_MXFP4>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass2<MOE_MXFP4>(int, int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2c<MOE_F32>(int, int, hipStream_t, const Pass2cArgs &);
extern template hipError_t launch_pass2c<MOE_BF16>(int, int, hipStream_t, const Pass2cArgs &);
extern template hipError_t launch_pass2c<MOE_FP8_E4M3>(int, int, hipStream_t, const Pass2cArgs &);
extern template hipError_t launch_pass2c<MOE_MXFP4>(int, int, hipStream_t, const Pass2cArgs &);
extern template hipError_t launch_pass1<MOE_Q4_0>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass2<MOE_Q4_0>(int, int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2c<MOE_Q4_0>(int, int, hipStream_t, const Pass2cArgs &);

}  // namespace moe
