// Templates of the GEMV expert passes, instantiated once per weight dtype in
// experts_<dtype>.hip.  See experts.hip for what the passes compute.
#pragma once

#include "common.h"

namespace moe {

struct SegArgs {
    const int32_t *ids, *counts, *offsets, *sorted, *uniq, *n_uniq;
    int grouped;  // 1: segment = unique expert, 0: segment = one route
    int R;        // routes
    int E;        // experts (ids outside [0, E) make an empty segment)
};

// Expert, first sorted slot and route count of segment s.
__device__ __forceinline__ void segment(const SegArgs &sa, int s, int &e, int &first, int &n) {
    if (sa.grouped) {
        e = sa.uniq[s];
        first = sa.offsets[e];
        n = sa.counts[e];
    } else {
        e = sa.ids[s];
        first = s;
        n = 1;
    }
    if (e < 0 || e >= sa.E) {
        e = 0;
        n = 0;
    }
}

__device__ __forceinline__ int segment_route(const SegArgs &sa, int first, int i) {
    return sa.grouped ? sa.sorted[first + i] : first + i;
}

__device__ __forceinline__ int segment_count(const SegArgs &sa) { return sa.grouped ? *sa.n_uniq : sa.R; }

// Loads chunk c of rows rows[r] (byte pointers), zero where invalid.
template <int NC, int NR>
__device__ __forceinline__ void load_rows(u32x4 (&w)[NR][NC], const char *const (&rows)[NR], const bool (&ok)[NR],
                                          int nq, int lane) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = lane + kWave * c;
            w[r][c] = (ok[r] && q < nq) ? load_weight_chunk(reinterpret_cast<const u32x4 *>(rows[r]) + q)
                                        : u32x4{0u, 0u, 0u, 0u};
        }
}

// acc[r] = lane partial of rows r . xv (chunk order), fp8 chunks scaled by
// their block scale.
template <int WDT, int NC, int NR>
__device__ __forceinline__ void dot_rows(const u32x4 (&w)[NR][NC], const float (&sc)[NR][NC],
                                         const float *__restrict__ xv, int nq, int lane, float (&acc)[NR]) {
    constexpr int EPC = WT<WDT>::kEpc;
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int q = lane + kWave * c;
        if (q < nq) {
            float xs[EPC];
            const float4 *xp = reinterpret_cast<const float4 *>(xv + q * EPC);
#pragma unroll
            for (int v = 0; v < EPC / 4; ++v) {
                const float4 f = xp[v];
                xs[4 * v] = f.x; xs[4 * v + 1] = f.y; xs[4 * v + 2] = f.z; xs[4 * v + 3] = f.w;
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (WDT == MOE_FP8_E4M3) acc[r] = fmaf(sc[r][c], chunk_dot<WDT>(w[r][c], xs, 0.f), acc[r]);
                else acc[r] = chunk_dot<WDT>(w[r][c], xs, acc[r]);
            }
        }
    }
}

// ---- pass 1: gate_up rows, activation ------------------------------------
struct Pass1Args {
    const void *gate_up;
    const float *s_gate_up;
    const float *x;
    float *act;
    int H, I, k;
    SegArgs sa;
};

template <int WDT, int NC>
__global__ __launch_bounds__(kBlock) void pass1_kernel(Pass1Args a) {
    constexpr int P = rows_per_wave(NC) / 2;  // gate/up pairs per wave
    constexpr int NR = 2 * P;
    constexpr int EPC = WT<WDT>::kEpc;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int H = a.H, I = a.I, nq = H / EPC;
    const int pairs_per_item = 4 * P;
    const int items_per_seg = (I + pairs_per_item - 1) / pairs_per_item;
    const int n_items = segment_count(a.sa) * items_per_seg;
    const size_t row_bytes = (size_t)H * WT<WDT>::kBytes;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int s = item / items_per_seg, blk = item % items_per_seg;
        int e, first, n;
        segment(a.sa, s, e, first, n);
        const int i0 = blk * pairs_per_item + wave * P;
        const char *rows[NR];
        bool ok[NR];
        float sc[NR][NC];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p;
            ok[p] = ok[P + p] = i < I;
            const char *base = static_cast<const char *>(a.gate_up) + (size_t)e * 2 * I * row_bytes;
            rows[p] = base + (size_t)i * row_bytes;
            rows[P + p] = base + (size_t)(I + i) * row_bytes;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) sc[r][c] = 1.f;
        if (WDT == MOE_FP8_E4M3) {
            const int nbh = H / 128;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int i = min(i0 + p, I - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int hb = min((lane + kWave * c) * EPC / 128, nbh - 1);
                    sc[p][c] = a.s_gate_up[((size_t)e * (2 * I / 128) + i / 128) * nbh + hb] * kE4m3Unscale;
                    sc[P + p][c] = a.s_gate_up[((size_t)e * (2 * I / 128) + (I + i) / 128) * nbh + hb] * kE4m3Unscale;
                }
            }
        }
        u32x4 w[NR][NC];
        load_rows<NC, NR>(w, rows, ok, nq, lane);
        for (int m = 0; m < n; ++m) {
            const int r = segment_route(a.sa, first, m);
            const int t = r / a.k;
            float acc[NR];
            dot_rows<WDT, NC, NR>(w, sc, a.x + (size_t)t * H, nq, lane, acc);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float g = wave_sum(acc[p]);
                const float u = wave_sum(acc[P + p]);
                if (lane == p && ok[p]) a.act[(size_t)r * I + i0 + p] = silu(g) * u;
            }
        }
    }
}

// ---- pass 2: down rows ---------------------------------------------------
struct Pass2Args {
    const void *down;
    const float *s_down;
    const float *act;
    float *y;
    int H, I;
    SegArgs sa;
};

template <int WDT, int NC>
__global__ __launch_bounds__(kBlock) void pass2_kernel(Pass2Args a) {
    constexpr int NR = rows_per_wave(NC);
    constexpr int EPC = WT<WDT>::kEpc;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int H = a.H, I = a.I, nq = I / EPC;
    const int rows_per_item = 4 * NR;
    const int items_per_seg = (H + rows_per_item - 1) / rows_per_item;
    const int n_items = segment_count(a.sa) * items_per_seg;
    const size_t row_bytes = (size_t)I * WT<WDT>::kBytes;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int s = item / items_per_seg, blk = item % items_per_seg;
        int e, first, n;
        segment(a.sa, s, e, first, n);
        const int h0 = blk * rows_per_item + wave * NR;
        const char *rows[NR];
        bool ok[NR];
        float sc[NR][NC];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            ok[r] = h0 + r < H;
            rows[r] = static_cast<const char *>(a.down) + ((size_t)e * H + h0 + r) * row_bytes;
#pragma unroll
            for (int c = 0; c < NC; ++c) sc[r][c] = 1.f;
        }
        if (WDT == MOE_FP8_E4M3) {
            const int nbi = I / 128;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int h = min(h0 + r, H - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ib = min((lane + kWave * c) * EPC / 128, nbi - 1);
                    sc[r][c] = a.s_down[((size_t)e * (H / 128) + h / 128) * nbi + ib] * kE4m3Unscale;
                }
            }
        }
        u32x4 w[NR][NC];
        load_rows<NC, NR>(w, rows, ok, nq, lane);
        for (int m = 0; m < n; ++m) {
            const int r = segment_route(a.sa, first, m);
            float acc[NR];
            dot_rows<WDT, NC, NR>(w, sc, a.act + (size_t)r * I, nq, lane, acc);
#pragma unroll
            for (int rr = 0; rr < NR; ++rr) {
                const float v = wave_sum(acc[rr]);
                if (lane == rr && ok[rr]) a.y[(size_t)r * H + h0 + rr] = v;
            }
        }
    }
}


// Chunks per lane are instantiated for 1, 2, 3, 4 and 8; other counts run on
// the next larger instance (chunks past the row end are masked).
__host__ __device__ constexpr int nc_instance(int nc) { return nc <= 4 ? nc : 8; }

template <int WDT>
hipError_t launch_pass1(int nc, int grid, hipStream_t st, const Pass1Args &a) {
    switch (nc_instance(nc)) {
        case 1: hipLaunchKernelGGL((pass1_kernel<WDT, 1>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 2: hipLaunchKernelGGL((pass1_kernel<WDT, 2>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 3: hipLaunchKernelGGL((pass1_kernel<WDT, 3>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 4: hipLaunchKernelGGL((pass1_kernel<WDT, 4>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 8: hipLaunchKernelGGL((pass1_kernel<WDT, 8>), dim3(grid), dim3(kBlock), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int WDT>
hipError_t launch_pass2(int nc, int grid, hipStream_t st, const Pass2Args &a) {
    switch (nc_instance(nc)) {
        case 1: hipLaunchKernelGGL((pass2_kernel<WDT, 1>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 2: hipLaunchKernelGGL((pass2_kernel<WDT, 2>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 3: hipLaunchKernelGGL((pass2_kernel<WDT, 3>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 4: hipLaunchKernelGGL((pass2_kernel<WDT, 4>), dim3(grid), dim3(kBlock), 0, st, a); break;
        case 8: hipLaunchKernelGGL((pass2_kernel<WDT, 8>), dim3(grid), dim3(kBlock), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Defined in experts_<dtype>.hip.
extern template hipError_t launch_pass1<MOE_F32>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass1<MOE_BF16>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass1<MOE_FP8_E4M3>(int, int, hipStream_t, const Pass1Args &);
extern template hipError_t launch_pass2<MOE_F32>(int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2<MOE_BF16>(int, int, hipStream_t, const Pass2Args &);
extern template hipError_t launch_pass2<MOE_FP8_E4M3>(int, int, hipStream_t, const Pass2Args &);

}  // namespace moe
