// Routing of one MoE layer in one launch: [RMSNorm] -> router GEMV ->
// top-k selection -> counting sort, with no host read anywhere.
//
// "MoE Performance Optimization Analysis" (markbaseengine), Root Cause and
// Option 1: the per-layer host read of the router scores and the host-side
// top-2 are the cost; the fix is a device router with device selection and
// dispatch.  "TEXT Generation Optimization Report", Phase 2: fewer, fused
// dispatches.  Here the router, the selection and the sort are one kernel:
//
//  * Workgroup (eb, tb) computes the logits of 16 experts (4 per wave, rows
//    held in registers; 4 experts, one per wave, for batches of up to
//    kRouteSmallT tokens, so that four times as many workgroups stream the
//    router rows) for a tile of up to 8 tokens (32 KiB, 64 KiB for
//    batches of 128 tokens or more) staged in LDS
//    (normalised there first for the RMSNorm form; workgroup eb = 0 also
//    writes the normalised rows for the expert passes).  In a layer stack
//    the staged rows can be the previous layer's combine plus its residual,
//    formed here with the combine kernel's arithmetic (workgroup eb = 0
//    writes them out as the next residual), which saves that kernel.
//  * The last workgroup to finish a token tile (per-tile arrival counter)
//    selects the top k for those tokens, two tokens per wave at once.
//  * The last tile to be selected (arrival counter over tiles) runs the
//    counting sort in that workgroup.
// Nothing waits: a workgroup that is not last simply exits.  The arrival
// counters are reset by the workgroup that consumed them, so they are zero
// again when the launch ends (a fresh workspace is zeroed once by
// moe_workspace_init).
#include <type_traits>

#include "route_impl.h"

namespace moe {

constexpr int kRouteRows = 4;                      // router rows per wave
constexpr int kRouteSmallT = 16;                   // up to here: one row per wave
constexpr int kRouteTileFloats = 8192;             // token tile: 32 KiB of LDS
constexpr int kRouteTileFloatsLarge = 16384;       // from kRouteLargeT tokens: 64 KiB
constexpr int kRouteLargeT = 128;

// Tokens per tile: up to 8, in 32 KiB of LDS (64 KiB for large batches,
// which have tiles enough to fill the chip and re-read the router rows once
// per tile).
__host__ __device__ constexpr int route_tile_tokens(int H, int T) {
    const int f = T >= kRouteLargeT ? kRouteTileFloatsLarge : kRouteTileFloats;
    return H >= f ? 1 : (f / H < 8 ? f / H : 8);
}

struct RouteArgs {
    const void *wr;          // router weights [E, H] (null: logits_in given)
    const float *bias;       // [E] or null
    const float *x;          // [T, H]
    const float *logits_in;  // [T, E] or null
    float *xn;               // normalised rows [T, H] (RMSNorm form) or null
    // previous layer's combine, fused (prev_y null: x is the input):
    // rows = prev_h + sum_j prev_w[t, j] * prev_y[t * prev_k + j]
    const float *prev_y;     // [T * prev_k, H]
    const float *prev_w;     // [T, prev_k]
    const float *prev_h;     // [T, H] residual
    float *h_out;            // [T, H] the combined rows (written by eb = 0)
    uint32_t *xb;            // bf16 copy of the staged rows [T, H] (written by eb = 0) or null
    int prev_k;
    float *logits;           // [T, E] out (when computed)
    int32_t *ids;            // [T, k]
    float *w;                // [T, k]
    int32_t *counts, *offsets, *sorted, *uniq, *n_uniq, *stats;  // counts null: no sort
    unsigned *arrive;        // [n_tblk + 1] arrival counters, zero on entry and exit
    unsigned *zero;          // counters of the kernels that follow, zeroed by the sort
    int n_zero;
    int T, E, H, k, n_eblk, n_tblk, tile;
    int rmsnorm;
    float eps;
};

template <int RDT, int NC, int RR>
__global__ __launch_bounds__(kBlock) void route_kernel(RouteArgs a) {
    extern __shared__ float4 dyn_lds[];
    float *tile = reinterpret_cast<float *>(dyn_lds);
    __shared__ int s_last;
    constexpr int EPC = WT<RDT>::kEpc;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int eb = blockIdx.x % a.n_eblk, tb = blockIdx.x / a.n_eblk;
    const int t0 = tb * a.tile, t1 = min(a.T, t0 + a.tile);
    const int H = a.H, E = a.E;

    if (!a.logits_in) {
        // router rows e0 .. e0+RR-1 of this wave, issued first (they do not
        // depend on the tokens)
        const int e0 = (eb * (kBlock / kWave) + wave) * RR;
        const int nq = H / EPC;
        const size_t row_bytes = (size_t)H * WT<RDT>::kBytes;
        u32x4 wr[RR][NC];
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int q = lane + kWave * c;
                wr[r][c] = (e0 + r < E && q < nq)
                               ? load_weight_chunk(reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.wr) +
                                                                                    (size_t)(e0 + r) * row_bytes) + q)
                               : u32x4{0u, 0u, 0u, 0u};
            }
        // this lane's router bias (lane r stores row r of the wave), read
        // before the token loop: a load inside it would wait behind the
        // previous tokens' logit stores (vector memory counts in order)
        const float bias_r = (a.bias && lane < RR && e0 + lane < E) ? a.bias[e0 + lane] : 0.f;
        // token tile -> LDS
        const int h4 = H / 4;
        if (a.prev_y) {
            // the previous layer's combine: per element the FMAs over its
            // routes in slot order from zero, then the residual added, as in
            // combine_kernel; 4 elements per thread and 2 routes at a time,
            // with every load of a group issued before its FMAs (8 elements
            // per thread took 241-290 VGPRs and was slower at bs=1)
            constexpr int kU = 4, kJ = 2;
            const int n4 = (t1 - t0) * h4, pk = a.prev_k;
            const float4 *py = reinterpret_cast<const float4 *>(a.prev_y);
            const float4 *ph = reinterpret_cast<const float4 *>(a.prev_h);
            float4 *dst = reinterpret_cast<float4 *>(tile);
            for (int base = 0; base < n4; base += kU * kBlock) {
                int tq[kU], qq[kU];
                float4 acc[kU], res[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int idx = min(base + u * kBlock + (int)threadIdx.x, n4 - 1);
                    tq[u] = t0 + idx / h4;
                    qq[u] = idx - (idx / h4) * h4;
                    acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                    res[u] = ph[(size_t)tq[u] * h4 + qq[u]];
                }
                for (int j0 = 0; j0 < pk; j0 += kJ) {
                    float wj[kU][kJ];
                    float4 v[kU][kJ];
#pragma unroll
                    for (int u = 0; u < kU; ++u)
#pragma unroll
                        for (int jj = 0; jj < kJ; ++jj) {
                            const size_t r = (size_t)tq[u] * pk + min(j0 + jj, pk - 1);
                            wj[u][jj] = a.prev_w[r];
                            v[u][jj] = py[r * h4 + qq[u]];
                        }
#pragma unroll
                    for (int u = 0; u < kU; ++u)
#pragma unroll
                        for (int jj = 0; jj < kJ; ++jj)
                            if (j0 + jj < pk) {
                                acc[u].x = fmaf(wj[u][jj], v[u][jj].x, acc[u].x);
                                acc[u].y = fmaf(wj[u][jj], v[u][jj].y, acc[u].y);
                                acc[u].z = fmaf(wj[u][jj], v[u][jj].z, acc[u].z);
                                acc[u].w = fmaf(wj[u][jj], v[u][jj].w, acc[u].w);
                            }
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int idx = base + u * kBlock + threadIdx.x;
                    if (idx < n4) {
                        acc[u].x += res[u].x; acc[u].y += res[u].y; acc[u].z += res[u].z; acc[u].w += res[u].w;
                        dst[idx] = acc[u];
                        if (eb == 0) reinterpret_cast<float4 *>(a.h_out)[(size_t)tq[u] * h4 + qq[u]] = acc[u];
                    }
                }
            }
        } else {  // the input rows, 8 loads in flight per thread
            const int n4 = (t1 - t0) * h4;
            const float4 *src = reinterpret_cast<const float4 *>(a.x + (size_t)t0 * H);
            float4 *dst = reinterpret_cast<float4 *>(tile);
            for (int base = 0; base < n4; base += 8 * kBlock) {
                float4 v[8];
                // unconditional loads (index clamped), all in flight at once:
                // the empty asm uses every value before any store, so the
                // compiler cannot sink a load under its store's condition
                // (which would wait for each load in turn)
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = src[min(base + u * kBlock + (int)threadIdx.x, n4 - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int idx = base + u * kBlock + threadIdx.x;
                    if (idx < n4) dst[idx] = v[u];
                }
            }
        }
        __syncthreads();
        if (a.rmsnorm) {
            for (int t = wave; t < t1 - t0; t += kBlock / kWave) {
                float4 *row = reinterpret_cast<float4 *>(tile + (size_t)t * H);
                float ss = 0.f;
                for (int q = lane; q < h4; q += kWave) {
                    const float4 v = row[q];
                    ss = fmaf(v.x, v.x, ss);
                    ss = fmaf(v.y, v.y, ss);
                    ss = fmaf(v.z, v.z, ss);
                    ss = fmaf(v.w, v.w, ss);
                }
                ss = wave_sum_dpp(ss);
                const float rs = 1.0f / sqrtf(ss / (float)H + a.eps);
                for (int q = lane; q < h4; q += kWave) {
                    float4 v = row[q];
                    v.x *= rs; v.y *= rs; v.z *= rs; v.w *= rs;
                    row[q] = v;
                    if (eb == 0) reinterpret_cast<float4 *>(a.xn + (size_t)(t0 + t) * H)[q] = v;
                }
            }
            __syncthreads();
        }
        // the bf16 copy of the rows the experts read (for their MFMA
        // segments), pairs rounded to nearest even
        if (a.xb && eb == 0) {
            const int n2 = (t1 - t0) * H / 2;
            const float2 *src2 = reinterpret_cast<const float2 *>(tile);
            uint32_t *dst2 = a.xb + (size_t)t0 * H / 2;
            for (int i = threadIdx.x; i < n2; i += kBlock) {
                const float2 v = src2[i];
                dst2[i] = bf16_pair_rne(v.x, v.y);
            }
        }
        // two tokens per pass (independent chains); each token reduced on its
        // own, so a logit never depends on its position in the tile
        const int nt = t1 - t0;
        for (int t = 0; t < nt; t += 2) {
            const bool two = t + 1 < nt;
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(wr[r][c]));
            float acc0[RR][1], acc1[RR][1];
#pragma unroll
            for (int r = 0; r < RR; ++r) { acc0[r][0] = 0.f; acc1[r][0] = 0.f; }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int q = lane + kWave * c;
                if (q < nq) {
                    float xs0[EPC], xs1[EPC];
                    const float4 *xp0 = reinterpret_cast<const float4 *>(tile + (size_t)t * H + q * EPC);
                    const float4 *xp1 = reinterpret_cast<const float4 *>(tile + (size_t)(two ? t + 1 : t) * H + q * EPC);
#pragma unroll
                    for (int v = 0; v < EPC / 4; ++v) {
                        const float4 f0 = xp0[v], f1 = xp1[v];
                        xs0[4 * v] = f0.x; xs0[4 * v + 1] = f0.y; xs0[4 * v + 2] = f0.z; xs0[4 * v + 3] = f0.w;
                        xs1[4 * v] = f1.x; xs1[4 * v + 1] = f1.y; xs1[4 * v + 2] = f1.z; xs1[4 * v + 3] = f1.w;
                    }
#pragma unroll
                    for (int r = 0; r < RR; ++r) {
                        acc0[r][0] = chunk_dot<RDT>(wr[r][c], xs0, acc0[r][0]);
                        acc1[r][0] = chunk_dot<RDT>(wr[r][c], xs1, acc1[r][0]);
                    }
                }
            }
            // one DPP sum over the wave per row and token; lane r stores row r
            float l0 = 0.f, l1 = 0.f;
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const float s0 = wave_sum_dpp(acc0[r][0]), s1 = wave_sum_dpp(acc1[r][0]);
                if (lane == r) {
                    l0 = s0;
                    l1 = s1;
                }
            }
            if (lane < RR && e0 + lane < E) {
                store_shared(a.logits + (size_t)(t0 + t) * E + e0 + lane, a.bias ? l0 + bias_r : l0);
                if (two) store_shared(a.logits + (size_t)(t0 + t + 1) * E + e0 + lane, a.bias ? l1 + bias_r : l1);
            }
        }
        wait_vm_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
            s_last = atomicAdd(a.arrive + tb, 1u) + 1u == (unsigned)a.n_eblk;
            if (s_last) store_shared(a.arrive + tb, 0u);
        }
        __syncthreads();
        if (!s_last) return;
    }

    // selection for the tile's tokens, two per wave; with a single tile
    // the ids also go to LDS, where the sort below reads them
    const float *lg = a.logits_in ? a.logits_in : a.logits;
    int *lds_ids = a.counts && a.n_tblk == 1 ? reinterpret_cast<int *>(dyn_lds) + sort_lds_ints(E) : nullptr;
    // tokens t and t + 4 of a wave together (their chains overlap), then a
    // last single one
    constexpr int WPB = kBlock / kWave;
    auto sel = [&](auto nt_tag, int t) {
        constexpr int NT = decltype(nt_tag)::value;
        const float *l[NT];
        int32_t *ids[NT], *li[NT];
        float *w[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int tq = t + q * WPB;
            l[q] = lg + (size_t)tq * E;
            ids[q] = a.ids + (size_t)tq * a.k;
            w[q] = a.w + (size_t)tq * a.k;
            li[q] = lds_ids ? lds_ids + (size_t)(tq - t0) * a.k : nullptr;
        }
        if (a.logits_in)
            select_tokens<false, NT>(l, E, a.k, ids, w, li, lane);
        else
            select_tokens<true, NT>(l, E, a.k, ids, w, li, lane);
    };
    int t = t0 + wave;
    for (; t + WPB < t1; t += 2 * WPB) sel(std::integral_constant<int, 2>{}, t);
    if (t < t1) sel(std::integral_constant<int, 1>{}, t);
    if (!a.counts) return;
    if (a.n_tblk == 1) {
        // one tile: this workgroup selected every token, no second arrival;
        // the sort reads the ids from LDS, so the global stores need not have
        // completed
        __syncthreads();
        sort_routes<false>(lds_ids, a.T * a.k, E, a.counts, a.offsets, a.sorted, a.uniq, a.n_uniq, a.stats,
                           reinterpret_cast<int *>(dyn_lds), a.zero, a.n_zero);
        return;
    }
    wait_vm_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        s_last = atomicAdd(a.arrive + a.n_tblk, 1u) + 1u == (unsigned)a.n_tblk;
        if (s_last) store_shared(a.arrive + a.n_tblk, 0u);
    }
    __syncthreads();
    if (!s_last) return;
    sort_routes<true>(a.ids, a.T * a.k, E, a.counts, a.offsets, a.sorted, a.uniq, a.n_uniq, a.stats,
                      reinterpret_cast<int *>(dyn_lds), a.zero, a.n_zero);
}

template <int RDT, int RR>
static hipError_t route_dispatch(int nc, dim3 g, size_t lds, hipStream_t st, const RouteArgs &a) {
    switch (nc) {
#define MOE_RC(N) \
    case N: hipLaunchKernelGGL((route_kernel<RDT, N, RR>), g, dim3(kBlock), lds, st, a); break;
        MOE_RC(1) MOE_RC(2) MOE_RC(3) MOE_RC(4) MOE_RC(5) MOE_RC(6) MOE_RC(7) MOE_RC(8)
#undef MOE_RC
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_route(const moe_layer_t &L, const float *x, const float *logits_in, int T, float *xn,
                        float *logits, int32_t *ids, float *w, int32_t *counts, int32_t *offsets, int32_t *sorted,
                        int32_t *uniq, int32_t *n_uniq, int32_t *stats, unsigned *arrive, bool rmsnorm,
                        unsigned *zero, int n_zero, hipStream_t st, const PrevCombine *prev, uint32_t *xb) {
    RouteArgs a;
    a.prev_y = prev ? prev->y : nullptr;
    a.prev_w = prev ? prev->w : nullptr;
    a.prev_h = prev ? prev->h : nullptr;
    a.h_out = prev ? prev->h_out : nullptr;
    a.prev_k = prev ? prev->k : 0;
    a.zero = zero;
    a.n_zero = n_zero;
    a.wr = L.w_router;
    a.bias = L.router_bias;
    a.x = x;
    a.logits_in = logits_in;
    a.xn = xn;
    a.xb = logits_in ? nullptr : xb;
    a.logits = logits;
    a.ids = ids;
    a.w = w;
    a.counts = counts;
    a.offsets = offsets;
    a.sorted = sorted;
    a.uniq = uniq;
    a.n_uniq = n_uniq;
    a.stats = stats;
    a.arrive = arrive;
    a.T = T;
    a.E = L.E;
    a.H = L.H;
    a.k = L.top_k;
    a.rmsnorm = rmsnorm ? 1 : 0;
    a.eps = 1e-6f;
    a.tile = logits_in ? (kBlock / kWave) : route_tile_tokens(L.H, T);
    // router rows per wave: one for small batches (more workgroups stream the
    // router rows), four otherwise (each row is re-read once per token tile)
    const int rr = T <= kRouteSmallT ? 1 : kRouteRows;
    const int experts_per_wg = rr * (kBlock / kWave);
    a.n_eblk = logits_in ? 1 : (L.E + experts_per_wg - 1) / experts_per_wg;
    a.n_tblk = (T + a.tile - 1) / a.tile;
    // the sort's LDS, then (single tile) the selected ids
    size_t lds = ((size_t)sort_lds_ints(L.E) + (size_t)a.tile * L.top_k) * 4;
    if (!logits_in) {
        const size_t tb = (size_t)a.tile * L.H * 4;
        lds = tb > lds ? tb : lds;
    }
    const int epc = elems_per_chunk(L.router_dtype);
    const int nc = logits_in ? 1 : (L.H / epc + kWave - 1) / kWave;
    const dim3 g(a.n_eblk * a.n_tblk);
    if (L.router_dtype == MOE_BF16)
        return rr == 1 ? route_dispatch<MOE_BF16, 1>(nc, g, lds, st, a)
                       : route_dispatch<MOE_BF16, kRouteRows>(nc, g, lds, st, a);
    return rr == 1 ? route_dispatch<MOE_F32, 1>(nc, g, lds, st, a)
                   : route_dispatch<MOE_F32, kRouteRows>(nc, g, lds, st, a);
}

// ---- fill kernel (workspace initialisation) ----------------------------------
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(unsigned *p, int n) {
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < n; i += gridDim.x * kBlock) p[i] = 0u;
}

hipError_t launch_zero(unsigned *p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((n + kBlock - 1) / kBlock < 64 ? (n + kBlock - 1) / kBlock : 64),
                       dim3(kBlock), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace moe
