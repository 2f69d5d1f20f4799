// Expert passes and combine: grouped GEMV over the unique experts.
//
// "perf(cpu-moe): dedup experts across the batch in pass 1" (FreeToken PR
// #46), commit message: pass 1 is split by (unique expert, row block) with
// the expert's routes as the inner loop, so each gate_up row is read from
// memory once and reused for every token routed to that expert; pass 2 reads
// down [H, I]; the follow-up change deduplicates pass 2 the same way.  Here:
//
//  * A segment is one expert with its routes: a unique expert and its slice
//    of the sorted route list (grouped walk), or a single route (per-route
//    walk).  Work items are (segment, row block); a persistent grid strides
//    over the items, whose count depends on the device-side n_uniq.
//  * A wave keeps its weight rows in registers as raw 16-byte chunks (lane l
//    holds chunks l, l+64, ...), loaded once with streaming loads, and then
//    walks the segment's routes: each (row, route) dot product is one lane
//    partial in chunk order followed by one butterfly reduction.  The same
//    (row, route) pair is computed the same way whatever segment it sits in,
//    so every walk gives bitwise the same result.
//  * Pass 1 keeps gate row i and up row I+i in the same wave and writes the
//    activation a[r, i] = silu(g) * u directly; pass 2 writes y[r, h]; rows of
//    both workspaces are indexed by route r = t*k + j.
//  * Combine: out[t, h] = sum_j w[t, j] * y[t*k + j, h], j ascending
//    ("MoE Performance Optimization Analysis", Root Cause, step 6, combine
//    on the device), plus x[t, h] for the residual form.
#include <limits.h>

#include <algorithm>

#include "experts_impl.h"

namespace moe {

// ---- combine ------------------------------------------------------------------
// out may alias xres: each thread reads its residual before storing there.
__global__ __launch_bounds__(kBlock) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                         const float *xres, float *out, int k, int H) {
    const int t = blockIdx.x;
    const int h = (blockIdx.y * kBlock + threadIdx.x) * 4;
    if (h >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)t * k + j) * H + h);
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    if (xres) {
        const float4 r = *reinterpret_cast<const float4 *>(xres + (size_t)t * H + h);
        acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
    }
    *reinterpret_cast<float4 *>(out + (size_t)t * H + h) = acc;
}

// ---- launchers -------------------------------------------------------------------
static int persistent_grid(long long max_items) {
    const long long cap = (long long)num_cus() * 8;
    long long g = max_items < cap ? max_items : cap;
    return (int)(g < 1 ? 1 : g);
}

// Segments with at least kMfmaMinRoutes routes go to the MFMA kernels when the
// weights are bf16 or fp8 with H and I multiples of 128, unless the caller
// asked for the GEMV path only.  A segment cannot hold more routes than there
// are tokens, so below kMfmaMinRoutes tokens no MFMA kernel is launched.
static bool mfma_eligible(const moe_layer_t &L, int T, uint32_t flags) {
    // the narrow kernels address activation rows with 32-bit byte offsets
    const bool offsets32 = (unsigned long long)T * L.H * 2 < (1ull << 32) &&
                           (unsigned long long)T * L.top_k * L.I * 4 < (1ull << 32);
    return (L.expert_dtype == MOE_BF16 || L.expert_dtype == MOE_FP8_E4M3) && L.H % 128 == 0 && L.I % 128 == 0 &&
           !(flags & MOE_NO_MFMA) && T >= kMfmaMinRoutes && (int)(flags & MOE_WALK_MASK) != MOE_WALK_PER_ROUTE &&
           offsets32;
}

// Small batches have few hot experts: narrow items (32 weight rows) spread
// them over the chip.  Large batches have many items anyway, and wide items
// (128 weight rows) read each staged activation row for 4x more weights.
static hipError_t launch_mfma_pass(const moe_layer_t &L, int pass, int T, const MfmaArgs &a, hipStream_t st) {
    const bool wide = T >= kMfmaWideTokens;
    // items <= row blocks x (segments that can reach the threshold + extra token blocks)
    const long long R = (long long)T * L.top_k;
    const long long segs = std::min<long long>(L.E, R / kMfmaMinRoutes);
    const long long n_rb = pass == 1 ? L.I / (wide ? 64 : 16) : L.H / (wide ? 128 : 32);
    const long long items = n_rb * (segs + R / kMfmaTokens);
    const long long cap = (long long)num_cus() * 2;
    const int grid = (int)std::max<long long>(1, std::min(items, cap));
    if (wide)
        return L.expert_dtype == MOE_BF16 ? launch_mfma_wide<MOE_BF16>(pass, grid, st, a)
                                          : launch_mfma_wide<MOE_FP8_E4M3>(pass, grid, st, a);
    return L.expert_dtype == MOE_BF16 ? launch_mfma<MOE_BF16>(pass, grid, st, a)
                                      : launch_mfma<MOE_FP8_E4M3>(pass, grid, st, a);
}

hipError_t launch_experts(const moe_layer_t &L, const float *x, const float *xres, int T, const Routing &rt,
                          void *xb, float *act, float *y, float *out, uint32_t flags, hipStream_t st,
                          const hipEvent_t *ev) {
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
    const int R = T * L.top_k;
    const int walk = (int)(flags & MOE_WALK_MASK);
    const int epc = elems_per_chunk(L.expert_dtype);
    const int max_uniq = R < L.E ? R : L.E;
    const bool mfma = mfma_eligible(L, T, flags);
    SegArgs grouped{rt.ids, rt.counts, rt.offsets, rt.sorted, rt.uniq, rt.n_uniq, 1, R, L.E, INT_MAX};
    SegArgs per_route = grouped;
    per_route.grouped = 0;
    SegArgs split = grouped;  // the GEMV share of a pass that also has MFMA segments
    if (mfma) split.gemv_below = kMfmaMinRoutes;

    // pass 1: one wave item = P gate/up pairs of one segment
    Pass1Args p1{L.w_gate_up, L.s_gate_up, x, act, L.H, L.I, L.top_k, walk == MOE_WALK_PER_ROUTE ? per_route : split,
                 mfma ? static_cast<uint32_t *>(xb) : nullptr, lds_batch_rows(L.H)};
    const int nq1 = L.H / epc;
    const int nc1 = nc_instance((nq1 + kWave - 1) / kWave);
    const int pairs = slots_for(nc1) / 2 * (kBlock / kWave);  // per workgroup item
    const long long items1 = (long long)(p1.sa.grouped ? max_uniq : R) * ((L.I + pairs - 1) / pairs);
    hipError_t err;
    switch (L.expert_dtype) {
        case MOE_F32: err = launch_pass1<MOE_F32>(nc1, persistent_grid(items1), st, p1); break;
        case MOE_BF16: err = launch_pass1<MOE_BF16>(nc1, persistent_grid(items1), st, p1); break;
        default: err = launch_pass1<MOE_FP8_E4M3>(nc1, persistent_grid(items1), st, p1); break;
    }
    if (err != hipSuccess || (err = mark(0)) != hipSuccess) return err;
    const bool mfma2 = mfma && walk == MOE_WALK_DEDUP;
    if (mfma) {
        MfmaArgs m1{L.w_gate_up, L.s_gate_up, xb, act, L.H, L.I, L.top_k, kMfmaMinRoutes, mfma2 ? 1 : 0, grouped,
                    rt.max_count};
        if ((err = launch_mfma_pass(L, 1, T, m1, st)) != hipSuccess) return err;
    }
    if ((err = mark(1)) != hipSuccess) return err;

    // pass 2: one wave item = slots x (64 / lanes) down rows of one segment
    Pass2Args p2{L.w_down, L.s_down, act, y, L.H, L.I, walk == MOE_WALK_DEDUP ? (mfma2 ? split : grouped) : per_route,
                 lds_batch_rows(L.I)};
    const int nq2 = L.I / epc;
    const int lanes = pass2_lanes(nq2);
    const int nc2 = nc_instance((nq2 + lanes - 1) / lanes);
    const int rows2 = slots_for(nc2) * (kWave / lanes) * (kBlock / kWave);  // per workgroup item
    const long long items2 = (long long)(p2.sa.grouped ? max_uniq : R) * ((L.H + rows2 - 1) / rows2);
    switch (L.expert_dtype) {
        case MOE_F32: err = launch_pass2<MOE_F32>(nc2, lanes, persistent_grid(items2), st, p2); break;
        case MOE_BF16: err = launch_pass2<MOE_BF16>(nc2, lanes, persistent_grid(items2), st, p2); break;
        default: err = launch_pass2<MOE_FP8_E4M3>(nc2, lanes, persistent_grid(items2), st, p2); break;
    }
    if (err != hipSuccess || (err = mark(2)) != hipSuccess) return err;
    if (mfma2) {
        MfmaArgs m2{L.w_down, L.s_down, act, y, L.H, L.I, L.top_k, kMfmaMinRoutes, 0, grouped, rt.max_count};
        if ((err = launch_mfma_pass(L, 2, T, m2, st)) != hipSuccess) return err;
    }
    if ((err = mark(3)) != hipSuccess) return err;

    hipLaunchKernelGGL(combine_kernel, dim3(T, (L.H / 4 + kBlock - 1) / kBlock), dim3(kBlock), 0, st, y, rt.w, xres,
                       out, L.top_k, L.H);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return mark(4);
}

}  // namespace moe
