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
#include <mutex>

#include "experts_impl.h"

namespace moe {

// ---- bf16 copy of the activations (MFMA pass 1 operand) ----------------------
// Stored as float-typed words: no store of this kernel may alias the int32
// routing arrays.
__global__ __launch_bounds__(kBlock) void to_bf16_kernel(const float2 *__restrict__ x, float *__restrict__ xb,
                                                         int npairs) {
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < npairs; i += gridDim.x * kBlock) {
        const float2 v = x[i];
        xb[i] = __uint_as_float(bf16_pair_rne(v.x, v.y));
    }
}

// ---- second stream for the MFMA segments -------------------------------------
// The GEMV segments and the MFMA segments of a pass read disjoint experts and
// write disjoint routes, so for large batches the MFMA kernels run on a
// second stream, forked from the caller's stream after routing and joined
// before the combine; both halves then share the HBM bandwidth instead of
// taking turns (2-4 % per step at 128-512 tokens).  Each (device, caller
// stream) pair gets its own side stream and fork/join events, created on the
// first such call made outside a graph capture and kept until the process
// ends (at most kMaxSides pairs; further pairs, and a first call made under
// capture, run the passes in order on the caller's stream).  The table
// mutex is held from the lookup through the join, so the whole fork ->
// record -> wait -> launches -> join sequence of one call is enqueued
// without interleaving with another thread's; and since a side stream
// serves a single caller stream, a caller stream under capture takes only
// its own side stream into that capture.
struct SideStream {
    int dev = -1;
    hipStream_t caller = nullptr;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

constexpr int kMaxSides = 64;
static std::mutex g_side_mu;
static SideStream g_sides[kMaxSides];
static int g_nsides = 0;

// The side stream of (current device, caller stream st), created if needed;
// null when none can be used.  The caller holds g_side_mu.
static SideStream *side_stream_locked(hipStream_t st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    for (int i = 0; i < g_nsides; ++i)
        if (g_sides[i].dev == dev && g_sides[i].caller == st) return &g_sides[i];
    if (g_nsides == kMaxSides) return nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    SideStream sd;
    sd.dev = dev;
    sd.caller = st;
    if (hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) != hipSuccess) {
        if (sd.fork) (void)hipEventDestroy(sd.fork);
        (void)hipStreamDestroy(sd.s);
        return nullptr;
    }
    g_sides[g_nsides] = sd;
    return &g_sides[g_nsides++];
}

// ---- combine ------------------------------------------------------------------
// out may alias xres: each thread reads its residual before storing there.
// reject (a caller-supplied routing's n_uniq, or null): when it is negative
// the sort rejected the routing, no expert pass ran, and out is left as it
// was.  It is read alongside the y rows and tested only before the store, so
// it adds no round trip.
__global__ __launch_bounds__(kBlock) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                         const float *xres, float *out, int k, int H,
                                                         const int32_t *reject) {
    const int t = blockIdx.x;
    const int h = (blockIdx.y * kBlock + threadIdx.x) * 4;
    if (h >= H) return;
    const int nu = reject ? __builtin_nontemporal_load(reject) : 0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // routes in groups of 8 with every load of a group issued before its
    // FMAs (j ascending): one memory round trip per group, not per route
    constexpr int kG = 8;
    for (int j0 = 0; j0 < k; j0 += kG) {
        float wj[kG];
        float4 v[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int j = min(j0 + u, k - 1);
            wj[u] = w[(size_t)t * k + j];
            v[u] = *reinterpret_cast<const float4 *>(y + ((size_t)t * k + j) * H + h);
        }
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            if (j0 + u < k) {
                acc.x = fmaf(wj[u], v[u].x, acc.x);
                acc.y = fmaf(wj[u], v[u].y, acc.y);
                acc.z = fmaf(wj[u], v[u].z, acc.z);
                acc.w = fmaf(wj[u], v[u].w, acc.w);
            }
        }
    }
    if (xres) {
        const float4 r = *reinterpret_cast<const float4 *>(xres + (size_t)t * H + h);
        acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
    }
    if (nu < 0) return;
    *reinterpret_cast<float4 *>(out + (size_t)t * H + h) = acc;
}

// ---- launchers -------------------------------------------------------------------
// GEMV grids: up to 32 workgroups of 256 threads per CU (8192 threads), of
// which an eighth are resident at a time; the later ones start as the first
// finish, which evens out the tail (16 per CU: 1 % slower at bs = 64 in bf16,
// MXFP4 and q4_0; 8 per CU slower again, 48 per CU slower on skewed routing).
static int persistent_grid(long long max_items) {
    const long long cap = (long long)num_cus() * (32 * 256 / kGemvBlock);
    long long g = max_items < cap ? max_items : cap;
    return (int)(g < 1 ? 1 : g);
}

// Segments with at least mfma_min_routes routes go to the MFMA kernels when
// the weights are bf16, fp8, MXFP4 or q4_0 with H and I multiples of 128, unless the
// caller asked for the GEMV path only, and from kMfmaMinTokens tokens on
// (below that the MFMA launches would mostly be idle, and batches up to
// kPass2cMaxT tokens run pass 2 with the combine, on GEMV segments only).
static bool mfma_eligible(const moe_layer_t &L, int T, uint32_t flags) {
    // the MFMA kernels address activation rows with 32-bit byte offsets, and
    // the wide ones mark unused rows with offsets from 2 GiB up
    const bool offsets32 = (unsigned long long)T * L.H * 2 < (1ull << 31) &&
                           (unsigned long long)T * L.top_k * L.I * 4 < (1ull << 31);
    // MXFP4 and q4_0 scale words are copied 4 bytes at a time
    const bool s4 = (reinterpret_cast<uintptr_t>(L.s_gate_up) & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(L.s_down) & 3) == 0;
    const bool fp4_ok = L.expert_dtype == MOE_MXFP4 && s4;
    const bool q4_ok = L.expert_dtype == MOE_Q4_0 && s4;
    return (L.expert_dtype == MOE_BF16 || L.expert_dtype == MOE_FP8_E4M3 || fp4_ok || q4_ok) && L.H % 128 == 0 &&
           L.I % 128 == 0 &&
           !(flags & MOE_NO_MFMA) && T >= kMfmaMinTokens && (int)(flags & MOE_WALK_MASK) != MOE_WALK_PER_ROUTE &&
           offsets32;
}

int mfma_min_routes(const moe_layer_t &L, int T, uint32_t flags) {
    if (!mfma_eligible(L, T, flags)) return 0;
    return T >= kMfmaWideTokens ? kMfmaMinRoutesWide : kMfmaMinRoutes;
}

int mfma_hot_routes(const moe_layer_t &L, int T, uint32_t flags) {
    if (!mfma_eligible(L, T, flags)) return 0;
    return T >= kMfmaWideTokens ? kMfmaMinRoutesWide : kMfmaHotRoutes;
}

// Pass 2 and the combine in one launch (pass2c_kernel) for small batches with
// an output to write: the y block of a workgroup ([R][rows] floats) must fit
// in 64 KiB of LDS, and down rows must take 32 or 64 lanes.  Short rows (16
// or 8 lanes, 4-bit formats) give a workgroup 4-8x more rows, so the launch
// would cover a quarter of the CUs or less (H = 2048: 64 workgroups of 8
// waves); they take pass2_kernel and the combine launch.  The same predicate
// tells a layer stack whether each layer writes its output rows itself.
bool fused_combine(const moe_layer_t &L, int T) {
    if (T > kPass2cMaxT) return false;
    const int nq2 = L.I / elems_per_chunk(L.expert_dtype);
    const int lanes = pass2_lanes(nq2, L.expert_dtype);
    if (lanes < 32) return false;
    const int nr = pass2c_rows(nc_instance((nq2 + lanes - 1) / lanes), lanes);
    return (size_t)T * L.top_k * (nr * 4 + 1) <= 64 * 1024;
}

// Small batches have few hot experts: narrow items (32 weight rows) spread
// them over the chip.  Large batches have many items anyway, and wide items
// (128 weight rows) read each staged activation row for 4x more weights.
static hipError_t launch_mfma_pass(const moe_layer_t &L, int pass, int T, const MfmaArgs &a, hipStream_t st) {
    const bool wide = T >= kMfmaWideTokens;
    // items <= row blocks x (segments that can reach the threshold + extra token blocks)
    const long long R = (long long)T * L.top_k;
    const long long segs = std::min<long long>(L.E, R / a.min_n);
    const long long n_rb = pass == 1 ? L.I / (wide ? 64 : 16) : L.H / (wide ? 128 : 32);
    const long long items = n_rb * (segs + R / (wide ? kMfmaTokens : kMfmaNarrowTokens));
    const long long cap = (long long)num_cus() * 2;
    const int grid = (int)std::max<long long>(1, std::min(items, cap));
    if (wide) switch (L.expert_dtype) {
            case MOE_BF16: return launch_mfma_wide<MOE_BF16>(pass, grid, st, a);
            case MOE_FP8_E4M3: return launch_mfma_wide<MOE_FP8_E4M3>(pass, grid, st, a);
            case MOE_Q4_0: return launch_mfma_wide<MOE_Q4_0>(pass, grid, st, a);
            default: return launch_mfma_wide<MOE_MXFP4>(pass, grid, st, a);
        }
    switch (L.expert_dtype) {
        case MOE_BF16: return launch_mfma<MOE_BF16>(pass, grid, st, a);
        case MOE_FP8_E4M3: return launch_mfma<MOE_FP8_E4M3>(pass, grid, st, a);
        case MOE_Q4_0: return launch_mfma<MOE_Q4_0>(pass, grid, st, a);
        default: return launch_mfma<MOE_MXFP4>(pass, grid, st, a);
    }
}

hipError_t launch_experts(const moe_layer_t &L, const float *x, const float *xres, int T, const Routing &rt,
                          void *xb, float *act, float *y, float *out, uint32_t flags, hipStream_t st,
                          const hipEvent_t *ev, bool may_fork) {
    const int R = T * L.top_k;
    const int walk = (int)(flags & MOE_WALK_MASK);
    const int epc = elems_per_chunk(L.expert_dtype);
    const int max_uniq = R < L.E ? R : L.E;
    const int min_n = mfma_min_routes(L, T, flags);  // 0: no MFMA segments
    const bool mfma = min_n > 0;
    const bool mfma2 = mfma && walk == MOE_WALK_DEDUP;
    // without the sort's statistics (a caller-supplied routing) every segment
    // of min_n routes or more takes the MFMA path
    const int hot = rt.max_count ? mfma_hot_routes(L, T, flags) : min_n;
    SegArgs grouped{rt.ids, rt.counts, rt.offsets, rt.sorted, rt.uniq, rt.n_uniq, 1, R, L.E, INT_MAX, nullptr, 0};
    SegArgs per_route = grouped;
    per_route.grouped = 0;
    SegArgs split = grouped;  // the GEMV share of a pass that also has MFMA segments
    if (mfma) {
        split.gemv_below = min_n;
        split.max_count = rt.max_count;
        split.hot = hot;
    }

    // pass 1 on the GEMV kernel: one wave item = P gate/up pairs of one segment
    // xb_first: the GEMV kernel writes the bf16 copy of x in its prologue
    // (in-order path); otherwise mfma_1 converts it on its own stream
    auto gemv1 = [&](hipStream_t s, bool xb_first) {
        Pass1Args p1{L.w_gate_up, L.s_gate_up, x, act, L.H, L.I, L.top_k,
                     walk == MOE_WALK_PER_ROUTE ? per_route : split,
                     xb_first ? static_cast<uint32_t *>(xb) : nullptr, lds_batch_rows(L.H)};
        const int nq1 = L.H / epc;
        const int nc1 = nc_instance((nq1 + kWave - 1) / kWave);
        const int pairs = slots_for(nc1) / 2 * (kGemvBlock / kWave);  // per workgroup item
        const long long items1 = (long long)(p1.sa.grouped ? max_uniq : R) * ((L.I + pairs - 1) / pairs);
        switch (L.expert_dtype) {
            case MOE_F32: return launch_pass1<MOE_F32>(nc1, persistent_grid(items1), s, p1);
            case MOE_BF16: return launch_pass1<MOE_BF16>(nc1, persistent_grid(items1), s, p1);
            case MOE_FP8_E4M3: return launch_pass1<MOE_FP8_E4M3>(nc1, persistent_grid(items1), s, p1);
            case MOE_MXFP4: return launch_pass1<MOE_MXFP4>(nc1, persistent_grid(items1), s, p1);
            default: return launch_pass1<MOE_Q4_0>(nc1, persistent_grid(items1), s, p1);
        }
    };
    // pass 1 of the MFMA segments, on a bf16 copy of x (converted here unless
    // the GEMV pass 1 did it)
    auto mfma_1 = [&](hipStream_t s, bool convert) {
        if (convert) {
            const int npairs = T * L.H / 2;
            const int g = std::max(1, std::min((npairs + kBlock - 1) / kBlock, num_cus() * 4));
            hipLaunchKernelGGL(to_bf16_kernel, dim3(g), dim3(kBlock), 0, s, reinterpret_cast<const float2 *>(x),
                               static_cast<float *>(xb), npairs);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        MfmaArgs m1{L.w_gate_up, L.s_gate_up, xb, act, L.H, L.I, L.top_k, min_n, hot, mfma2 ? 1 : 0, grouped,
                    rt.max_count};
        return launch_mfma_pass(L, 1, T, m1, s);
    };
    // pass 2 on the GEMV kernel: one wave item = slots x (64 / lanes) down rows of one segment
    auto gemv2 = [&](hipStream_t s) {
        Pass2Args p2{L.w_down, L.s_down, act, y, L.H, L.I,
                     walk == MOE_WALK_DEDUP ? (mfma2 ? split : grouped) : per_route, lds_batch_rows(L.I)};
        const int nq2 = L.I / epc;
        const int lanes = pass2_lanes(nq2, L.expert_dtype);
        const int nc2 = nc_instance((nq2 + lanes - 1) / lanes);
        const int rows2 = slots_for(nc2) * (kWave / lanes) * (kGemvBlock / kWave);  // per workgroup item
        const long long items2 = (long long)(p2.sa.grouped ? max_uniq : R) * ((L.H + rows2 - 1) / rows2);
        switch (L.expert_dtype) {
            case MOE_F32: return launch_pass2<MOE_F32>(nc2, lanes, persistent_grid(items2), s, p2);
            case MOE_BF16: return launch_pass2<MOE_BF16>(nc2, lanes, persistent_grid(items2), s, p2);
            case MOE_FP8_E4M3: return launch_pass2<MOE_FP8_E4M3>(nc2, lanes, persistent_grid(items2), s, p2);
            case MOE_MXFP4: return launch_pass2<MOE_MXFP4>(nc2, lanes, persistent_grid(items2), s, p2);
            default: return launch_pass2<MOE_Q4_0>(nc2, lanes, persistent_grid(items2), s, p2);
        }
    };
    // pass 2 with the combine (small batches): writes out directly; the
    // routes on the matrix cores come from y, written by mfma_2 before it
    const bool p2c = out && fused_combine(L, T);
    auto gemv2c = [&](hipStream_t s) {
        Pass2cArgs p{L.w_down, L.s_down, act, rt.w, xres, out, rt.reject, mfma2 ? y : nullptr, L.H, L.I, L.top_k, T,
                     walk == MOE_WALK_DEDUP ? (mfma2 ? split : grouped) : per_route};
        const int nq2 = L.I / epc;
        const int lanes = pass2_lanes(nq2, L.expert_dtype);
        const int nc2 = (nq2 + lanes - 1) / lanes;
        switch (L.expert_dtype) {
            case MOE_F32: return launch_pass2c<MOE_F32>(nc2, lanes, s, p);
            case MOE_BF16: return launch_pass2c<MOE_BF16>(nc2, lanes, s, p);
            case MOE_FP8_E4M3: return launch_pass2c<MOE_FP8_E4M3>(nc2, lanes, s, p);
            case MOE_MXFP4: return launch_pass2c<MOE_MXFP4>(nc2, lanes, s, p);
            default: return launch_pass2c<MOE_Q4_0>(nc2, lanes, s, p);
        }
    };
    auto mfma_2 = [&](hipStream_t s) {
        MfmaArgs m2{L.w_down, L.s_down, act, y, L.H, L.I, L.top_k, min_n, hot, 0, grouped, rt.max_count};
        return launch_mfma_pass(L, 2, T, m2, s);
    };
    auto combine = [&]() {
        if (!out || p2c) return hipSuccess;  // a stack: the next layer's routing launch combines
        hipLaunchKernelGGL(combine_kernel, dim3(T, (L.H / 4 + kBlock - 1) / kBlock), dim3(kBlock), 0, st, y, rt.w,
                           xres, out, L.top_k, L.H, rt.reject);
        return hipGetLastError();
    };
    hipError_t err;
#define MOE_TRY(expr) \
    if ((err = (expr)) != hipSuccess) return err

    // GEMV and MFMA segments side by side for large batches, which always
    // have hot experts.  Below that the MFMA launches are often idle (they
    // exit on the sort's maximum count), and an idle launch running beside
    // the GEMV pass costs it more than it costs in order.  Not when the
    // caller times the stages: then everything runs in order on its stream.
    std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
    SideStream *sd = nullptr;
    if (mfma && !ev && may_fork && T >= kMfmaWideTokens) {
        side_lock.lock();  // held until this call's join is enqueued
        sd = side_stream_locked(st);
        if (!sd) side_lock.unlock();
    }
    if (sd) {
        MOE_TRY(hipEventRecord(sd->fork, st));
        MOE_TRY(hipStreamWaitEvent(sd->s, sd->fork, 0));
        MOE_TRY(mfma_1(sd->s, !rt.xb_ready));
        if (mfma2) MOE_TRY(mfma_2(sd->s));
        MOE_TRY(gemv1(st, false));
        // pass 2 of the DEDUP_PASS1 walk reads every segment's pass-1 rows
        if (!mfma2) {
            MOE_TRY(hipEventRecord(sd->join, sd->s));
            MOE_TRY(hipStreamWaitEvent(st, sd->join, 0));
        }
        MOE_TRY(gemv2(st));
        if (mfma2) {
            MOE_TRY(hipEventRecord(sd->join, sd->s));
            MOE_TRY(hipStreamWaitEvent(st, sd->join, 0));
        }
        return combine();
    }
    // In order: pass 2 on the matrix cores before pass 2 on the GEMV kernels
    // (they write disjoint routes; pass 2 with the combine reads the MFMA
    // routes' y rows).
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
    MOE_TRY(gemv1(st, mfma && !rt.xb_ready));
    MOE_TRY(mark(0));
    if (mfma) MOE_TRY(mfma_1(st, false));
    MOE_TRY(mark(1));
    if (mfma2) MOE_TRY(mfma_2(st));
    MOE_TRY(mark(2));
    MOE_TRY(p2c ? gemv2c(st) : gemv2(st));
    MOE_TRY(mark(3));
    MOE_TRY(combine());
    return mark(4);
#undef MOE_TRY
}

}  // namespace moe
