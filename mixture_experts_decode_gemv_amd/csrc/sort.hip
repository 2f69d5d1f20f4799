// Stable counting sort of the (token, route) pairs by expert id.
//
// "perf(cpu-moe): dedup experts across the batch in pass 1" (FreeToken PR
// #46), commit message: the routes are grouped by expert with a counting sort
// over their ids, built once per layer per step, and the grouped list drives
// the pass-1 walk.  Here the sort is one workgroup working in LDS:
//   1. histogram of the ids (integer LDS atomics, order-free),
//   2. exclusive scans: offsets over the counts, uniq slots over count > 0,
//   3. stable scatter in windows of 256 routes: a route's slot is its
//      expert's offset + routes of that expert in earlier windows + in
//      earlier waves of this window + earlier lanes of its own wave.
#include "common.h"

namespace moe {

// Exclusive scan of one int per thread over the workgroup; returns the
// prefix and writes the total to *total (all threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_tmp, int *total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) {
        if (w < wave) before += s_tmp[w];
        all += s_tmp[w];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kBlock) void sort_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ sorted, int32_t *__restrict__ uniq,
                                                      int32_t *__restrict__ n_uniq, int32_t *__restrict__ stats) {
    __shared__ int s_cnt[kMaxE];
    __shared__ int s_off[kMaxE];
    __shared__ int s_run[kMaxE];
    __shared__ int s_wc[kBlock / kWave][kMaxE];
    __shared__ int s_tmp[kBlock / kWave];
    __shared__ int s_bad, s_max;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    for (int e = tid; e < E; e += kBlock) {
        s_cnt[e] = 0;
        s_run[e] = 0;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) s_wc[w][e] = 0;
    }
    if (tid == 0) { s_bad = 0; s_max = 0; }
    __syncthreads();
    for (int r = tid; r < R; r += kBlock) {
        const int v = ids[r];
        if (v < 0 || v >= E) s_bad = 1;
        else atomicAdd(&s_cnt[v], 1);
    }
    __syncthreads();
    if (s_bad) {
        if (tid == 0) {
            *n_uniq = -1;
            if (stats) { stats[0] = -1; stats[1] = R; stats[2] = 0; stats[3] = 0; }
        }
        return;
    }

    // Scans: thread tid owns experts [lo, hi).
    const int per = (E + kBlock - 1) / kBlock;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int csum = 0, usum = 0, cmax = 0;
    for (int e = lo; e < hi; ++e) {
        csum += s_cnt[e];
        usum += s_cnt[e] > 0;
        cmax = max(cmax, s_cnt[e]);
    }
    int ctot, utot;
    int cpre = block_exclusive_scan(csum, s_tmp, &ctot);
    int upre = block_exclusive_scan(usum, s_tmp, &utot);
    atomicMax(&s_max, cmax);
    for (int e = lo; e < hi; ++e) {
        const int c = s_cnt[e];
        s_off[e] = cpre;
        offsets[e] = cpre;
        counts[e] = c;
        if (c > 0) uniq[upre++] = e;
        cpre += c;
    }
    __syncthreads();
    if (tid == 0) {
        offsets[E] = R;
        *n_uniq = utot;
        if (stats) { stats[0] = utot; stats[1] = R; stats[2] = s_max; stats[3] = 0; }
    }

    // Stable scatter, 256 routes per window.
    for (int base = 0; base < R; base += kBlock) {
        const int r = base + tid;
        const int v = r < R ? ids[r] : -1;
        int rank = 0, later = 0;
        for (int l = 0; l < kWave; ++l) {
            const int o = __shfl(v, l, kWave);
            if (o == v) {
                rank += l < lane;
                later += l > lane;
            }
        }
        if (v >= 0 && later == 0) s_wc[wave][v] = rank + 1;
        __syncthreads();
        if (v >= 0) {
            int pre = s_run[v];
            for (int w = 0; w < wave; ++w) pre += s_wc[w][v];
            sorted[s_off[v] + pre + rank] = r;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kBlock) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kBlock / kWave; ++w) {
                add += s_wc[w][e];
                s_wc[w][e] = 0;
            }
            s_run[e] += add;
        }
        __syncthreads();
    }
}

hipError_t launch_sort(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                       int32_t *uniq, int32_t *n_uniq, int32_t *stats, hipStream_t st) {
    hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kBlock), 0, st, ids, R, E, counts, offsets, sorted, uniq, n_uniq,
                       stats);
    return hipGetLastError();
}

}  // namespace moe
