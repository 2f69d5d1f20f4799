// Stable counting sort of the (token, route) pairs by expert id, as its own
// launch (the moe_sort entry point); the layer path sorts inside the routing
// kernel.  See route_impl.h for the method.
#include "route_impl.h"

namespace moe {

__global__ __launch_bounds__(kBlock) void sort_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ sorted, int32_t *__restrict__ uniq,
                                                      int32_t *__restrict__ n_uniq) {
    extern __shared__ float4 dyn_lds[];
    sort_routes<false>(ids, R, E, counts, offsets, sorted, uniq, n_uniq, nullptr, reinterpret_cast<int *>(dyn_lds),
                       nullptr, 0);
}

hipError_t launch_sort(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                       int32_t *uniq, int32_t *n_uniq, hipStream_t st) {
    hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kBlock), (size_t)sort_lds_ints(E) * 4, st, ids, R, E, counts,
                       offsets, sorted, uniq, n_uniq);
    return hipGetLastError();
}

// ---- expert-usage telemetry ---------------------------------------------------
// hist[e] += counts[e] for the E experts of one routing ("MoE Performance
// Optimization Analysis", Option 3 and Phase 3: track how often each expert
// is used, per layer).  Skipped when the sort rejected the routing
// (*n_uniq < 0).  One thread per expert: every word has one writer.
__global__ __launch_bounds__(kBlock) void usage_kernel(const int32_t *__restrict__ counts,
                                                       const int32_t *__restrict__ n_uniq, int E,
                                                       unsigned long long *__restrict__ hist) {
    const int e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= E || *n_uniq < 0) return;
    hist[e] += (unsigned long long)counts[e];
}

hipError_t launch_usage(const int32_t *counts, const int32_t *n_uniq, int E, unsigned long long *hist,
                        hipStream_t st) {
    hipLaunchKernelGGL(usage_kernel, dim3((E + kBlock - 1) / kBlock), dim3(kBlock), 0, st, counts, n_uniq, E, hist);
    return hipGetLastError();
}

}  // namespace moe
