// Router GEMV, RMSNorm prologue and top-k selection on the device.
//
// "MoE Performance Optimization Analysis" (markbaseengine), Option 1 and GPU
// Router Design: router scores, expert selection and the expert dispatch all
// stay on the device so no host read or wait sits between the router and the
// experts.  Selection: the k largest logits by (logit descending, expert
// index ascending); weights are a softmax over all E logits renormalised over
// the k chosen, which equals a softmax over the chosen logits alone.
#include "common.h"

namespace moe {

// ---- RMSNorm: xn[t] = x[t] / sqrt(mean(x[t]^2) + eps) (gamma = 1) ---------
__global__ __launch_bounds__(kBlock) void rmsnorm_kernel(const float *__restrict__ x, float *__restrict__ xn,
                                                         int H, float eps) {
    __shared__ float part[kBlock / kWave];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H);
    float ss = 0.f;
    for (int q = tid; q < H / 4; q += kBlock) {
        float4 v = xr[q];
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) part[tid / kWave] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    float4 *o = reinterpret_cast<float4 *>(xn + (size_t)t * H);
    for (int q = tid; q < H / 4; q += kBlock) {
        float4 v = xr[q];
        o[q] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
    }
}

hipError_t launch_rmsnorm(const float *x, float *xn, int T, int H, float eps, hipStream_t st) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(kBlock), 0, st, x, xn, H, eps);
    return hipGetLastError();
}

// ---- router GEMV --------------------------------------------------------------
// Workgroup = 16 experts x up to 8 tokens.  Each wave keeps 4 router rows in
// registers (lane l holds 16-byte chunks l, l+64, ...) and dots them with the
// token rows read through the cache; one butterfly reduction per (row, token).
constexpr int kRouterRows = 4;
constexpr int kRouterTok = 8;

template <int RDT, int NC>
__global__ __launch_bounds__(kBlock) void router_kernel(const void *__restrict__ wr, const float *__restrict__ bias,
                                                        const float *__restrict__ x, float *__restrict__ logits,
                                                        int T, int E, int H) {
    constexpr int EPC = WT<RDT>::kEpc;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int e0 = blockIdx.x * (4 * kRouterRows) + wave * kRouterRows;
    const int t0 = blockIdx.y * kRouterTok, t1 = min(T, t0 + kRouterTok);
    const int nq = H / EPC;
    const size_t row_bytes = (size_t)H * WT<RDT>::kBytes;
    u32x4 w[kRouterRows][NC];
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = lane + kWave * c;
            if (e0 + r < E && q < nq)
                w[r][c] = load_weight_chunk(
                    reinterpret_cast<const u32x4 *>(static_cast<const char *>(wr) + (size_t)(e0 + r) * row_bytes) + q);
            else
                w[r][c] = u32x4{0u, 0u, 0u, 0u};
        }
    for (int t = t0; t < t1; ++t) {
        const float *xv = x + (size_t)t * H;
        float acc[kRouterRows];
#pragma unroll
        for (int r = 0; r < kRouterRows; ++r) acc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int q = lane + kWave * c;
            if (q < nq) {
                float xs[EPC];
                const float4 *xp = reinterpret_cast<const float4 *>(xv + q * EPC);
#pragma unroll
                for (int v = 0; v < EPC / 4; ++v) {
                    float4 f = xp[v];
                    xs[4 * v] = f.x; xs[4 * v + 1] = f.y; xs[4 * v + 2] = f.z; xs[4 * v + 3] = f.w;
                }
#pragma unroll
                for (int r = 0; r < kRouterRows; ++r) acc[r] = chunk_dot<RDT>(w[r][c], xs, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < kRouterRows; ++r) {
            const float s = wave_sum(acc[r]);
            if (lane == r && e0 + r < E) logits[(size_t)t * E + e0 + r] = bias ? s + bias[e0 + r] : s;
        }
    }
}

template <int RDT>
static hipError_t router_dispatch(int nc, dim3 g, hipStream_t st, const void *wr, const float *bias,
                                  const float *x, float *logits, int T, int E, int H) {
    switch (nc) {
#define MOE_RC(N) \
    case N: hipLaunchKernelGGL((router_kernel<RDT, N>), g, dim3(kBlock), 0, st, wr, bias, x, logits, T, E, H); break;
        MOE_RC(1) MOE_RC(2) MOE_RC(3) MOE_RC(4) MOE_RC(5) MOE_RC(6) MOE_RC(7) MOE_RC(8)
#undef MOE_RC
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_router(const moe_layer_t &L, const float *x, float *logits, int T, hipStream_t st) {
    const int epc = elems_per_chunk(L.router_dtype);
    const int nc = (L.H / epc + kWave - 1) / kWave;
    dim3 g((L.E + 4 * kRouterRows - 1) / (4 * kRouterRows), (T + kRouterTok - 1) / kRouterTok);
    if (L.router_dtype == MOE_BF16)
        return router_dispatch<MOE_BF16>(nc, g, st, L.w_router, L.router_bias, x, logits, T, L.E, L.H);
    return router_dispatch<MOE_F32>(nc, g, st, L.w_router, L.router_bias, x, logits, T, L.E, L.H);
}

// ---- top-k selection: one wave per token ------------------------------------
// Lane l holds logits e = l + 64c.  Round j: each lane offers its best
// unchosen (value, index); a butterfly keeps the larger value, the lower
// index on ties, so every lane agrees on the winner.  Lane j remembers the
// winner of round j and finally writes slot j.
constexpr int kSelPerLane = kMaxE / kWave;

__global__ __launch_bounds__(kBlock) void select_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                        int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const float *l = logits + (size_t)t * E;
    float v[kSelPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int c = 0; c < kSelPerLane; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? l[e] : 0.f;
    }
    float top = 0.f, sum = 0.f, mine = 0.f;
    int mine_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < kSelPerLane; ++c) {
            const int e = lane + kWave * c;
            if (e < E && !((taken >> c) & 1u) && (bi == 0x7fffffff || v[c] > bv)) {
                bv = v[c];
                bi = e;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, kWave);
            const int oi = __shfl_xor(bi, m, kWave);
            const bool better = oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
            if (better) { bv = ov; bi = oi; }
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        if (j == 0) top = bv;
        const float p = expf(bv - top);
        sum += p;
        if (lane == j) { mine = p; mine_id = bi; }
    }
    if (lane < k) {
        ids[(size_t)t * k + lane] = mine_id;
        w[(size_t)t * k + lane] = mine / sum;
    }
}

hipError_t launch_select(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t st) {
    const int per_block = kBlock / kWave;
    hipLaunchKernelGGL(select_kernel, dim3((T + per_block - 1) / per_block), dim3(kBlock), 0, st, logits, T, E, k,
                       ids, w);
    return hipGetLastError();
}

}  // namespace moe
