// Expert passes on the matrix cores for segments with many routes.
//
// Once an expert holds n >= kMfmaMinRoutes routes, pass 1 of its segment is
// the product [n x H] . [H x 2I] and pass 2 is [n x I] . [I x H]; the GEMV
// walk would spend n fp32 FMAs per weight element, which outruns the VALU
// long before it outruns HBM, so such segments run here on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Weights are still read
// once per unique expert and token block, as in the grouped GEMV ("perf(
// cpu-moe): dedup experts across the batch in pass 1", commit message: the
// expert's routes are the inner loop over each weight row block).
//
// Work item = (segment, row block, token block of up to kMfmaTokens routes).
// A workgroup of 4 waves owns 64 gate/up row pairs (pass 1) or 128 down rows
// (pass 2); each wave holds two 16-row weight tiles:
//   pass 1: gate rows i0..i0+15 and up rows I+i0..I+i0+15, so the MFMA
//           outputs of a pair sit in the same lane and register and
//           a[r, i] = silu(g) * u is formed in registers;
//   pass 2: down rows h0..h0+31.
// K runs in stages of 128.  Each wave loads its weight tiles for stage s+1
// straight from HBM into registers in the MFMA operand layout (lane l: row
// l % 16, 16 bytes at k-group l / 16) while it computes stage s; the
// activation rows of the token block (x[t] for pass 1, a[r] for pass 2,
// fp32) are converted to bf16 into a padded LDS tile shared by the 4 waves.
// The k order inside an MFMA operand only has to agree between the two
// operands, so fp8 rows are loaded as 16 consecutive codes per lane and used
// for two k-steps.
//
// fp8 e4m3 weights (W8A16): each code is converted to fp32 by the hardware
// (OCP E4M3 on gfx950), multiplied by its 128x128 block scale and rounded to
// bf16; the MFMA then runs on bf16 exactly as for bf16 weights.
#include "experts_impl.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kTB = kMfmaTokens;                 // routes per token block
constexpr int kTT = kTB / 16;                    // 16-token MFMA tiles per block
constexpr int kKS = 128;                         // K per stage
constexpr int kRowLds = kKS * 2 + 16;            // padded bf16 activation row (bytes)
constexpr int kBufLds = kTB * kRowLds;           // one stage of activations
constexpr int kStageF4 = kTB * kKS / 4 / kBlock; // float4 loads per thread per stage
constexpr int kThrPerRow = kKS / 4;              // threads per activation row in staging

__device__ __forceinline__ f32x4_t mfma16(const u32x4 &a, const u32x4 &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(unsigned, v);
}

// 8 E4M3 codes (two words, element 0 in the low byte) times s, as 8 bf16.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(unsigned w0, unsigned w1, float s) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    return u32x4{pack_bf16(a[0] * s, a[1] * s), pack_bf16(b[0] * s, b[1] * s), pack_bf16(c[0] * s, c[1] * s),
                 pack_bf16(d[0] * s, d[1] * s)};
}

// Workgroup barrier that waits for this wave's LDS traffic only: the global
// loads of the next stage stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix over the unique segments of the items each one yields
// (segments below min_n yield none); returns the total.  pre has nu + 1
// entries.
__device__ int build_item_table(const MfmaArgs &a, int nu, int n_rb, int *pre, int *wsum) {
    const int tid = threadIdx.x;
    constexpr int kPer = (kMaxE + kBlock - 1) / kBlock;
    int c[kPer], loc = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int s = tid * kPer + q;
        int items = 0;
        if (s < nu) {
            const int e = a.sa.uniq[s];
            if (e >= 0 && e < a.sa.E) {
                const int n = a.sa.counts[e];
                if (n >= a.min_n) items = n_rb * ((n + kTB - 1) / kTB);
            }
        }
        c[q] = items;
        loc += items;
    }
    int v = loc;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if ((tid & (kWave - 1)) >= d) v += o;
    }
    if ((tid & (kWave - 1)) == kWave - 1) wsum[tid / kWave] = v;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) {
        base += w < tid / kWave ? wsum[w] : 0;
        total += wsum[w];
    }
    int ex = base + v - loc;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int s = tid * kPer + q;
        if (s < nu) pre[s] = ex;
        ex += c[q];
    }
    if (tid == 0) pre[nu] = total;
    __syncthreads();
    return total;
}

}  // namespace

template <int WDT, int PASS>
__global__ __launch_bounds__(kBlock, 2) void mfma_kernel(MfmaArgs a) {
    constexpr bool kFp8 = WDT == MOE_FP8_E4M3;
    constexpr int NWL = kFp8 ? 2 : 4;  // 16-byte weight loads per tile per stage
    __shared__ __align__(16) unsigned char xs[2 * kBufLds];
    __shared__ int pre[kMaxE + 1];
    __shared__ int wsum[kBlock / kWave];
    __shared__ int rts[kTB];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int K = PASS == 1 ? a.H : a.I;
    const int nst = K / kKS;
    const int n_rb = PASS == 1 ? a.I / 64 : a.H / 128;
    const int w_rows = PASS == 1 ? 2 * a.I : a.H;
    const size_t row_bytes = (size_t)K * WT<WDT>::kBytes;
    const int nu = min(segment_count(a.sa), a.sa.E);
    const int total = build_item_table(a, nu, n_rb, pre, wsum);

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int lo = 0, hi = nu;  // pre[lo] <= item < pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= item) lo = mid;
            else hi = mid;
        }
        const int local = item - pre[lo];
        const int e = a.sa.uniq[lo];
        const int first = a.sa.offsets[e], n = a.sa.counts[e];
        const int ntb = (n + kTB - 1) / kTB;
        const int rb = local / ntb, tb = local - rb * ntb;
        const int nv = min(kTB, n - tb * kTB);
        const int ntt = (nv + 15) >> 4;

        __syncthreads();  // the previous item is done with rts and the LDS tiles
        if (tid < kTB) rts[tid] = tid < nv ? a.sa.sorted[first + tb * kTB + tid] : 0;
        __syncthreads();

        // the wave's two weight tiles
        const int r0 = PASS == 1 ? rb * 64 + 16 * wv : rb * 128 + 32 * wv;
        const int r1 = PASS == 1 ? a.I + r0 : r0 + 16;
        const char *wbase = static_cast<const char *>(a.w) + (size_t)e * w_rows * row_bytes;
        const char *wp0 = wbase + (size_t)(r0 + (lane & 15)) * row_bytes + (lane >> 4) * 16;
        const char *wp1 = wbase + (size_t)(r1 + (lane & 15)) * row_bytes + (lane >> 4) * 16;
        const float *sp0 = nullptr, *sp1 = nullptr;
        if (kFp8) {
            const int kb = K / 128;
            sp0 = a.scales + ((size_t)e * (w_rows / 128) + r0 / 128) * kb;
            sp1 = a.scales + ((size_t)e * (w_rows / 128) + r1 / 128) * kb;
        }

        // activation rows this thread stages: token it*8 + tid/32, float4 tid%32
        float4 X[kStageF4];
        auto load_x = [&](int ks) {
#pragma unroll
            for (int it = 0; it < kStageF4; ++it) {
                const int tok = it * (kBlock / kThrPerRow) + tid / kThrPerRow;
                X[it] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (it * (kBlock / kThrPerRow) < nv && tok < nv) {
                    const int r = rts[tok];
                    const int row = PASS == 1 ? r / a.k : r;
                    X[it] = *reinterpret_cast<const float4 *>(a.src + (size_t)row * K + ks * kKS +
                                                              4 * (tid % kThrPerRow));
                }
            }
        };
        auto store_x = [&](int buf) {
            unsigned char *xb = xs + buf * kBufLds + (tid % kThrPerRow) * 8;
#pragma unroll
            for (int it = 0; it < kStageF4; ++it) {
                const int tok = it * (kBlock / kThrPerRow) + tid / kThrPerRow;
                if (it * (kBlock / kThrPerRow) < nv)
                    *reinterpret_cast<uint2 *>(xb + tok * kRowLds) =
                        make_uint2(pack_bf16(X[it].x, X[it].y), pack_bf16(X[it].z, X[it].w));
            }
        };
        auto load_w = [&](int ks, u32x4(&W)[2][NWL]) {
            const size_t off = (size_t)ks * kKS * WT<WDT>::kBytes;
#pragma unroll
            for (int c = 0; c < NWL; ++c) {
                W[0][c] = load_weight_chunk(reinterpret_cast<const u32x4 *>(wp0 + off + c * 64));
                W[1][c] = load_weight_chunk(reinterpret_cast<const u32x4 *>(wp1 + off + c * 64));
            }
        };

        f32x4_t acc0[kTT], acc1[kTT];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) acc0[tt] = acc1[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](int buf, u32x4(&W)[2][NWL], float s0, float s1) {
            const unsigned char *xb = xs + buf * kBufLds + (lane & 15) * kRowLds;
            const int g = lane >> 4;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4 a0, a1;
                int koff;
                if (kFp8) {
                    const u32x4 &c0 = W[0][s >> 1], &c1 = W[1][s >> 1];
                    a0 = (s & 1) ? e4m3x8_to_bf16(c0.z, c0.w, s0) : e4m3x8_to_bf16(c0.x, c0.y, s0);
                    a1 = (s & 1) ? e4m3x8_to_bf16(c1.z, c1.w, s1) : e4m3x8_to_bf16(c1.x, c1.y, s1);
                    koff = 64 * (s >> 1) + 16 * g + 8 * (s & 1);
                } else {
                    a0 = W[0][s];
                    a1 = W[1][s];
                    koff = 32 * s + 8 * g;
                }
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt) {
                    if (tt < ntt) {
                        const u32x4 b = *reinterpret_cast<const u32x4 *>(xb + tt * 16 * kRowLds + koff * 2);
                        acc0[tt] = mfma16(a0, b, acc0[tt]);
                        acc1[tt] = mfma16(a1, b, acc1[tt]);
                    }
                }
            }
        };

        u32x4 Wa[2][NWL], Wb[2][NWL];
        float sa0 = 1.f, sa1 = 1.f, sb0 = 1.f, sb1 = 1.f;
        load_w(0, Wa);
        if (kFp8) { sa0 = sp0[0]; sa1 = sp1[0]; }
        load_x(0);
        store_x(0);
        auto stage = [&](int ks, u32x4(&Wc)[2][NWL], float sc0, float sc1, u32x4(&Wn)[2][NWL], float &sn0,
                         float &sn1) {
            if (ks + 1 < nst) {
                load_w(ks + 1, Wn);
                if (kFp8) { sn0 = sp0[ks + 1]; sn1 = sp1[ks + 1]; }
                load_x(ks + 1);
            }
            lds_barrier();
            compute(ks & 1, Wc, sc0, sc1);
            if (ks + 1 < nst) store_x((ks + 1) & 1);
        };
        for (int ks = 0; ks < nst; ks += 2) {
            stage(ks, Wa, sa0, sa1, Wb, sb0, sb1);
            if (ks + 1 < nst) stage(ks + 1, Wb, sb0, sb1, Wa, sa0, sa1);
        }

        // epilogue: lane holds rows 4*(lane/16)+v of both tiles for token lane%16
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) {
            const int tok = tt * 16 + (lane & 15);
            if (tt < ntt && tok < nv) {
                const int r = rts[tok];
                const int row = r0 + 4 * (lane >> 4);
                if (PASS == 1) {
                    float4 o;
                    o.x = silu(acc0[tt][0]) * acc1[tt][0];
                    o.y = silu(acc0[tt][1]) * acc1[tt][1];
                    o.z = silu(acc0[tt][2]) * acc1[tt][2];
                    o.w = silu(acc0[tt][3]) * acc1[tt][3];
                    *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.I + row) = o;
                } else {
                    *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row) =
                        make_float4(acc0[tt][0], acc0[tt][1], acc0[tt][2], acc0[tt][3]);
                    *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row + 16) =
                        make_float4(acc1[tt][0], acc1[tt][1], acc1[tt][2], acc1[tt][3]);
                }
            }
        }
    }
}

template <int WDT>
hipError_t launch_mfma(int pass, int grid, hipStream_t st, const MfmaArgs &a) {
    if (pass == 1) hipLaunchKernelGGL((mfma_kernel<WDT, 1>), dim3(grid), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((mfma_kernel<WDT, 2>), dim3(grid), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template hipError_t launch_mfma<MOE_BF16>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma<MOE_FP8_E4M3>(int, int, hipStream_t, const MfmaArgs &);

}  // namespace moe
