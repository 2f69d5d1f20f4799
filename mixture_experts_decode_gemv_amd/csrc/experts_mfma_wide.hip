// Expert passes on the matrix cores, wide tiles: the variant for large
// batches, where the hot experts carry many token blocks and there are
// plenty of work items to fill the chip.
//
// Same products as the narrow variant (experts_mfma.hip: [n x H] . [H x 2I]
// and [n x I] . [I x H] on v_mfma_f32_16x16x32_bf16 for segments with
// n >= kMfmaMinRoutes, weights read once per unique expert and token block,
// as in "perf(cpu-moe): dedup experts across the batch in pass 1", commit
// message), with a 4x larger weight tile per work item, so that each staged
// activation row serves 4x more weight rows:
//
// Work item = (segment, row block, token block of up to kMfmaTokens routes).
// A workgroup of 4 waves owns 64 gate/up row pairs (pass 1) or 128 down rows
// (pass 2); each wave holds two 16-row weight tiles over the whole K:
//   pass 1: gate rows i0..i0+15 and up rows I+i0..I+i0+15, so the MFMA
//           outputs of a pair sit in the same lane and register and
//           a[r, i] = silu(g) * u is formed in registers;
//   pass 2: down rows h0..h0+31.
// K runs in stages of 128.  The weights of a stage are loaded from HBM into
// registers with each load instruction covering whole 256-byte (bf16) or
// 128-byte (fp8) row segments of 4 or 8 rows: loads that give each lane 16
// bytes of a different row, as the MFMA operand layout (lane l: row l % 16)
// would, reach only about half the HBM bandwidth on gfx950.  The loads run
// through a ring of three stages held in registers (stage s+2 is issued while
// stage s is computed); each stage is written to a wave-private LDS tile and
// read back in the operand layout.  The activation rows of the token block
// are bf16 in memory; each stage of them is loaded two stages ahead into
// registers and written into a padded LDS tile shared by the 4 waves.  The k
// order inside an MFMA operand only has to agree between the two operands,
// so fp8 rows are loaded as 16 consecutive codes per lane and used for two
// k-steps.  A (row, route) result is one accumulator over K in order, so it
// does not depend on the segment's size or the route's place in it.
//
// Items are numbered (segment, row block, token block) with the token block
// fastest and dealt out in contiguous ranges per XCD (workgroup b runs on
// XCD b % 8), so the token blocks of one row block, which read the same
// weights, run at the same time behind the same L2.
//
// fp8 e4m3 weights (W8A16): the codes are converted to bf16 by the hardware
// (OCP E4M3 on gfx950), which is exact, and the MFMAs of a stage (128 along
// K, one block of the 128x128 block scales) add into sums of their own that
// are multiplied by the tile's block scale and added to the accumulator at
// the stage's end.
//
// MXFP4 weights (W4A16; OCP Microscaling Formats v1.0: E2M1 codes, an E8M0
// scale per 32 along K): a stage of a row is 64 bytes of codes, so one load
// covers a whole 16-row tile (4 lanes per row), and each lane also loads its
// row's 4 scale bytes of the stage (one aligned word: a row's scale array
// is K/32 bytes and K is a multiple of 128).  MFMA k-step s of the stage is
// scale block 4 ks + s; the hardware converts the codes to bf16 with that
// scale applied (a power of two), which is exact.
#include <type_traits>

#include "experts_impl.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kTB = kMfmaTokens;                     // routes per token block
constexpr int kTT = kTB / 16;                        // 16-token MFMA tiles per block
constexpr int kKS = 128;                             // K per stage
constexpr int kRowLds = kKS * 2 + 16;                // padded bf16 activation row (bytes)
constexpr int kBufLds = kTB * kRowLds;               // one stage of activations
constexpr int kChunksPerRow = kKS * 2 / 16;           // 16-byte chunks of a staged row (16)
constexpr int kRowsPerPass = kBlock / kChunksPerRow;  // rows staged per pass of the workgroup (16)
constexpr int kXChunks = kTB / kRowsPerPass;          // rows (one chunk each) per thread per stage
constexpr int kXcds = 8;
// Buffer descriptor word 3 for raw 32-bit loads on gfx9 (CDNA), and a byte
// offset beyond every activation buffer here (< 2 GiB, with room for K)
constexpr int kBufferFlags = 0x00020000;
constexpr unsigned kOutside = 0x80000000u;
// wave-private weight tile of one stage: 32 rows (two 16-row MFMA tiles)
constexpr int kWRow = kKS * 2 + 16;  // bf16 row segment + pad (bytes); fp8 uses kKS + 16
constexpr int kWTile = 32 * kWRow;

__device__ __forceinline__ f32x4_t mfma16(const u32x4 &a, const u32x4 &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// 8 E2M1 codes (one word, element 0 in the low nibble) times the E8M0 scale
// s (a power of two, or NaN for the code 0xFF), as 8 bf16: the hardware
// conversion applies the scale's exponent, which is exact.
__device__ __forceinline__ u32x4 e2m1x8_to_bf16(unsigned w, float s) {
    return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
}

// 8 E4M3 codes (two words, element 0 in the low byte) as 8 bf16, exactly:
// every E4M3 value is a bf16 value (the conversion's scale is 1).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(unsigned w0, unsigned w1) {
    return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
}

// Workgroup barrier that waits for this wave's LDS traffic only: the global
// loads of later stages stay in flight across it.
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
__global__ __launch_bounds__(kBlock, 2) void mfma_wide_kernel(MfmaArgs a) {
    constexpr bool kFp8 = WDT == MOE_FP8_E4M3, kFp4 = WDT == MOE_MXFP4, kQ4 = WDT == MOE_Q4_0;
    constexpr int NWL = kFp4 || kQ4 ? 1 : kFp8 ? 2 : 4;  // 16-byte weight loads per tile per stage
    // stages in the register ring (kD - 1 in flight); deeper rings for the
    // narrower fp8 and MXFP4 stages measured slower (4 and 5 stages)
    constexpr int kD = 3;
    constexpr int kStageB = kFp4 || kQ4 ? kKS / 2 : kKS * WT<WDT>::kBytes;  // bytes of a row per stage
    // per tile and stage: fp8 its block scale; MXFP4 the lane's row's 4 scale bytes
    // q4_0: the lane's row's 4 binary16 scales of the stage
    using ScaleT = std::conditional_t<kFp4, unsigned, std::conditional_t<kQ4, uint2, float>>;
    __shared__ __align__(16) unsigned char xs[2 * kBufLds];
    __shared__ __align__(16) unsigned char wls[kBlock / kWave][kWTile];
    __shared__ int pre[kMaxE + 1];
    __shared__ int wsum[kBlock / kWave];
    __shared__ int rts[kTB];

    // no expert reaches the threshold (known from the sort's statistics):
    // nothing to do, without building the item table
    if (a.max_count && load_uniform(a.max_count) < a.hot) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int K = PASS == 1 ? a.H : a.I;
    const int nst = K / kKS;
    const int n_rb = PASS == 1 ? a.I / 64 : a.H / 128;
    const int w_rows = PASS == 1 ? 2 * a.I : a.H;
    const size_t row_bytes = kFp4 || kQ4 ? (size_t)K / 2 : (size_t)K * WT<WDT>::kBytes;  // 4-bit: 2 codes a byte
    // bf16 activation rows: pass 1 reads xb [T, H]; pass 2 reads a[r] from the
    // first half of the fp32 activation row r (4I bytes apart)
    const size_t src_stride = PASS == 1 ? (size_t)a.H * 2 : (size_t)a.I * 4;
    // the activation rows as a buffer: pass 1 x [T, H] bf16, pass 2 R rows
    // of 4I bytes (offsets from kOutside on read as zeros)
    const unsigned src_bytes = PASS == 1 ? (unsigned)(a.sa.R / a.k) * a.H * 2 : (unsigned)a.sa.R * a.I * 4;
    const auto xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.src), 0, (int)src_bytes, kBufferFlags);
    const int nu = min(segment_count(a.sa), a.sa.E);
    const int total = build_item_table(a, nu, n_rb, pre, wsum);
    // contiguous item ranges per XCD (the grid is a multiple of kXcds)
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int slots = per_xcd * kXcds;

    for (int it = blockIdx.x; it < slots; it += gridDim.x) {
        const int item = (it % kXcds) * per_xcd + it / kXcds;
        if (item >= total) continue;  // uniform over the workgroup
        int lo = 0, hi = nu;          // pre[lo] <= item < pre[hi]
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

        // the wave's two weight tiles: rows r0.. (tile 0) and r1.. (tile 1)
        const int r0 = PASS == 1 ? rb * 64 + 16 * wv : rb * 128 + 32 * wv;
        const int r1 = PASS == 1 ? a.I + r0 : r0 + 16;
        const char *wbase = static_cast<const char *>(a.w) + (size_t)e * w_rows * row_bytes;
        // load c covers rows RPL*(c % (16/RPL)) + lane / (64/RPL) of tile c / (16/RPL):
        // bf16 4 rows x 256 B (16 lanes per row), fp8 8 rows x 128 B (8 lanes
        // per row), MXFP4 16 rows x 64 B (4 lanes per row)
        constexpr int LPR = kStageB / 16;      // lanes per row segment
        constexpr int RPL = kWave / LPR;       // rows per load
        constexpr int WROW = kStageB + 16;     // padded LDS row of the wave's tile
        static_assert(WROW <= kWRow && NWL * RPL == 16, "two 16-row tiles per wave");
        const char *wsrc[NWL * 2];
        int wdst[NWL * 2];
#pragma unroll
        for (int c = 0; c < 2 * NWL; ++c) {
            const int t = c / (16 / RPL);
            const int rho = RPL * (c % (16 / RPL)) + lane / LPR;
            wsrc[c] = wbase + (size_t)((t ? r1 : r0) + rho) * row_bytes + (lane % LPR) * 16;
            wdst[c] = (t * 16 + rho) * WROW + (lane % LPR) * 16;
        }
        unsigned char *wl = wls[wv];
        const ScaleT *sp0 = nullptr, *sp1 = nullptr;
        if constexpr (kFp8) {
            const int kb = K / 128;
            sp0 = static_cast<const float *>(a.scales) + ((size_t)e * (w_rows / 128) + r0 / 128) * kb;
            sp1 = static_cast<const float *>(a.scales) + ((size_t)e * (w_rows / 128) + r1 / 128) * kb;
        } else if constexpr (kFp4) {  // the scale words of rows r0 + lane % 16 and r1 + lane % 16
            const size_t sk = (size_t)K / 32;
            const unsigned char *sb = static_cast<const unsigned char *>(a.scales) + (size_t)e * w_rows * sk;
            sp0 = reinterpret_cast<const unsigned *>(sb + (size_t)(r0 + (lane & 15)) * sk);
            sp1 = reinterpret_cast<const unsigned *>(sb + (size_t)(r1 + (lane & 15)) * sk);
        }
        // q4_0: the scale words of rows r0 + lane % 16 and r1 + lane % 16 (two
        // words, four binary16 scales, a row and stage; arrays 4-byte aligned)
        const unsigned *sq0 = nullptr, *sq1 = nullptr;
        if constexpr (kQ4) {
            const size_t sk = (size_t)K / 16;  // bytes of scales per row
            const unsigned char *sb = static_cast<const unsigned char *>(a.scales) + (size_t)e * w_rows * sk;
            sq0 = reinterpret_cast<const unsigned *>(sb + (size_t)(r0 + (lane & 15)) * sk);
            sq1 = reinterpret_cast<const unsigned *>(sb + (size_t)(r1 + (lane & 15)) * sk);
        }
        // activation rows this thread stages: chunk tid % 16 of tokens
        // tid / 16 + 16 j (16 lanes fill one 256-byte row segment: contiguous
        // global reads and conflict-free LDS writes).  They are buffer loads:
        // rows past the block's routes take an offset outside the buffer,
        // which reads zeros without touching memory (their LDS rows only
        // feed output columns that are never stored), so every lane issues
        // the same loads and the wait counts stay exact.
        const int xq = tid % kChunksPerRow, xt0 = tid / kChunksPerRow;
        unsigned xoff[kXChunks];
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int tok = xt0 + kRowsPerPass * j;
            const int xr = rts[tok < nv ? tok : 0];
            xoff[j] = tok < nv ? (unsigned)(xq * 16 + (size_t)(PASS == 1 ? xr / a.k : xr) * src_stride) : kOutside;
        }
        unsigned char *xdst = xs + xt0 * kRowLds + xq * 16;

        auto load_x = [&](int ks, u32x4(&X)[kXChunks]) {
#pragma unroll
            for (int j = 0; j < kXChunks; ++j)
                X[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)(xoff[j] + ks * kKS * 2), 0, 0));
        };
        auto store_x = [&](int buf, const u32x4(&X)[kXChunks]) {
#pragma unroll
            for (int j = 0; j < kXChunks; ++j)
                *reinterpret_cast<u32x4 *>(xdst + buf * kBufLds + kRowsPerPass * j * kRowLds) = X[j];
        };
        // Ordinary (not streaming) loads: the other token blocks of this row
        // block read the same lines at about the same time on this XCD, and
        // streaming loads leave them out of L2 (the experts with more than
        // kTB routes were then read once per token block from HBM).
        auto load_w = [&](int ks, u32x4(&W)[2 * NWL], ScaleT(&S)[2]) {
            const size_t off = (size_t)ks * kStageB;  // kKS elements
#pragma unroll
            for (int c = 0; c < 2 * NWL; ++c) W[c] = *reinterpret_cast<const u32x4 *>(wsrc[c] + off);
            if constexpr (kFp8 || kFp4) {
                S[0] = sp0[ks];
                S[1] = sp1[ks];
            }
            if constexpr (kQ4) {
                S[0] = make_uint2(sq0[2 * ks], sq0[2 * ks + 1]);
                S[1] = make_uint2(sq1[2 * ks], sq1[2 * ks + 1]);
            }
        };

        // The rest of the item for NT token tiles, a compile-time count: no
        // tile past them costs a branch, an LDS read or an MFMA, and each
        // count has its own accumulators.
        auto run = [&](auto ntc) {
            constexpr int NT = decltype(ntc)::value;
            f32x4_t acc0[NT], acc1[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) acc0[tt] = acc1[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            // the stage's weights into the wave's LDS tile, then the MFMAs reading
            // both operands from LDS (A: lane (m, g) row m, k-group g of the step)
            auto compute = [&](int buf, const u32x4(&W)[2 * NWL], const ScaleT(&S)[2]) {
#pragma unroll
                for (int c = 0; c < 2 * NWL; ++c) *reinterpret_cast<u32x4 *>(wl + wdst[c]) = W[c];
                const unsigned char *xb = xs + buf * kBufLds + (lane & 15) * kRowLds;
                const int g = lane >> 4;
                const unsigned char *wa0 = wl + (lane & 15) * WROW;
                const unsigned char *wa1 = wl + (16 + (lane & 15)) * WROW;
                // fp8: the stage's products in sums of their own (from zero at
                // k-step 0), scaled by the tiles' block scales at the stage's end
                f32x4_t p0[NT], p1[NT];
                const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int koff = 32 * s + 8 * g;  // k of this lane's 8 elements within the stage
                    u32x4 a0, a1;
                    if constexpr (kQ4) {  // (code - 8) * the row's scale of block s, rounded to bf16
                        const unsigned c0 = *reinterpret_cast<const unsigned *>(wa0 + koff / 2);
                        const unsigned c1 = *reinterpret_cast<const unsigned *>(wa1 + koff / 2);
                        const unsigned h0 = s < 2 ? S[0].x : S[0].y, h1 = s < 2 ? S[1].x : S[1].y;
                        a0 = q4x8_to_bf16(c0, f16_value((h0 >> (16 * (s & 1))) & 0xffffu));
                        a1 = q4x8_to_bf16(c1, f16_value((h1 >> (16 * (s & 1))) & 0xffffu));
                    } else if constexpr (kFp4) {
                        const unsigned c0 = *reinterpret_cast<const unsigned *>(wa0 + koff / 2);
                        const unsigned c1 = *reinterpret_cast<const unsigned *>(wa1 + koff / 2);
                        a0 = e2m1x8_to_bf16(c0, e8m0_value((S[0] >> (8 * s)) & 0xffu));
                        a1 = e2m1x8_to_bf16(c1, e8m0_value((S[1] >> (8 * s)) & 0xffu));
                    } else if constexpr (kFp8) {
                        const uint2 c0 = *reinterpret_cast<const uint2 *>(wa0 + koff);
                        const uint2 c1 = *reinterpret_cast<const uint2 *>(wa1 + koff);
                        a0 = e4m3x8_to_bf16(c0.x, c0.y);
                        a1 = e4m3x8_to_bf16(c1.x, c1.y);
                    } else {
                        a0 = *reinterpret_cast<const u32x4 *>(wa0 + koff * 2);
                        a1 = *reinterpret_cast<const u32x4 *>(wa1 + koff * 2);
                    }
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        u32x4 b;
                        if constexpr (kQ4) {  // elements 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 of block s
                            const uint2 u0 = *reinterpret_cast<const uint2 *>(xb + tt * 16 * kRowLds + 64 * s + 8 * g);
                            const uint2 u1 =
                                *reinterpret_cast<const uint2 *>(xb + tt * 16 * kRowLds + 64 * s + 32 + 8 * g);
                            b = u32x4{u0.x, u0.y, u1.x, u1.y};
                        } else {
                            b = *reinterpret_cast<const u32x4 *>(xb + tt * 16 * kRowLds + koff * 2);
                        }
                        if constexpr (kFp8) {
                            p0[tt] = mfma16(a0, b, s == 0 ? zero : p0[tt]);
                            p1[tt] = mfma16(a1, b, s == 0 ? zero : p1[tt]);
                        } else {
                            acc0[tt] = mfma16(a0, b, acc0[tt]);
                            acc1[tt] = mfma16(a1, b, acc1[tt]);
                        }
                    }
                }
                if constexpr (kFp8) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            acc0[tt][v] = fmaf(S[0], p0[tt][v], acc0[tt][v]);
                            acc1[tt][v] = fmaf(S[1], p1[tt][v], acc1[tt][v]);
                        }
                    }
                }
            };

            // ring of kD stages: W/X/S slot ks % kD
            u32x4 W[kD][2 * NWL], X[kD][kXChunks];
            ScaleT S[kD][2];
#pragma unroll
            for (int d = 0; d < kD; ++d) {
                if constexpr (kQ4) S[d][0] = S[d][1] = make_uint2(0u, 0u);
                else S[d][0] = S[d][1] = 1;
            }
            // Every stage issues the same loads (stage indices past the end are
            // clamped to the last stage) and the loop runs a multiple of kD
            // stages, so the compiler's wait counts see the same load sequence on
            // every path and only wait for the stage being consumed.
            {
#pragma unroll
                for (int d = 0; d + 1 < kD; ++d) {
                    load_x(min(d, nst - 1), X[d]);
                    load_w(min(d, nst - 1), W[d], S[d]);
                }
                store_x(0, X[0]);
                for (int ks = 0; ks < nst; ks += kD) {
                    // stage k: issue stage k + kD - 1, compute stage k, stage k +
                    // 1's activations into LDS
#pragma unroll
                    for (int d = 0; d < kD; ++d) {
                        const int k = ks + d, kl = min(k + kD - 1, nst - 1);
                        load_x(kl, X[(d + kD - 1) % kD]);
                        load_w(kl, W[(d + kD - 1) % kD], S[(d + kD - 1) % kD]);
                        lds_barrier();
                        if (k < nst) compute(k & 1, W[d], S[d]);
                        if (k + 1 < nst) store_x((k + 1) & 1, X[(d + 1) % kD]);
                    }
                }
            }

            // epilogue: lane holds rows 4*(lane/16)+v of both tiles for token lane%16
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int tok = tt * 16 + (lane & 15);
                if (tok < nv) {
                    const int r = rts[tok];
                    const int row = r0 + 4 * (lane >> 4);
                    if (PASS == 1) {
                        float o[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) o[v] = silu(acc0[tt][v]) * acc1[tt][v];
                        if (a.act_bf16) {  // bf16 into the first half of the fp32 row r
                            *reinterpret_cast<uint2 *>(reinterpret_cast<char *>(a.dst) + (size_t)r * a.I * 4 + row * 2) =
                                make_uint2(bf16_pair_rne(o[0], o[1]), bf16_pair_rne(o[2], o[3]));
                        } else {
                            *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.I + row) =
                                make_float4(o[0], o[1], o[2], o[3]);
                        }
                    } else {
                        *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row) =
                            make_float4(acc0[tt][0], acc0[tt][1], acc0[tt][2], acc0[tt][3]);
                        *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row + 16) =
                            make_float4(acc1[tt][0], acc1[tt][1], acc1[tt][2], acc1[tt][3]);
                    }
                }
            }
        };
        // (bf16: one body for all counts; four took more than 256 VGPRs)
        static_assert(kTT == 4, "token tiles 1 to 4");
        if constexpr (kFp8 || kFp4 || kQ4) {
            switch (ntt) {
                case 1: run(std::integral_constant<int, 1>{}); break;
                case 2: run(std::integral_constant<int, 2>{}); break;
                case 3: run(std::integral_constant<int, 3>{}); break;
                default: run(std::integral_constant<int, 4>{}); break;
            }
        } else {
            run(std::integral_constant<int, 4>{});
        }
    }
}

template <int WDT>
hipError_t launch_mfma_wide(int pass, int grid, hipStream_t st, const MfmaArgs &a) {
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    if (pass == 1) hipLaunchKernelGGL((mfma_wide_kernel<WDT, 1>), dim3(grid), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((mfma_wide_kernel<WDT, 2>), dim3(grid), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template hipError_t launch_mfma_wide<MOE_BF16>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma_wide<MOE_FP8_E4M3>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma_wide<MOE_MXFP4>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma_wide<MOE_Q4_0>(int, int, hipStream_t, const MfmaArgs &);

}  // namespace moe
