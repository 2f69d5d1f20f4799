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
// Work item = (segment, row block of 32 weight rows, token block of up to
// kMfmaTokens routes).  The 32 rows are two 16-row MFMA tiles:
//   pass 1: gate rows i0..i0+15 and up rows I+i0..I+i0+15, so the outputs of
//           a gate/up pair sit in the same lane and register and
//           a[r, i] = silu(g) * u is formed in registers;
//   pass 2: down rows h0..h0+31.
// Small items keep every CU busy even when only a few experts are hot.
//
// K runs in stages of 128.  Each stage of the weight tile and of the bf16
// activation rows of the token block is copied from memory straight into LDS
// (global_load_lds_dwordx4: no register staging, so the depth of the
// pipeline is set by LDS, not by VGPRs), through a ring of as many stages as
// 76 KiB hold (4 for bf16 weights, 6 for fp8 and MXFP4; two workgroups per
// CU), all but one in flight while a stage is computed.  Token blocks hold 32
// routes, so a stage's activation rows take 8 KiB.  A lane's 16-byte chunk is
// stored at chunk position (chunk ^ row) of its LDS row: the copies stay
// coalesced (a row's 16 chunks are still read by 16 adjacent lanes) and the
// operand reads (16 rows, same chunk) hit 16 different bank groups.
//
// The four waves split every stage by k: wave w runs the MFMA k-step
// 32w..32w+31 of each stage for both tiles and all token tiles, so all four
// share one copy of the weights and of the activations.  At the end the four
// partial sums are added through LDS in the fixed order w = 0, 1, 2, 3, so
// the result of a (row, route) pair depends on nothing but its own operands:
// not on the segment's size, the token block or the position in it.
//
// Items are numbered (segment, row block, token block) with the token block
// fastest and dealt out in contiguous ranges per XCD (workgroup b runs on
// XCD b % 8), so the token blocks of one row block, which read the same
// weights, run at the same time behind the same L2.
//
// fp8 e4m3 weights (W8A16): each code is converted to fp32 by the hardware
// (OCP E4M3 on gfx950), multiplied by its 128x128 block scale and rounded to
// bf16; the MFMA then runs on bf16 exactly as for bf16 weights.
//
// MXFP4 weights (W4A16; OCP Microscaling Formats v1.0, E2M1 elements with an
// E8M0 scale per 32 along K): a wave's k-step of 32 is one scale block, so a
// lane's 8 codes share one scale.  The hardware converts them to bf16 with
// the scale applied (a power of two), which is exact (an E2M1 value has 2
// significant bits).  A 128-wide stage of a row is 64 bytes
// of codes and 4 scale bytes (one aligned word: the rows' scale arrays are
// K/32 bytes long and K is a multiple of 128); every wave copies the 32
// rows' scale words of the stage into its own LDS area.
#include "experts_impl.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kTB = kMfmaNarrowTokens;  // routes per token block
constexpr int kTT = kTB / 16;         // 16-token MFMA tiles per block
constexpr int kKS = 128;              // K per stage
constexpr int kWaves = kBlock / kWave;
constexpr int kXRowB = kKS * 2;       // bytes of a staged activation row (bf16)
constexpr int kXBytes = kTB * kXRowB;  // activations of one stage (8 KiB)
constexpr int kXcds = 8;
constexpr int kRedBytes = kWaves * 2 * kTT * kWave * 16;  // partial sums of an item's four waves
static_assert(kTT <= kWaves, "one token tile per wave in the epilogue");

template <int WDT>
struct Stage {
    static constexpr bool kFp8 = WDT == MOE_FP8_E4M3;
    static constexpr bool kFp4 = WDT == MOE_MXFP4;
    static constexpr bool kQ4 = WDT == MOE_Q4_0;
    static constexpr int kRowB = kFp4 || kQ4 ? kKS / 2 : kKS * (kFp8 ? 1 : 2);  // bytes of a weight row per stage
    static constexpr int kChunks = kRowB / 16;                // 16-byte chunks per weight row
    static constexpr int kWBytes = 32 * kRowB;                // weights of one stage
    static constexpr int kWLanes = kWBytes / kWaves / 16 < kWave ? kWBytes / kWaves / 16 : kWave;  // lanes per copy
    static constexpr int kWLoads = kWBytes / (kWLanes * 16) / kWaves;  // weight copies per wave per stage
    static constexpr int kXLoads = kXBytes / 1024 / kWaves;   // activation copies per wave per stage
    static constexpr int kSLoads = kFp4 || kQ4 ? 1 : 0;       // scale-word copies per wave per stage
    // MXFP4: each wave's 32 scale words (4 E8M0 bytes a row); q4_0: 64 words
    // (4 binary16 scales a row)
    static constexpr int kSWave = kFp4 ? 32 * 4 : kQ4 ? 32 * 8 : 0;
    static constexpr int kSBytes = kWaves * kSWave;
    static constexpr int kLoads = kWLoads + kXLoads + kSLoads;  // copies per wave per stage
    static constexpr int kBytes = kWBytes + kXBytes + kSBytes;
    // bytes past the last slot so that it holds the partial sums of an item
    static constexpr int kPad = kRedBytes > kBytes ? kRedBytes - kBytes : 0;
    // LDS stages of the ring (kRing - 1 in flight), as many as 76 KiB hold
    // with the pad (two workgroups per CU): 4 for bf16, 6 for fp8 and MXFP4
    static constexpr int kRing = (76 * 1024 - kPad) / kBytes < 6 ? (76 * 1024 - kPad) / kBytes : 6;
    static_assert(kWLoads >= 1 && kWLoads * kWLanes * 16 * kWaves == kWBytes, "weight copies cover the stage");
    static_assert(kWLanes % kChunks == 0, "a copy covers whole rows");
};

__device__ __forceinline__ f32x4_t mfma16(const u32x4 &a, const u32x4 &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// 8 E4M3 codes (two words, element 0 in the low byte) times s, as 8 bf16.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(unsigned w0, unsigned w1, float s) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    return u32x4{bf16_pair_rne(a[0] * s, a[1] * s), bf16_pair_rne(b[0] * s, b[1] * s),
                 bf16_pair_rne(c[0] * s, c[1] * s), bf16_pair_rne(d[0] * s, d[1] * s)};
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

// A wave-uniform pointer (kept in scalar registers).
template <typename P>
__device__ __forceinline__ P *uniform_ptr(P *p) {
    const unsigned long long v = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return reinterpret_cast<P *>(((unsigned long long)hi << 32) | lo);
}

// Copy of 16 bytes per lane from base + off (base wave-uniform, off this
// lane's byte offset) into LDS at dst + 16 * lane (dst wave-uniform; M0
// carries it and is restored afterwards).  Issued from asm: the compiler,
// which tracks the LDS writes of its own copies, would wait for every copy in
// flight (vmcnt(0)) before the next LDS read and so drain the ring at each
// stage; the waits here are explicit (wait_copies_and_sync).  Its own waits
// stay correct: copies issued after one of its loads only make a vmcnt wait
// for that load stricter.
__device__ __forceinline__ void copy_to_lds(const void *base, unsigned off, const unsigned char *dst) {
    const unsigned l = __builtin_amdgcn_readfirstlane(
        (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned char *)dst);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(uniform_ptr(base)), "s"(l)
        : "memory");
}

// The same for 4 bytes per lane (LDS at dst + 4 * lane).
__device__ __forceinline__ void copy_word_to_lds(const void *base, unsigned off, const unsigned char *dst) {
    const unsigned l = __builtin_amdgcn_readfirstlane(
        (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned char *)dst);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(uniform_ptr(base)), "s"(l)
        : "memory");
}


// Wait until at most N of this wave's global loads are outstanding and all
// of its LDS operations are done, then meet the other waves.  The copies
// complete in issue order, so N = the copies issued after the stage that is
// needed.
template <int N>
__device__ __forceinline__ void wait_copies_and_sync() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// wait_copies_and_sync for n (wave-uniform, 0 <= n <= MAXN) stages of P
// copies each, then X more copies, issued after the needed one.
template <int MAXN, int P, int X>
__device__ __forceinline__ void wait_stages(int n) {
    if constexpr (MAXN > 0) {
        if (n == MAXN) {
            wait_copies_and_sync<MAXN * P + X>();
            return;
        }
        wait_stages<MAXN - 1, P, X>(n);
    } else {
        wait_copies_and_sync<X>();
    }
}

// Workgroup barrier that waits for this wave's LDS traffic only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Item and route tables over the experts, from the counts alone: pre[e] =
// items of the experts below e (an expert with n >= min_n routes yields
// n_rb x token blocks items, others none), pre[E] = total; off[e] = routes
// of the experts below e, which is where the sorted routes of e start (the
// counting sort lays the segments out in expert order).  Returns the total.
__device__ int build_tables(const MfmaArgs &a, int n_rb, int *pre, int *off, int *wsum) {
    const int tid = threadIdx.x, E = a.sa.E;
    constexpr int kPer = (kMaxE + kBlock - 1) / kBlock;
    const int per = (E + kBlock - 1) / kBlock;  // experts per thread, contiguous
    int it[kPer], ct[kPer], li = 0, lc = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * per + q;
        const int n = (q < per && e < E) ? a.sa.counts[e] : 0;
        ct[q] = n;
        it[q] = n >= a.min_n ? n_rb * ((n + kTB - 1) / kTB) : 0;
        li += it[q];
        lc += n;
    }
    int vi = li, vc = lc;  // inclusive scans over the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int oi = __shfl_up(vi, d, kWave), oc = __shfl_up(vc, d, kWave);
        if ((tid & (kWave - 1)) >= d) {
            vi += oi;
            vc += oc;
        }
    }
    if ((tid & (kWave - 1)) == kWave - 1) {
        wsum[tid / kWave] = vi;
        wsum[kWaves + tid / kWave] = vc;
    }
    __syncthreads();
    int bi = 0, bc = 0, total = 0, routes = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < tid / kWave) {
            bi += wsum[w];
            bc += wsum[kWaves + w];
        }
        total += wsum[w];
        routes += wsum[kWaves + w];
    }
    int xi = bi + vi - li, xc = bc + vc - lc;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * per + q;
        if (q < per && e < E) {
            pre[e] = xi;
            off[e] = xc;
        }
        xi += it[q];
        xc += ct[q];
    }
    if (tid == 0) {
        pre[E] = total;
        off[E] = routes;
    }
    __syncthreads();
    return total;
}

}  // namespace

// The end of an item: the four waves' partial sums (acc0, acc1: this wave's
// k-steps of the two weight tiles, per token tile) go through red (LDS,
// 2 x kWaves x kTT x 64 x 16 bytes) and are added in wave order
// w = 0, 1, 2, 3; wave tt then writes token tile tt: pass 1 a[r, i] =
// silu(gate) * up (fp32, or bf16 into the first half of the fp32 row for the
// MFMA pass 2), pass 2 the y rows.  A lane (m, g) holds rows 4g .. 4g+3 of
// both tiles for token m of its tile; r is that token's route.
template <int PASS>
__device__ __forceinline__ void mfma_epilogue(const MfmaArgs &a, f32x4_t *red, const f32x4_t (&acc0)[kTT],
                                              const f32x4_t (&acc1)[kTT], int ntt, int nv, int r, int r0, int wv,
                                              int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
        if (tt < ntt) {
            red[((wv * 2 + 0) * kTT + tt) * kWave + lane] = acc0[tt];
            red[((wv * 2 + 1) * kTT + tt) * kWave + lane] = acc1[tt];
        }
    }
    lds_barrier();
    const int tt = wv;  // this wave's token tile in the epilogue (waves < kTT)
    const int tok = tt * 16 + m;
    if (tt < ntt && tok < nv) {
        f32x4_t s0 = red[((0 * 2 + 0) * kTT + tt) * kWave + lane];
        f32x4_t s1 = red[((0 * 2 + 1) * kTT + tt) * kWave + lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            s0 += red[((w * 2 + 0) * kTT + tt) * kWave + lane];
            s1 += red[((w * 2 + 1) * kTT + tt) * kWave + lane];
        }
        const int row = r0 + 4 * g;
        if (PASS == 1) {
            float o[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = silu(s0[v]) * s1[v];
            if (a.act_bf16) {  // bf16 into the first half of the fp32 row r
                *reinterpret_cast<uint2 *>(reinterpret_cast<char *>(a.dst) + (size_t)r * a.I * 4 + row * 2) =
                    make_uint2(bf16_pair_rne(o[0], o[1]), bf16_pair_rne(o[2], o[3]));
            } else {
                *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.I + row) = make_float4(o[0], o[1], o[2], o[3]);
            }
        } else {
            *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row) = make_float4(s0[0], s0[1], s0[2], s0[3]);
            *reinterpret_cast<float4 *>(a.dst + (size_t)r * a.H + row + 16) = make_float4(s1[0], s1[1], s1[2], s1[3]);
        }
    }
}

// Items follow each other without a gap in the copy stream.  During the last
// stages of an item, once its final copies are issued, each wave copies the
// next item's route ids into its own LDS row (one 4-byte copy per lane, which
// the stage waits count) and loads the next fp8 scales; after the item's
// last stage, the next item's first kRing - 1 stages are issued into ring
// slots 0 .. kRing - 2, and only then are the item's partial sums reduced,
// in slot kRing - 1 (extended by kPad bytes where a stage is smaller than
// the reduction).  So the route-id round trip and the ring's fill latency of
// an item overlap the previous item's last stages and epilogue.
template <int WDT, int PASS>
__global__ __launch_bounds__(kBlock, 2) void mfma_kernel(MfmaArgs a) {
    using S = Stage<WDT>;
    constexpr bool kFp8 = S::kFp8, kFp4 = S::kFp4, kQ4 = S::kQ4;
    constexpr int kRing = S::kRing;
    static_assert(kRing >= 3 && (kRing - 2) * S::kLoads + 1 <= 63, "ring depth");
    __shared__ __align__(1024) unsigned char ring[kRing * S::kBytes + S::kPad];
    __shared__ int ids[kWaves][kWave];  // each wave's copy of an item's route ids
    __shared__ int wsum[2 * kWaves];
    extern __shared__ int tables[];  // pre [E + 1], off [E + 1]
    static_assert(S::kBytes + S::kPad >= kRedBytes, "partial sums fit in the last slot");

    // no expert reaches the threshold (known from the sort's statistics), or
    // the routing was rejected: nothing to do
    if (a.max_count && load_uniform(a.max_count) < a.hot) return;
    if (segment_count(a.sa) == 0) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int E = a.sa.E;
    int *pre = tables, *off = tables + E + 1;
    const int K = PASS == 1 ? a.H : a.I;
    const int nst = K / kKS;
    const int n_rb = PASS == 1 ? a.I / 16 : a.H / 32;
    const int w_rows = PASS == 1 ? 2 * a.I : a.H;
    // MXFP4 and q4_0: 2 codes a byte
    const unsigned row_bytes = kFp4 || kQ4 ? (unsigned)K / 2 : (unsigned)K * WT<WDT>::kBytes;
    // bf16 activation rows: pass 1 reads xb [T, H]; pass 2 reads a[r] from the
    // first half of the fp32 activation row r (4I bytes apart)
    const unsigned src_stride = PASS == 1 ? (unsigned)a.H * 2 : (unsigned)a.I * 4;
    const int total = __builtin_amdgcn_readfirstlane(build_tables(a, n_rb, pre, off, wsum));
    // contiguous item ranges per XCD (the grid is a multiple of kXcds, so a
    // workgroup's items ascend and stay inside its XCD's range)
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int slots = per_xcd * kXcds;
    const int m = lane & 15, g = lane >> 4;
    auto item_of = [&](int it) { return (it % kXcds) * per_xcd + it / kXcds; };

    // item -> (expert, row block, token block)
    struct Item {
        int e, first, rb, tb, nv;
    };
    auto decode = [&](int item) {
        int lo = 0, hi = E;  // pre[lo] <= item < pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= item) lo = mid;
            else hi = mid;
        }
        Item d;
        d.e = __builtin_amdgcn_readfirstlane(lo);
        const int local = item - pre[d.e];
        d.first = off[d.e];
        const int n = off[d.e + 1] - d.first;
        const int ntb = (n + kTB - 1) / kTB;
        d.rb = local / ntb;
        d.tb = local - d.rb * ntb;
        d.nv = min(kTB, n - d.tb * kTB);
        return d;
    };
    // the item's route ids into this wave's row of ids: lane l copies route
    // l & 31 of the token block; positions past its routes take the first
    // route (their LDS rows only feed outputs that are never stored)
    const char *sorted = uniform_ptr(reinterpret_cast<const char *>(a.sa.sorted));
    const unsigned char *idrow = reinterpret_cast<const unsigned char *>(&ids[wv][0]);
    auto copy_ids = [&](const Item &d) {
        const int tau = lane & (kTB - 1);
        copy_word_to_lds(sorted, (unsigned)(d.first + d.tb * kTB + (tau < d.nv ? tau : 0)) * 4u, idrow);
    };
    // fp8 block scales of the item's two tiles, stage ks in lane ks (K <= 64 *
    // 128; lanes past the stages repeat the last).  Nothing else writes s0
    // and s1 here: a register write while an earlier load into the same
    // register may be in flight would make the compiler wait for every load.
    auto load_scales = [&](const Item &d, float &s0, float &s1) {
        if (kFp8) {
            const int kb = K / 128;
            const int q0 = PASS == 1 ? d.rb * 16 : d.rb * 32;
            const int q1 = PASS == 1 ? a.I + q0 : q0 + 16;
            const float *sp0 = static_cast<const float *>(a.scales) + ((size_t)d.e * (w_rows / 128) + q0 / 128) * kb;
            const float *sp1 = static_cast<const float *>(a.scales) + ((size_t)d.e * (w_rows / 128) + q1 / 128) * kb;
            const int l = lane < kb ? lane : kb - 1;
            s0 = sp0[l];
            s1 = sp1[l];
        }
    };

    // per-item state: the item, its copy offsets and its fp8 scales
    struct St {
        Item d;
        int ntt, r0, r_out;
        bool xw;
        const char *wbase;
        const unsigned char *sbase;
        unsigned soff;
        unsigned woff[S::kWLoads];
        unsigned xoff[S::kXLoads];
        float sc0, sc1;
    };
    const int sk = K / 32;  // MXFP4 scale bytes per weight row
    const char *xbase = uniform_ptr(static_cast<const char *>(a.src));
    // the state of item d once its id copy (and scale loads) are complete
    auto setup = [&](const Item &d, float s0, float s1) {
        St c;
        c.d = d;
        c.ntt = (d.nv + 15) >> 4;
        c.sc0 = s0;
        c.sc1 = s1;
        int rn[S::kXLoads];
#pragma unroll
        for (int j = 0; j < S::kXLoads; ++j) rn[j] = ids[wv][(wv * S::kXLoads + j) * 4 + (lane >> 4)];
        c.r_out = ids[wv][wv * 16 + m];  // this lane's route in the epilogue (waves < kTT)
        // the reads are done before a later copy rewrites the row
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // weight rows of the item: row rho < 16 of tile 0, rho >= 16 of tile 1.
        // This lane's weight copy c covers rows (kWLanes / kChunks) apart; its
        // chunk is the one that lands at its LDS position (position ^ row).
        c.r0 = PASS == 1 ? d.rb * 16 : d.rb * 32;
        const int r1 = PASS == 1 ? a.I + c.r0 : c.r0 + 16;
        c.wbase = uniform_ptr(static_cast<const char *>(a.w) + (size_t)d.e * w_rows * row_bytes);
#pragma unroll
        for (int q = 0; q < S::kWLoads; ++q) {
            const int rho = (wv * S::kWLoads + q) * (S::kWLanes / S::kChunks) + (lane % S::kWLanes) / S::kChunks;
            const int pos = lane % S::kChunks;
            const int chunk = pos ^ (rho & (S::kChunks - 1));
            c.woff[q] = (unsigned)(rho < 16 ? c.r0 + rho : r1 + rho - 16) * row_bytes + chunk * 16;
        }
        // MXFP4 scale words: lane l < 32 copies the stage's word of row l;
        // q4_0: lane l copies word l & 1 of row l / 2 (a row's 4 binary16
        // scales of the stage are two words)
        c.sbase = nullptr;
        c.soff = 0;
        if (kFp4) {
            c.sbase = uniform_ptr(static_cast<const unsigned char *>(a.scales) + (size_t)d.e * w_rows * sk);
            c.soff = (unsigned)((lane < 16 ? c.r0 + lane : r1 + (lane & 31) - 16) * sk);
        }
        if (kQ4) {
            const int rho = lane >> 1;
            c.sbase = uniform_ptr(static_cast<const unsigned char *>(a.scales) + (size_t)d.e * w_rows * (2 * sk));
            c.soff = (unsigned)((rho < 16 ? c.r0 + rho : r1 + rho - 16) * (2 * sk) + (lane & 1) * 4);
        }
        // activation copies: only the waves whose token tile holds routes copy
        c.xw = wv * kTB / (16 * kWaves) < c.ntt;
#pragma unroll
        for (int j = 0; j < S::kXLoads; ++j) {
            const int tau = (wv * S::kXLoads + j) * 4 + (lane >> 4);
            const int chunk = (lane & 15) ^ (tau & 15);
            c.xoff[j] = (unsigned)(PASS == 1 ? rn[j] / a.k : rn[j]) * src_stride + chunk * 16;
        }
        return c;
    };
    // stage ks of item c into ring slot sl
    auto issue = [&](const St &c, int ks, int sl) {
        const unsigned char *wd = ring + sl * S::kBytes;
        if (S::kWLanes == kWave || lane < S::kWLanes)
#pragma unroll
            for (int q = 0; q < S::kWLoads; ++q)
                copy_to_lds(uniform_ptr(c.wbase) + (size_t)ks * S::kRowB, c.woff[q],
                            wd + (wv * S::kWLoads + q) * S::kWLanes * 16);
        if (c.xw)
#pragma unroll
            for (int j = 0; j < S::kXLoads; ++j)
                copy_to_lds(xbase + (size_t)ks * kXRowB, c.xoff[j], wd + S::kWBytes + (wv * S::kXLoads + j) * 1024);
        if (kFp4 && lane < 32)
            copy_word_to_lds(uniform_ptr(c.sbase) + (size_t)ks * 4, c.soff, wd + S::kWBytes + kXBytes + wv * S::kSWave);
        if (kQ4)
            copy_word_to_lds(uniform_ptr(c.sbase) + (size_t)ks * 8, c.soff, wd + S::kWBytes + kXBytes + wv * S::kSWave);
    };
    // stages 0 .. kRing - 2 of item c in flight, in slots 0 .. kRing - 2
    auto prologue = [&](const St &c) {
#pragma unroll
        for (int s = 0; s + 1 < kRing; ++s)
            if (s < nst) issue(c, s, s);
    };

    int it = blockIdx.x;
    if (it >= slots || item_of(it) >= total) return;  // uniform over the workgroup
    St cur;
    {
        const Item d = decode(item_of(it));
        float s0 = 1.f, s1 = 1.f;
        load_scales(d, s0, s1);
        copy_ids(d);
        // Redefining the values in an asm statement tells the compiler that
        // the loads are complete; it would otherwise wait for them (vmcnt) at
        // their first use inside the stage loop, and its count, which does
        // not know the copies, would drain the ring there.
        asm volatile("s_waitcnt vmcnt(0)" : "+v"(s0), "+v"(s1)::"memory");
        cur = setup(d, s0, s1);
    }
    prologue(cur);

    // k-step wv of stage ks from slot sl: A lane (m, g) holds row m of a
    // tile at k 32 wv + 8 g .. +7, B lane (m, g) token m of a token tile.
    // Every operand of the stage is read before the copies of a later stage
    // are issued and before the first MFMA, so the LDS latency is paid once
    // per stage; tiles past ntt read rows that feed no output.
    const int aoff = kFp4 || kQ4 ? ((wv ^ (m & 3)) << 4) + (g << 2)
                     : kFp8 ? (((2 * wv + (g >> 1)) ^ (m & 7)) << 4) + ((g & 1) << 3)
                            : ((4 * wv + g) ^ m) << 4;
    const int boff = m * kXRowB + (((4 * wv + g) ^ m) << 4);
    // q4_0: the activations of block elements 4g .. 4g + 3 and 16 + 4g ..
    // 16 + 4g + 3 of k-step wv, in the order of the lane's weight codes
    const int boffq0 = m * kXRowB + (((4 * wv + (g >> 1)) ^ m) << 4) + ((g & 1) << 3);
    const int boffq1 = m * kXRowB + (((4 * wv + 2 + (g >> 1)) ^ m) << 4) + ((g & 1) << 3);
    // the next item's fp8 scales, written only by their loads inside the
    // loop (see load_scales)
    float n0 = 1.f, n1 = 1.f;
    for (;;) {
        // the next item of this workgroup, if any: its id copy (and scale
        // loads) are issued once this item's last copies are
        const int nit = it + (int)gridDim.x;
        const bool more = nit < slots && item_of(nit) < total;
        Item dn = cur.d;
        bool pf = false;  // issued, and counted by the stage waits
        auto prefetch = [&]() {
            if (more) {
                dn = decode(item_of(nit));
                load_scales(dn, n0, n1);
                copy_ids(dn);
                pf = true;
            }
        };
        if (nst <= kRing - 1) prefetch();

        const int ntt = cur.ntt;
        f32x4_t acc0[kTT], acc1[kTT];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) acc0[tt] = acc1[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        int sl = 0;
        for (int ks = 0; ks < nst; ++ks) {
            // copies issued after the stage that is needed: those of stages
            // ks + 1 .. ks + after, then the next item's id copy
            const int after = min(kRing - 2, nst - 1 - ks);
            if (pf) {
                if (cur.xw) wait_stages<kRing - 2, S::kLoads, 1>(after);
                else wait_stages<kRing - 2, S::kWLoads + S::kSLoads, 1>(after);
            } else {
                if (cur.xw) wait_stages<kRing - 2, S::kLoads, 0>(after);
                else wait_stages<kRing - 2, S::kWLoads + S::kSLoads, 0>(after);
            }

            const unsigned char *wd = ring + sl * S::kBytes;
            const unsigned char *xd = wd + S::kWBytes;
            u32x4 a0, a1, b[kTT];
            uint2 c0, c1;
            unsigned f0 = 0, f1 = 0, e0 = 0, e1 = 0;
            float d0[4], d1[4];  // q4_0: scales of rows 4g .. 4g + 3 of both tiles, block wv
            if (kQ4) {
                const unsigned char *sd = wd + S::kWBytes + kXBytes + wv * S::kSWave;
                f0 = *reinterpret_cast<const unsigned *>(wd + m * S::kRowB + aoff);
                f1 = *reinterpret_cast<const unsigned *>(wd + (16 + m) * S::kRowB + aoff);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    d0[v] = f16_value(*reinterpret_cast<const unsigned short *>(sd + (4 * g + v) * 8 + 2 * wv));
                    d1[v] = f16_value(*reinterpret_cast<const unsigned short *>(sd + (16 + 4 * g + v) * 8 + 2 * wv));
                }
            } else if (kFp4) {
                const unsigned char *sd = wd + S::kWBytes + kXBytes + wv * 128;
                f0 = *reinterpret_cast<const unsigned *>(wd + m * S::kRowB + aoff);
                f1 = *reinterpret_cast<const unsigned *>(wd + (16 + m) * S::kRowB + aoff);
                e0 = sd[4 * m + wv];  // scale block 4 ks + wv of row m (tile 0) and 16 + m (tile 1)
                e1 = sd[4 * (16 + m) + wv];
            } else if (kFp8) {
                c0 = *reinterpret_cast<const uint2 *>(wd + m * S::kRowB + aoff);
                c1 = *reinterpret_cast<const uint2 *>(wd + (16 + m) * S::kRowB + aoff);
            } else {
                a0 = *reinterpret_cast<const u32x4 *>(wd + m * S::kRowB + aoff);
                a1 = *reinterpret_cast<const u32x4 *>(wd + (16 + m) * S::kRowB + aoff);
            }
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
                if (kQ4) {
                    const uint2 u0 = *reinterpret_cast<const uint2 *>(xd + tt * 16 * kXRowB + boffq0);
                    const uint2 u1 = *reinterpret_cast<const uint2 *>(xd + tt * 16 * kXRowB + boffq1);
                    b[tt] = u32x4{u0.x, u0.y, u1.x, u1.y};
                } else {
                    b[tt] = *reinterpret_cast<const u32x4 *>(xd + tt * 16 * kXRowB + boff);
                }
            }

            if (ks + kRing - 1 < nst) {
                issue(cur, ks + kRing - 1, sl == 0 ? kRing - 1 : sl - 1);
                if (ks + kRing == nst) prefetch();  // the item's last copies are issued
            }
            if (kFp4) {
                a0 = e2m1x8_to_bf16(f0, e8m0_value(e0));
                a1 = e2m1x8_to_bf16(f1, e8m0_value(e1));
            }
            if (kQ4) {
                a0 = q4x8_to_bf16(f0);
                a1 = q4x8_to_bf16(f1);
            }
            if (kFp8) {
                a0 = e4m3x8_to_bf16(c0.x, c0.y,
                                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.sc0), ks)));
                a1 = e4m3x8_to_bf16(c1.x, c1.y,
                                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.sc1), ks)));
            }
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
                if (tt < ntt) {
                    if (kQ4) {  // one block per row: the k-step's sums times the rows' scales
                        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
                        const f32x4_t p0 = mfma16(a0, b[tt], zero), p1 = mfma16(a1, b[tt], zero);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            acc0[tt][v] = fmaf(d0[v], p0[v], acc0[tt][v]);
                            acc1[tt][v] = fmaf(d1[v], p1[v], acc1[tt][v]);
                        }
                    } else {
                        acc0[tt] = mfma16(a0, b[tt], acc0[tt]);
                        acc1[tt] = mfma16(a1, b[tt], acc1[tt]);
                    }
                }
            }
            sl = sl == kRing - 1 ? 0 : sl + 1;
        }

        lds_barrier();  // every wave is done reading the ring
        St nxt = cur;
        if (more) {
            // the next item's first stages go out before this item's partial
            // sums are added: slots 0 .. kRing - 2, slot kRing - 1 is left
            // for the sums
            asm volatile("s_waitcnt vmcnt(0)" : "+v"(n0), "+v"(n1)::"memory");
            nxt = setup(dn, n0, n1);
            prologue(nxt);
        }
        mfma_epilogue<PASS>(a, reinterpret_cast<f32x4_t *>(ring + (kRing - 1) * S::kBytes), acc0, acc1, ntt,
                            cur.d.nv, cur.r_out, cur.r0, wv, lane);
        if (!more) break;
        it = nit;
        cur = nxt;
    }
}

template <int WDT>
hipError_t launch_mfma(int pass, int grid, hipStream_t st, const MfmaArgs &a) {
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    const size_t lds = (size_t)2 * (a.sa.E + 1) * sizeof(int);
    if (pass == 1) hipLaunchKernelGGL((mfma_kernel<WDT, 1>), dim3(grid), dim3(kBlock), lds, st, a);
    else hipLaunchKernelGGL((mfma_kernel<WDT, 2>), dim3(grid), dim3(kBlock), lds, st, a);
    return hipGetLastError();
}

template hipError_t launch_mfma<MOE_BF16>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma<MOE_FP8_E4M3>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma<MOE_MXFP4>(int, int, hipStream_t, const MfmaArgs &);
template hipError_t launch_mfma<MOE_Q4_0>(int, int, hipStream_t, const MfmaArgs &);

}  // namespace moe
