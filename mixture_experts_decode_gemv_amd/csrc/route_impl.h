// Device pieces of routing: exact top-k selection of one token by one wave,
// and the stable counting sort of the routes by one workgroup.
//
// Selection ("MoE Performance Optimization Analysis", GPU Router Design:
// router compute, argmax and selection on the device).  The k largest logits
// by (logit descending, expert index ascending), one or two tokens per wave: logits
// map to order-preserving 32-bit keys (-0 and +0 share one key, as IEEE
// comparison has them equal); each lane keeps its best untaken (key, index);
// round j takes the wave maximum key and, among lanes holding it, the lowest
// index (two DPP reductions), and only the winning lane rescans its logits.
// Slot j is the winner of round j.  The weights are a softmax over the k
// chosen logits, which equals the softmax over all E logits renormalised over
// the chosen k.
//
// Sort ("perf(cpu-moe): dedup experts across the batch in pass 1", commit
// message: a counting sort of the routes by expert id, built once per layer
// and step).  Up to kSortOneWaveMax routes, one wave sorts alone, with no
// barrier (sort_wave): rounds of 64 routes in route order, each route's rank
// among the equal ids of its round from ballots over the id bits, plus the
// per-expert running count in LDS; then one scan over the experts.  Up to
// 4 kSortWaveRoutes routes, four waves do the same on their quarters of the
// routes and combine their per-expert counts (sort_waves4).  Larger sorts
// use the whole workgroup (sort_block): histogram with LDS integer
// atomics, exclusive scans for the offsets and the unique-expert list, then a
// stable scatter in windows of 256 routes: each window sets one bit per route
// in a per-expert bitmask, and a route's rank inside its expert is the
// expert's count in earlier windows plus the bits below its own.
#pragma once

#include "common.h"

namespace moe {

constexpr int kSelPerLane = kMaxE / kWave;

__device__ __forceinline__ uint32_t logit_key(float f) {
    if (f == 0.0f) f = 0.0f;  // -0 -> +0
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Wave-wide unsigned max / min: DPP row_shr 1, 2, 4, 8 inside each row of 16
// lanes, then row_bcast15 and row_bcast31 across rows; lane 63 holds the
// result.  Lanes outside a row's range read the identity.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
    const int id = MAX ? 0 : (int)0xFFFFFFFFu;
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Wave-wide float sum by the same DPP pattern (fixed order, so the result is
// deterministic); every lane receives lane 63's total.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    auto add = [](float a, int b) { return a + __int_as_float(b); };
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// One wave selects for NT tokens at once (their chains are independent, so
// their memory round trips and reduction latencies overlap).  l[q]: token
// q's E logits (COHERENT: written by other workgroups of this launch).
// Writes ids[q][0..k) and w[q][0..k) with device-scope stores, and the ids
// also to lds_ids[q][0..k) when it is set.  Each lane sorts its own keys once
// (descending key, ascending index); a round then takes the wave maximum of
// the lanes' heads, finds its lane by ballot, and only on an exact tie
// between lanes runs a second reduction for the lowest index; the winning
// lane advances its head.  Every token's result is the same as when it is
// selected alone.
template <bool COHERENT, int NCS, int NT>
__device__ __forceinline__ void select_tokens_n(const float *const (&l)[NT], int E, int k, int32_t *const (&ids)[NT],
                                                float *const (&w)[NT], int32_t *const (&lds_ids)[NT], int lane) {
    uint32_t key[NT][NCS];
    uint32_t idx[NT][NCS];
    const int nc = (E + kWave - 1) / kWave;
    // unconditional loads (index clamped), all in flight at once
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int c = 0; c < NCS; ++c) {
            const int e = lane + kWave * c;
            const bool valid = c < nc && e < E;
            const int ec = min(e, E - 1);
            const float v = COHERENT ? load_shared(l[q] + ec) : l[q][ec];
            key[q][c] = valid ? logit_key(v) : 0u;  // 0: no expert
            idx[q][c] = (uint32_t)e;
        }
    // per-lane insertion sort, descending key (stable: equal keys keep the
    // ascending index order they were generated in)
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int i = 1; i < NCS; ++i) {
#pragma unroll
            for (int j = i; j > 0; --j) {
                if (key[q][j] > key[q][j - 1]) {
                    const uint32_t tk = key[q][j]; key[q][j] = key[q][j - 1]; key[q][j - 1] = tk;
                    const uint32_t ti = idx[q][j]; idx[q][j] = idx[q][j - 1]; idx[q][j - 1] = ti;
                }
            }
        }
    int head[NT];
    uint32_t my_key[NT], my_idx[NT], top[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        head[q] = 0;
        my_key[q] = my_idx[q] = top[q] = 0u;
    }
    for (int j = 0; j < k; ++j) {
        uint32_t hk[NT], hi[NT], m[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            hk[q] = 0u;
            hi[q] = 0xFFFFFFFFu;
#pragma unroll
            for (int c = 0; c < NCS; ++c)
                if (c == head[q]) { hk[q] = key[q][c]; hi[q] = idx[q][c]; }
        }
#pragma unroll
        for (int q = 0; q < NT; ++q) m[q] = wave_reduce_u32<true>(hk[q]);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const unsigned long long holders = __ballot(hk[q] == m[q]);
            uint32_t win;
            if (__popcll(holders) == 1) win = (uint32_t)__shfl((int)hi[q], __ffsll((long long)holders) - 1, kWave);
            else win = wave_reduce_u32<false>(hk[q] == m[q] ? hi[q] : 0xFFFFFFFFu);
            if (j == 0) top[q] = m[q];
            if (lane == j) { my_key[q] = m[q]; my_idx[q] = win; }
            if (hi[q] == win) ++head[q];
        }
    }
    float p[NT], sum[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) p[q] = lane < k ? expf(key_logit(my_key[q]) - key_logit(top[q])) : 0.f;
#pragma unroll
    for (int q = 0; q < NT; ++q) sum[q] = wave_sum_dpp(p[q]);
    if (lane < k) {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            store_shared(ids[q] + lane, (int32_t)my_idx[q]);
            store_shared(w[q] + lane, p[q] / sum[q]);
            if (lds_ids[q]) lds_ids[q][lane] = (int32_t)my_idx[q];
        }
    }
}

// Logits per lane instantiated for 1, 2, 4, 8 and 16 (E <= 1024).
template <bool COHERENT, int NT>
__device__ __forceinline__ void select_tokens(const float *const (&l)[NT], int E, int k, int32_t *const (&ids)[NT],
                                              float *const (&w)[NT], int32_t *const (&lds_ids)[NT], int lane) {
    const int nc = (E + kWave - 1) / kWave;
    if (nc <= 1) select_tokens_n<COHERENT, 1, NT>(l, E, k, ids, w, lds_ids, lane);
    else if (nc <= 2) select_tokens_n<COHERENT, 2, NT>(l, E, k, ids, w, lds_ids, lane);
    else if (nc <= 4) select_tokens_n<COHERENT, 4, NT>(l, E, k, ids, w, lds_ids, lane);
    else if (nc <= 8) select_tokens_n<COHERENT, 8, NT>(l, E, k, ids, w, lds_ids, lane);
    else select_tokens_n<COHERENT, 16, NT>(l, E, k, ids, w, lds_ids, lane);
}

// LDS ints needed by sort_block for E experts.
__host__ __device__ constexpr int sort_lds_ints(int E) { return 11 * E; }

// One workgroup sorts R routes.  ids COHERENT: written by other workgroups
// of this launch; otherwise global memory written before the launch or this
// workgroup's LDS.  lds: sort_lds_ints(E) ints.  Each thread loads its routes
// r = tid + 256 w once (up to 16 windows held in registers).  Also zeroes
// n_zero words at zero (counters of the kernels that follow).
template <bool COHERENT>
__device__ __forceinline__ void sort_block(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                           int32_t *uniq, int32_t *n_uniq, int32_t *stats, int *lds, unsigned *zero, int n_zero) {
    constexpr int kWin = 16;
    __shared__ int s_bad, s_max;
    __shared__ int s_wc[kBlock / kWave], s_wu[kBlock / kWave];
    int *s_cnt = lds, *s_off = lds + E, *s_run = lds + 2 * E;
    unsigned *s_bits = reinterpret_cast<unsigned *>(lds + 3 * E);  // [E][8]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nwin = (R + kBlock - 1) / kBlock;

    int v[kWin];
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
        const int r = tid + kBlock * w;
        v[w] = (w < nwin && r < R) ? (COHERENT ? load_shared(ids + r) : ids[r]) : -1;
    }
    for (int i = tid; i < n_zero; i += kBlock) zero[i] = 0u;
    for (int e = tid; e < E; e += kBlock) {
        s_cnt[e] = 0;
        s_run[e] = 0;
    }
    if (tid == 0) { s_bad = 0; s_max = 0; }
    __syncthreads();
    for (int w = 0; w < nwin; ++w) {
        const int r = tid + kBlock * w;
        const int vv = w < kWin ? v[w] : (r < R ? (COHERENT ? load_shared(ids + r) : ids[r]) : -1);
        if (r < R) {
            if (vv < 0 || vv >= E) s_bad = 1;
            else atomicAdd(&s_cnt[vv], 1);
        }
    }
    __syncthreads();
    if (s_bad) {
        if (tid == 0) {
            *n_uniq = -1;
            if (stats) { stats[0] = -1; stats[1] = R; stats[2] = 0; stats[3] = 0; }
        }
        return;
    }
    // exclusive scans of the counts and of (count > 0); thread tid owns [lo, hi)
    const int per = (E + kBlock - 1) / kBlock;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int csum = 0, usum = 0, cmax = 0;
    for (int e = lo; e < hi; ++e) {
        csum += s_cnt[e];
        usum += s_cnt[e] > 0;
        cmax = max(cmax, s_cnt[e]);
    }
    int cinc = csum, uinc = usum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int oc = __shfl_up(cinc, d, kWave), ou = __shfl_up(uinc, d, kWave);
        if (lane >= d) { cinc += oc; uinc += ou; }
    }
    if (lane == kWave - 1) { s_wc[wave] = cinc; s_wu[wave] = uinc; }
    atomicMax(&s_max, cmax);
    __syncthreads();
    int cpre = cinc - csum, upre = uinc - usum, utot = 0;
    for (int wv = 0; wv < kBlock / kWave; ++wv) {
        if (wv < wave) { cpre += s_wc[wv]; upre += s_wu[wv]; }
        utot += s_wu[wv];
    }
    for (int e = lo; e < hi; ++e) {
        const int c = s_cnt[e];
        s_off[e] = cpre;
        offsets[e] = cpre;
        counts[e] = c;
        if (c > 0) uniq[upre++] = e;
        cpre += c;
    }
    if (tid == 0) {
        offsets[E] = R;
        *n_uniq = utot;
        if (stats) { stats[0] = utot; stats[1] = R; stats[2] = s_max; stats[3] = 0; }
    }
    // stable scatter, 256 routes per window
    for (int w = 0; w < nwin; ++w) {
        for (int i = tid; i < E * 8; i += kBlock) s_bits[i] = 0u;
        __syncthreads();
        const int r = tid + kBlock * w;
        int vv = -1;
#pragma unroll
        for (int u = 0; u < kWin; ++u)
            if (u == w) vv = v[u];
        if (w >= kWin && r < R) vv = COHERENT ? load_shared(ids + r) : ids[r];
        const int word = tid >> 5, bit = tid & 31;
        if (vv >= 0) atomicOr(&s_bits[vv * 8 + word], 1u << bit);
        __syncthreads();
        if (vv >= 0) {
            int rank = s_run[vv];
            for (int wd = 0; wd < word; ++wd) rank += __popc(s_bits[vv * 8 + wd]);
            rank += __popc(s_bits[vv * 8 + word] & ((1u << bit) - 1u));
            sorted[s_off[vv] + rank] = r;
        }
        __syncthreads();
        if (w + 1 < nwin) {
            for (int e = tid; e < E; e += kBlock) {
                int add = 0;
#pragma unroll
                for (int wd = 0; wd < 8; ++wd) add += __popc(s_bits[e * 8 + wd]);
                s_run[e] += add;
            }
            __syncthreads();
        }
    }
}


// Inclusive prefix sum over the wave by DPP (row_shr 1, 2, 4, 8 inside rows
// of 16, then row_bcast15 and row_bcast31 across rows).
__device__ __forceinline__ int wave_scan_incl(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

constexpr int kSortWaveRounds = 16;
constexpr int kSortWaveRoutes = kSortWaveRounds * kWave;  // routes one wave of sort_waves4 handles
// The sorts' per-lane route arrays and their unrolled rounds are sized at
// compile time; fewer rounds make a much shorter code path, which the one
// workgroup that sorts runs once per call (4 rounds instead of 16: -4.4 us
// per step with 512 and 1024 routes), so short sorts get their own.
constexpr int kSortShortRounds = 4;
// Above this many routes four waves sort faster than one (measured with
// moe_sort back to back: 1024 routes 9.7 -> 7.0 us, 512 routes 6.5 -> 6.2 us).
constexpr int kSortOneWaveMax = 256;
constexpr int kOneWaveRounds = kSortOneWaveMax / kWave;

// LDS ints needed by sort_wave for E experts.
__host__ __device__ constexpr int sort_wave_lds_ints(int E) { return 2 * E; }

// One wave sorts R <= kSortOneWaveMax routes (same outputs as sort_block).
// Route r = 64 j + lane is handled in round j.  Within a round, the lanes
// holding the same id are found by ballots over the id bits; a route's rank
// is the number of earlier routes with its id: the running count of that id
// from earlier rounds (LDS, updated by the lowest lane of each group) plus
// the group's lanes below it.  A wave's LDS accesses complete in program
// order, so no barrier is needed.  lds: sort_wave_lds_ints(E) ints.
template <bool COHERENT>
__device__ __forceinline__ void sort_wave(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                          int32_t *uniq, int32_t *n_uniq, int32_t *stats, int *lds, int lane) {
    int *s_run = lds, *s_off = lds + E;
    const int nr = (R + kWave - 1) / kWave;
    int id[kOneWaveRounds], rk[kOneWaveRounds];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kOneWaveRounds; ++j) {
        const int r = j * kWave + lane;
        id[j] = (j < nr && r < R) ? (COHERENT ? load_shared(ids + r) : ids[r]) : -1;
        if (j < nr && r < R && (id[j] < 0 || id[j] >= E)) bad = true;
    }
    for (int e = lane; e < E; e += kWave) s_run[e] = 0;
    if (__ballot(bad)) {
        if (lane == 0) {
            *n_uniq = -1;
            if (stats) { stats[0] = -1; stats[1] = R; stats[2] = 0; stats[3] = 0; }
        }
        return;
    }
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kOneWaveRounds; ++j) {
        if (j < nr) {
            const int v = id[j];
            const bool valid = v >= 0;
            unsigned long long same = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = ((v >> b) & 1) != 0;
                const unsigned long long on = __ballot(bit);
                same &= bit ? on : ~on;
            }
            const int before = __popcll(same & below);
            const int base = valid ? s_run[v] : 0;
            rk[j] = base + before;
            if (valid && before == 0) s_run[v] = base + __popcll(same);
        }
    }
    // exclusive scans over the experts of the counts and of (count > 0); lane
    // l owns experts [l * per, l * per + per)
    const int per = (E + kWave - 1) / kWave;
    const int lo = min(E, lane * per), hi = min(E, lo + per);
    int csum = 0, usum = 0, cmax = 0;
    for (int e = lo; e < hi; ++e) {
        const int c = s_run[e];
        csum += c;
        usum += c > 0;
        cmax = max(cmax, c);
    }
    const int cinc = wave_scan_incl(csum), uinc = wave_scan_incl(usum);
    const int utot = __builtin_amdgcn_readlane(uinc, kWave - 1);
    const int mx = (int)wave_reduce_u32<true>((uint32_t)cmax);
    int cpre = cinc - csum, upre = uinc - usum;
    for (int e = lo; e < hi; ++e) {
        const int c = s_run[e];
        s_off[e] = cpre;
        offsets[e] = cpre;
        counts[e] = c;
        if (c > 0) uniq[upre++] = e;
        cpre += c;
    }
    if (lane == 0) {
        offsets[E] = R;
        *n_uniq = utot;
        if (stats) { stats[0] = utot; stats[1] = R; stats[2] = mx; stats[3] = 0; }
    }
#pragma unroll
    for (int j = 0; j < kOneWaveRounds; ++j)
        if (j < nr && id[j] >= 0) sorted[s_off[id[j]] + rk[j]] = j * kWave + lane;
}

// Four waves sort R <= 4 * ROUNDS * 64 routes: wave w ranks the routes
// of its contiguous quarter [w Q, w Q + Q) as sort_wave does (ballots over
// the id bits per round of 64, a per-wave running count per expert in LDS),
// with no barrier; then one barrier, and each expert's count is the sum of
// the four per-wave counts, whose exclusive prefix over the waves is added to
// a route's rank within its wave.  Earlier waves hold earlier routes, so the
// order is the stable one.  Same outputs as sort_block.  lds: 5 E ints.
template <int ROUNDS, bool COHERENT>
__device__ __forceinline__ void sort_waves4(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets,
                                            int32_t *sorted, int32_t *uniq, int32_t *n_uniq, int32_t *stats, int *lds,
                                            unsigned *zero, int n_zero) {
    constexpr int kW = kBlock / kWave;
    __shared__ int s_bad, s_max;
    __shared__ int s_wc[kW], s_wu[kW];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int *s_runw = lds + wave * E, *s_off = lds + kW * E;
    const int q = ((R + kW - 1) / kW + kWave - 1) / kWave * kWave;  // routes per wave, a multiple of 64
    const int r0 = wave * q, r1 = min(R, r0 + q);
    const int nr = r1 > r0 ? (r1 - r0 + kWave - 1) / kWave : 0;
    if (tid == 0) { s_bad = 0; s_max = 0; }
    for (int i = tid; i < n_zero; i += kBlock) zero[i] = 0u;
    int id[ROUNDS], rk[ROUNDS];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
        const int r = r0 + j * kWave + lane;
        id[j] = (j < nr && r < r1) ? (COHERENT ? load_shared(ids + r) : ids[r]) : -1;
        if (j < nr && r < r1 && (id[j] < 0 || id[j] >= E)) bad = true;
    }
    for (int e = lane; e < E; e += kWave) s_runw[e] = 0;
    __syncthreads();  // s_bad, s_max initialised
    if (__ballot(bad)) {
        if (lane == 0) s_bad = 1;
    } else {
        const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j) {
            if (j < nr) {
                const int v = id[j];
                const bool valid = v >= 0;
                unsigned long long same = __ballot(valid);
                for (int b = 0; b < nbits; ++b) {
                    const bool bit = ((v >> b) & 1) != 0;
                    const unsigned long long on = __ballot(bit);
                    same &= bit ? on : ~on;
                }
                const int before = __popcll(same & below);
                const int base = valid ? s_runw[v] : 0;
                rk[j] = base + before;
                if (valid && before == 0) s_runw[v] = base + __popcll(same);
            }
        }
    }
    __syncthreads();
    if (s_bad) {
        if (tid == 0) {
            *n_uniq = -1;
            if (stats) { stats[0] = -1; stats[1] = R; stats[2] = 0; stats[3] = 0; }
        }
        return;
    }
    // per expert: the count is the sum over the waves; the waves' counts
    // become their exclusive prefixes; then exclusive scans over the experts
    // of the counts and of (count > 0).  Thread tid owns experts [lo, hi).
    const int per = (E + kBlock - 1) / kBlock;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int csum = 0, usum = 0, cmax = 0;
    for (int e = lo; e < hi; ++e) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            const int cw = lds[w * E + e];
            lds[w * E + e] = c;
            c += cw;
        }
        s_off[e] = c;  // the count, for now
        csum += c;
        usum += c > 0;
        cmax = max(cmax, c);
    }
    int cinc = csum, uinc = usum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int oc = __shfl_up(cinc, d, kWave), ou = __shfl_up(uinc, d, kWave);
        if (lane >= d) { cinc += oc; uinc += ou; }
    }
    if (lane == kWave - 1) { s_wc[wave] = cinc; s_wu[wave] = uinc; }
    atomicMax(&s_max, cmax);
    __syncthreads();
    int cpre = cinc - csum, upre = uinc - usum, utot = 0;
    for (int wv = 0; wv < kW; ++wv) {
        if (wv < wave) { cpre += s_wc[wv]; upre += s_wu[wv]; }
        utot += s_wu[wv];
    }
    for (int e = lo; e < hi; ++e) {
        const int c = s_off[e];
        s_off[e] = cpre;
        offsets[e] = cpre;
        counts[e] = c;
        if (c > 0) uniq[upre++] = e;
        cpre += c;
    }
    if (tid == 0) {
        offsets[E] = R;
        *n_uniq = utot;
        if (stats) { stats[0] = utot; stats[1] = R; stats[2] = s_max; stats[3] = 0; }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j)
        if (j < nr && id[j] >= 0) sorted[s_off[id[j]] + s_runw[id[j]] + rk[j]] = r0 + j * kWave + lane;
}



// LDS ints needed by sort_routes for E experts and R routes (callers reserve
// sort_lds_ints(E), the largest of the three).
__host__ __device__ constexpr int sort_routes_lds_ints(int E, int R) {
    return R <= kSortOneWaveMax ? sort_wave_lds_ints(E)
           : R <= (kBlock / kWave) * kSortWaveRoutes ? (kBlock / kWave + 1) * E
                                                    : sort_lds_ints(E);
}
static_assert(sort_routes_lds_ints(1, kSortOneWaveMax) <= sort_lds_ints(1) &&
                  sort_routes_lds_ints(1, kSortWaveRoutes) <= sort_lds_ints(1),
              "sort_lds_ints(E) covers every sort variant");

// Sort by one workgroup (every thread calls this): one wave up to
// kSortOneWaveMax routes, four waves up to 4 kSortWaveRoutes, the whole
// workgroup's windows otherwise.
// Also zeroes n_zero words at zero.
template <bool COHERENT>
__device__ __forceinline__ void sort_routes(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                            int32_t *uniq, int32_t *n_uniq, int32_t *stats, int *lds, unsigned *zero, int n_zero) {
    if (R > kSortOneWaveMax && R <= (kBlock / kWave) * kSortShortRounds * kWave) {
        sort_waves4<kSortShortRounds, COHERENT>(ids, R, E, counts, offsets, sorted, uniq, n_uniq, stats, lds, zero,
                                                n_zero);
        return;
    }
    if (R > kSortOneWaveMax && R <= (kBlock / kWave) * kSortWaveRoutes) {
        sort_waves4<kSortWaveRounds, COHERENT>(ids, R, E, counts, offsets, sorted, uniq, n_uniq, stats, lds, zero,
                                               n_zero);
        return;
    }
    if (R > kSortWaveRoutes) {
        sort_block<COHERENT>(ids, R, E, counts, offsets, sorted, uniq, n_uniq, stats, lds, zero, n_zero);
        return;
    }
    const int tid = threadIdx.x;
    if (tid < kWave) {
        sort_wave<COHERENT>(ids, R, E, counts, offsets, sorted, uniq, n_uniq, stats, lds, tid);
    } else {
        for (int i = tid - kWave; i < n_zero; i += kBlock - kWave) zero[i] = 0u;
    }
}

}  // namespace moe
