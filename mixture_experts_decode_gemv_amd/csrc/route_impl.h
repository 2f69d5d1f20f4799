// Device pieces of routing: exact top-k selection of one token by one wave,
// and the stable counting sort of the routes by one workgroup.
//
// Selection ("MoE Performance Optimization Analysis", GPU Router Design:
// router compute, argmax and selection on the device).  The k largest logits
// by (logit descending, expert index ascending), one wave per token: logits
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
// and step).  Histogram with LDS integer atomics, exclusive scans for the
// offsets and the unique-expert list, then a stable scatter in windows of 256
// routes: each window sets one bit per route in a per-expert bitmask, and a
// route's rank inside its expert is the expert's count in earlier windows
// plus the bits below its own.
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

// This lane's best untaken (key, index) over its logits e = lane + 64c;
// key 0 means none.  Strictly greater wins, so the lowest c (lowest index)
// keeps a tie.
__device__ __forceinline__ void lane_best(const uint32_t (&key)[kSelPerLane], uint32_t taken, int nc, int E, int lane,
                                          uint32_t &kb, uint32_t &ib) {
    kb = 0u;
    ib = 0xFFFFFFFFu;
#pragma unroll
    for (int c = 0; c < kSelPerLane; ++c) {
        if (c < nc && lane + kWave * c < E && !((taken >> c) & 1u) && key[c] > kb) {
            kb = key[c];
            ib = (uint32_t)(lane + kWave * c);
        }
    }
}

// One wave selects for one token.  l: the token's E logits (COHERENT: written
// by other workgroups of this launch).  Writes ids[0..k) and w[0..k) with
// device-scope stores.
template <bool COHERENT>
__device__ void select_token(const float *l, int E, int k, int32_t *ids, float *w, int lane) {
    uint32_t key[kSelPerLane];
    const int nc = (E + kWave - 1) / kWave;
#pragma unroll
    for (int c = 0; c < kSelPerLane; ++c) {
        const int e = lane + kWave * c;
        float v = 0.f;
        if (c < nc && e < E) v = COHERENT ? load_shared(l + e) : l[e];
        key[c] = logit_key(v);
    }
    uint32_t taken = 0u, kb, ib;
    lane_best(key, taken, nc, E, lane, kb, ib);
    uint32_t my_key = 0u, my_idx = 0u, top = 0u;
    for (int j = 0; j < k; ++j) {
        const uint32_t m = wave_reduce_u32<true>(kb);
        const uint32_t idx = wave_reduce_u32<false>(kb == m ? ib : 0xFFFFFFFFu);
        if (j == 0) top = m;
        if (lane == j) { my_key = m; my_idx = idx; }
        if ((int)(idx & (kWave - 1)) == lane) {
            taken |= 1u << (idx / kWave);
            lane_best(key, taken, nc, E, lane, kb, ib);
        }
    }
    const float p = lane < k ? expf(key_logit(my_key) - key_logit(top)) : 0.f;
    const float sum = wave_sum(p);
    if (lane < k) {
        store_shared(ids + lane, (int32_t)my_idx);
        store_shared(w + lane, p / sum);
    }
}

// LDS ints needed by sort_block for E experts.
__host__ __device__ constexpr int sort_lds_ints(int E) { return 11 * E; }

// One workgroup sorts R routes.  ids COHERENT: written by other workgroups
// of this launch.  lds: sort_lds_ints(E) ints.
template <bool COHERENT>
__device__ void sort_block(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *sorted,
                           int32_t *uniq, int32_t *n_uniq, int32_t *stats, int *lds) {
    __shared__ int s_tmp[kBlock / kWave];
    __shared__ int s_bad, s_max;
    int *s_cnt = lds, *s_off = lds + E, *s_run = lds + 2 * E;
    unsigned *s_bits = reinterpret_cast<unsigned *>(lds + 3 * E);  // [E][8]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    for (int e = tid; e < E; e += kBlock) {
        s_cnt[e] = 0;
        s_run[e] = 0;
    }
    if (tid == 0) { s_bad = 0; s_max = 0; }
    __syncthreads();
    for (int r = tid; r < R; r += kBlock) {
        const int v = COHERENT ? load_shared(ids + r) : ids[r];
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
    __shared__ int s_wc[kBlock / kWave], s_wu[kBlock / kWave];
    if (lane == kWave - 1) { s_wc[wave] = cinc; s_wu[wave] = uinc; }
    atomicMax(&s_max, cmax);
    __syncthreads();
    int cpre = cinc - csum, upre = uinc - usum, utot = 0;
    for (int wv = 0; wv < kBlock / kWave; ++wv) {
        if (wv < wave) { cpre += s_wc[wv]; upre += s_wu[wv]; }
        utot += s_wu[wv];
    }
    (void)s_tmp;
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
    __syncthreads();
    // stable scatter, 256 routes per window
    for (int base = 0; base < R; base += kBlock) {
        for (int i = tid; i < E * 8; i += kBlock) s_bits[i] = 0u;
        __syncthreads();
        const int r = base + tid;
        const int v = r < R ? (COHERENT ? load_shared(ids + r) : ids[r]) : -1;
        const int word = tid >> 5, bit = tid & 31;
        if (v >= 0) atomicOr(&s_bits[v * 8 + word], 1u << bit);
        __syncthreads();
        if (v >= 0) {
            int rank = s_run[v];
            for (int wd = 0; wd < word; ++wd) rank += __popc(s_bits[v * 8 + wd]);
            rank += __popc(s_bits[v * 8 + word] & ((1u << bit) - 1u));
            sorted[s_off[v] + rank] = r;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kBlock) {
            int add = 0;
#pragma unroll
            for (int wd = 0; wd < 8; ++wd) add += __popc(s_bits[e * 8 + wd]);
            s_run[e] += add;
        }
        __syncthreads();
    }
}

}  // namespace moe
