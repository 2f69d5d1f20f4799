// C ABI of the gfx950 MoE decode library: host-side validation, workspace
// carving and the launch sequence.  Nothing here allocates, synchronises or
// reads device memory back; every call only enqueues work on the caller's
// stream, so a stack of layers can be recorded into one HIP graph
// ("TEXT Generation Optimization Report", Phase 1: one submission and one
// wait per forward; "MoE Performance Optimization Analysis", Option 1: no
// host read between router and experts).
#include <stdint.h>

#include <mutex>

#include "common.h"

// ---- scratch of the allocation-free entry point -----------------------------
// Device memory the library holds for moe_layer_fwd_static: each GPU the
// library runs on has its own copy, for as long as the process runs.  In host
// code this name is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress (static_scratch below), and only that address is
// ever passed to a kernel or a fill.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace moe {

int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev >= 64) dev = 63;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static moe_status check_layer(const moe_layer_t *L) {
    if (!L) return MOE_ERR_ARG;
    if (L->E < 1 || L->top_k < 1 || L->top_k > L->E || L->H < 1 || L->I < 1) return MOE_ERR_ARG;
    if (L->E > kMaxE || L->top_k > kMaxK) return MOE_ERR_SHAPE;
    if (L->router_dtype != MOE_F32 && L->router_dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (L->expert_dtype != MOE_F32 && L->expert_dtype != MOE_BF16 && L->expert_dtype != MOE_FP8_E4M3 &&
        L->expert_dtype != MOE_MXFP4 && L->expert_dtype != MOE_Q4_0)
        return MOE_ERR_DTYPE;
    const int epc = elems_per_chunk(L->expert_dtype), repc = elems_per_chunk(L->router_dtype);
    if (L->H % epc || L->I % epc || L->H % repc || L->H % 4 || L->I % 4) return MOE_ERR_SHAPE;
    if (L->expert_dtype == MOE_FP8_E4M3 && (L->H % 128 || L->I % 128)) return MOE_ERR_SHAPE;
    const int mc = max_chunks_per_lane(L->expert_dtype);
    if (L->H / epc > kWave * mc || L->I / epc > kWave * mc || L->H / repc > kWave * kMaxChunksPerLane)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

static moe_status check_weights(const moe_layer_t *L, bool router, bool experts) {
    if (router && !L->w_router) return MOE_ERR_ARG;
    if (router && !aligned16(L->w_router)) return MOE_ERR_ALIGN;
    if (experts) {
        if (!L->w_gate_up || !L->w_down) return MOE_ERR_ARG;
        if (!aligned16(L->w_gate_up) || !aligned16(L->w_down)) return MOE_ERR_ALIGN;
        if ((L->expert_dtype == MOE_FP8_E4M3 || L->expert_dtype == MOE_MXFP4 || L->expert_dtype == MOE_Q4_0) &&
            (!L->s_gate_up || !L->s_down))
            return MOE_ERR_ARG;
        // q4_0 scales are read as 2-byte words
        if (L->expert_dtype == MOE_Q4_0 &&
            (((uintptr_t)L->s_gate_up & 1u) != 0 || ((uintptr_t)L->s_down & 1u) != 0))
            return MOE_ERR_ALIGN;
    }
    return MOE_OK;
}

static moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// A layer workspace for T tokens: present, large enough and aligned.
static moe_status check_ws(const moe_layer_t &L, int32_t T, const void *ws, size_t ws_bytes) {
    if (T > kMaxTokens) return MOE_ERR_SHAPE;
    if (!ws || ws_bytes < ws_bytes_for(L, T)) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens) {
    if (check_layer(layer) != MOE_OK || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
    return ws_bytes_for(*layer, max_tokens);
}

moe_status moe_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                              void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (max_tokens < 0 || !ws) return MOE_ERR_ARG;
    if ((s = check_ws(*layer, max_tokens, ws, ws_bytes)) != MOE_OK) return s;
    // the statistics and synchronisation words: the fixed front
    return hip_status(launch_zero(static_cast<unsigned *>(ws), (int)(kWsFrontBytes / 4), (hipStream_t)stream));
}

moe_status moe_route(const moe_layer_t *layer, const float *x, const float *logits_in, int32_t T,
                     float *logits_out, int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                     void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (T < 0 || !topk_ids || !topk_w || (!x && !logits_in)) return MOE_ERR_ARG;
    if (T == 0) return MOE_OK;
    hipStream_t st = (hipStream_t)stream;
    if (logits_in) {
        if (logits_out && logits_out != logits_in &&
            hipMemcpyAsync(logits_out, logits_in, (size_t)T * layer->E * 4, hipMemcpyDeviceToDevice, st) !=
                hipSuccess)
            return MOE_ERR_HIP;
        return hip_status(launch_route(*layer, nullptr, logits_in, T, nullptr, nullptr, topk_ids, topk_w, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false, nullptr, 0, st));
    }
    if ((s = check_weights(layer, true, false)) != MOE_OK) return s;
    if (!aligned16(x)) return MOE_ERR_ALIGN;
    if ((s = check_ws(*layer, T, ws, ws_bytes)) != MOE_OK) return s;
    const WsLayout wl = ws_layout(*layer, T);
    char *b = static_cast<char *>(ws);
    float *dst = logits_out ? logits_out : reinterpret_cast<float *>(b + wl.logits);
    return hip_status(launch_route(*layer, x, nullptr, T, nullptr, dst, topk_ids, topk_w, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, reinterpret_cast<unsigned *>(b + wl.arrive), false,
                                   nullptr, 0, st));
}

int32_t moe_mfma_min_routes(const moe_layer_t *layer, int32_t T, uint32_t flags) {
    if (check_layer(layer) != MOE_OK || T < 0 || (flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return -1;
    return mfma_min_routes(*layer, T, flags);
}

int32_t moe_mfma_hot_routes(const moe_layer_t *layer, int32_t T, uint32_t flags) {
    if (check_layer(layer) != MOE_OK || T < 0 || (flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return -1;
    return mfma_hot_routes(*layer, T, flags);
}

moe_status moe_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t *counts, int32_t *offsets,
                    int32_t *sorted_routes, int32_t *uniq, int32_t *n_uniq, void *stream) {
    if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_ARG;
    if (E > kMaxE || k > kMaxK) return MOE_ERR_SHAPE;
    if (!topk_ids || !counts || !offsets || !sorted_routes || !uniq || !n_uniq) return MOE_ERR_ARG;
    if ((int64_t)T * k > INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    return hip_status(launch_sort(topk_ids, T * k, E, counts, offsets, sorted_routes, uniq, n_uniq,
                                  (hipStream_t)stream));
}

moe_status moe_expert_fwd(const moe_layer_t *layer, const float *x, int32_t T, const int32_t *topk_ids,
                          const float *topk_w, const int32_t *counts, const int32_t *offsets,
                          const int32_t *sorted_routes, const int32_t *uniq, const int32_t *n_uniq, float *out,
                          uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if ((s = check_weights(layer, false, true)) != MOE_OK) return s;
    if (T < 0 || !x || !topk_ids || !topk_w || !counts || !offsets || !sorted_routes || !uniq || !n_uniq || !out)
        return MOE_ERR_ARG;
    if ((flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if ((s = check_ws(*layer, T, ws, ws_bytes)) != MOE_OK) return s;
    const WsLayout wl = ws_layout(*layer, T);
    char *b = static_cast<char *>(ws);
    Routing rt{topk_ids, counts, offsets, sorted_routes, uniq, n_uniq, topk_w, nullptr, n_uniq};
    return hip_status(launch_experts(*layer, x, (flags & MOE_ACCUM_RESIDUAL) ? x : nullptr, T, rt, b + wl.xb,
                                     reinterpret_cast<float *>(b + wl.act), reinterpret_cast<float *>(b + wl.y), out,
                                     flags, (hipStream_t)stream));
}

static moe_status layer_fwd(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                            void *ws, size_t ws_bytes, void *stream, const hipEvent_t *ev, bool may_fork = true) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if ((s = check_weights(layer, true, true)) != MOE_OK) return s;
    if (T < 0 || !x || !out) return MOE_ERR_ARG;
    if ((flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if ((s = check_ws(*layer, T, ws, ws_bytes)) != MOE_OK) return s;
    const WsLayout wl = ws_layout(*layer, T);
    hipStream_t st = (hipStream_t)stream;
    char *b = static_cast<char *>(ws);
    auto F = [&](size_t o) { return reinterpret_cast<float *>(b + o); };
    auto I32 = [&](size_t o) { return reinterpret_cast<int32_t *>(b + o); };

    const bool norm = (flags & MOE_RMSNORM_IN) != 0;
    const float *xin = norm ? F(wl.xn) : x;
    if (ev && (s = hip_status(hipEventRecord(ev[0], st))) != MOE_OK) return s;
    // the routing launch also writes the bf16 copy of x when segments may
    // take the MFMA path
    const bool xb = mfma_min_routes(*layer, T, flags) > 0;
    if ((s = hip_status(launch_route(*layer, x, nullptr, T, norm ? F(wl.xn) : nullptr, F(wl.logits), I32(wl.ids),
                                     F(wl.w), I32(wl.counts), I32(wl.offsets), I32(wl.sorted), I32(wl.uniq),
                                     I32(wl.nuniq), I32(wl.stats), reinterpret_cast<unsigned *>(b + wl.arrive), norm,
                                     nullptr, 0, st, nullptr,
                                     xb ? reinterpret_cast<uint32_t *>(b + wl.xb) : nullptr))) != MOE_OK)
        return s;
    if (ev && (s = hip_status(hipEventRecord(ev[1], st))) != MOE_OK) return s;
    Routing rt{I32(wl.ids),  I32(wl.counts), I32(wl.offsets), I32(wl.sorted),
               I32(wl.uniq), I32(wl.nuniq),  F(wl.w),         I32(wl.stats) + 2, nullptr, xb};
    return hip_status(launch_experts(*layer, xin, (flags & MOE_ACCUM_RESIDUAL) ? x : nullptr, T, rt, b + wl.xb,
                                     F(wl.act), F(wl.y), out, flags, st, ev ? ev + 2 : nullptr, may_fork));
}

moe_status moe_layer_fwd(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags, void *ws,
                         size_t ws_bytes, void *stream) {
    return layer_fwd(layer, x, T, out, flags, ws, ws_bytes, stream, nullptr);
}

// The device address of this GPU's scratch array, looked up on the first
// call on the device (with the device current), when its synchronisation
// front is also cleared by a fill kernel on `st`; kept per device after that.
static moe_status static_scratch(hipStream_t st, void **out) {
    static std::mutex mu;
    static void *ptr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        if (launch_zero(static_cast<unsigned *>(p), (int)(kWsFrontBytes / 4), st) != hipSuccess) return MOE_ERR_HIP;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return MOE_OK;
}

moe_status moe_layer_fwd_static(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                                void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if ((s = check_weights(layer, true, true)) != MOE_OK) return s;
    if (T < 0 || !x || !out) return MOE_ERR_ARG;
    if ((flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if (T > kMaxTokens) return MOE_ERR_SHAPE;
    if (ws_bytes_for(*layer, T) > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((s = static_scratch((hipStream_t)stream, &ws)) != MOE_OK) return s;
    return layer_fwd(layer, x, T, out, flags, ws, MOE_STATIC_SCRATCH_BYTES, stream, nullptr, false);
}

moe_status moe_layer_fwd_events(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream, void *const *events) {
    if (events)
        for (int i = 0; i <= MOE_N_STAGES; ++i)
            if (!events[i]) return MOE_ERR_ARG;
    return layer_fwd(layer, x, T, out, flags, ws, ws_bytes, stream, reinterpret_cast<const hipEvent_t *>(events));
}

moe_status moe_layer_routing(const moe_layer_t *layer, int32_t T, void *ws, size_t ws_bytes, int32_t **topk_ids,
                             float **topk_w, int32_t **counts, int32_t **offsets, int32_t **sorted_routes,
                             int32_t **uniq, int32_t **n_uniq) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (T < 0 || !ws) return MOE_ERR_ARG;
    if ((s = check_ws(*layer, T, ws, ws_bytes)) != MOE_OK) return s;
    const WsLayout wl = ws_layout(*layer, T);
    char *b = static_cast<char *>(ws);
    if (topk_ids) *topk_ids = reinterpret_cast<int32_t *>(b + wl.ids);
    if (topk_w) *topk_w = reinterpret_cast<float *>(b + wl.w);
    if (counts) *counts = reinterpret_cast<int32_t *>(b + wl.counts);
    if (offsets) *offsets = reinterpret_cast<int32_t *>(b + wl.offsets);
    if (sorted_routes) *sorted_routes = reinterpret_cast<int32_t *>(b + wl.sorted);
    if (uniq) *uniq = reinterpret_cast<int32_t *>(b + wl.uniq);
    if (n_uniq) *n_uniq = reinterpret_cast<int32_t *>(b + wl.nuniq);
    return MOE_OK;
}

// ---- layer stack ----------------------------------------------------------------
// A stack's workspace: the fixed fronts of two layer workspaces, then their
// data arrays (layers alternate between them, so layer l + 1's routing launch
// can read layer l's y and weights while writing its own routing), then two
// residual buffers [T, H] fp32.  Only the fronts must stay in place from call
// to call; the rest is laid out for each call's batch.

struct StackLayout {
    WsLayout half[2];
    size_t h[2], total;
};

static StackLayout stack_layout(const moe_layer_t &L, int64_t T) {
    StackLayout sl;
    const size_t data = align256(ws_data_bytes(L, T)), hb = align256((size_t)T * L.H * 4);
    for (int i = 0; i < 2; ++i) sl.half[i] = ws_layout_at(L, T, i * kWsFrontBytes, 2 * kWsFrontBytes + i * data);
    sl.h[0] = 2 * kWsFrontBytes + 2 * data;
    sl.h[1] = sl.h[0] + hb;
    sl.total = sl.h[1] + hb;
    return sl;
}

size_t moe_stack_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens) {
    if (check_layer(layer) != MOE_OK || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
    return stack_layout(*layer, max_tokens).total;
}

static moe_status check_stack_ws(const moe_layer_t &L, int32_t T, const void *ws, size_t ws_bytes) {
    if (T > kMaxTokens) return MOE_ERR_SHAPE;
    if (!ws || ws_bytes < stack_layout(L, T).total) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status moe_stack_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                                    void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (max_tokens < 0 || !ws) return MOE_ERR_ARG;
    if ((s = check_stack_ws(*layer, max_tokens, ws, ws_bytes)) != MOE_OK) return s;
    return hip_status(launch_zero(static_cast<unsigned *>(ws), (int)(2 * kWsFrontBytes / 4), (hipStream_t)stream));
}

moe_status moe_stack_fwd(const moe_layer_t *layers, int32_t n_layers, const float *x, int32_t T, float *out,
                         uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
    if (!layers || n_layers < 1) return MOE_ERR_ARG;
    moe_status s;
    const moe_layer_t &L0 = layers[0];
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer_t &L = layers[l];
        if ((s = check_layer(&L)) != MOE_OK) return s;
        if ((s = check_weights(&L, true, true)) != MOE_OK) return s;
        if (L.E != L0.E || L.top_k != L0.top_k || L.H != L0.H || L.I != L0.I || L.router_dtype != L0.router_dtype ||
            L.expert_dtype != L0.expert_dtype)
            return MOE_ERR_SHAPE;
    }
    if (T < 0 || !x || !out) return MOE_ERR_ARG;
    if ((flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if ((s = check_stack_ws(L0, T, ws, ws_bytes)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const StackLayout sl = stack_layout(L0, T);
    char *b = static_cast<char *>(ws);
    float *hbuf[2] = {reinterpret_cast<float *>(b + sl.h[0]), reinterpret_cast<float *>(b + sl.h[1])};
    auto F = [](char *p, size_t o) { return reinterpret_cast<float *>(p + o); };
    auto I32 = [](char *p, size_t o) { return reinterpret_cast<int32_t *>(p + o); };
    const uint32_t lf = (flags & (MOE_WALK_MASK | MOE_NO_MFMA)) | MOE_RMSNORM_IN | MOE_ACCUM_RESIDUAL;

    // Small batches: every layer writes its output rows itself (pass 2 and
    // the combine in one launch).  Otherwise each layer's combine runs in the
    // next layer's routing launch and only the last layer launches one.
    const bool direct = fused_combine(L0, T);
    const float *h = x;  // the current layer's input, the residual of its combine
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer_t &L = layers[l];
        const WsLayout &wl = sl.half[l & 1];
        const bool last = l == n_layers - 1;
        PrevCombine pc{};
        if (l > 0 && !direct) {
            const WsLayout &pl = sl.half[(l - 1) & 1];
            pc = PrevCombine{F(b, pl.y), F(b, pl.w), h, hbuf[l & 1], L.top_k};
            h = hbuf[l & 1];
        }
        const bool xb = mfma_min_routes(L, T, lf) > 0;
        if ((s = hip_status(launch_route(L, h, nullptr, T, F(b, wl.xn), F(b, wl.logits), I32(b, wl.ids),
                                         F(b, wl.w), I32(b, wl.counts), I32(b, wl.offsets), I32(b, wl.sorted),
                                         I32(b, wl.uniq), I32(b, wl.nuniq), I32(b, wl.stats),
                                         reinterpret_cast<unsigned *>(b + wl.arrive), true, nullptr, 0, st,
                                         l > 0 && !direct ? &pc : nullptr,
                                         xb ? reinterpret_cast<uint32_t *>(b + wl.xb) : nullptr))) != MOE_OK)
            return s;
        Routing rt{I32(b, wl.ids),  I32(b, wl.counts), I32(b, wl.offsets), I32(b, wl.sorted),
                   I32(b, wl.uniq), I32(b, wl.nuniq),  F(b, wl.w),         I32(b, wl.stats) + 2, nullptr, xb};
        float *dst = last ? out : direct ? hbuf[l & 1] : nullptr;
        if ((s = hip_status(launch_experts(L, F(b, wl.xn), h, T, rt, b + wl.xb, F(b, wl.act), F(b, wl.y), dst, lf,
                                           st))) != MOE_OK)
            return s;
        if (direct) h = dst;
    }
    return MOE_OK;
}

moe_status moe_expert_usage(const int32_t *counts, const int32_t *n_uniq, int32_t E, uint64_t *hist,
                            void *stream) {
    if (!counts || !n_uniq || !hist) return MOE_ERR_ARG;
    if (E < 1) return MOE_ERR_ARG;
    if (E > kMaxE) return MOE_ERR_SHAPE;
    if (((uintptr_t)hist & 7u) != 0) return MOE_ERR_ALIGN;
    return hip_status(launch_usage(counts, n_uniq, E, reinterpret_cast<unsigned long long *>(hist),
                                   (hipStream_t)stream));
}

const char *moe_status_str(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_SHAPE: return "unsupported or inconsistent shape";
        case MOE_ERR_DTYPE: return "unsupported dtype";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch error";
        case MOE_ERR_UNSUPPORTED: return "not supported by this library";
        case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    }
    return "unknown status";
}

}  // extern "C"
