// C ABI of the gfx950 MoE decode library: host-side validation, workspace
// carving and the launch sequence.  Nothing here allocates, synchronises or
// reads device memory back; every call only enqueues work on the caller's
// stream, so a stack of layers can be recorded into one HIP graph
// ("TEXT Generation Optimization Report", Phase 1: one submission and one
// wait per forward; "MoE Performance Optimization Analysis", Option 1: no
// host read between router and experts).
#include <stdint.h>

#include "common.h"

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
        L->expert_dtype != MOE_MXFP4)
        return MOE_ERR_DTYPE;
    const int epc = elems_per_chunk(L->expert_dtype), repc = elems_per_chunk(L->router_dtype);
    if (L->H % epc || L->I % epc || L->H % repc || L->H % 4 || L->I % 4) return MOE_ERR_SHAPE;
    if (L->expert_dtype == MOE_FP8_E4M3 && (L->H % 128 || L->I % 128)) return MOE_ERR_SHAPE;
    if (L->H / epc > kWave * kMaxChunksPerLane || L->I / epc > kWave * kMaxChunksPerLane ||
        L->H / repc > kWave * kMaxChunksPerLane)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

static moe_status check_weights(const moe_layer_t *L, bool router, bool experts) {
    if (router && !L->w_router) return MOE_ERR_ARG;
    if (router && !aligned16(L->w_router)) return MOE_ERR_ALIGN;
    if (experts) {
        if (!L->w_gate_up || !L->w_down) return MOE_ERR_ARG;
        if (!aligned16(L->w_gate_up) || !aligned16(L->w_down)) return MOE_ERR_ALIGN;
        if ((L->expert_dtype == MOE_FP8_E4M3 || L->expert_dtype == MOE_MXFP4) && (!L->s_gate_up || !L->s_down))
            return MOE_ERR_ARG;
    }
    return MOE_OK;
}

static moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens) {
    if (check_layer(layer) != MOE_OK || max_tokens < 0) return 0;
    return ws_bytes_for(*layer, max_tokens);
}

moe_status moe_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                              void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (max_tokens < 0 || !ws) return MOE_ERR_ARG;
    const int64_t cap = ws_capacity(*layer, ws_bytes);
    if (cap < max_tokens) return MOE_ERR_WORKSPACE;
    const WsLayout wl = ws_layout(*layer, cap, cap);
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    // stats and synchronisation words sit at the front of the workspace
    return hip_status(launch_zero(static_cast<unsigned *>(ws), (int)(wl.logits / 4), (hipStream_t)stream));
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
    const int64_t cap = ws ? ws_capacity(*layer, ws_bytes) : -1;
    if (cap < T) return MOE_ERR_WORKSPACE;
    const WsLayout wl = ws_layout(*layer, T, cap);
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    char *b = static_cast<char *>(ws);
    float *dst = logits_out ? logits_out : reinterpret_cast<float *>(b + wl.logits);
    return hip_status(launch_route(*layer, x, nullptr, T, nullptr, dst, topk_ids, topk_w, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, reinterpret_cast<unsigned *>(b + wl.arrive), false,
                                   nullptr, 0, st));
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
    const int64_t cap = ws ? ws_capacity(*layer, ws_bytes) : -1;
    if (cap < T) return MOE_ERR_WORKSPACE;
    const WsLayout wl = ws_layout(*layer, T, cap);
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    char *b = static_cast<char *>(ws);
    Routing rt{topk_ids, counts, offsets, sorted_routes, uniq, n_uniq, topk_w, nullptr};
    return hip_status(launch_experts(*layer, x, (flags & MOE_ACCUM_RESIDUAL) ? x : nullptr, T, rt, b + wl.xb,
                                     reinterpret_cast<float *>(b + wl.act), reinterpret_cast<float *>(b + wl.y), out,
                                     flags, (hipStream_t)stream));
}

static moe_status layer_fwd(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                            void *ws, size_t ws_bytes, void *stream, const hipEvent_t *ev) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if ((s = check_weights(layer, true, true)) != MOE_OK) return s;
    if (T < 0 || !x || !out) return MOE_ERR_ARG;
    if ((flags & MOE_WALK_MASK) > MOE_WALK_DEDUP_PASS1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    const int64_t cap = ws ? ws_capacity(*layer, ws_bytes) : -1;
    if (cap < T) return MOE_ERR_WORKSPACE;
    const WsLayout wl = ws_layout(*layer, T, cap);
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    char *b = static_cast<char *>(ws);
    auto F = [&](size_t o) { return reinterpret_cast<float *>(b + o); };
    auto I32 = [&](size_t o) { return reinterpret_cast<int32_t *>(b + o); };

    const bool norm = (flags & MOE_RMSNORM_IN) != 0;
    const float *xin = norm ? F(wl.xn) : x;
    if (ev && (s = hip_status(hipEventRecord(ev[0], st))) != MOE_OK) return s;
    if ((s = hip_status(launch_route(*layer, x, nullptr, T, norm ? F(wl.xn) : nullptr, F(wl.logits), I32(wl.ids),
                                     F(wl.w), I32(wl.counts), I32(wl.offsets), I32(wl.sorted), I32(wl.uniq),
                                     I32(wl.nuniq), I32(wl.stats), reinterpret_cast<unsigned *>(b + wl.arrive), norm,
                                     nullptr, 0, st))) != MOE_OK)
        return s;
    if (ev && (s = hip_status(hipEventRecord(ev[1], st))) != MOE_OK) return s;
    Routing rt{I32(wl.ids),  I32(wl.counts), I32(wl.offsets), I32(wl.sorted),
               I32(wl.uniq), I32(wl.nuniq),  F(wl.w),         I32(wl.stats) + 2};
    return hip_status(launch_experts(*layer, xin, (flags & MOE_ACCUM_RESIDUAL) ? x : nullptr, T, rt, b + wl.xb,
                                     F(wl.act), F(wl.y), out, flags, st, ev ? ev + 2 : nullptr));
}

moe_status moe_layer_fwd(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags, void *ws,
                         size_t ws_bytes, void *stream) {
    return layer_fwd(layer, x, T, out, flags, ws, ws_bytes, stream, nullptr);
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
    const int64_t cap = ws_capacity(*layer, ws_bytes);
    if (cap < T) return MOE_ERR_WORKSPACE;
    const WsLayout wl = ws_layout(*layer, T, cap);
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
// A stack's workspace: two layer workspaces (layers alternate between them,
// so layer l + 1's routing launch can read layer l's y and weights while
// writing its own routing), then two residual buffers [cap, H] fp32; all laid
// out for the capacity cap, the largest batch ws_bytes holds.

static size_t stack_bytes_for(const moe_layer_t &L, int64_t T) {
    return 2 * align256(ws_bytes_for(L, T)) + 2 * align256((size_t)T * L.H * 4);
}

static int64_t stack_capacity(const moe_layer_t &L, size_t bytes) {
    if (bytes < stack_bytes_for(L, 0)) return -1;
    int64_t lo = 0, hi = 1;
    while (hi < (int64_t)1 << 30 && stack_bytes_for(L, hi) <= bytes) {
        lo = hi;
        hi *= 2;
    }
    while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (stack_bytes_for(L, mid) <= bytes) lo = mid;
        else hi = mid;
    }
    return lo;
}

size_t moe_stack_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens) {
    if (check_layer(layer) != MOE_OK || max_tokens < 0) return 0;
    return stack_bytes_for(*layer, max_tokens);
}

moe_status moe_stack_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                                    void *stream) {
    moe_status s = check_layer(layer);
    if (s != MOE_OK) return s;
    if (max_tokens < 0 || !ws) return MOE_ERR_ARG;
    const int64_t cap = stack_capacity(*layer, ws_bytes);
    if (cap < max_tokens) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    const WsLayout wl = ws_layout(*layer, cap, cap);
    const size_t half = align256(ws_bytes_for(*layer, cap));
    for (int i = 0; i < 2; ++i)
        if ((s = hip_status(launch_zero(reinterpret_cast<unsigned *>(static_cast<char *>(ws) + i * half),
                                        (int)(wl.logits / 4), (hipStream_t)stream))) != MOE_OK)
            return s;
    return MOE_OK;
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
    const int64_t cap = ws ? stack_capacity(L0, ws_bytes) : -1;
    if (cap < T) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    const WsLayout wl = ws_layout(L0, T, cap);
    const size_t half = align256(ws_bytes_for(L0, cap)), hb = align256((size_t)cap * L0.H * 4);
    char *b = static_cast<char *>(ws);
    char *wsl[2] = {b, b + half};
    float *hbuf[2] = {reinterpret_cast<float *>(b + 2 * half), reinterpret_cast<float *>(b + 2 * half + hb)};
    auto F = [](char *p, size_t o) { return reinterpret_cast<float *>(p + o); };
    auto I32 = [](char *p, size_t o) { return reinterpret_cast<int32_t *>(p + o); };
    const uint32_t lf = (flags & (MOE_WALK_MASK | MOE_NO_MFMA)) | MOE_RMSNORM_IN | MOE_ACCUM_RESIDUAL;

    const float *h = x;  // the current layer's input, the residual of its combine
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer_t &L = layers[l];
        char *wb = wsl[l & 1];
        PrevCombine pc{};
        if (l > 0) {
            char *pb = wsl[(l - 1) & 1];
            pc = PrevCombine{F(pb, wl.y), F(pb, wl.w), h, hbuf[l & 1], L.top_k};
            h = hbuf[l & 1];
        }
        if ((s = hip_status(launch_route(L, h, nullptr, T, F(wb, wl.xn), F(wb, wl.logits), I32(wb, wl.ids),
                                         F(wb, wl.w), I32(wb, wl.counts), I32(wb, wl.offsets), I32(wb, wl.sorted),
                                         I32(wb, wl.uniq), I32(wb, wl.nuniq), I32(wb, wl.stats),
                                         reinterpret_cast<unsigned *>(wb + wl.arrive), true, nullptr, 0, st,
                                         l > 0 ? &pc : nullptr))) != MOE_OK)
            return s;
        Routing rt{I32(wb, wl.ids),  I32(wb, wl.counts), I32(wb, wl.offsets), I32(wb, wl.sorted),
                   I32(wb, wl.uniq), I32(wb, wl.nuniq),  F(wb, wl.w),         I32(wb, wl.stats) + 2};
        // the last layer combines here; the others in the next routing launch
        if ((s = hip_status(launch_experts(L, F(wb, wl.xn), h, T, rt, wb + wl.xb, F(wb, wl.act), F(wb, wl.y),
                                           l == n_layers - 1 ? out : nullptr, lf, st))) != MOE_OK)
            return s;
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
