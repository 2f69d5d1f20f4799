/*
 * moe_oracle.c -- plain, slow CPU oracle of the sparse-MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two meet only in the
 * seeded inputs both read.
 *
 * Every sum is accumulated in double in ascending index order; outputs are
 * returned in double.  Weights are decoded exactly to double first: fp32 as
 * is, bf16 as the upper half of an fp32 bit pattern, OCP E4M3 from its bit
 * fields times the fp32 scale of its 128x128 block, and MXFP4 (OCP
 * microscaling: E2M1 elements, two per byte with the first in the low
 * nibble, sharing an E8M0 scale per block of 32 along a row) from its bit
 * fields times 2^(scale - 127), and q4_0 (blocks of 32 elements along a row
 * with one IEEE binary16 scale d; element j of a block is the 4-bit code in
 * the low nibble of the block's byte j, element j + 16 the code in its high
 * nibble; the value is (code - 8) * d) from its codes and the binary16 bit
 * fields of d.
 *
 * Sources (page title, section):
 *  - "MoE Performance Optimization Analysis" (markbaseengine), Root Cause:
 *    the layer computes router scores, selects the top experts, runs the
 *    experts and combines their outputs; GPU Router Design: router compute,
 *    selection and combination, all on the device.
 *  - "perf(cpu-moe): dedup experts across the batch in pass 1" (FreeToken
 *    PR #46), commit message: routes are grouped per expert by a counting sort
 *    over their expert ids; pass 1 reads gate_up [2I, H] (a gate row and an up
 *    row per intermediate index) and pass 2 reads down [H, I]; the grouped walk
 *    only changes the loop order, so it computes exactly what the per-route
 *    walk computes.
 *  - Where the pages are silent the readings are: softmax over all E logits,
 *    top-k by (logit descending, expert index ascending), weights renormalised
 *    over the k selected; gate rows [0, I) and up rows [I, 2I) of gate_up;
 *    activation SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z)); combine in
 *    slot order; RMSNorm x / sqrt(mean(x^2) + eps) * gamma before the router
 *    and a residual add after the combine for the layer-stack workload.
 *
 * Pins: every function here is checked by tests against brute force, closed
 * forms, library routines on special cases and invariants (tests/test_oracle*.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_MXFP4 = 3, OR_Q4_0 = 4 };
enum { OR_RMSNORM = 1, OR_RESIDUAL = 2 };

typedef struct {
    int32_t E, top_k, H, I;
    int32_t router_dtype, expert_dtype;
    const void *w_router;     /* [E, H]                          */
    const void *w_gate_up;    /* [E, 2I, H]                      */
    const void *w_down;       /* [E, H, I]                       */
    const void *s_gate_up;    /* fp8: float [E, 2I/128, H/128]; mxfp4: uint8, q4_0: binary16 [E, 2I, H/32] */
    const void *s_down;       /* fp8: float [E, H/128, I/128];  mxfp4: uint8, q4_0: binary16 [E, H, I/32]  */
    const float *router_bias; /* [E] or NULL                     */
} oracle_layer;

/* ---- exact decoders ------------------------------------------------------- */

double oracle_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities. */
double oracle_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 0xF && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* OCP E2M1 (MX element): sign, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent 0 is subnormal (m * 2^-1); no infinities or NaN. */
double oracle_e2m1_value(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* OCP E8M0 (MX shared scale): 2^(s - 127); 255 is NaN. */
double oracle_e8m0_value(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* IEEE 754 binary16: sign, 5 exponent bits (bias 15), 10 fraction bits;
 * exponent 0 is subnormal (f * 2^-24), exponent 31 is infinity (f = 0) or
 * NaN. */
double oracle_f16_value(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double mag;
    if (e == 0x1F) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)f, -24);
    else mag = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return s ? -mag : mag;
}

/* Element idx of a row-major matrix (idx = row * cols + col).  MXFP4: the
 * code is nibble (idx & 1) of byte idx / 2, its scale byte idx / 32 (cols is
 * a multiple of 32, so the blocks of 32 never cross a row). */
static double decode(int dtype, const void *base, const void *scales, size_t idx) {
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    if (dtype == OR_BF16) return oracle_bf16_value(((const uint16_t *)base)[idx]);
    if (dtype == OR_Q4_0) {
        /* block idx / 32 is 16 code bytes; element j < 16 in the low nibble of
         * byte j, element j >= 16 in the high nibble of byte j - 16 */
        const size_t blk = idx / 32, j = idx % 32;
        const uint8_t b = ((const uint8_t *)base)[blk * 16 + (j & 15)];
        const int code = j < 16 ? (b & 15) : (b >> 4);
        return (double)(code - 8) * oracle_f16_value(((const uint16_t *)scales)[blk]);
    }
    if (dtype == OR_MXFP4) {
        const uint8_t b = ((const uint8_t *)base)[idx / 2];
        return oracle_e2m1_value((idx & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15)) *
               oracle_e8m0_value(((const uint8_t *)scales)[idx / 32]);
    }
    return oracle_e4m3_value(((const uint8_t *)base)[idx]);
}

/* gate_up[e][row][h], row < 2I */
static double w_gu(const oracle_layer *L, int e, int row, int h) {
    size_t idx = ((size_t)e * 2 * L->I + row) * L->H + h;
    double v = decode(L->expert_dtype, L->w_gate_up, L->s_gate_up, idx);
    if (L->expert_dtype == OR_FP8) {
        size_t sb = ((size_t)e * (2 * L->I / 128) + row / 128) * (L->H / 128) + h / 128;
        v *= (double)((const float *)L->s_gate_up)[sb];
    }
    return v;
}

/* down[e][h][i] */
static double w_dn(const oracle_layer *L, int e, int h, int i) {
    size_t idx = ((size_t)e * L->H + h) * L->I + i;
    double v = decode(L->expert_dtype, L->w_down, L->s_down, idx);
    if (L->expert_dtype == OR_FP8) {
        size_t sb = ((size_t)e * (L->H / 128) + h / 128) * (L->I / 128) + i / 128;
        v *= (double)((const float *)L->s_down)[sb];
    }
    return v;
}

int oracle_check_layer(const oracle_layer *L) {
    if (!L || L->E < 1 || L->top_k < 1 || L->top_k > L->E || L->H < 1 || L->I < 1) return 1;
    if (!L->w_router || !L->w_gate_up || !L->w_down) return 1;
    if (L->expert_dtype == OR_FP8 && (L->H % 128 || L->I % 128 || !L->s_gate_up || !L->s_down)) return 1;
    if ((L->expert_dtype == OR_MXFP4 || L->expert_dtype == OR_Q4_0) &&
        (L->H % 32 || L->I % 32 || !L->s_gate_up || !L->s_down))
        return 1;
    if (L->expert_dtype < OR_F32 || L->expert_dtype > OR_Q4_0) return 1;
    if (L->router_dtype != OR_F32 && L->router_dtype != OR_BF16) return 1;
    return 0;
}

/* ---- step 0: RMSNorm (layer-stack workload only) ------------------------- */

void oracle_rmsnorm(int T, int H, const double *x, double eps, double *xhat) {
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int h = 0; h < H; ++h) ss += x[(size_t)t * H + h] * x[(size_t)t * H + h];
        double r = 1.0 / sqrt(ss / (double)H + eps); /* gamma = 1 */
        for (int h = 0; h < H; ++h) xhat[(size_t)t * H + h] = x[(size_t)t * H + h] * r;
    }
}

/* ---- step 1: router GEMV ---------------------------------------------------- */

void oracle_router_logits(const oracle_layer *L, int T, const double *x, double *logits) {
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < L->E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < L->H; ++h)
                acc += decode(L->router_dtype, L->w_router, NULL, (size_t)e * L->H + h) * x[(size_t)t * L->H + h];
            if (L->router_bias) acc += (double)L->router_bias[e];
            logits[(size_t)t * L->E + e] = acc;
        }
}

/* ---- steps 2-3: top-k selection and renormalised softmax weights --------- */

/* Slot j takes the largest remaining logit; a later expert replaces the
 * current best only when strictly greater, so ties keep the lower index.
 * IEEE comparison: -0 == +0. */
void oracle_select(int T, int E, int k, const double *logits, int32_t *ids, double *w) {
    char *taken = (char *)malloc((size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        /* full softmax over all E, then renormalise over the selected k */
        double m = l[0];
        for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - m); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += p[ids[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = p[ids[(size_t)t * k + j]] / s;
    }
    free(p);
    free(taken);
}

/* ---- step 4: counting sort of the routes by expert ---------------------- */

/* Route r = t*k + j carries expert ids[r].  counts[e] = routes of expert e;
 * offsets = exclusive prefix sum (offsets[E] = R); sorted_routes lists the
 * routes of expert 0, then 1, ..., each in ascending r; uniq = experts with a
 * nonzero count, ascending; *n_uniq = their number. */
int oracle_sort(int T, int k, int E, const int32_t *ids, int32_t *counts, int32_t *offsets,
                int32_t *sorted_routes, int32_t *uniq, int32_t *n_uniq) {
    int R = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int r = 0; r < R; ++r) {
        if (ids[r] < 0 || ids[r] >= E) return 1;
        counts[ids[r]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int r = 0; r < R; ++r) {
        int e = ids[r];
        sorted_routes[offsets[e] + fill[e]] = r;
        fill[e] += 1;
    }
    free(fill);
    int n = 0;
    for (int e = 0; e < E; ++e) if (counts[e] > 0) uniq[n++] = e;
    *n_uniq = n;
    return 0;
}

/* ---- step 5: the per-route walk (the definition) -------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y[r][:] for one route: expert e applied to the activation row xr. */
static void expert_route(const oracle_layer *L, int e, const double *xr, double *a, double *yr) {
    int H = L->H, I = L->I;
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) g += w_gu(L, e, i, h) * xr[h];
        for (int h = 0; h < H; ++h) u += w_gu(L, e, I + i, h) * xr[h];
        a[i] = silu(g) * u;
    }
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += w_dn(L, e, h, i) * a[i];
        yr[h] = acc;
    }
}

typedef struct {
    const oracle_layer *L;
    int k, lo, hi;
    const double *x;
    const int32_t *ids;
    double *y;
} route_job;

static void *route_worker(void *arg) {
    route_job *j = (route_job *)arg;
    double *a = (double *)malloc(sizeof(double) * (size_t)j->L->I);
    for (int r = j->lo; r < j->hi; ++r) {
        int t = r / j->k;
        expert_route(j->L, j->ids[r], j->x + (size_t)t * j->L->H, a, j->y + (size_t)r * j->L->H);
    }
    free(a);
    return NULL;
}

/* y[r, h] for every route r = t*k + j (expert ids[r], activation row x[t]).
 * Routes are independent, so the optional thread split changes nothing. */
void oracle_walk_per_route(const oracle_layer *L, int T, const double *x, const int32_t *ids, double *y,
                           int nthreads) {
    int R = T * L->top_k;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > R) nthreads = R > 0 ? R : 1;
    route_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i)
        jobs[i] = (route_job){L, L->top_k, R * i / nthreads, R * (i + 1) / nthreads, x, ids, y};
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, route_worker, &jobs[i]);
    route_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ---- step 6: the grouped walk (one pass over each unique expert) --------- */

/* Same sums as the per-route walk with the loop nest reordered: unique expert
 * outermost, then the weight row, then the expert's routes innermost, so each
 * weight row is visited once per expert and applied to every route of the
 * segment.  The order inside every dot product is unchanged, so y is bitwise
 * the per-route result. */
void oracle_walk_grouped(const oracle_layer *L, int T, const double *x, const int32_t *ids, double *y) {
    int E = L->E, k = L->top_k, H = L->H, I = L->I, R = T * k;
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    int32_t *uniq = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t nu = 0;
    oracle_sort(T, k, E, ids, counts, offsets, sorted, uniq, &nu);
    int maxc = 0;
    for (int e = 0; e < E; ++e) if (counts[e] > maxc) maxc = counts[e];
    double *g = (double *)malloc(sizeof(double) * (size_t)(maxc > 0 ? maxc : 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)(maxc > 0 ? maxc : 1));
    double *a = (double *)malloc(sizeof(double) * (size_t)(maxc > 0 ? maxc : 1) * (size_t)I);
    for (int q = 0; q < nu; ++q) {
        int e = uniq[q], n = counts[e];
        const int32_t *seg = sorted + offsets[e];
        /* pass 1: gate row i and up row I+i, each applied to all n routes */
        for (int i = 0; i < I; ++i) {
            for (int s = 0; s < n; ++s) { g[s] = 0.0; u[s] = 0.0; }
            for (int s = 0; s < n; ++s) {
                const double *xr = x + (size_t)(seg[s] / k) * H;
                for (int h = 0; h < H; ++h) g[s] += w_gu(L, e, i, h) * xr[h];
            }
            for (int s = 0; s < n; ++s) {
                const double *xr = x + (size_t)(seg[s] / k) * H;
                for (int h = 0; h < H; ++h) u[s] += w_gu(L, e, I + i, h) * xr[h];
            }
            for (int s = 0; s < n; ++s) a[(size_t)s * I + i] = silu(g[s]) * u[s];
        }
        /* pass 2: down row h applied to all n routes */
        for (int h = 0; h < H; ++h)
            for (int s = 0; s < n; ++s) {
                double acc = 0.0;
                for (int i = 0; i < I; ++i) acc += w_dn(L, e, h, i) * a[(size_t)s * I + i];
                y[(size_t)seg[s] * H + h] = acc;
            }
    }
    free(a); free(u); free(g); free(uniq); free(sorted); free(offsets); free(counts);
}

/* ---- step 7: router-weighted combine -------------------------------------- */

void oracle_combine(int T, int k, int H, const double *w, const double *y, double *out) {
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * y[((size_t)t * k + j) * H + h];
            out[(size_t)t * H + h] = acc;
        }
}

/* ---- the experts and combine for a given routing -------------------------- */

/* out[T, H] from activations x (double), routing ids/w; walk 0 = per route,
 * 1 = grouped.  Returns 0, or 1 on bad arguments. */
int oracle_expert_fwd(const oracle_layer *L, int T, const double *x, const int32_t *ids, const double *w,
                      int walk, double *out, int nthreads) {
    if (oracle_check_layer(L) || T < 0) return 1;
    int R = T * L->top_k;
    for (int r = 0; r < R; ++r) if (ids[r] < 0 || ids[r] >= L->E) return 1;
    if (T == 0) return 0;
    double *y = (double *)malloc(sizeof(double) * (size_t)R * (size_t)L->H);
    if (walk == 1) oracle_walk_grouped(L, T, x, ids, y);
    else oracle_walk_per_route(L, T, x, ids, y, nthreads);
    oracle_combine(T, L->top_k, L->H, w, y, out);
    free(y);
    return 0;
}

/* ---- the whole layer --------------------------------------------------------- */

/* x [T, H] fp32 -> out [T, H] double.  flags: OR_RMSNORM normalises x before
 * the router and the experts (gamma = 1, eps given); OR_RESIDUAL adds x to the
 * combined output.  If logits_in is given it replaces steps 0-1 (selection fed
 * straight from given logits).  logits_out, ids_out, w_out may be NULL. */
int oracle_moe_layer(const oracle_layer *L, int T, const float *x, const double *logits_in, int flags, double eps,
                     int walk, double *logits_out, int32_t *ids_out, double *w_out, double *out, int nthreads) {
    if (oracle_check_layer(L) || T < 0) return 1;
    if (T == 0) return 0;
    int E = L->E, k = L->top_k, H = L->H;
    double *xd = (double *)malloc(sizeof(double) * (size_t)T * H);
    double *xh = (double *)malloc(sizeof(double) * (size_t)T * H);
    double *lg = (double *)malloc(sizeof(double) * (size_t)T * E);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)T * k);
    for (size_t i = 0; i < (size_t)T * H; ++i) xd[i] = (double)x[i];
    if (flags & OR_RMSNORM) oracle_rmsnorm(T, H, xd, eps, xh);
    else memcpy(xh, xd, sizeof(double) * (size_t)T * H);
    if (logits_in) memcpy(lg, logits_in, sizeof(double) * (size_t)T * E);
    else oracle_router_logits(L, T, xh, lg);
    oracle_select(T, E, k, lg, ids, w);
    int rc = oracle_expert_fwd(L, T, xh, ids, w, walk, out, nthreads);
    if (!rc && (flags & OR_RESIDUAL))
        for (size_t i = 0; i < (size_t)T * H; ++i) out[i] += xd[i];
    if (logits_out) memcpy(logits_out, lg, sizeof(double) * (size_t)T * E);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)T * k);
    free(w); free(ids); free(lg); free(xh); free(xd);
    return rc;
}
