/*
 * Drives the host C code of the test infrastructure -- the CPU oracle
 * (oracle/moe_oracle.c) and the seeded input generator (workload/moegen.c)
 * -- through every entry point on small inputs, for sanitizer builds
 * (AddressSanitizer + UndefinedBehaviorSanitizer, ThreadSanitizer) made by
 * tests/test_sanitizers.py.  Exits non-zero if a result is inconsistent (the
 * two oracle walks must agree bitwise, a bad routing id must be refused); the
 * sanitizers abort on any memory or undefined-behaviour error or data race.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t E, top_k, H, I;
    int32_t router_dtype, expert_dtype;
    const void *w_router, *w_gate_up, *w_down, *s_gate_up, *s_down;
    const float *router_bias;
} layer_t;

/* oracle/moe_oracle.c */
double oracle_bf16_value(uint16_t b);
double oracle_e4m3_value(uint8_t c);
double oracle_e2m1_value(uint8_t c);
double oracle_e8m0_value(uint8_t s);
int oracle_check_layer(const layer_t *L);
void oracle_rmsnorm(int T, int H, const double *x, double eps, double *xhat);
void oracle_router_logits(const layer_t *L, int T, const double *x, double *logits);
void oracle_select(int T, int E, int k, const double *logits, int32_t *ids, double *w);
int oracle_sort(int T, int k, int E, const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *sorted,
                int32_t *uniq, int32_t *n_uniq);
int oracle_moe_layer(const layer_t *L, int T, const float *x, const double *logits_in, int flags, double eps,
                     int walk, double *logits_out, int32_t *ids_out, double *w_out, double *out, int nthreads);

/* workload/moegen.c */
uint64_t moegen_key(uint64_t seed, uint32_t layer, uint32_t tensor);
void moegen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float *out, int nthreads);
void moegen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t *out, int nthreads);
int moegen_fp8_matrix(uint64_t key, uint64_t start, int rows, int cols, double sigma, uint8_t *q, float *scales,
                      int nthreads);
int moegen_mxfp4_matrix(uint64_t key, uint64_t start, int rows, int cols, double sigma, uint8_t *q,
                        uint8_t *scales, int nthreads);
uint8_t moegen_e4m3_encode(double v);
uint8_t moegen_e2m1_encode(double v);
void moegen_permutation(uint64_t key, int n, int32_t *perm);
double moegen_normal_one(uint64_t key, uint64_t i);
double moegen_uniform_one(uint64_t key, uint64_t i);

enum { F32 = 0, BF16 = 1, FP8 = 2, MXFP4 = 3 };

static int failures = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                \
        }                                                              \
    } while (0)

/* The weights of one small layer, generated with several threads. */
typedef struct {
    layer_t L;
    void *wr, *gu, *dn, *sgu, *sdn;
    float *bias;
} owned_layer;

static size_t elem_bytes(int dtype) { return dtype == F32 ? 4 : dtype == BF16 ? 2 : 1; }

static void make_layer(owned_layer *o, int E, int k, int H, int I, int rdt, int edt, int with_bias, int nth) {
    memset(o, 0, sizeof(*o));
    o->L.E = E; o->L.top_k = k; o->L.H = H; o->L.I = I;
    o->L.router_dtype = rdt; o->L.expert_dtype = edt;
    const double sh = 1.0 / sqrt((double)H), si = 1.0 / sqrt((double)I);
    o->wr = malloc((size_t)E * H * elem_bytes(rdt));
    if (rdt == F32) moegen_normal_f32(moegen_key(0, 0, 1), 0, (uint64_t)E * H, sh, o->wr, nth);
    else moegen_normal_bf16(moegen_key(0, 0, 1), 0, (uint64_t)E * H, sh, o->wr, nth);
    const size_t ngu = (size_t)E * 2 * I * H, ndn = (size_t)E * H * I;
    if (edt == F32 || edt == BF16) {
        o->gu = malloc(ngu * elem_bytes(edt));
        o->dn = malloc(ndn * elem_bytes(edt));
        if (edt == F32) {
            moegen_normal_f32(moegen_key(0, 0, 2), 0, ngu, sh, o->gu, nth);
            moegen_normal_f32(moegen_key(0, 0, 3), 0, ndn, si, o->dn, nth);
        } else {
            moegen_normal_bf16(moegen_key(0, 0, 2), 0, ngu, sh, o->gu, nth);
            moegen_normal_bf16(moegen_key(0, 0, 3), 0, ndn, si, o->dn, nth);
        }
    } else if (edt == FP8) {
        o->gu = malloc(ngu);
        o->dn = malloc(ndn);
        o->sgu = malloc(sizeof(float) * (size_t)E * (2 * I / 128) * (H / 128));
        o->sdn = malloc(sizeof(float) * (size_t)E * (H / 128) * (I / 128));
        for (int e = 0; e < E; ++e) {
            CHECK(moegen_fp8_matrix(moegen_key(0, 0, 2), (uint64_t)e * 2 * I * H, 2 * I, H, sh,
                                    (uint8_t *)o->gu + (size_t)e * 2 * I * H,
                                    (float *)o->sgu + (size_t)e * (2 * I / 128) * (H / 128), nth) == 0);
            CHECK(moegen_fp8_matrix(moegen_key(0, 0, 3), (uint64_t)e * H * I, H, I, si,
                                    (uint8_t *)o->dn + (size_t)e * H * I,
                                    (float *)o->sdn + (size_t)e * (H / 128) * (I / 128), nth) == 0);
        }
    } else {
        o->gu = malloc(ngu / 2);
        o->dn = malloc(ndn / 2);
        o->sgu = malloc(ngu / 32);
        o->sdn = malloc(ndn / 32);
        CHECK(moegen_mxfp4_matrix(moegen_key(0, 0, 2), 0, E * 2 * I, H, sh, o->gu, o->sgu, nth) == 0);
        CHECK(moegen_mxfp4_matrix(moegen_key(0, 0, 3), 0, E * H, I, si, o->dn, o->sdn, nth) == 0);
    }
    if (with_bias) {
        o->bias = malloc(sizeof(float) * E);
        int32_t *perm = malloc(sizeof(int32_t) * E);
        moegen_permutation(moegen_key(2, 0, 9), E, perm);
        for (int r = 0; r < E; ++r) o->bias[perm[r]] = (float)(-1.1 * log(r + 1.0));
        free(perm);
    }
    o->L.w_router = o->wr; o->L.w_gate_up = o->gu; o->L.w_down = o->dn;
    o->L.s_gate_up = o->sgu; o->L.s_down = o->sdn; o->L.router_bias = o->bias;
}

static void free_layer(owned_layer *o) {
    free(o->wr); free(o->gu); free(o->dn); free(o->sgu); free(o->sdn); free(o->bias);
}

/* Every walk, flag combination and thread count of the whole layer. */
static void exercise_layer(const owned_layer *o) {
    const layer_t *L = &o->L;
    CHECK(oracle_check_layer(L) == 0);
    const int Ts[3] = {0, 1, 5};
    for (int ti = 0; ti < 3; ++ti) {
        const int T = Ts[ti], H = L->H, E = L->E, k = L->top_k;
        float *x = malloc(sizeof(float) * (size_t)(T ? T : 1) * H);
        moegen_normal_f32(moegen_key(1, 0, 5), 0, (uint64_t)T * H, 1.0, x, 2);
        double *out[2], *lg = malloc(sizeof(double) * (size_t)(T ? T : 1) * E);
        double *w = malloc(sizeof(double) * (size_t)(T ? T : 1) * k);
        int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T ? T : 1) * k);
        for (int flags = 0; flags < 4; ++flags) {
            for (int walk = 0; walk < 2; ++walk) {
                out[walk] = calloc((size_t)(T ? T : 1) * H, sizeof(double));
                CHECK(oracle_moe_layer(L, T, x, NULL, flags, 1e-6, walk, lg, ids, w, out[walk], walk ? 1 : 3) == 0);
            }
            CHECK(memcmp(out[0], out[1], sizeof(double) * (size_t)T * H) == 0);
            free(out[0]);
            free(out[1]);
        }
        /* selection fed with given logits */
        double *out2 = calloc((size_t)(T ? T : 1) * H, sizeof(double));
        CHECK(oracle_moe_layer(L, T, x, lg, 0, 1e-6, 0, NULL, NULL, NULL, out2, 2) == 0);
        free(out2);
        free(x); free(lg); free(w); free(ids);
    }
}

int main(void) {
    /* decoders over every code */
    for (int b = 0; b < 65536; b += 7) (void)oracle_bf16_value((uint16_t)b);
    for (int c = 0; c < 256; ++c) {
        (void)oracle_e4m3_value((uint8_t)c);
        (void)oracle_e8m0_value((uint8_t)c);
    }
    for (int c = 0; c < 16; ++c) (void)oracle_e2m1_value((uint8_t)c);
    for (int i = -40; i <= 40; ++i) {
        (void)moegen_e4m3_encode(i * 13.7);
        (void)moegen_e2m1_encode(i * 0.31);
    }
    (void)moegen_normal_one(moegen_key(3, 1, 2), 12345);
    (void)moegen_uniform_one(moegen_key(3, 1, 2), 54321);

    /* selection with ties and signed zeros; sort with repeats and a bad id */
    {
        const int T = 3, E = 8, k = 3;
        double lg[24];
        for (int i = 0; i < 24; ++i) lg[i] = (i % 3 == 0) ? 0.25 : (i % 2 ? -0.0 : 0.0);
        int32_t ids[9];
        double w[9];
        oracle_select(T, E, k, lg, ids, w);
        int32_t counts[8], offsets[9], sorted[9], uniq[8], n_uniq = 0;
        CHECK(oracle_sort(T, k, E, ids, counts, offsets, sorted, uniq, &n_uniq) == 0);
        CHECK(offsets[E] == T * k);
        ids[4] = E;  /* out of range: refused */
        CHECK(oracle_sort(T, k, E, ids, counts, offsets, sorted, uniq, &n_uniq) == 1);
        double x[2 * 16], xh[2 * 16];
        for (int i = 0; i < 32; ++i) x[i] = i * 0.1 - 1.0;
        oracle_rmsnorm(2, 16, x, 1e-6, xh);
    }

    owned_layer o;
    make_layer(&o, 8, 2, 64, 32, F32, F32, 0, 3);
    exercise_layer(&o);
    free_layer(&o);
    make_layer(&o, 16, 4, 128, 64, BF16, BF16, 1, 4);
    exercise_layer(&o);
    free_layer(&o);
    make_layer(&o, 4, 2, 128, 128, BF16, FP8, 0, 3);
    exercise_layer(&o);
    free_layer(&o);
    make_layer(&o, 4, 2, 64, 64, BF16, MXFP4, 1, 3);
    exercise_layer(&o);
    free_layer(&o);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("sanitizer driver ok\n");
    return 0;
}
