/*
 * moegen.c -- seeded synthetic inputs for the sparse-MoE decode layer.
 *
 * This file generates inputs only: activations, router and expert weights,
 * per-expert router biases and the fp8 block encoding of weights.  It holds
 * none of the layer's arithmetic.  Both the CPU oracle (through the Python
 * wrapper in this folder) and the GPU harness consume what it writes, so the
 * two sides always see the same bytes.
 *
 * Random numbers are counter-based: element i of tensor (seed, layer, tensor)
 * is a pure function of those four integers, so any slice (one expert of one
 * layer, one token row) can be regenerated on its own and the output does not
 * depend on the thread count.
 *
 *   mix64     : the SplitMix64 finaliser (Steele, Lea and Flood, "Fast
 *               splittable pseudorandom number generators", OOPSLA 2014;
 *               constants as in Vigna's public-domain splitmix64.c).
 *   uniforms  : u = (mix64(key + c * golden) >> 11) * 2^-53.
 *   normals   : Box-Muller (1958) in double, pair p = i/2 uses counters 2p and
 *               2p+1; even i takes the cosine branch, odd i the sine branch.
 *   bf16      : value = sigma * z in double -> fp32 (round to nearest even,
 *               the C cast) -> bf16 (round to nearest even on the bit pattern).
 *   fp8 e4m3  : OCP 8-bit floating point (OFP8) E4M3: bias 7, 3 mantissa bits,
 *               subnormals, max 448, S.1111.111 is NaN, no infinities.  Block
 *               scale s = fp32(amax / 448) over a 128x128 tile; the code is the
 *               nearest E4M3 value to w / s (ties to even code, saturating).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Stream key of one tensor: (seed, layer, tensor id). */
uint64_t moegen_key(uint64_t seed, uint32_t layer, uint32_t tensor) {
    uint64_t k = mix64(seed + GOLDEN);
    k = mix64(k ^ ((uint64_t)layer * 0xD1B54A32D192ED03ULL + GOLDEN));
    k = mix64(k ^ ((uint64_t)tensor * 0xAEF17502108EF2D9ULL + GOLDEN));
    return k;
}

static inline uint64_t draw64(uint64_t key, uint64_t ctr) {
    return mix64(key + (ctr + 1) * GOLDEN);
}

/* u in [0, 1) with 53 random bits. */
static inline double uniform01(uint64_t key, uint64_t ctr) {
    return (double)(draw64(key, ctr) >> 11) * (1.0 / 9007199254740992.0);
}

/* Standard normal number i of the stream. */
static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = 1.0 - uniform01(key, 2 * p); /* (0, 1] so log is finite */
    double u2 = uniform01(key, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

double moegen_normal_one(uint64_t key, uint64_t i) { return normal_at(key, i); }
double moegen_uniform_one(uint64_t key, uint64_t i) { return uniform01(key, i); }

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---- thread fan-out over [0, n) with a static split ---------------------- */

typedef struct {
    int kind;            /* 0 f32, 1 bf16 */
    uint64_t key, start, lo, hi;
    double sigma;
    void *out;
} fill_job;

static void *fill_worker(void *arg) {
    fill_job *j = (fill_job *)arg;
    if (j->kind == 0) {
        float *o = (float *)j->out;
        for (uint64_t i = j->lo; i < j->hi; ++i) o[i] = (float)(j->sigma * normal_at(j->key, j->start + i));
    } else {
        uint16_t *o = (uint16_t *)j->out;
        for (uint64_t i = j->lo; i < j->hi; ++i)
            o[i] = f32_to_bf16_rne((float)(j->sigma * normal_at(j->key, j->start + i)));
    }
    return NULL;
}

static void fill_parallel(int kind, uint64_t key, uint64_t start, uint64_t n, double sigma, void *out,
                          int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > n / 65536 + 1) nthreads = (int)(n / 65536 + 1);
    fill_job jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].kind = kind;
        jobs[t].key = key;
        jobs[t].start = start;
        jobs[t].lo = n * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].hi = n * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].sigma = sigma;
        jobs[t].out = out;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fill_worker, &jobs[t]);
    fill_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* out[i] = fp32(sigma * z_{start+i}), i < n. */
void moegen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float *out, int nthreads) {
    fill_parallel(0, key, start, n, sigma, out, nthreads);
}

/* out[i] = bf16(fp32(sigma * z_{start+i})), i < n, as raw bit patterns. */
void moegen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t *out, int nthreads) {
    fill_parallel(1, key, start, n, sigma, out, nthreads);
}

/* ---- OCP E4M3 encoder ----------------------------------------------------- */

static double e4m3_mag[127]; /* magnitude of codes 0x00..0x7E */
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;

static void e4m3_table_init(void) {
    for (int c = 0; c < 127; ++c) {
        int e = (c >> 3) & 0xF, m = c & 7;
        e4m3_mag[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    }
}

/* Nearest E4M3 code to v, ties to the even code, |v| >= 448 saturates. */
static uint8_t e4m3_encode(double v) {
    uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
    double a = fabs(v);
    if (!(a < 448.0)) return sign | 0x7E;
    int lo = 0, hi = 126; /* invariant: mag[lo] <= a < mag[hi] or a == mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (e4m3_mag[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - e4m3_mag[lo], dhi = e4m3_mag[hi] - a;
    int c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) ? hi : lo);
    return sign | (uint8_t)c;
}

uint8_t moegen_e4m3_encode(double v) {
    pthread_once(&e4m3_once, e4m3_table_init);
    return e4m3_encode(v);
}

typedef struct {
    uint64_t key, start;
    int rows, cols, blk_lo, blk_hi;
    double sigma;
    uint8_t *q;
    float *scales;
} fp8_job;

static void *fp8_worker(void *arg) {
    fp8_job *j = (fp8_job *)arg;
    int nbc = j->cols / 128;
    double *tile = (double *)malloc(sizeof(double) * 128 * 128);
    for (int b = j->blk_lo; b < j->blk_hi; ++b) {
        int br = b / nbc, bc = b % nbc;
        double amax = 0.0;
        for (int r = 0; r < 128; ++r)
            for (int c = 0; c < 128; ++c) {
                uint64_t idx = (uint64_t)(br * 128 + r) * (uint64_t)j->cols + (uint64_t)(bc * 128 + c);
                double w = j->sigma * normal_at(j->key, j->start + idx);
                tile[r * 128 + c] = w;
                if (fabs(w) > amax) amax = fabs(w);
            }
        float s = (float)(amax / 448.0);
        if (s == 0.0f) s = 1.0f;
        j->scales[b] = s;
        for (int r = 0; r < 128; ++r)
            for (int c = 0; c < 128; ++c) {
                uint64_t idx = (uint64_t)(br * 128 + r) * (uint64_t)j->cols + (uint64_t)(bc * 128 + c);
                j->q[idx] = e4m3_encode(tile[r * 128 + c] / (double)s);
            }
    }
    free(tile);
    return NULL;
}

/*
 * One [rows, cols] matrix (rows, cols multiples of 128) whose element
 * (r, c) is sigma * z_{start + r*cols + c}, encoded as E4M3 codes q[r*cols+c]
 * with fp32 block scales scales[(r/128)*(cols/128) + c/128].
 */
int moegen_fp8_matrix(uint64_t key, uint64_t start, int rows, int cols, double sigma, uint8_t *q, float *scales,
                      int nthreads) {
    if (rows % 128 || cols % 128 || rows <= 0 || cols <= 0) return 1;
    pthread_once(&e4m3_once, e4m3_table_init);
    int nblk = (rows / 128) * (cols / 128);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nblk) nthreads = nblk;
    fp8_job jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (fp8_job){key, start, rows, cols, nblk * t / nthreads, nblk * (t + 1) / nthreads, sigma, q, scales};
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fp8_worker, &jobs[t]);
    fp8_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ---- MXFP4 (OCP microscaling: E2M1 elements, E8M0 scale per 32) -------- */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Nearest E2M1 code to v, ties to the even code, |v| >= 6 saturates. */
static uint8_t e2m1_encode(double v) {
    uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 8 : 0;
    double a = fabs(v);
    if (!(a < 6.0)) return sign | 7;
    int lo = 0;
    while (lo < 6 && e2m1_mag[lo + 1] <= a) ++lo;
    int hi = lo + 1;
    double dlo = a - e2m1_mag[lo], dhi = e2m1_mag[hi] - a;
    int c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) ? hi : lo);
    return sign | (uint8_t)c;
}

typedef struct {
    uint64_t key, start;
    int cols;
    int64_t blk_lo, blk_hi;
    double sigma;
    uint8_t *q, *scales;
} mx_job;

static void *mx_worker(void *arg) {
    mx_job *j = (mx_job *)arg;
    double w[32];
    for (int64_t b = j->blk_lo; b < j->blk_hi; ++b) {
        double amax = 0.0;
        for (int c = 0; c < 32; ++c) {
            w[c] = j->sigma * normal_at(j->key, j->start + (uint64_t)b * 32 + (uint64_t)c);
            if (fabs(w[c]) > amax) amax = fabs(w[c]);
        }
        /* shared exponent: floor(log2(amax)) minus the largest E2M1
         * exponent (2), clamped to the E8M0 range */
        int se = 0;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
            se = (ex - 1) - 2;
        }
        if (se < -127) se = -127;
        if (se > 127) se = 127;
        j->scales[b] = (uint8_t)(se + 127);
        for (int c = 0; c < 32; c += 2) {
            uint8_t lo = e2m1_encode(ldexp(w[c], -se)), hi = e2m1_encode(ldexp(w[c + 1], -se));
            j->q[b * 16 + c / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
    return NULL;
}

/*
 * One [rows, cols] matrix (cols a multiple of 32) whose element (r, c) is
 * sigma * z_{start + r*cols + c}, encoded as MXFP4: codes two per byte
 * (q[(r*cols + c)/2], element c even in the low nibble) and one E8M0 scale
 * byte per block of 32 along a row (scales[(r*cols + c)/32]).  The scale is
 * 2^(floor(log2 amax) - 2); codes are the nearest E2M1 values of w / scale.
 */
int moegen_mxfp4_matrix(uint64_t key, uint64_t start, int rows, int cols, double sigma, uint8_t *q,
                        uint8_t *scales, int nthreads) {
    if (cols % 32 || rows <= 0 || cols <= 0) return 1;
    int64_t nblk = (int64_t)rows * cols / 32;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nblk) nthreads = (int)nblk;
    mx_job jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t)
        jobs[t] = (mx_job){key, start, cols, nblk * t / nthreads, nblk * (t + 1) / nthreads, sigma, q, scales};
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, mx_worker, &jobs[t]);
    mx_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

uint8_t moegen_e2m1_encode(double v) { return e2m1_encode(v); }

/* ---- q4_0 (blocks of 32 with one binary16 scale, 4-bit codes offset by 8) */

/* Nearest IEEE binary16 value of v as its bit pattern, ties to even
 * (rint in the default rounding mode); beyond the largest finite value,
 * the largest finite value. */
static uint16_t f16_encode(double v) {
    uint16_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x8000 : 0;
    double a = fabs(v);
    if (a < ldexp(1.0, -14)) return sign | (uint16_t)rint(ldexp(a, 24)); /* subnormal (1024 carries into 2^-14) */
    int ex;
    double m = frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;
    double frac = rint((2.0 * m - 1.0) * 1024.0);
    if (frac == 1024.0) {
        frac = 0.0;
        ++e;
    }
    if (e > 15) return sign | 0x7BFF;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)frac;
}

static double f16_decode(uint16_t h) {
    int e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double mag = e == 0 ? ldexp((double)f, -24) : ldexp(1.0 + f / 1024.0, e - 15);
    return (h & 0x8000) ? -mag : mag;
}

typedef struct {
    uint64_t key, start;
    int64_t blk_lo, blk_hi;
    double sigma;
    uint8_t *q;
    uint16_t *scales;
} q4_job;

static void *q4_worker(void *arg) {
    q4_job *j = (q4_job *)arg;
    double w[32];
    for (int64_t b = j->blk_lo; b < j->blk_hi; ++b) {
        double amax = 0.0;
        for (int c = 0; c < 32; ++c) {
            w[c] = j->sigma * normal_at(j->key, j->start + (uint64_t)b * 32 + (uint64_t)c);
            if (fabs(w[c]) > amax) amax = fabs(w[c]);
        }
        /* the scale maps the largest magnitude to code 8 +- 7 */
        const uint16_t h = f16_encode(amax / 7.0);
        const double d = f16_decode(h);
        j->scales[b] = h;
        uint8_t code[32];
        for (int c = 0; c < 32; ++c) {
            double qv = d > 0.0 ? rint(w[c] / d) + 8.0 : 8.0;
            code[c] = (uint8_t)(qv < 0.0 ? 0.0 : qv > 15.0 ? 15.0 : qv);
        }
        for (int c = 0; c < 16; ++c) j->q[b * 16 + c] = (uint8_t)(code[c] | (code[c + 16] << 4));
    }
    return NULL;
}

/*
 * One [rows, cols] matrix (cols a multiple of 32) whose element (r, c) is
 * sigma * z_{start + r*cols + c}, encoded as q4_0: per block of 32 along a row
 * one binary16 scale d = amax / 7 (scales[(r*cols + c)/32]) and 16 code bytes
 * (q[(r*cols + c)/32 * 16 + j]: element j of the block in the low nibble of
 * byte j, element j + 16 in its high nibble); each code is the nearest
 * integer to w / d plus 8 (ties to even), clamped to 0..15.
 */
int moegen_q4_0_matrix(uint64_t key, uint64_t start, int rows, int cols, double sigma, uint8_t *q,
                       uint16_t *scales, int nthreads) {
    if (cols % 32 || rows <= 0 || cols <= 0) return 1;
    int64_t nblk = (int64_t)rows * cols / 32;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nblk) nthreads = (int)nblk;
    q4_job jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t)
        jobs[t] = (q4_job){key, start, nblk * t / nthreads, nblk * (t + 1) / nthreads, sigma, q, scales};
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, q4_worker, &jobs[t]);
    q4_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

uint16_t moegen_f16_encode(double v) { return f16_encode(v); }

/* Seeded permutation of 0..n-1 (Fisher-Yates driven by the uniform stream). */
void moegen_permutation(uint64_t key, int n, int32_t *perm) {
    for (int i = 0; i < n; ++i) perm[i] = i;
    for (int i = n - 1; i > 0; --i) {
        int j = (int)(uniform01(key, (uint64_t)i) * (double)(i + 1));
        if (j > i) j = i;
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
}
