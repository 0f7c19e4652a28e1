/*
 * Plain CPU oracle for the mixed-precision training hot path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library. No code, table
 * or constant is shared with the HIP path.
 *
 * Sources (page titles as published):
 *   [A]  "Mixed Precision Training" — long-form analysis page
 *        (paper-graph-ui.vercel.app).
 *   [E]  "Mixed Precision Training" — explainer page (azimuth.plus).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -pthread.
 * On x86-64 every float operation below is a single SSE operation rounded to
 * nearest-even, with denormals neither flushed nor treated as zero.
 *
 * Parity status per function (see the tests for each pin):
 *   codec ............ pinned (exhaustive against numpy float16; format constants)
 *   GEMM definitions . pinned (exact integer sums; FP64 error bound; K=4096 ones)
 *   overflow flag .... pinned (injected +-inf/NaN at head/middle/tail)
 *   SGD update ....... pinned (worked examples and closed forms)
 *   scaler ........... pinned (closed-form traces)
 *   relu/gelu/losses . pinned (library erf/softmax, finite differences, closed forms)
 *   Nesterov/Adagrad . pinned (exact-rational closed forms; reductions to plain SGD and to
 *                      a sign step; fp64 bounds where a square root enters)
 *   max|g|, S from it  pinned (numpy over the finite elements; closed forms; largest
 *                      fitting power of two)
 *   batch-norm stats . pinned (constant channels, arithmetic progressions, exact rationals)
 *   normalization .... pinned (dyadic cases exact in FP32; special cases)
 *   softmax .......... pinned (constant and two-valued rows in closed form; shift
 *                      invariance; infinities and NaN)
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------- */
/* A minimal parallel-for over [0, n).                                        */
/* ------------------------------------------------------------------------- */
static int32_t g_threads = 0;

void or_set_threads(int32_t n) { g_threads = n; }

int32_t or_get_threads(void) {
    if (g_threads > 0) return g_threads;
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int32_t)c : 1;
}

typedef void (*range_fn)(int64_t lo, int64_t hi, void* ctx);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } range_job;

static void* range_worker(void* p) {
    range_job* j = (range_job*)p;
    j->fn(j->lo, j->hi, j->ctx);
    return NULL;
}

static void parallel_for(int64_t n, int64_t min_per_thread, range_fn fn, void* ctx) {
    int32_t t = or_get_threads();
    if (min_per_thread < 1) min_per_thread = 1;
    if ((int64_t)t > n / min_per_thread) t = (int32_t)(n / min_per_thread);
    if (t <= 1) { if (n > 0) fn(0, n, ctx); return; }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)t);
    range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)t);
    for (int32_t i = 0; i < t; ++i) {
        jobs[i].fn = fn; jobs[i].ctx = ctx;
        jobs[i].lo = n * i / t; jobs[i].hi = n * (i + 1) / t;
        pthread_create(&th[i], NULL, range_worker, &jobs[i]);
    }
    for (int32_t i = 0; i < t; ++i) pthread_join(th[i], NULL);
    free(th); free(jobs);
}

/* ------------------------------------------------------------------------- */
/* binary16 codec.                                                             */
/* [A] §2 and §3.4 "FP32 Master Copy of Weights": 1 sign bit, 5 exponent bits,   */
/* 10 mantissa bits; normal exponents -14..15; the smallest subnormal is 2^-24; */
/* the largest finite value 65504 has exponent 15 and every mantissa bit set     */
/* ([A] §3.4 "Choosing the Loss Scaling Factor", method 2).                      */
/* ------------------------------------------------------------------------- */

/* Exact decode: exponent field 0 is the subnormal m * 2^-24, 31 is inf/NaN,
 * anything else (1024 + m) * 2^(e - 25). */
float or_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)       v = ldexp((double)m, -24);
    else if (e == 31) v = m ? (double)NAN : (double)INFINITY;
    else              v = ldexp((double)(1024 + m), e - 25);
    float f = (float)v;                 /* exact: at most 11 significant bits */
    return sign ? -f : f;
}

/* Round to the nearest binary16 value, ties to the even significand
 * ([A] §3.4 "The Integrated Training Procedure", Step 1, rounds each master
 * weight to the closest binary16 value), with gradual underflow and overflow
 * to infinity.
 * Written from the definition: find the spacing q of binary16 values around
 * |x|, take the two neighbours floor(|x|/q)*q and the next one up, keep the
 * nearer, and on an exact tie the one whose significand is even. All of it
 * is exact in double because |x| carries at most 24 significant bits. */
uint16_t or_f32_to_f16(float x) {
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);          /* quiet NaN */
    double a = fabs((double)x);
    /* 65504 is the largest finite value and its spacing is 32: everything at
     * or above the midpoint 65520 rounds away (the tie goes to the even
     * neighbour 65536, which is not finite). */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                    /* a in [2^(e2-1), 2^e2) */
    int binade = e2 - 1;
    if (binade < -14) binade = -14;   /* subnormals share the spacing 2^-24 */
    double q = ldexp(1.0, binade - 10);
    double n = floor(a / q);
    double r = a - n * q;
    double half = 0.5 * q;
    if (r > half || (r == half && fmod(n, 2.0) != 0.0)) n += 1.0;
    double v = n * q;
    if (v < ldexp(1.0, -14)) {
        /* subnormal (or rounded up to exactly 2^-14, which encodes as 0x0400) */
        return (uint16_t)(sign | (uint16_t)ldexp(v, 24));
    }
    int ev;
    frexp(v, &ev);
    int E = ev - 1;                   /* v in [2^E, 2^(E+1)) */
    uint16_t mant = (uint16_t)(ldexp(v, 10 - E) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | mant);
}

typedef struct { const float* x; uint16_t* h; const uint16_t* hi; float* xo; uint64_t base; } codec_ctx;

static void enc_range(int64_t lo, int64_t hi, void* p) {
    codec_ctx* c = (codec_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) c->h[i] = or_f32_to_f16(c->x[i]);
}
static void dec_range(int64_t lo, int64_t hi, void* p) {
    codec_ctx* c = (codec_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) c->xo[i] = or_f16_to_f32(c->hi[i]);
}
static void bits_range(int64_t lo, int64_t hi, void* p) {
    codec_ctx* c = (codec_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) {
        uint32_t b = (uint32_t)(c->base + (uint64_t)i);
        float f;
        memcpy(&f, &b, sizeof f);
        c->h[i] = or_f32_to_f16(f);
    }
}

void or_f32_to_f16_array(const float* x, uint16_t* h, int64_t n) {
    codec_ctx c = { x, h, NULL, NULL, 0 };
    parallel_for(n, 1 << 16, enc_range, &c);
}
void or_f16_to_f32_array(const uint16_t* h, float* x, int64_t n) {
    codec_ctx c = { NULL, NULL, h, x, 0 };
    parallel_for(n, 1 << 16, dec_range, &c);
}
void or_f32bits_to_f16_range(uint64_t lo, uint64_t hi, uint16_t* out) {
    codec_ctx c = { NULL, out, NULL, NULL, lo };
    parallel_for((int64_t)(hi - lo), 1 << 16, bits_range, &c);
}

/* ------------------------------------------------------------------------- */
/* Dot-product layers.                                                         */
/* [A] §3.4 "FP16 Arithmetic with FP32 Accumulation": c = sum_i a_i * b_i with  */
/* binary16 a_i, b_i and the running sum held in FP32, rounded to binary16     */
/* only when stored. A product of two binary16 values has at most 22           */
/* significant bits and lies in [2^-48, 2^32], so the FP32 multiply is exact.   */
/* The three layers of a linear map Y = X W^T are                              */
/*   forward  Y[i,j]  = sum_k X[i,k]  W[j,k]   (Step 2)                         */
/*   dgrad    dX[i,k] = sum_n dY[i,n] W[n,k]   (Step 4, activation gradient)   */
/*   wgrad    dW[n,k] = sum_m dY[m,n] X[m,k]   (Step 4, weight gradient)       */
/* ------------------------------------------------------------------------- */

static float dot_f32acc(const uint16_t* a, int64_t sa, const uint16_t* b, int64_t sb, int64_t n) {
    float acc = 0.0f;
    for (int64_t r = 0; r < n; ++r) {
        float p = or_f16_to_f32(a[r * sa]) * or_f16_to_f32(b[r * sb]);
        acc = acc + p;
    }
    return acc;
}

typedef struct {
    const uint16_t *a, *b;
    int64_t lda, ldb;      /* row strides of the two operands              */
    int64_t ldo;           /* row stride of the output                     */
    int64_t ncols, red;    /* output columns; reduction length             */
    int kind;              /* 0 fwd, 1 dgrad, 2 wgrad                      */
    int out_f16;
    void* out;
    const int64_t *rows, *cols;
    float* outs;
} gemm_ctx;

static float gemm_at(const gemm_ctx* g, int64_t i, int64_t j) {
    switch (g->kind) {
    case 0:  return dot_f32acc(g->a + i * g->lda, 1, g->b + j * g->ldb, 1, g->red);
    case 1:  return dot_f32acc(g->a + i * g->lda, 1, g->b + j, g->ldb, g->red);
    default: return dot_f32acc(g->a + i, g->lda, g->b + j, g->ldb, g->red);
    }
}

static void gemm_rows(int64_t lo, int64_t hi, void* p) {
    gemm_ctx* g = (gemm_ctx*)p;
    for (int64_t i = lo; i < hi; ++i)
        for (int64_t j = 0; j < g->ncols; ++j) {
            float acc = gemm_at(g, i, j);
            if (g->out_f16) ((uint16_t*)g->out)[i * g->ldo + j] = or_f32_to_f16(acc);
            else            ((float*)g->out)[i * g->ldo + j] = acc;
        }
}

static void gemm_points(int64_t lo, int64_t hi, void* p) {
    gemm_ctx* g = (gemm_ctx*)p;
    for (int64_t t = lo; t < hi; ++t) g->outs[t] = gemm_at(g, g->rows[t], g->cols[t]);
}

static void run_full(gemm_ctx* g, int64_t nrows) { parallel_for(nrows, 1, gemm_rows, g); }

void or_linear_fwd(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                   void* Y, int64_t ldy, int out_f16, int64_t M, int64_t N, int64_t K) {
    gemm_ctx g = { X, W, ldx, ldw, ldy, N, K, 0, out_f16, Y, NULL, NULL, NULL };
    run_full(&g, M);
}
void or_linear_dgrad(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                     void* dX, int64_t lddx, int out_f16, int64_t M, int64_t N, int64_t K) {
    gemm_ctx g = { dY, W, lddy, ldw, lddx, K, N, 1, out_f16, dX, NULL, NULL, NULL };
    run_full(&g, M);
}
void or_linear_wgrad(const uint16_t* dY, int64_t lddy, const uint16_t* X, int64_t ldx,
                     void* dW, int64_t lddw, int out_f16, int64_t M, int64_t N, int64_t K) {
    gemm_ctx g = { dY, X, lddy, ldx, lddw, K, M, 2, out_f16, dW, NULL, NULL, NULL };
    run_full(&g, N);
}
void or_linear_fwd_at(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                      int64_t K, const int64_t* rows, const int64_t* cols, int64_t count,
                      float* out) {
    gemm_ctx g = { X, W, ldx, ldw, 0, 0, K, 0, 0, NULL, rows, cols, out };
    parallel_for(count, 64, gemm_points, &g);
}
void or_linear_dgrad_at(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                        int64_t N, const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out) {
    gemm_ctx g = { dY, W, lddy, ldw, 0, 0, N, 1, 0, NULL, rows, cols, out };
    parallel_for(count, 64, gemm_points, &g);
}
void or_linear_wgrad_at(const uint16_t* dY, int64_t lddy, const uint16_t* X, int64_t ldx,
                        int64_t M, const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out) {
    gemm_ctx g = { dY, X, lddy, ldx, 0, 0, M, 2, 0, NULL, rows, cols, out };
    parallel_for(count, 64, gemm_points, &g);
}

/* ------------------------------------------------------------------------- */
/* Optimizer sweep.                                                            */
/* [A] §3.4 "The Integrated Training Procedure":                               */
/*   Step 5  g_true = g_scaled / S                                             */
/*   Step 6  if any weight gradient is +-inf or NaN, skip the whole update;    */
/*           the FP32 master weights are not modified                           */
/*   Step 7  v_t = mu v_{t-1} + g_true ;  w = w - eta v_t   (all FP32)          */
/*   weight decay: g_eff = g_true + lambda w, with the FP32 master w, applied  */
/*           after unscaling and before the update                              */
/*   Step 1 (next iteration): w16 = nearest binary16 of the master.             */
/* S is a power of two, so multiplying by 1/S is the same number as dividing.  */
/* ------------------------------------------------------------------------- */

typedef struct {
    const or_param* p;
    int32_t n;
    const int64_t* first;      /* prefix sums of numel                */
    float lr, mu, wd, inv_scale;
    uint32_t flag;             /* OR of every range's check result    */
    int32_t kind;              /* OR_OPT_*                            */
    float eps;                 /* Adagrad's denominator term          */
} step_ctx;

static int find_tensor(const step_ctx* s, int64_t gidx) {
    int lo = 0, hi = s->n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (s->first[mid] <= gidx) lo = mid; else hi = mid - 1;
    }
    return lo;
}

static void update_range(int64_t lo, int64_t hi, void* p) {
    step_ctx* s = (step_ctx*)p;
    if (lo >= hi) return;
    int t = find_tensor(s, lo);
    for (int64_t gi = lo; gi < hi; ++gi) {
        while (gi >= s->first[t] + s->p[t].numel) ++t;
        const or_param* q = &s->p[t];
        int64_t i = gi - s->first[t];
        float w = q->master[i];
        float v = q->momentum[i];
        float gs = or_f16_to_f32(q->grad[i]);   /* Step 5: to FP32        */
        float g  = gs * s->inv_scale;           /* Step 5: unscale        */
        float t1 = s->wd * w;                   /* weight decay term      */
        g = g + t1;
        if (s->kind == OR_OPT_ADAGRAD) {
            float t2 = g * g;                   /* accumulate g^2         */
            v = v + t2;
            float r = sqrtf(v);
            float d = r + s->eps;
            float u = g / d;
            float t3 = s->lr * u;
            w = w - t3;
        } else {
            float t2 = s->mu * v;               /* Step 7: momentum       */
            v = t2 + g;
            float step = v;
            if (s->kind == OR_OPT_NESTEROV) {   /* look-ahead: g + mu v   */
                float t4 = s->mu * v;
                step = g + t4;
            }
            float t3 = s->lr * step;            /* Step 7: master update  */
            w = w - t3;
        }
        q->master[i] = w;
        q->momentum[i] = v;
        q->weight16[i] = or_f32_to_f16(w);      /* Step 1: nearest FP16   */
    }
}

static void check_range(int64_t lo, int64_t hi, void* p) {
    step_ctx* s = (step_ctx*)p;
    if (lo >= hi) return;
    int t = find_tensor(s, lo);
    uint32_t bad = 0;
    for (int64_t gi = lo; gi < hi; ++gi) {
        while (gi >= s->first[t] + s->p[t].numel) ++t;
        float g = or_f16_to_f32(s->p[t].grad[gi - s->first[t]]);
        if (isinf(g) || isnan(g)) bad = 1;
    }
    if (bad) __atomic_or_fetch(&s->flag, 1u, __ATOMIC_RELAXED);
}

static int64_t* prefix_numel(const or_param* params, int32_t n) {
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    int64_t acc = 0;
    for (int32_t i = 0; i < n; ++i) { first[i] = acc; acc += params[i].numel; }
    return first;
}

static int64_t total_numel(const int64_t* first, const or_param* params, int32_t n) {
    return first[n - 1] + params[n - 1].numel;
}

uint32_t or_check_overflow(const or_param* params, int32_t n) {
    if (n <= 0) return 0;
    int64_t* first = prefix_numel(params, n);
    step_ctx s = { params, n, first, 0, 0, 0, 0, 0, OR_OPT_SGD, 0.0f };
    parallel_for(total_numel(first, params, n), 1 << 16, check_range, &s);
    free(first);
    return s.flag;
}

void or_sgd_update(const or_param* params, int32_t n, float lr, float momentum,
                   float weight_decay, float inv_scale) {
    if (n <= 0) return;
    int64_t* first = prefix_numel(params, n);
    step_ctx s = { params, n, first, lr, momentum, weight_decay, inv_scale, 0, OR_OPT_SGD, 0.0f };
    parallel_for(total_numel(first, params, n), 1 << 16, update_range, &s);
    free(first);
}

void or_opt_update(const or_param* params, int32_t n, int32_t kind, float lr, float momentum,
                   float weight_decay, float eps, float inv_scale) {
    if (n <= 0) return;
    int64_t* first = prefix_numel(params, n);
    step_ctx s = { params, n, first, lr, momentum, weight_decay, inv_scale, 0, kind, eps };
    parallel_for(total_numel(first, params, n), 1 << 16, update_range, &s);
    free(first);
}

uint32_t or_step_opt(const or_param* params, int32_t n, int32_t kind, float lr, float momentum,
                     float weight_decay, float eps, float inv_scale) {
    uint32_t flag = or_check_overflow(params, n);
    if (!flag) or_opt_update(params, n, kind, lr, momentum, weight_decay, eps, inv_scale);
    return flag;
}

uint32_t or_step(const or_param* params, int32_t n, float lr, float momentum,
                 float weight_decay, float inv_scale) {
    uint32_t flag = or_check_overflow(params, n);
    if (!flag) or_sgd_update(params, n, lr, momentum, weight_decay, inv_scale);
    return flag;
}

/* ------------------------------------------------------------------------- */
/* Loss-scale method 2 ([A] §3.4, the direct statistical approach).            */
/* ------------------------------------------------------------------------- */

float or_absmax_f32(const float* x, int64_t n, float running, uint32_t* nonfinite) {
    float m = running;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(x[i])) {
            if (nonfinite) *nonfinite = 1;
            continue;
        }
        float a = fabsf(x[i]);
        if (a > m) m = a;
    }
    return m;
}

float or_absmax_f16(const uint16_t* x, int64_t n, float running, uint32_t* nonfinite) {
    float m = running;
    for (int64_t i = 0; i < n; ++i) {
        float v = or_f16_to_f32(x[i]);
        if (!isfinite(v)) {
            if (nonfinite) *nonfinite = 1;
            continue;
        }
        float a = fabsf(v);
        if (a > m) m = a;
    }
    return m;
}

float or_scale_from_absmax(float amax, float headroom) {
    /* S = 2^64 down to 1: the first S with S * headroom * amax <= 65504. With
       power-of-two S and headroom both products are exact (or overflow to
       +inf, which fails the test), so the comparison is exact. */
    float x = headroom * amax;
    float S = ldexpf(1.0f, 64);
    while (S > 1.0f && S * x > 65504.0f) S = S * 0.5f;
    return S;
}

/* ------------------------------------------------------------------------- */
/* Loss scaler.                                                                */
/* [A] §3.4 "Choosing the Loss Scaling Factor": method 1 keeps S constant (an  */
/* overflowing step is skipped); method 3 multiplies S by beta = 0.5 and skips */
/* on overflow and multiplies it by alpha = 2 otherwise. [E] "Loss scaling":   */
/* the increase happens after a run of clean steps, which growth_interval      */
/* counts. S stays a power of two, clamped to [1, 2^64].                        */
/* ------------------------------------------------------------------------- */

void or_scaler_init(or_scaler* s, float init_scale, int32_t dynamic, int32_t growth_interval) {
    s->scale = init_scale;
    s->inv_scale = 1.0f / init_scale;
    s->count = 0;
    s->growth_interval = growth_interval;
    s->found_inf = 0;
    s->dynamic = dynamic ? 1u : 0u;
    s->skipped_steps = 0;
}

void or_scaler_update(or_scaler* s) {
    const float lo = 1.0f, hi = ldexpf(1.0f, 64);
    if (s->found_inf) s->skipped_steps += 1;
    if (s->dynamic) {
        if (s->found_inf) {
            s->scale = s->scale * 0.5f;
            if (s->scale < lo) s->scale = lo;
            s->count = 0;
        } else {
            s->count += 1;
            if (s->count >= s->growth_interval) {
                s->scale = s->scale * 2.0f;
                if (s->scale > hi) s->scale = hi;
                s->count = 0;
            }
        }
    }
    s->inv_scale = 1.0f / s->scale;
    s->found_inf = 0;
}

/* ------------------------------------------------------------------------- */
/* Point-wise ops and losses ([A] §3.4: point-wise ops may run in either       */
/* precision; large reductions in FP32 or wider). Evaluated in double here and */
/* rounded once to binary16 (via float, exact for these magnitudes in all but  */
/* double-rounding ties, which the tolerances absorb).                         */
/* ------------------------------------------------------------------------- */

static uint16_t d_to_f16(double v) { return or_f32_to_f16((float)v); }

void or_relu_fwd(const uint16_t* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        float v = or_f16_to_f32(x[i]);
        y[i] = (v > 0.0f || isnan(v)) ? x[i] : (uint16_t)0;
    }
}
void or_relu_bwd(const uint16_t* x, const uint16_t* dy, uint16_t* dx, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        float v = or_f16_to_f32(x[i]);
        dx[i] = (v > 0.0f) ? dy[i] : (uint16_t)0;
    }
}

static const double kInvSqrt2 = 0.70710678118654752440;
static const double kInvSqrt2Pi = 0.39894228040143267794;

typedef struct { const uint16_t *x, *dy; uint16_t* out; } pw_ctx;

static void gelu_f_range(int64_t lo, int64_t hi, void* p) {
    pw_ctx* c = (pw_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) {
        double v = (double)or_f16_to_f32(c->x[i]);
        c->out[i] = d_to_f16(0.5 * v * (1.0 + erf(v * kInvSqrt2)));
    }
}
static void gelu_b_range(int64_t lo, int64_t hi, void* p) {
    pw_ctx* c = (pw_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) {
        double v = (double)or_f16_to_f32(c->x[i]);
        double g = (double)or_f16_to_f32(c->dy[i]);
        double d = 0.5 * (1.0 + erf(v * kInvSqrt2)) + v * kInvSqrt2Pi * exp(-0.5 * v * v);
        c->out[i] = d_to_f16(g * d);
    }
}
void or_gelu_fwd(const uint16_t* x, uint16_t* y, int64_t n) {
    pw_ctx c = { x, NULL, y };
    parallel_for(n, 1 << 14, gelu_f_range, &c);
}
void or_gelu_bwd(const uint16_t* x, const uint16_t* dy, uint16_t* dx, int64_t n) {
    pw_ctx c = { x, dy, dx };
    parallel_for(n, 1 << 14, gelu_b_range, &c);
}

/* L = (1/B) sum_b [ log sum_c exp(z_bc) - z_{b,y_b} ];
 * dL/dz_bc = (softmax(z_b)_c - [c == y_b]) / B;  dz16 = RNE16(S * dL/dz). */
double or_softmax_ce(const uint16_t* logits, const int32_t* labels, int64_t B, int64_t C,
                     double scale, uint16_t* dlogits) {
    double total = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t* z = logits + b * C;
        double mx = -INFINITY;
        for (int64_t c = 0; c < C; ++c) {
            double v = (double)or_f16_to_f32(z[c]);
            if (v > mx) mx = v;
        }
        double se = 0.0;
        for (int64_t c = 0; c < C; ++c) se += exp((double)or_f16_to_f32(z[c]) - mx);
        double lse = mx + log(se);
        total += lse - (double)or_f16_to_f32(z[labels[b]]);
        if (dlogits) {
            for (int64_t c = 0; c < C; ++c) {
                double p = exp((double)or_f16_to_f32(z[c]) - lse);
                double d = (p - (c == labels[b] ? 1.0 : 0.0)) / (double)B;
                dlogits[b * C + c] = d_to_f16(scale * d);
            }
        }
    }
    return total / (double)B;
}

/* L = c * (1/(M N)) sum (y - t)^2;  dL/dy = c * 2 (y - t) / (M N). */
double or_mse(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, double c,
              double scale, uint16_t* dy) {
    double total = 0.0;
    double mn = (double)M * (double)N;
    for (int64_t i = 0; i < M * N; ++i) {
        double d = (double)or_f16_to_f32(y[i]) - (double)or_f16_to_f32(t[i]);
        total += d * d;
        if (dy) dy[i] = d_to_f16(scale * (c * 2.0 * d / mn));
    }
    return c * total / mn;
}

void or_mse_grad_f64(const uint16_t* y, const uint16_t* t, int64_t M_rows, int64_t N,
                     int64_t M_total, double c, double* dy) {
    double mn = (double)M_total * (double)N;
    for (int64_t i = 0; i < M_rows * N; ++i) {
        double d = (double)or_f16_to_f32(y[i]) - (double)or_f16_to_f32(t[i]);
        dy[i] = c * 2.0 * d / mn;
    }
}

/* ------------------------------------------------------------------------- */
/* Large reductions ([A] §3.4 "FP16 Arithmetic with FP32 Accumulation": batch-  */
/* normalization statistics and softmax sums are summed in FP32 from binary16   */
/* tensors, and the normalization arithmetic is FP32).                         */
/* ------------------------------------------------------------------------- */

void or_bn_stats(const uint16_t* x, int64_t rows, int64_t C, int64_t ldx, double* mean, double* var) {
    for (int64_t c = 0; c < C; ++c) { mean[c] = 0.0; var[c] = 0.0; }
    if (rows <= 0) return;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < C; ++c) mean[c] += (double)or_f16_to_f32(x[r * ldx + c]);
    for (int64_t c = 0; c < C; ++c) mean[c] /= (double)rows;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < C; ++c) {
            double d = (double)or_f16_to_f32(x[r * ldx + c]) - mean[c];
            var[c] += d * d;
        }
    for (int64_t c = 0; c < C; ++c) var[c] /= (double)rows;
}

void or_bn_apply(const uint16_t* x, int64_t rows, int64_t C, int64_t ldx, const float* mean,
                 const float* var, const float* gamma, const float* beta, float eps,
                 uint16_t* y, int64_t ldy) {
    for (int64_t c = 0; c < C; ++c) {
        float s = var[c] + eps;
        float r = sqrtf(s);
        float inv = 1.0f / r;
        for (int64_t i = 0; i < rows; ++i) {
            float t = or_f16_to_f32(x[i * ldx + c]) - mean[c];
            float u = t * inv;
            float v = u * gamma[c];
            float w = v + beta[c];
            y[i * ldy + c] = or_f32_to_f16(w);
        }
    }
}

typedef struct { const uint16_t* x; uint16_t* y; int64_t cols, ldx, ldy; } sm_ctx;

static void softmax_rows(int64_t lo, int64_t hi, void* p) {
    sm_ctx* c = (sm_ctx*)p;
    for (int64_t r = lo; r < hi; ++r) {
        const uint16_t* xr = c->x + r * c->ldx;
        uint16_t* yr = c->y + r * c->ldy;
        double m = -INFINITY;
        int bad = 0;
        for (int64_t j = 0; j < c->cols; ++j) {
            double v = (double)or_f16_to_f32(xr[j]);
            if (isnan(v) || v == INFINITY) bad = 1;
            if (v > m) m = v;
        }
        double s = 0.0;
        for (int64_t j = 0; j < c->cols; ++j) s += exp((double)or_f16_to_f32(xr[j]) - m);
        for (int64_t j = 0; j < c->cols; ++j)
            yr[j] = bad ? d_to_f16(NAN) : d_to_f16(exp((double)or_f16_to_f32(xr[j]) - m) / s);
    }
}

void or_softmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy) {
    sm_ctx c = {x, y, cols, ldx, ldy};
    parallel_for(rows, 1, softmax_rows, &c);
}
