/*
 * Plain CPU oracle for the mixed-precision training hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this code; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no source, header, table or helper with the
 * HIP path.
 *
 * Sources cited in this file (page titles as published):
 *   [A]  "Mixed Precision Training" — long-form analysis page
 *        (paper-graph-ui.vercel.app), sections §2, §3.2, §3.4.
 *   [E]  "Mixed Precision Training" — explainer page (azimuth.plus),
 *        sections "The problem", "Loss scaling", "Which operations stay in FP32?".
 *
 * Every floating-point step is one IEEE operation in the stated precision;
 * the translation unit is built with -ffp-contract=off and without
 * fast-math so that no multiply-add is fused.
 */
#ifndef MP_ORACLE_H
#define MP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- binary16 codec, [A] §2 and §3.4 "FP32 Master Copy of Weights" ---- */
float    or_f16_to_f32(uint16_t h);
uint16_t or_f32_to_f16(float x);
void     or_f32_to_f16_array(const float* x, uint16_t* h, int64_t n);
void     or_f16_to_f32_array(const uint16_t* h, float* x, int64_t n);
/* All 2^32 float32 bit patterns in [lo, hi) -> binary16, written to out[0..hi-lo). */
void     or_f32bits_to_f16_range(uint64_t lo, uint64_t hi, uint16_t* out);

/* ---- dot-product layers, [A] §3.4 "FP16 Arithmetic with FP32 Accumulation" ----
 * Every output is acc = 0; acc = acc + a_r * b_r for r ascending, in FP32.
 * out_f16 != 0 rounds each output to binary16 (bit patterns in a uint16 array),
 * otherwise float outputs are written.                                        */
void or_linear_fwd(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                   void* Y, int64_t ldy, int out_f16, int64_t M, int64_t N, int64_t K);
void or_linear_dgrad(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                     void* dX, int64_t lddx, int out_f16, int64_t M, int64_t N, int64_t K);
void or_linear_wgrad(const uint16_t* dY, int64_t lddy, const uint16_t* X, int64_t ldx,
                     void* dW, int64_t lddw, int out_f16, int64_t M, int64_t N, int64_t K);
/* The same three definitions evaluated only at the listed output coordinates. */
void or_linear_fwd_at(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                      int64_t K, const int64_t* rows, const int64_t* cols, int64_t count,
                      float* out);
void or_linear_dgrad_at(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                        int64_t N, const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out);
void or_linear_wgrad_at(const uint16_t* dY, int64_t lddy, const uint16_t* X, int64_t ldx,
                        int64_t M, const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out);

/* ---- optimizer sweep, [A] §3.4 "The Integrated Training Procedure", Steps 5-7 ---- */
typedef struct {
    float*          master;    /* FP32 master weights, updated in place      */
    float*          momentum;  /* FP32 velocity, updated in place            */
    const uint16_t* grad;      /* loss-scaled binary16 weight gradient       */
    uint16_t*       weight16;  /* binary16 working copy, rewritten           */
    int64_t         numel;
} or_param;

/* Step 6: 1 if any gradient element of any tensor is +-inf or NaN. */
uint32_t or_check_overflow(const or_param* params, int32_t n);
/* Steps 5 and 7 (+ weight decay) for every element, unconditionally. */
void or_sgd_update(const or_param* params, int32_t n, float lr, float momentum,
                   float weight_decay, float inv_scale);
/* Steps 5-7 together: check first, update only when the check is clean.
 * Returns the flag. */
uint32_t or_step(const or_param* params, int32_t n, float lr, float momentum,
                 float weight_decay, float inv_scale);

/* ---- optimizer variants of the same sweep ----
 * The pages name the optimizers their experiments used but print no update
 * rule for them: Nesterov-momentum SGD ([A] §3.1 "Empirical validation
 * (Figure 2a)", §4.3, §6.4) and Adagrad ([A] §4.5 (Figure 5), §6.4). The rules
 * below are the textbook forms (readings, see the test-suite's pins):
 *   OR_OPT_SGD       v = mu v + g;           w = w - lr v
 *   OR_OPT_NESTEROV  v = mu v + g;           w = w - lr (g + mu v)
 *   OR_OPT_ADAGRAD   G = G + g g;            w = w - lr (g / (sqrt(G) + eps))
 * with g = g16 / S + weight_decay w, every operation one IEEE FP32 rounding in
 * the order written (sqrt and division correctly rounded), `momentum` holding
 * v or G. Steps 5, 6 and 1 are as for or_step.                              */
enum { OR_OPT_SGD = 0, OR_OPT_NESTEROV = 1, OR_OPT_ADAGRAD = 2 };
void or_opt_update(const or_param* params, int32_t n, int32_t kind, float lr, float momentum,
                   float weight_decay, float eps, float inv_scale);
uint32_t or_step_opt(const or_param* params, int32_t n, int32_t kind, float lr, float momentum,
                     float weight_decay, float eps, float inv_scale);

/* ---- loss-scale method 2, [A] §3.4 "Choosing the scaling factor — the direct
 * statistical approach" and the gradient-statistics recipe after it:
 * record g_max = max |gradient| over all layers (and iterations), then
 * S = 65504 / (h g_max), h = 2 leaving one bit of headroom.
 * or_absmax_*: max(running, max |x| over the finite elements of x); any
 * +-inf/NaN element sets *nonfinite (when not NULL) and is left out.
 * or_scale_from_absmax: the largest power of two S with S h amax <= 65504
 * (a power of two keeps the unscale exact), clamped to [1, 2^64]; h must be
 * a power of two, so every product here is exact.                            */
float or_absmax_f32(const float* x, int64_t n, float running, uint32_t* nonfinite);
float or_absmax_f16(const uint16_t* x, int64_t n, float running, uint32_t* nonfinite);
float or_scale_from_absmax(float amax, float headroom);

/* ---- loss scaler, [A] §3.4 "Choosing the Loss Scaling Factor" ---- */
typedef struct {
    float    scale;
    float    inv_scale;
    int32_t  count;            /* consecutive clean steps since the last change */
    int32_t  growth_interval;  /* clean steps before the scale doubles          */
    uint32_t found_inf;
    uint32_t dynamic;
    uint32_t skipped_steps;
} or_scaler;

void or_scaler_init(or_scaler* s, float init_scale, int32_t dynamic, int32_t growth_interval);
void or_scaler_update(or_scaler* s);

/* ---- point-wise ops and losses, [A] §3.4 (point-wise ops, large reductions) ----
 * Computed in double from the binary16 inputs, rounded once to binary16.      */
void or_relu_fwd(const uint16_t* x, uint16_t* y, int64_t n);
void or_relu_bwd(const uint16_t* x, const uint16_t* dy, uint16_t* dx, int64_t n);
void or_gelu_fwd(const uint16_t* x, uint16_t* y, int64_t n);
void or_gelu_bwd(const uint16_t* x, const uint16_t* dy, uint16_t* dx, int64_t n);
/* dY[b, c] = RNE16(S * dL/dlogits), L = mean over the batch of the cross-entropy;
 * returns L.                                                                    */
double or_softmax_ce(const uint16_t* logits, const int32_t* labels, int64_t B, int64_t C,
                     double scale, uint16_t* dlogits);
/* L = c * mean((y - t)^2) over all M*N elements; dY = RNE16(S * dL/dy); returns L. */
double or_mse(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, double c,
              double scale, uint16_t* dy);
/* Same loss gradient without the final rounding (FP64), for calibration. */
void or_mse_grad_f64(const uint16_t* y, const uint16_t* t, int64_t M_rows, int64_t N,
                     int64_t M_total, double c, double* dy);

/* ---- large reductions, [A] §3.4 "FP16 Arithmetic with FP32 Accumulation" (large
 * reductions: batch-normalization statistics and softmax sums in FP32 from binary16
 * tensors). The statistics and the softmax are evaluated in double (their exact
 * values, to which a device's FP32 reductions in any order are compared within a
 * bound); the normalization is element-wise, so it follows the pages' FP32 with one
 * rounding per operation in a fixed order.                                       */
/* Per-channel mean and population variance over the rows of x[rows, C] (row pitch
 * ldx elements): mean = sum(x) / rows, var = sum((x - mean)^2) / rows (two passes). */
void or_bn_stats(const uint16_t* x, int64_t rows, int64_t C, int64_t ldx, double* mean, double* var);
/* y = RNE16(w) with, per channel c, s = var + eps, r = sqrt(s), inv = 1 / r, and per
 * element t = x - mean, u = t * inv, v = u * gamma, w = v + beta: FP32, one rounding
 * per operation, in this order.                                                 */
void or_bn_apply(const uint16_t* x, int64_t rows, int64_t C, int64_t ldx, const float* mean,
                 const float* var, const float* gamma, const float* beta, float eps,
                 uint16_t* y, int64_t ldy);
/* Row-wise softmax of x[rows, cols]: y = RNE16(exp(x - m) / sum exp(x - m)), m the row
 * maximum, in double. A row with a NaN or +inf gives NaN throughout; -inf gives 0
 * (a row of only -inf gives NaN).                                               */
void or_softmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy);

/* Worker threads used by the parallel loops (0 = all online CPUs). */
void or_set_threads(int32_t n);
int32_t or_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
