/*
 * libmp — the mixed-precision training hot path on AMD Instinct MI355X (gfx950).
 *
 * The method ("Mixed Precision Training", long-form analysis page,
 * paper-graph-ui.vercel.app, §3.2 and §3.4 "The Integrated Training
 * Procedure", Steps 1-7):
 *   binary16 weights, activations and gradients; dot products with binary16
 *   inputs and FP32 accumulation; an FP32 master copy of every weight; the
 *   loss multiplied by a scale S before back-propagation; weight gradients
 *   divided by S, checked for inf/NaN, the whole update skipped on overflow,
 *   otherwise SGD with momentum (and coupled weight decay) on the FP32
 *   masters, which are rounded back to binary16; S adjusted afterwards.
 *
 * Conventions shared by every entry point
 *   - Device pointers unless stated otherwise. binary16 data is passed as
 *     uint16_t bit patterns (IEEE 754 binary16), FP32 as float.
 *   - Matrices are row-major with an explicit leading dimension (elements
 *     between consecutive rows). Weights follow the out x in convention:
 *     W[N, K] maps K inputs to N outputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is stream-ordered and asynchronous: no entry point
 *     synchronises the host or reads device results on the host.
 *   - Argument errors are detected on the host before anything is launched
 *     and returned as a status; a launch failure returns MP_ERR_HIP and
 *     mp_last_hip_error() names it. Faults inside kernels surface at the
 *     caller's next synchronisation. No C++ exception crosses this ABI.
 *   - A zero M, N, numel or list length is a successful no-op; K = 0 (an
 *     empty reduction) writes zeros.
 *   - The caller owns every data buffer and every mp_scaler. The library
 *     owns only mp_param_list and mp_tensor_list handles (created and
 *     destroyed here).
 *   - Outputs must not alias inputs, except that master weights and momentum
 *     are updated in place by design.
 *   - Calls on different streams are safe when their buffers are disjoint;
 *     one mp_scaler belongs to one stream at a time.
 *   - Device words the kernels update atomically or read whole (an
 *     mp_scaler, wgrad's found_inf, the |g| maximum and its non-finite flag,
 *     a loss value) must be 4-byte aligned, and workspaces aligned as each
 *     call states; a misaligned one is MP_ERR_INVALID_ARGUMENT. Data buffers
 *     may be unaligned (such calls take an element-wise path).
 */
#ifndef MP_H
#define MP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MP_OK = 0,
    MP_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad leading dim, bad scale */
    MP_ERR_MISALIGNED = 2,         /* reserved: every entry point has an unaligned path      */
    MP_ERR_UNSUPPORTED = 3,        /* a flag or dtype that is not implemented                 */
    MP_ERR_HIP = 4,                /* a HIP runtime call failed; see mp_last_hip_error()     */
    MP_ERR_OUT_OF_MEMORY = 5       /* allocation of a library-owned handle failed            */
} mp_status;

typedef enum { MP_F16 = 0, MP_F32 = 1 } mp_dtype;

/* Loss-scaler state, resident in device memory (caller-allocated, 32 bytes,
 * 4-byte aligned). `scale` is always a power of two in [1, 2^64];
 * `inv_scale` is its exact reciprocal. `found_inf` is the overflow flag of
 * the step in progress: it must be 0 when a step starts (mp_scaler_init and
 * mp_scaler_update leave it 0) and only ever goes 0 -> 1 during a step. */
typedef struct mp_scaler {
    float    scale;
    float    inv_scale;
    int32_t  count;            /* consecutive clean steps since the last change */
    int32_t  growth_interval;  /* clean steps after which S doubles (dynamic)   */
    uint32_t found_inf;
    uint32_t dynamic;          /* 0: constant S (method 1); 1: dynamic (method 3) */
    uint32_t skipped_steps;    /* steps skipped because of overflow             */
    uint32_t reserved;
} mp_scaler;

/* SGD-with-momentum hyper-parameters, passed by value. */
typedef struct mp_sgd {
    float lr;
    float momentum;
    float weight_decay;
} mp_sgd;

/* Update rules of the sweep (mp_step_opt). The pages name Nesterov-momentum
 * SGD and Adagrad as the optimizers of their experiments (the analysis page,
 * §3.1 "Empirical validation (Figure 2a)", §4.5 (Figure 5), §6.4) without
 * printing the rules; these are the textbook forms:
 *   MP_OPT_SGD       v = mu v + g;  w = w - lr v
 *   MP_OPT_NESTEROV  v = mu v + g;  w = w - lr (g + mu v)
 *   MP_OPT_ADAGRAD   G = G + g g;   w = w - lr (g / (sqrt(G) + eps))
 * with g = grad16 / S + weight_decay w, one FP32 rounding per operation in
 * the order written (square root and division correctly rounded). */
typedef enum { MP_OPT_SGD = 0, MP_OPT_NESTEROV = 1, MP_OPT_ADAGRAD = 2 } mp_opt_kind;

/* Optimizer hyper-parameters, passed by value. momentum is ignored by
 * Adagrad, eps by the others. */
typedef struct mp_optim {
    int32_t kind;              /* mp_opt_kind */
    float   lr;
    float   momentum;
    float   weight_decay;
    float   eps;               /* Adagrad: > 0 */
} mp_optim;

/* One parameter tensor of the optimizer sweep (host-side description). */
typedef struct mp_param {
    float*          master;    /* FP32 master weights [numel], updated in place */
    float*          momentum;  /* FP32 optimizer state [numel], updated in place:
                                  the velocity v, or Adagrad's sum G of squares */
    const uint16_t* grad;      /* binary16 loss-scaled gradient [numel], read   */
    uint16_t*       weight16;  /* binary16 working copy [numel], rewritten      */
    int64_t         numel;
} mp_param;

typedef struct mp_param_list mp_param_list;

/* A list of device tensors of one element type (FP32 or binary16), for the
 * gradient statistics of loss-scale method 2. */
typedef struct mp_tensor_list mp_tensor_list;

typedef void* mp_stream;

/* ------------------------------------------------------------------------
 * Dot-product layers: binary16 inputs, exact products, FP32 accumulation,
 * output rounded to nearest-even binary16 (overflow gives +-inf, never a
 * saturated 65504) or written as FP32. Source: the analysis page, §3.4
 * "FP16 Arithmetic with FP32 Accumulation" and "The Integrated Training
 * Procedure", Steps 2 and 4. Summation order inside a dot product is the
 * kernel's (tiled); results agree with an ascending-order FP32 sum within
 * the rounding error of FP32 accumulation.
 * ------------------------------------------------------------------------ */

/* Point-wise activation of the fused epilogues and of mp_act_fwd/bwd. */
typedef enum { MP_ACT_RELU = 0, MP_ACT_GELU = 1 } mp_act;

/* Forward: Y[M, N] = X[M, K] . W[N, K]^T.
 * X: ldx >= K; W: ldw >= K; Y: ldy >= N, element type y_dtype.
 * Errors: MP_ERR_INVALID_ARGUMENT for negative sizes, a leading dimension
 * smaller than its row, or a null pointer with a non-empty matrix. */
mp_status mp_linear_fwd(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                        void* Y, int64_t ldy, mp_dtype y_dtype,
                        int64_t M, int64_t N, int64_t K, mp_stream stream);

/* Activation gradient: dX[M, K] = dY[M, N] . W[N, K]. The result stays
 * multiplied by the loss scale (Step 4: activation gradients are never
 * unscaled). dY: lddy >= N; W: ldw >= K; dX: lddx >= K. */
mp_status mp_linear_dgrad(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                          void* dX, int64_t lddx, mp_dtype dx_dtype,
                          int64_t M, int64_t N, int64_t K, mp_stream stream);

/* Weight gradient: dW[N, K] = dY[M, N]^T . X[M, K] (overwritten, not
 * accumulated). dY: lddy >= N; X: ldx >= K; dW: lddw >= K.
 * found_inf (nullable, device uint32): when given, the kernel ORs 1 into it
 * if any stored binary16 output is +-inf or NaN, so that mp_step can be
 * called with MP_GRADS_PRECHECKED (Step 6 fused into the producer). With an
 * FP32 output found_inf must be NULL (MP_ERR_INVALID_ARGUMENT otherwise). */
mp_status mp_linear_wgrad(const uint16_t* dY, int64_t lddy, const uint16_t* X, int64_t ldx,
                          void* dW, int64_t lddw, mp_dtype dw_dtype,
                          int64_t M, int64_t N, int64_t K, uint32_t* found_inf,
                          mp_stream stream);

/* Forward of an activated layer in one pass: Z[M, N] = RNE16(X . W^T) as in
 * mp_linear_fwd with a binary16 output, and H = act(Z) elementwise, both
 * stored. The bits of Z and H equal those of mp_linear_fwd followed by
 * mp_act_fwd; the activation is applied while the output tile is written,
 * so Z is not read back from memory. Source: the analysis page, §3.4 "The
 * Integrated Training Procedure", Step 2 (the forward pass, whose point-wise
 * operations are memory-bound and may run in binary16 or FP32).
 * X: ldx >= K; W: ldw >= K; Z: ldz >= N; H: ldh >= N. Z and H must not
 * overlap each other or the inputs.
 * Errors: MP_ERR_INVALID_ARGUMENT for an unknown kind and as mp_linear_fwd. */
mp_status mp_linear_fwd_act(mp_act kind, const uint16_t* X, int64_t ldx, const uint16_t* W,
                            int64_t ldw, uint16_t* Z, int64_t ldz, uint16_t* H, int64_t ldh,
                            int64_t M, int64_t N, int64_t K, mp_stream stream);

/* Activation gradient through an activated layer in one pass:
 * dZ[M, K] = RNE16(act'(Z) * RNE16(dY . W)), i.e. the bits of mp_linear_dgrad
 * (binary16 output) followed by mp_act_bwd with the saved pre-activation Z,
 * without storing the intermediate. Stays multiplied by the loss scale.
 * Source: the analysis page, §3.4 "The Integrated Training Procedure",
 * Step 4. dY: lddy >= N; W: ldw >= K; Z: ldz >= K; dZ: lddz >= K. dZ must
 * not overlap the inputs.
 * Errors: MP_ERR_INVALID_ARGUMENT for an unknown kind and as mp_linear_dgrad. */
mp_status mp_linear_dgrad_act(mp_act kind, const uint16_t* dY, int64_t lddy, const uint16_t* W,
                              int64_t ldw, const uint16_t* Z, int64_t ldz, uint16_t* dZ,
                              int64_t lddz, int64_t M, int64_t N, int64_t K, mp_stream stream);

/* Forward of an activated layer that keeps the activation's derivative instead
 * of the pre-activation: with Z = RNE16(X . W^T) (not stored), H = act(Z) and
 * D = RNE16(act'(Z)), both [M, N] binary16: the bits of mp_act_fwd(Z) and of
 * mp_act_bwd(Z, 1.0), from one evaluation of the activation. The layer's
 * backward then needs only D (mp_linear_dgrad_mul): D takes the bytes Z would.
 * Source: as mp_linear_fwd_act (Steps 2 and 4 of the analysis page's §3.4).
 * X: ldx >= K; W: ldw >= K; H: ldh >= N; D: ldd >= N. H and D must not overlap
 * each other or the inputs.
 * Errors: MP_ERR_INVALID_ARGUMENT for an unknown kind and as mp_linear_fwd. */
mp_status mp_linear_fwd_act_deriv(mp_act kind, const uint16_t* X, int64_t ldx, const uint16_t* W,
                                  int64_t ldw, uint16_t* H, int64_t ldh, uint16_t* D, int64_t ldd,
                                  int64_t M, int64_t N, int64_t K, mp_stream stream);

/* Activation gradient with the saved derivative:
 * dZ[M, K] = RNE16(f32(RNE16(dY . W)) * f32(D)), one FP32 product of the
 * binary16 dgrad output and D from mp_linear_fwd_act_deriv, rounded once (an
 * IEEE product: signs, zeros, infinities and NaN as FP32 multiplication gives
 * them). Against mp_linear_dgrad_act it adds the rounding of act' to binary16,
 * so the result is within two binary16 ulps of the exact act'(Z) * RNE16(dY.W).
 * Stays multiplied by the loss scale. dY: lddy >= N; W: ldw >= K; D: ldd >= K;
 * dZ: lddz >= K. dZ must not overlap the inputs.
 * Errors: as mp_linear_dgrad. */
mp_status mp_linear_dgrad_mul(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                              const uint16_t* D, int64_t ldd, uint16_t* dZ, int64_t lddz, int64_t M,
                              int64_t N, int64_t K, mp_stream stream);

/* ------------------------------------------------------------------------
 * The optimizer sweep over a ragged list of parameter tensors.
 * Source: the analysis page, §3.4 "The Integrated Training Procedure",
 * Steps 5-7 and the weight-decay paragraph.
 * ------------------------------------------------------------------------ */

/* Copies the n descriptors (host array, read during the call only) into a
 * library-owned device table and chunk map. Tensors may have any length; a
 * tensor whose four base addresses are all 16-byte aligned takes the
 * vectorised path, any other tensor a scalar path with the same results.
 * Every non-empty tensor needs four non-null pointers; empty tensors are
 * allowed and ignored. The list remembers the pointers, not the data: the
 * buffers must stay allocated while the list is used.
 * Errors: MP_ERR_INVALID_ARGUMENT (n < 0, out == NULL, null pointer with
 * numel > 0, numel < 0), MP_ERR_OUT_OF_MEMORY, MP_ERR_HIP. */
mp_status mp_param_list_create(const mp_param* host_params, int32_t n,
                               mp_param_list** out, mp_stream stream);

/* Frees the handle after the work queued on `stream` at creation has
 * finished (it synchronises that stream). NULL is accepted. */
mp_status mp_param_list_destroy(mp_param_list* list);

/* Total number of elements in the list (host value). */
int64_t mp_param_list_numel(const mp_param_list* list);

enum {
    MP_STEP_DEFAULT = 0,
    /* Skip the check pass: the gradients were produced by mp_linear_wgrad
     * with found_inf = &scaler->found_inf, which already holds the flag. */
    MP_GRADS_PRECHECKED = 1u << 0,
    /* Only the check pass (Step 6): OR the overflow flag into scaler->found_inf
     * and write nothing else (no unscale, no update). With
     * MP_GRADS_PRECHECKED as well the call does nothing. */
    MP_CHECK_ONLY = 1u << 1
};

/* One optimizer step. For every element of every tensor, in FP32 with one
 * rounding per operation and no fused multiply-add:
 *     g  = f32(grad16) * inv_scale         (Step 5: unscale, exact)
 *     g  = g + weight_decay * master       (coupled L2 on the FP32 master)
 *     v  = momentum * v + g                (Step 7)
 *     w  = w - lr * v                      (Step 7)
 *     weight16 = round-to-nearest-even binary16 of w   (Step 1)
 * but only if no gradient element of any tensor is +-inf or NaN (Step 6).
 * Otherwise nothing is written (masters, momentum and binary16 copies keep
 * their bits) and scaler->found_inf is 1 afterwards. inv_scale and the flag
 * are read from `scaler` on the device. The gradients are never written.
 * Implementation: a read-only check pass over all gradients (skipped with
 * MP_GRADS_PRECHECKED) followed by one fused update pass that exits at once
 * when the flag is set.
 * Errors: MP_ERR_INVALID_ARGUMENT (list or scaler NULL), MP_ERR_UNSUPPORTED
 * (unknown flag bits), MP_ERR_HIP. */
mp_status mp_step(const mp_param_list* list, mp_sgd hyper, mp_scaler* scaler,
                  uint32_t flags, mp_stream stream);

/* The sweep of mp_step with the update rule hyper.kind (see mp_opt_kind):
 * Steps 5-7 and 1 as for mp_step, the same skip on overflow (nothing written,
 * Adagrad's sum included), the same check pass and MP_GRADS_PRECHECKED flag.
 * MP_OPT_SGD gives the bits of mp_step.
 * Errors: MP_ERR_INVALID_ARGUMENT (list or scaler NULL, unknown kind,
 * Adagrad with eps not > 0 or not finite), MP_ERR_UNSUPPORTED (unknown flag
 * bits), MP_ERR_HIP. */
mp_status mp_step_opt(const mp_param_list* list, mp_optim hyper, mp_scaler* scaler,
                      uint32_t flags, mp_stream stream);

/* ------------------------------------------------------------------------
 * Loss scaler. Source: the analysis page, §3.4 "Choosing the Loss Scaling
 * Factor": method 1 (constant S, an overflowing step is skipped) and
 * method 3 (dynamic: on overflow skip and halve S; after growth_interval
 * consecutive clean steps double S).
 * ------------------------------------------------------------------------ */

/* Writes a fresh state: scale = init_scale, count = 0, found_inf = 0,
 * skipped_steps = 0. init_scale must be a power of two in [1, 2^64];
 * growth_interval >= 1 when dynamic. */
mp_status mp_scaler_init(mp_scaler* scaler, float init_scale, int32_t dynamic,
                         int32_t growth_interval, mp_stream stream);

/* Consumes found_inf of the finished step: on overflow skipped_steps += 1
 * and, when dynamic, scale halves (not below 1) and count = 0; on a clean
 * dynamic step count += 1 and, when it reaches growth_interval, scale
 * doubles (not above 2^64) and count = 0. Then inv_scale = 1/scale and
 * found_inf = 0. One single-lane kernel; no host round trip. */
mp_status mp_scaler_update(mp_scaler* scaler, mp_stream stream);

/* ------------------------------------------------------------------------
 * Loss-scale method 2. Source: the analysis page, §3.4 "Choosing the scaling
 * factor — the direct statistical approach" and the gradient-statistics
 * recipe after it: record g_max = max |gradient| over all layers during a
 * short FP32 run, then S = 65504 / g_max, or 65504 / (2 g_max) to leave one
 * bit of headroom.
 * ------------------------------------------------------------------------ */

/* Copies n (pointer, length) pairs (host arrays, read during the call) into a
 * library-owned device table. dtype: MP_F32 or MP_F16 (binary16 bits) for
 * every tensor. The list remembers pointers, not data.
 * Errors: MP_ERR_INVALID_ARGUMENT (n < 0, out NULL, null pointer with
 * numel > 0, numel < 0, other dtype), MP_ERR_OUT_OF_MEMORY, MP_ERR_HIP. */
mp_status mp_tensor_list_create(const void* const* host_ptrs, const int64_t* host_numel, int32_t n,
                                mp_dtype dtype, mp_tensor_list** out, mp_stream stream);
/* Frees the handle after the work queued on its stream at creation (it
 * synchronises that stream). NULL is accepted. */
mp_status mp_tensor_list_destroy(mp_tensor_list* list);

/* *amax (device FP32, >= 0 on entry) = max(*amax, |x|) over the finite
 * elements of every tensor: a running maximum over layers and iterations.
 * Elements that are +-inf or NaN are left out and, when nonfinite (device
 * uint32) is not NULL, OR 1 into it. Exact (no rounding is involved).
 * Errors: MP_ERR_INVALID_ARGUMENT (list or amax NULL), MP_ERR_HIP. */
mp_status mp_absmax(const mp_tensor_list* list, float* amax, uint32_t* nonfinite, mp_stream stream);

/* Writes a fresh scaler whose scale is the largest power of two S with
 * S * headroom * (*amax) <= 65504, clamped to [1, 2^64] (a power of two keeps
 * the unscale exact; headroom 2 is the page's one bit of headroom); count,
 * found_inf and skipped_steps are 0. amax is read on the device.
 * headroom must be a power of two in [1, 2^64]; growth_interval >= 1 when
 * dynamic. Errors: MP_ERR_INVALID_ARGUMENT. */
mp_status mp_scaler_init_from_absmax(mp_scaler* scaler, const float* amax, float headroom,
                                     int32_t dynamic, int32_t growth_interval, mp_stream stream);

/* ------------------------------------------------------------------------
 * Large reductions. Source: the analysis page, §3.4 "FP16 Arithmetic with
 * FP32 Accumulation": batch normalization's mean and variance and the
 * softmax normalization constant are summed in FP32 from binary16 tensors,
 * all of their arithmetic is FP32, and binary16 results are written back.
 * Matrices are row-major with a row pitch (ld*) in elements, ld >= columns.
 * The sums run in a fixed order, so results do not vary from run to run;
 * that order is not the sequential one, so they are not bit-equal to a
 * sequential FP32 sum. Every entry point is asynchronous on `stream`.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace mp_bn_stats needs for these sizes (0 when there
 * is nothing to do). */
size_t mp_bn_stats_workspace(int64_t rows, int64_t channels);

/* Batch-normalization statistics of x[rows, channels] (binary16; channels
 * contiguous, e.g. NHWC with rows = N*H*W): per channel, mean = sum(x) / rows
 * and the population variance var = sum((x - mean)^2) / rows, written as FP32
 * to the device arrays mean[channels] and var[channels]. Computed in FP32 with
 * per-thread sums of shifted values (the shift is one of the thread's own
 * values) and Chan's pairwise merge, in a fixed order.
 * `workspace` is caller-owned device memory of at least
 * mp_bn_stats_workspace(rows, channels) bytes, 4-byte aligned, overwritten.
 * Errors: MP_ERR_INVALID_ARGUMENT (rows < 1, channels < 0, ldx < channels, a
 * null pointer or too small or misaligned a workspace when channels > 0),
 * MP_ERR_HIP. */
mp_status mp_bn_stats(const uint16_t* x, int64_t rows, int64_t channels, int64_t ldx, float* mean,
                      float* var, void* workspace, size_t workspace_bytes, mp_stream stream);

/* Batch-normalization: y = RNE16(((x - mean) * inv) * gamma + beta) with
 * inv = 1 / sqrt(var + eps) per channel: FP32, one rounding per operation in
 * this order (correctly rounded square root and division), then round to
 * nearest even binary16. mean, var, gamma, beta: device FP32 [channels].
 * x and y may not overlap unless x == y with ldx == ldy.
 * Errors: MP_ERR_INVALID_ARGUMENT (negative sizes, ldx or ldy < channels, a
 * null pointer with rows * channels > 0), MP_ERR_HIP. */
mp_status mp_bn_apply(const uint16_t* x, int64_t rows, int64_t channels, int64_t ldx, const float* mean,
                      const float* var, const float* gamma, const float* beta, float eps, uint16_t* y,
                      int64_t ldy, mp_stream stream);

/* Bytes of device workspace mp_softmax needs for these sizes (0 when there is
 * nothing to do). */
size_t mp_softmax_workspace(int64_t rows, int64_t cols);

/* Row-wise softmax of x[rows, cols] (binary16): y = RNE16(exp(x - m) / s), m
 * the row maximum and s the sum of exp(x - m) over the row, in FP32 (the
 * quotient as exp(x - m) * (1 / s)). Rows are cut into segments merged in a
 * fixed order. A row containing NaN or +inf gives NaN throughout; -inf entries
 * give 0, and a row of only -inf gives NaN. `workspace`: caller-owned device
 * memory of at least mp_softmax_workspace(rows, cols) bytes, 8-byte aligned,
 * overwritten. x and y may be the same matrix (ldx == ldy); no other overlap.
 * Two forms, chosen per call from the sizes: when x and y are distinct,
 * 16-byte aligned with pitches that are multiples of 8, and every row fits in
 * at most 256 blocks of 204,800 values with the whole grid at most one block
 * per compute unit, x is read once (each block keeps its segment on chip and
 * exchanges its (max, sum) through the workspace); otherwise a two-pass form
 * reads x twice; so does a call made while the stream is being captured into
 * a graph (the single-read form's per-call tag would repeat on every replay).
 * The result does not depend on timing, but the forms cut rows differently,
 * so their outputs may differ in the last bit. Calls that share a workspace
 * must not overlap.
 * Errors: MP_ERR_INVALID_ARGUMENT (negative sizes, rows > 2^31 - 1, ldx or ldy
 * < cols, a null pointer or too small or misaligned a workspace when
 * rows * cols > 0), MP_ERR_HIP. */
mp_status mp_softmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, mp_stream stream);

/* Tuning of mp_softmax's single-read form: how long, in microseconds, a block
 * waits for the (max, sum) of its row's other blocks before computing the
 * missing ones itself from x (default 200; at most 100000; 0: never wait,
 * every block computes every other segment's pair). The wait ends either way,
 * so a block that is not resident yet costs time, never progress, and every
 * setting gives the same bits. Process-wide; applies to later calls. A
 * negative value only queries. Returns the previous setting. */
int64_t mp_softmax_wait_us(int64_t us);

/* ------------------------------------------------------------------------
 * Auxiliary steps that a full training step needs around the hot path.
 * Point-wise ops run in FP32 on binary16 data; the losses reduce in FP32
 * (the analysis page, §3.4: point-wise ops in either precision, large
 * reductions in FP32). Loss gradients are multiplied by the device-resident
 * scale S in FP32 and rounded once to binary16 (Step 3).
 * ------------------------------------------------------------------------ */

/* w16[i] = round-to-nearest-even binary16 of w32[i] (Step 1 at init). */
mp_status mp_round_f32_to_f16(const float* w32, uint16_t* w16, int64_t n, mp_stream stream);


/* y = act(x), elementwise over n binary16 values. GELU is x * Phi(x) with
 * the exact error function. */
mp_status mp_act_fwd(mp_act kind, const uint16_t* x, uint16_t* y, int64_t n, mp_stream stream);

/* dx = dy * act'(x), elementwise; x is the saved pre-activation. */
mp_status mp_act_bwd(mp_act kind, const uint16_t* x, const uint16_t* dy, uint16_t* dx,
                     int64_t n, mp_stream stream);

/* Bytes of device workspace mp_loss_softmax_ce needs for B rows of C logits
 * (at most 4096; 0 when there is nothing to do). */
size_t mp_loss_softmax_ce_workspace(int64_t B, int64_t C);

/* Mean softmax cross-entropy over B rows of C logits (binary16, row-major,
 * contiguous) with int32 labels in [0, C). Writes the FP32 loss to *loss
 * (device) and dlogits = RNE16(S * (softmax - onehot) / B) with S read from
 * `scaler`. Labels live on the device, so their range is the caller's
 * responsibility: a label outside [0, C) contributes no one-hot term.
 * The loss is reduced in a fixed order: per-block partials in `workspace`
 * (caller-owned device memory of at least mp_loss_softmax_ce_workspace(B, C)
 * bytes, 4-byte aligned, overwritten), then one block. Calls with disjoint
 * buffers and workspaces may run concurrently.
 * Errors: MP_ERR_INVALID_ARGUMENT (negative sizes, a null pointer, too small
 * or misaligned a workspace when B * C > 0), MP_ERR_HIP. */
mp_status mp_loss_softmax_ce(const uint16_t* logits, const int32_t* labels, int64_t B,
                             int64_t C, const mp_scaler* scaler, float* loss,
                             uint16_t* dlogits, void* workspace, size_t workspace_bytes,
                             mp_stream stream);

/* Bytes of device workspace mp_loss_mse needs for M x N elements (at most
 * 4096; 0 when there is nothing to do). */
size_t mp_loss_mse_workspace(int64_t M, int64_t N);

/* Mean squared error times c over the M x N elements (binary16, contiguous):
 * *loss = c * mean((y - t)^2) (FP32, device), dy = RNE16(S * c * 2 (y - t) / (M N)).
 * The sum is reduced in a fixed order: per-block partials in `workspace`
 * (caller-owned device memory of at least mp_loss_mse_workspace(M, N) bytes,
 * 4-byte aligned, overwritten), then one block; the loss is deterministic.
 * Calls with disjoint buffers and workspaces may run concurrently.
 * Errors: MP_ERR_INVALID_ARGUMENT (negative sizes, a null pointer, too small
 * or misaligned a workspace when M * N > 0), MP_ERR_HIP. */
mp_status mp_loss_mse(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, float c,
                      const mp_scaler* scaler, float* loss, uint16_t* dy, void* workspace,
                      size_t workspace_bytes, mp_stream stream);

/* mp_loss_mse for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * same kernels, results and errors as mp_loss_mse, with the per-block
 * partials in a device array of the library (1024 floats per GPU, the most
 * any size needs, kept until the process ends) instead of a workspace, so
 * neither the call nor the library allocates anything. The array's address
 * is looked up once per device on the first call there. Every call on one
 * GPU shares that array: calls that overlap on one GPU (other streams, other
 * host threads, replays of graphs that hold this call) race and must be
 * ordered by the caller.
 * Errors: as mp_loss_mse without the workspace ones; MP_ERR_UNSUPPORTED on a
 * device index of 64 or more. */
mp_status mp_loss_mse_noalloc(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, float c,
                              const mp_scaler* scaler, float* loss, uint16_t* dy, mp_stream stream);

/* ------------------------------------------------------------------------ */
const char* mp_status_string(mp_status status);
/* The last HIP error seen by this library on the calling thread ("" if none). */
const char* mp_last_hip_error(void);
/* Library version string. */
const char* mp_version(void);

#ifdef __cplusplus
}
#endif
#endif
