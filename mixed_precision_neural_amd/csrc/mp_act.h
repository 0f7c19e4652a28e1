// Point-wise activations on binary16 values, shared by the stand-alone
// activation kernels and the fused GEMM epilogues so that both give the same
// bits. Kept apart from mp_internal.h, which the optimizer sweeps and the
// statistics kernels include: a change here leaves those kernels' sources as
// they were.
#pragma once

#include "mp_internal.h"

namespace mp {

// GELU(x) = x Phi(x), Phi the standard normal CDF (the exact-erf GELU). For
// u = |x|, Phi(-u) = e G(u) with e = exp(-x^2/2) and G(u) = Phi(-u) exp(u^2/2)
// a smooth function; Phi(x) = 1 - Phi(-x) for x >= 0. G is a polynomial in
// z = A s + B, s = 1 / (1 + P u), fitted over u in [0, U] (constants from
// gelu_coefficients.py; u is clamped to U, where e has made the term
// negligible). GELU' = Phi(x) + x phi(x) shares e.
//   The forward uses degree 6 (relative fit error 4.7e-6): the result is
//   rounded to binary16, whose half ulp is 2^-11, so it stays within one ulp
//   of the correctly rounded value. The derivative uses degree 8 (1.0e-7):
//   Phi(x) + x phi(x) cancels near its zero at x = -0.7518, where the nearest
//   binary16 inputs give values of ~1e-4 and Phi needs ~1e-7 absolute accuracy.
//   e is one v_exp_f32 of x^2 times -log2(e)/2 (a single rounded product: the
//   factor 1/2 is exact).
constexpr float kGeluP = 0x1.333334p-2f, kGeluU = 0x1.cp+2f, kGeluA = 0x1.79e79ep+1f, kGeluB = -0x1.f3cf3cp+0f;
constexpr float kGeluE = -0x1.715476p-1f;            // -log2(e) / 2, from log2(e) in FP32
constexpr float kGeluC6[7] = {0x1.81febep-3f, 0x1.97f8ep-3f, 0x1.64aa14p-4f, 0x1.7d53aap-6f, 0x1.4a8ff6p-9f, -0x1.c03286p-12f, -0x1.09f21cp-13f};
constexpr float kGeluC8[9] = {0x1.81feaap-3f, 0x1.97f89cp-3f, 0x1.64adb6p-4f, 0x1.7d75f6p-6f, 0x1.4968e6p-9f, -0x1.d900bp-12f, -0x1.08bb14p-13f, 0x1.208f62p-16f, 0x1.9688d4p-18f};
struct NormalCdf {
    float cdf;      // Phi(x)
    float e;        // exp(-x^2 / 2)
};
template <int N>
__device__ __forceinline__ float horner(float z, const float (&c)[N]) {
    float g = c[N - 1];
#pragma unroll
    for (int k = N - 2; k >= 0; --k) g = __builtin_fmaf(g, z, c[k]);
    return g;
}
template <int DEG>
__device__ __forceinline__ NormalCdf std_normal(float x) {
    static_assert(DEG == 6 || DEG == 8, "fitted degrees");
    const float u = fminf(fabsf(x), kGeluU);
    const float e = __builtin_amdgcn_exp2f(kGeluE * (x * x));
    const float s = __builtin_amdgcn_rcpf(1.0f + kGeluP * u);
    const float z = __builtin_fmaf(s, kGeluA, kGeluB);
    float g;
    if constexpr (DEG == 6) g = horner(z, kGeluC6);
    else g = horner(z, kGeluC8);
    const float q = e * g;                           // Phi(-|x|)
    return {x < 0.0f ? q : 1.0f - q, e};
}
__device__ __forceinline__ float gelu_f(float x) { return x * std_normal<6>(x).cdf; }
__device__ __forceinline__ float gelu_d(float x) {
    const NormalCdf n = std_normal<8>(x);
    return n.cdf + (x * 0.39894228040143267794f) * n.e;
}
// kind: 0 = ReLU, 1 = GELU (the values of mp_act)
template <int KIND>
__device__ __forceinline__ uint16_t act_fwd1(uint16_t xh) {
    if (KIND == 0) {
        const float x = h2f(xh);
        return (x > 0.0f || x != x) ? xh : uint16_t(0);
    }
    return f2h(gelu_f(h2f(xh)));
}
template <int KIND>
__device__ __forceinline__ uint16_t act_bwd1(uint16_t xh, uint16_t dyh) {
    const float x = h2f(xh);
    if (KIND == 0) return x > 0.0f ? dyh : uint16_t(0);
    return f2h(h2f(dyh) * gelu_d(x));
}

}  // namespace mp
