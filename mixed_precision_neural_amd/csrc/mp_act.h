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
// a smooth function; Phi(x) = 1 - Phi(-x) for x >= 0. G is a degree-8
// polynomial in z = A s + B, s = 1 / (1 + P u), fitted over u in [0, U]
// (constants from gelu_coefficients.py, relative fit error 1.0e-7; u is clamped
// to U, where e has made the term negligible). GELU' = Phi(x) + x phi(x) shares
// e and Phi, so one evaluation gives both. The accuracy is set by GELU':
// Phi(x) + x phi(x) cancels near its zero at x = -0.7518, where the nearest
// binary16 inputs give values of ~1e-4 and Phi needs ~1e-7 absolute accuracy.
// e is one v_exp_f32 of x^2 times -log2(e)/2 (a single rounded product: the
// factor 1/2 is exact).
constexpr float kGeluP = 0x1.333334p-2f, kGeluU = 0x1.cp+2f, kGeluA = 0x1.79e79ep+1f, kGeluB = -0x1.f3cf3cp+0f;
constexpr float kGeluE = -0x1.715476p-1f;            // -log2(e) / 2, from log2(e) in FP32
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
__device__ __forceinline__ NormalCdf std_normal(float x) {
    const float u = fminf(fabsf(x), kGeluU);
    const float e = __builtin_amdgcn_exp2f(kGeluE * (x * x));
    const float s = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluP, u, 1.0f));
    const float z = __builtin_fmaf(s, kGeluA, kGeluB);
    const float q = e * horner(z, kGeluC8);          // Phi(-|x|)
    return {x < 0.0f ? q : 1.0f - q, e};
}
__device__ __forceinline__ float gelu_f(const NormalCdf& n, float x) { return x * n.cdf; }
__device__ __forceinline__ float gelu_d(const NormalCdf& n, float x) {
    return __builtin_fmaf(x * 0.39894228040143267794f, n.e, n.cdf);
}
// kind: 0 = ReLU, 1 = GELU (the values of mp_act)
template <int KIND>
__device__ __forceinline__ uint16_t act_fwd1(uint16_t xh) {
    if (KIND == 0) {
        const float x = h2f(xh);
        return (x > 0.0f || x != x) ? xh : uint16_t(0);
    }
    const float x = h2f(xh);
    return f2h(gelu_f(std_normal(x), x));
}
template <int KIND>
__device__ __forceinline__ uint16_t act_bwd1(uint16_t xh, uint16_t dyh) {
    const float x = h2f(xh);
    if (KIND == 0) return x > 0.0f ? dyh : uint16_t(0);
    return f2h(h2f(dyh) * gelu_d(std_normal(x), x));
}
// act(x) and act'(x) of one binary16 value, each rounded to binary16, from one
// evaluation: the bits of act_fwd1(x) and of act_bwd1(x, 1.0) (ReLU' is 1 for
// x > 0 and 0 otherwise, NaN included).
template <int KIND>
__device__ __forceinline__ void act_fwd_deriv1(uint16_t xh, uint16_t& a, uint16_t& d) {
    const float x = h2f(xh);
    if (KIND == 0) {
        a = (x > 0.0f || x != x) ? xh : uint16_t(0);
        d = x > 0.0f ? uint16_t(0x3C00) : uint16_t(0);
        return;
    }
    const NormalCdf n = std_normal(x);
    a = f2h(gelu_f(n, x));
    d = f2h(1.0f * gelu_d(n, x));
}
// act_fwd_deriv1 of two values, packed: a01 = act(x0) | act(x1) << 16, d01 the
// same for act'; the same bits, with one packed conversion per pair.
template <int KIND>
__device__ __forceinline__ void act_fwd_deriv2(uint16_t x0, uint16_t x1, uint32_t& a01, uint32_t& d01) {
    if (KIND == 0) {
        uint16_t a0, d0, a1, d1;
        act_fwd_deriv1<0>(x0, a0, d0);
        act_fwd_deriv1<0>(x1, a1, d1);
        a01 = uint32_t(a0) | uint32_t(a1) << 16;
        d01 = uint32_t(d0) | uint32_t(d1) << 16;
        return;
    }
    const float y0 = h2f(x0), y1 = h2f(x1);
    const NormalCdf n0 = std_normal(y0), n1 = std_normal(y1);
    a01 = f2h2(gelu_f(n0, y0), gelu_f(n1, y1));
    d01 = f2h2(1.0f * gelu_d(n0, y0), 1.0f * gelu_d(n1, y1));
}

}  // namespace mp
