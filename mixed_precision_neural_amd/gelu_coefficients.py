"""Generates the constants of the GELU evaluation in csrc/mp_act.h (run by hand; prints C).

GELU(x) = x Phi(x), Phi the standard normal CDF. For u = |x|:
    Phi(-u) = exp(-u^2 / 2) G(u),   G(u) = Phi(-u) exp(u^2 / 2),
and Phi(x) = 1 - Phi(-x) for x >= 0. G is smooth and slowly varying (G(0) = 1/2, G(u) ~
1 / (u sqrt(2 pi)) for large u), so it is fitted once, here, as a polynomial of degree 8 in
    z = A s + B,   s = 1 / (1 + P u),   u in [0, U],
with z spanning [-1, 1] (Chebyshev basis for the fit, then expanded to powers of z), by
relative least squares on a dense grid. Beyond U the kernel clamps u: exp(-u^2/2) has made
every term negligible there. Relative fit error 1.0e-7: the derivative Phi(x) + x phi(x),
which shares this evaluation, cancels near its zero (x = -0.7518), where the nearest binary16
inputs give values of ~1e-4. The GPU tests check every finite binary16 input against the
double-precision oracle.
"""
import numpy as np
from scipy.special import erfc

DEG, P, U = 8, 0.3, 7.0


def fit(deg=DEG, p=P, upper=U, n=400001):
    u = np.linspace(0.0, upper, n)
    g = 0.5 * erfc(u / np.sqrt(2.0)) * np.exp(u * u / 2.0)
    s = 1.0 / (1.0 + p * u)
    smin = 1.0 / (1.0 + p * upper)
    a, b = 2.0 / (1.0 - smin), -2.0 * smin / (1.0 - smin) - 1.0
    z = a * s + b
    v = np.polynomial.chebyshev.chebvander(z, deg)
    cheb, *_ = np.linalg.lstsq(v / g[:, None], np.ones_like(g), rcond=None)
    mono = np.polynomial.chebyshev.cheb2poly(cheb)
    rel = float(np.max(np.abs(v @ cheb / g - 1.0)))
    return mono, a, b, rel


def main():
    def f(v):
        h = float(np.float32(v)).hex()              # exact: every constant is rounded to FP32 first
        mant, exp = h.split("p")
        return (mant.rstrip("0").rstrip(".") if "." in mant else mant) + "p" + exp + "f"
    mono, a, b, rel = fit(deg=DEG)
    print(f"// degree {DEG}, P = {P}, U = {U}, relative fit error {rel:.2e}")
    print(f"constexpr float kGeluP = {f(P)}, kGeluU = {f(U)}, kGeluA = {f(a)}, kGeluB = {f(b)};")
    print(f"constexpr float kGeluE = {f(-0.5 * float(np.float32(np.log2(np.e))))};")
    print(f"constexpr float kGeluC8[{DEG + 1}] = {{" + ", ".join(f(c) for c in mono) + "};")

if __name__ == "__main__":
    main()
