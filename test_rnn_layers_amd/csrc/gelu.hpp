// gelu.hpp -- GELU and its derivative in fp32 for the TTT-MLP kernels (the
// erf form x * Phi(x) of the hidden layer of f).
#pragma once

namespace ttt {

// GELU(x) = x Phi(x) and GELU'(x) = Phi(x) + x phi(x) with the erf form of
// the normal CDF Phi.  erf comes from the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (absolute error <= 1.5e-7 over the real line): for z >= 0
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z).
// With z = |x| / sqrt(2), exp(-z^2) = exp(-x^2 / 2) is also the factor of
// the normal density phi, so GELU and GELU' share one exponential.
struct Gelu {
    float g, dg;
};
// With s = |x| sqrt(log2(e) / 2) (so that s^2 = x^2 log2(e) / 2):
//   t = 1 / (1 + p z) = 1 / (1 + p' s),       p' = p / (sqrt(2) sqrt(log2(e) / 2))
//   phi(x) = 2^(-s^2 + log2(1 / sqrt(2 pi)))  (the density, one exp2)
//   h = (1 - erf(z)) / 2 = (a1 t + ... + a5 t^5) exp(-z^2) / 2
//     = (a1' t + ... + a5' t^5) phi(x),      a_i' = a_i sqrt(2 pi) / 2
//   Phi(x) = 1 - h (x >= 0), h (x < 0);  GELU = x Phi;  GELU' = Phi + x phi
// (the constants fold the scalings of the two transcendentals and of the
// density; an fp32 emulation of this sequence agrees with the exact GELU and
// GELU' to 6e-7 on [-10, 10])
__device__ __forceinline__ Gelu gelu_both(float x) {
    constexpr float c1 = 0.8493218002880191f, pp = 0.27273747f, c2 = -1.3257480647361593f;
    constexpr float a1 = 0.31938153f, a2 = -0.35656378f, a3 = 1.7814779f, a4 = -1.8212559f, a5 = 1.3302745f;
    const float sx = fabsf(x) * c1;
    const float t = __builtin_amdgcn_rcpf(fmaf(pp, sx, 1.f));
    const float poly = t * fmaf(fmaf(fmaf(fmaf(a5, t, a4), t, a3), t, a2), t, a1);
    const float ph = __builtin_amdgcn_exp2f(fmaf(-sx, sx, c2));  // phi(x)
    const float h = poly * ph;
    const float cdf = x >= 0.f ? 1.f - h : h;
    return Gelu{x * cdf, fmaf(x, ph, cdf)};
}

// GELU alone needs no density, so it takes erf from formula 7.1.28 of the same
// handbook (absolute error <= 3e-7), which has a reciprocal but no exponential:
//   erf(z) = 1 - 1 / (1 + a1 z + ... + a6 z^6)^16,  z >= 0
// (the 16th power overflows to +inf for large z, where 1/inf = 0 is the limit)
__device__ __forceinline__ float gelu(float x) {
    constexpr float a1 = 0.0705230784f, a2 = 0.0422820123f, a3 = 0.0092705272f, a4 = 0.0001520143f,
                    a5 = 0.0002765672f, a6 = 0.0000430638f;
    const float z = fabsf(x) * 0.70710678118654752f;
    float pz = fmaf(fmaf(fmaf(fmaf(fmaf(fmaf(a6, z, a5), z, a4), z, a3), z, a2), z, a1), z, 1.f);
    pz *= pz;  // ^2
    pz *= pz;  // ^4
    pz *= pz;  // ^8
    pz *= pz;  // ^16
    const float h = 0.5f * __builtin_amdgcn_rcpf(pz);  // (1 - erf(|x| / sqrt(2))) / 2
    return x * (x >= 0.f ? 1.f - h : h);
}

}  // namespace ttt
