// SiTU-GLU elementwise math in fp32, shared by the streaming kernels and the GEMM epilogues.
//
// Definition ("Frontier-scale RL with Kimi K3", section "Streaming activations"):
//   gate' = beta * tanh(g / beta) * sigmoid(g),  lin' = lambda * tanh(l / lambda),
//   a = gate' * lin',  with g the first half and l the second half of the pre-activation.
// The custom op of the same section keeps only the bf16 pre-activation and recomputes tanh
// and sigmoid in the backward; this header is that recomputation.
//
// Evaluation (our own, chosen for gfx950, where these kernels are bound by vector ALU
// issue): every factor is written with a decaying exponential of |x|, so nothing overflows
// and no NaN can come from the tails:
//   e1 = exp(-2|g|/beta):  tanh(g/beta) = sgn(g) (1 - e1) / (1 + e1),
//                          1 - tanh^2   = 4 e1 / (1 + e1)^2
//   e2 = exp(-|g|):        sigmoid(g)   = (g >= 0 ? 1 : e2) / (1 + e2),
//                          s (1 - s)    = e2 / (1 + e2)^2
//   e3 = exp(-2|l|/lambda): tanh(l/lambda) = sgn(l) (1 - e3) / (1 + e3)
// With beta = 4 (the pages' default) e2 = e1^2, which saves one exponential (template flag
// B4, chosen on the host from beta). The numerators are kept scaled: U1 = beta (1 - e1) and
// U3 = lambda (1 - e3), each one fma. For tiny arguments 1 - e cancels, so beta (1 - exp(-y))
// with y = 2|g|/beta is taken as beta y = 2|g| when y < 2^-12 (relative error below
// y/2 < 2^-13, far under bf16's spacing), and likewise for l; results in fp32's denormal
// range may flush to zero.
// The forward folds its three denominators into one reciprocal; the backward takes one
// reciprocal of the square of their product. The backward calls the same forward routine
// for `a`, so a recomputed activation is bit-identical to the one the forward stored. Builds
// use -ffp-contract=off so the compiler cannot fuse these operations differently in
// different callers.
#pragma once

#include "common.h"

namespace moe {

struct SituCoef {
  float k1;      // 2 log2(e) / beta
  float k2;      // log2(e)
  float k3;      // 2 log2(e) / lambda
  float t1;      // beta 2^-13: |g| below it has 2|g|/beta < 2^-12
  float t3;      // lambda 2^-13
  float beta;
  float lam;
  int b4;        // beta == 4: exp(-|g|) = exp(-|g|/2)^2
};

inline SituCoef make_situ_coef(float beta, float lam) {
  const double log2e = 1.4426950408889634;
  SituCoef c;
  c.k1 = (float)(2.0 * log2e / beta);
  c.k2 = (float)log2e;
  c.k3 = (float)(2.0 * log2e / lam);
  c.t1 = (float)(beta * 0x1p-13);
  c.t3 = (float)(lam * 0x1p-13);
  c.beta = beta;
  c.lam = lam;
  c.b4 = (beta == 4.0f) ? 1 : 0;
  return c;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// scale (1 - exp(-y)) for y = 2 ax / scale >= 0, given e = exp(-y) and thr = scale 2^-13
// (y < 2^-12 exactly when ax < thr; there scale y = 2 ax)
__device__ __forceinline__ float scaled_one_minus_exp(float ax, float e, float scale,
                                                      float thr) {
  return (ax < thr) ? (ax + ax) : fmaf(-scale, e, scale);
}

// The three decaying exponentials of one (g, l) pair.
template <bool B4>
__device__ __forceinline__ void situ_exps(float ag, float al, const SituCoef& c, float& e1,
                                          float& e2, float& e3) {
  e1 = exp2_fast(-(ag * c.k1));
  e2 = B4 ? e1 * e1 : exp2_fast(-(ag * c.k2));
  e3 = exp2_fast(-(al * c.k3));
}

// a = gate'(g) * lin'(l)
template <bool B4>
__device__ __forceinline__ float situ_fwd(float g, float l, const SituCoef& c) {
  const float ag = fabsf(g), al = fabsf(l);
  float e1, e2, e3;
  situ_exps<B4>(ag, al, c, e1, e2, e3);
  const float sn = (g >= 0.0f) ? 1.0f : e2;
  const float u1 = scaled_one_minus_exp(ag, e1, c.beta, c.t1);
  const float u3 = scaled_one_minus_exp(al, e3, c.lam, c.t3);
  const float den = ((1.0f + e1) * (1.0f + e2)) * (1.0f + e3);
  const float mag = ((u1 * sn) * u3) * rcp_fast(den);
  // sign of tanh(g/beta) * tanh(l/lambda); sigmoid and the scales are positive
  const uint32_t sgn = (__float_as_uint(g) ^ __float_as_uint(l)) & 0x80000000u;
  return __uint_as_float(__float_as_uint(mag) ^ sgn);
}

// Backward: dL/dg, dL/dl for upstream da. With p1 = 1 + e1, p2 = 1 + e2, p3 = 1 + e3,
// u1 = beta (1 - e1), u3 = lambda (1 - e3) and sn = (g >= 0 ? 1 : e2):
//   beta tanh(g/beta) = sgn(g) u1 / p1,  sigmoid(g) = sn / p2,
//   lambda tanh(l/lambda) = sgn(l) u3 / p3,
//   1 - tanh^2(g/beta) = 4 e1 / p1^2,  s (1 - s) = e2 / p2^2,  1 - tanh^2(l/lambda) = 4 e3 / p3^2,
// so over the common denominator (p1 p2 p3)^2, with s1 = sgn(g) u1,
//   d gate'/dg = (4 e1 sn p2 + s1 e2 p1) / (p1 p2)^2,
//   dL/dg = da lin' d gate'/dg = da sgn(l) u3 (4 e1 sn p2 + s1 e2 p1) p3 / (p1 p2 p3)^2,
//   dL/dl = da gate' 4 e3 / p3^2 = da s1 sn 4 e3 p1 p2 / (p1 p2 p3)^2,
// one reciprocal in all (every p lies in [1, 2], so nothing overflows). u1, u3, sn, the p's
// and the reciprocal are the forward's own expressions, so a caller that needs both shares
// them.
template <bool B4>
__device__ __forceinline__ void situ_grad(float g, float l, float da, const SituCoef& c,
                                          float& dg, float& dl) {
  const float ag = fabsf(g), al = fabsf(l);
  float e1, e2, e3;
  situ_exps<B4>(ag, al, c, e1, e2, e3);
  const float sn = (g >= 0.0f) ? 1.0f : e2;
  const float u1 = scaled_one_minus_exp(ag, e1, c.beta, c.t1);
  const float u3 = scaled_one_minus_exp(al, e3, c.lam, c.t3);
  const float p1 = 1.0f + e1, p2 = 1.0f + e2, p3 = 1.0f + e3;
  const float p12 = p1 * p2;
  const float rd = rcp_fast(p12 * p3);
  const float rd2 = rd * rd;                         // 1 / (p1 p2 p3)^2
  const float s1 = copysignf(u1, g);
  const float ng = ((4.0f * e1) * sn) * p2 + (s1 * e2) * p1;
  dg = ((copysignf(u3, l) * da) * ng) * (rd2 * p3);
  dl = (((s1 * sn) * (4.0f * e3)) * da) * (rd2 * p12);
}

// Backward with the recomputed activation: a is bit-identical to situ_fwd<B4>(g, l, c).
template <bool B4>
__device__ __forceinline__ void situ_bwd(float g, float l, float da, const SituCoef& c,
                                         float& a, float& dg, float& dl) {
  a = situ_fwd<B4>(g, l, c);
  situ_grad<B4>(g, l, da, c, dg, dl);
}

}  // namespace moe
