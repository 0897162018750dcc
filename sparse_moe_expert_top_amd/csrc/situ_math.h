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
// B4, chosen on the host from beta). For tiny arguments 1 - e cancels, so 1 - exp(-y) is
// taken as y when y < 2^-12 (relative error below y/2 < 2^-13, far under bf16's spacing);
// results in fp32's denormal range may flush to zero.
// The forward folds its three denominators into one reciprocal; the backward takes one
// reciprocal of their product and recovers the three from it. The backward calls the same
// forward routine for `a`, so a recomputed activation is bit-identical to the one the
// forward stored. Builds use -ffp-contract=off so the compiler cannot fuse these operations
// differently in different callers.
#pragma once

#include "common.h"

namespace moe {

struct SituCoef {
  float k1;      // 2 log2(e) / beta
  float k2;      // log2(e)
  float k3;      // 2 log2(e) / lambda
  float y1;      // 2 / beta
  float y3;      // 2 / lambda
  float beta;
  float lam;
  float bl;      // beta * lambda
  int b4;        // beta == 4: exp(-|g|) = exp(-|g|/2)^2
};

inline SituCoef make_situ_coef(float beta, float lam) {
  const double log2e = 1.4426950408889634;
  SituCoef c;
  c.k1 = (float)(2.0 * log2e / beta);
  c.k2 = (float)log2e;
  c.k3 = (float)(2.0 * log2e / lam);
  c.y1 = (float)(2.0 / beta);
  c.y3 = (float)(2.0 / lam);
  c.beta = beta;
  c.lam = lam;
  c.bl = beta * lam;
  c.b4 = (beta == 4.0f) ? 1 : 0;
  return c;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// 1 - exp(-y) for y >= 0, given e = exp(-y)
__device__ __forceinline__ float one_minus_exp(float y, float e) {
  return (y < 0x1p-12f) ? y : (1.0f - e);
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
  const float snum = (g >= 0.0f) ? 1.0f : e2;
  const float num = (one_minus_exp(ag * c.y1, e1) * snum) * one_minus_exp(al * c.y3, e3);
  const float den = ((1.0f + e1) * (1.0f + e2)) * (1.0f + e3);
  const float mag = (c.bl * num) * rcp_fast(den);
  // sign of tanh(g/beta) * tanh(l/lambda); sigmoid and the scales are positive
  const uint32_t sgn = (__float_as_uint(g) ^ __float_as_uint(l)) & 0x80000000u;
  return __uint_as_float(__float_as_uint(mag) ^ sgn);
}

// Backward: dL/dg, dL/dl for upstream da.
template <bool B4>
__device__ __forceinline__ void situ_grad(float g, float l, float da, const SituCoef& c,
                                          float& dg, float& dl) {
  const float ag = fabsf(g), al = fabsf(l);
  float e1, e2, e3;
  situ_exps<B4>(ag, al, c, e1, e2, e3);
  const float p1 = 1.0f + e1, p2 = 1.0f + e2, p3 = 1.0f + e3;
  const float p12 = p1 * p2;
  const float rall = rcp_fast(p12 * p3);             // 1 / (p1 p2 p3)
  const float r12 = rall * p3;                       // 1 / (p1 p2)
  const float r1 = r12 * p2, r2 = r12 * p1, r3 = rall * p12;
  const float t1 = copysignf(one_minus_exp(ag * c.y1, e1) * r1, g);
  const float s = ((g >= 0.0f) ? 1.0f : e2) * r2;
  const float t2 = copysignf(one_minus_exp(al * c.y3, e3) * r3, l);
  const float gate = (c.beta * t1) * s;
  const float lin = c.lam * t2;
  const float sech2_g = (4.0f * e1) * (r1 * r1);       // 1 - tanh^2(g/beta)
  const float s1ms = e2 * (r2 * r2);                    // s (1 - s)
  const float sech2_l = (4.0f * e3) * (r3 * r3);       // 1 - tanh^2(l/lambda)
  const float dgate = sech2_g * s + (c.beta * t1) * s1ms;
  dg = (da * lin) * dgate;
  dl = (da * gate) * sech2_l;
}

// Backward with the recomputed activation: a is bit-identical to situ_fwd<B4>(g, l, c).
template <bool B4>
__device__ __forceinline__ void situ_bwd(float g, float l, float da, const SituCoef& c,
                                         float& a, float& dg, float& dl) {
  a = situ_fwd<B4>(g, l, c);
  situ_grad<B4>(g, l, da, c, dg, dl);
}

}  // namespace moe
