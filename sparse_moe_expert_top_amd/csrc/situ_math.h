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
//   e1 = exp(-2|g|/beta):  tanh(|g|/beta) = (1 - e1) / (1 + e1),
//                          1 - tanh^2     = 4 e1 / (1 + e1)^2
//   e2 = exp(-|g|):        sigmoid(g)     = sn / (1 + e2), sn = (g >= 0 ? 1 : e2),
//                          s (1 - s)      = e2 / (1 + e2)^2
//   e3 = exp(-2|l|/lambda): tanh(|l|/lambda) = (1 - e3) / (1 + e3)
// With beta = 4 (the pages' default) e2 = e1^2, which saves one exponential (template flag
// B4, chosen on the host from beta).
//
// Scaled terms. The kernels work with E3 = 2 e3 (the exponential of 1 - 2|l| log2(e)/lambda
// in base 2) and
//   v1 = beta (1 - e1) / 2,  v3 = lambda (1 - e3) / 2,  q1 = (1 + e1) / 4,
//   q12 = q1 (1 + e2),  p3 = 1 + e3,  r = 1 / (q12 p3) = 4 / ((1 + e1)(1 + e2)(1 + e3)),
// each one fma, multiply or reciprocal. The powers of two are chosen so they cancel:
//   a = sgn(g) sgn(l) v1 sn v3 r                       (the 1/2, 1/2 and 4 cancel)
//   dL/dl = da gate' 4 e3 / p3^2 = (sgn(g) v1 sn) E3 q12 (da r^2)
//   dL/dg = da lin' d gate'/dg = (da r^2) (sgn(l) v3) N p3,
//           N = e1 sn (1 + e2) / 2 + (sgn(g) v1) e2 q1
// (d gate'/dg = (1 - tanh^2) sigmoid + beta tanh s (1 - s) over the common denominator
// (1 + e1)^2 (1 + e2)^2, with 1/p3 = r q12 and 1/(q12^2 p3) = r^2 p3). Every 1 + e lies in
// [1, 2], so r lies in [1/2, 4] and no intermediate overflows or underflows beyond the inputs'
// own tails. Scaling by a power of two is exact, so a equals what the unscaled expressions give
// (barring fp32 denormals).
// For tiny arguments 1 - e cancels, so beta (1 - exp(-y)) / 2 with y = 2|g|/beta is taken as
// beta y / 2 = |g| when y < 2^-12 (relative error below y/2 < 2^-13, far under bf16's
// spacing), and likewise for l; results in fp32's denormal range may flush to zero.
// The backward with the activation (the dA epilogue) shares the forward's operations, so a
// recomputed activation is bit-identical to the one the forward stored. Builds use
// -ffp-contract=off so the compiler cannot fuse these operations differently in different
// callers; the fmas below are written out.
#pragma once

#include "common.h"

namespace moe {

struct SituCoef {
  float k1;      // 2 log2(e) / beta
  float k2;      // log2(e)
  float k3;      // 2 log2(e) / lambda
  float t1;      // beta 2^-13: |g| below it has 2|g|/beta < 2^-12
  float t3;      // lambda 2^-13
  float hb;      // beta / 2
  float hl;      // lambda / 2
  float ql;      // lambda / 4
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
  c.hb = 0.5f * beta;
  c.hl = 0.5f * lam;
  c.ql = 0.25f * lam;
  c.b4 = (beta == 4.0f) ? 1 : 0;
  return c;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// The scaled terms of one (g, l) pair (see the header comment).
struct SituTerms {
  float e1, e2, E3;   // exp(-2|g|/beta), exp(-|g|), 2 exp(-2|l|/lambda)
  float v1, v3;       // >= 0
  float q1, q12, p3, r;
};

template <bool B4>
__device__ __forceinline__ SituTerms situ_terms(float g, float l, const SituCoef& c) {
  SituTerms t;
  const float ag = fabsf(g), al = fabsf(l);
  t.e1 = exp2_fast(-(ag * c.k1));
  t.e2 = B4 ? t.e1 * t.e1 : exp2_fast(-(ag * c.k2));
  t.E3 = exp2_fast(fmaf(al, -c.k3, 1.0f));
  t.v1 = (ag < c.t1) ? ag : fmaf(-c.hb, t.e1, c.hb);
  t.v3 = (al < c.t3) ? al : fmaf(-c.ql, t.E3, c.hl);
  t.q1 = fmaf(0.25f, t.e1, 0.25f);
  t.q12 = fmaf(t.q1, t.e2, t.q1);
  t.p3 = fmaf(0.5f, t.E3, 1.0f);
  t.r = rcp_fast(t.q12 * t.p3);
  return t;
}

// sgn(g) sn in one select: 1 for g >= 0, else -e2.
__device__ __forceinline__ float situ_sns(const SituTerms& t, float g) {
  return (g >= 0.0f) ? 1.0f : -t.e2;
}

// a from the terms and As = v1 sns: (sgn(g) v1 sn) (sgn(l) v3) r.
__device__ __forceinline__ float situ_act(const SituTerms& t, float l, float As) {
  return (As * copysignf(t.v3, l)) * t.r;
}

// a = gate'(g) * lin'(l)
template <bool B4>
__device__ __forceinline__ float situ_fwd(float g, float l, const SituCoef& c) {
  const SituTerms t = situ_terms<B4>(g, l, c);
  return situ_act(t, l, t.v1 * situ_sns(t, g));
}

// dL/dg and dL/dl for upstream da, given the terms, sns and As = v1 sns.
__device__ __forceinline__ void situ_grad_terms(const SituTerms& t, float g, float l, float da,
                                                float sns, float As, float& dg, float& dl) {
  const float ds = (t.r * t.r) * da;
  dl = ((As * t.E3) * t.q12) * ds;
  const float n = fmaf(t.e1 * fabsf(sns), fmaf(0.5f, t.e2, 0.5f), (copysignf(t.v1, g) * t.e2) * t.q1);
  dg = ((ds * copysignf(t.v3, l)) * n) * t.p3;
}

// Backward: dL/dg, dL/dl for upstream da.
template <bool B4>
__device__ __forceinline__ void situ_grad(float g, float l, float da, const SituCoef& c,
                                          float& dg, float& dl) {
  const SituTerms t = situ_terms<B4>(g, l, c);
  const float sns = situ_sns(t, g);
  situ_grad_terms(t, g, l, da, sns, t.v1 * sns, dg, dl);
}

// Backward with the recomputed activation: a is bit-identical to situ_fwd<B4>(g, l, c).
template <bool B4>
__device__ __forceinline__ void situ_bwd(float g, float l, float da, const SituCoef& c,
                                         float& a, float& dg, float& dl) {
  const SituTerms t = situ_terms<B4>(g, l, c);
  const float sns = situ_sns(t, g);
  const float As = t.v1 * sns;
  a = situ_act(t, l, As);
  situ_grad_terms(t, g, l, da, sns, As, dg, dl);
}

}  // namespace moe
