// MXFP4 weights of the W4A8 expert forward, shared by the weight quantizer and its inverse.
//
// "Frontier-scale RL with Kimi K3", section "Low precision (MXFP4) rollouts", runs the MoE
// layers with 4-bit weights; the explainer's "Idea Four" describes MXFP4 as 4-bit floats
// whose small blocks share one scale. The pages fix no encoding; this library reads it as
// OCP Microscaling v1.0 MXFP4:
//   * E2M1 elements: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, magnitudes 0, 0.5, 1,
//     1.5, 2, 3, 4, 6 (codes 0..7), sign in bit 3. Encoding rounds to nearest, ties to the
//     even code, saturates to +-6 and keeps the sign of values that round to zero.
//   * 32 consecutive elements of a row share a scale 2^X, stored as the byte X + 127, with
//     X = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an all-zero block).
// A stored row of n elements is n/2 code bytes (element 2j in the low nibble of byte j, 2j+1
// in the high nibble) plus n/32 scale bytes.
#pragma once

#include "common.h"

namespace moe {

// E8M0 scale byte of a block from its largest magnitude (finite, non-negative fp32).
__device__ __forceinline__ uint32_t mx4_scale_byte(float amax) {
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);   // 0 for zero or subnormal
  int X = ex - 127 - 2;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  return (uint32_t)(X + 127);
}

// E2M1 code of a finite fp32 value (already divided by its block scale): the magnitude code
// is the number of rounding boundaries at or below |v|. Each boundary is the midpoint of two
// neighbouring magnitudes; a value exactly on one goes to the even code, so the boundaries
// above an odd code (0.75, 1.75, 3.5) count when reached and the others (0.25, 1.25, 2.5, 5)
// only when passed.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
  return ((__float_as_uint(v) >> 28) & 0x8u) | mag;
}

// Value of an E2M1 code.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const uint32_t ex = (c >> 1) & 3u, m = c & 1u;
  const float mag = ex ? __uint_as_float(((ex + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
  return (c & 8u) ? -mag : mag;
}

// 8 consecutive elements of one block -> 8 codes packed into one word (element i in bits
// 4i .. 4i+3).
__device__ __forceinline__ uint32_t mx4_encode8(const float (&v)[8], uint32_t scale_byte) {
  const int nx = 127 - (int)scale_byte;            // -X
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= e2m1_encode(__builtin_amdgcn_ldexpf(v[i], nx)) << (4 * i);
  return word;
}
__device__ __forceinline__ void mx4_decode8(uint32_t codes, uint32_t scale_byte, float (&v)[8]) {
  const int X = (int)scale_byte - 127;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_ldexpf(e2m1_decode((codes >> (4 * i)) & 0xFu), X);
}

}  // namespace moe
