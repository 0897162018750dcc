// MXFP8 storage of the saved pre-activation, shared by the GEMM epilogues and the standalone
// quantizer.
//
// "Kimi K3 ... Memory" (unified activation manager; ledger summary) keeps most saved
// activations block-wise in FP8, which halves them again. The pages do not fix the format;
// this library reads it as OCP Microscaling v1.0 MXFP8:
//   * E4M3 elements: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
//     largest finite 448, subnormal quantum 2^-9. Encoding rounds to nearest, ties to even,
//     saturates to +-448, and keeps the sign of values that round to zero.
//   * 32 consecutive elements of a row share a scale 2^X, stored as the byte X + 127, with
//     X = floor(log2(amax)) - 8 clamped to [-127, 127] (-127 for an all-zero block).
// A stored row of n elements is n code bytes plus n/32 scale bytes (1.03 bytes per element
// against 2 for bf16). Encoding uses gfx950's fp32 -> E4M3 conversion (v_cvt_pk_fp8_f32, OCP
// E4M3, round to nearest even) on values first clamped to +-448, which gives the saturation
// above. On every finite bf16 value at block exponents -10, 0 and 5 it agreed bit for bit
// with a bit-level encoder of the rule above (subnormals, signed zeros and the saturation
// band included).
#pragma once

#include "common.h"

namespace moe {

constexpr int kMxBlock = 32;

// E8M0 scale byte of a block from its largest magnitude (a finite, non-negative fp32).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  // biased fp32 exponent = floor(log2(amax)) + 127 for normal amax; 0 for zero or subnormal,
  // whose true X lies below the clamp anyway
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int X = ex - 127 - 8;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  return (uint32_t)(X + 127);
}

// Values of the E4M3 codes in bytes 2P and 2P + 1 of w, by gfx950's E4M3 -> fp32
// conversion (v_cvt_pk_f32_fp8, OCP E4M3): exact for every finite code, subnormals and signed
// zeros included (the encoder never produces the NaN codes).
template <int P>
__device__ __forceinline__ f32x2 e4m3_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, P == 1);
}
// Value of code i (0..3) of w.
__device__ __forceinline__ float e4m3_code(uint32_t w, int i) {
  const f32x2 v = ((i >> 1) & 1) ? e4m3_pair<1>(w) : e4m3_pair<0>(w);
  return v[i & 1];
}

// 8 consecutive elements of one block: codes packed little-endian into two words.
__device__ __forceinline__ u32x2 mx_encode8(const float (&v)[8], uint32_t scale_byte) {
  const int nx = 127 - (int)scale_byte;            // -X
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[i], nx), -448.0f), 448.0f);
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w], q[4 * w + 1], 0, false);
    out[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w + 2], q[4 * w + 3], lo, true);
  }
  return out;
}
__device__ __forceinline__ void mx_decode8(u32x2 codes, uint32_t scale_byte, float (&v)[8]) {
  const int X = (int)scale_byte - 127;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_amdgcn_ldexpf(e4m3_code(codes[i >> 2], i & 3), X);
}

// Largest magnitude over the 4 lanes (xor 1, 2) that hold one 32-element block.
__device__ __forceinline__ float mx_amax4(float m) {
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  return m;
}

}  // namespace moe
