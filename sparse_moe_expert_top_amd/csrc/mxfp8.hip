// Standalone MXFP8 quantizer and dequantizer of a bf16 [rows, n] tensor (n a multiple of 32),
// in the storage format the gate/up GEMM writes for the saved pre-activation (mxfp8.h).
//
// Each lane owns 8 consecutive elements (16 bytes of bf16 in, 8 code bytes out); the 4 lanes
// of a 32-element block are consecutive lanes, so the block maximum is two xor-shuffles.
// Chunk counts are multiples of 4 and so is the grid stride, so a block's lanes are always
// active together.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "mxfp8.h"

namespace moe {

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ v,
                                                          int64_t nchunks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const u32x4 raw = *(const u32x4*)(v + c * 8);
    float f[8];
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_lo(raw[q]);
      f[2 * q + 1] = bf16_hi(raw[q]);
      m = fmaxf(m, fmaxf(fabsf(f[2 * q]), fabsf(f[2 * q + 1])));
    }
    const uint32_t sb = mx_scale_byte(mx_amax4(m));
    *(u32x2*)(codes + c * 8) = mx_encode8(f, sb);
    if ((c & 3) == 0) scales[c >> 2] = (uint8_t)sb;
  }
}

__global__ __launch_bounds__(256) void mx_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nchunks,
                                                            uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    float f[8];
    mx_decode8(*(const u32x2*)(codes + c * 8), scales[c >> 2], f);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
    *(u32x4*)(out + c * 8) = o;
  }
}

static unsigned mx_grid(int64_t nchunks) {
  int64_t blocks = (nchunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 64;
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t launch_mx_quantize(const uint16_t* v, int64_t rows, int n, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nchunks = rows * (int64_t)(n / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(mx_grid(nchunks)), dim3(256), 0, s, v, nchunks,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int n,
                                uint16_t* out, hipStream_t s) {
  const int64_t nchunks = rows * (int64_t)(n / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_dequantize_kernel, dim3(mx_grid(nchunks)), dim3(256), 0, s, codes,
                     scales, nchunks, out);
  return hipGetLastError();
}

}  // namespace moe
