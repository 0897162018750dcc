// Streaming SiTU-GLU forward and backward (gfx950).
//
// "Frontier-scale RL with Kimi K3", section "Streaming activations": the custom op keeps
// only the bf16 pre-activation h = [g | l] of shape [R, 2H], streams over it with a
// constant-size fp32 working set, and recomputes tanh and sigmoid in the backward; this is
// valid because the activation is elementwise.
//
// Here each lane owns one 16-byte chunk (8 columns) of a row per step: it reads g and l
// (and da) with 16-byte loads, keeps all fp32 intermediates in registers and writes the
// bf16 result with 16-byte stores. The grid is persistent (a few workgroups per CU) and
// walks row-chunks in a grid-stride loop, so the fp32 working set is fixed by the launch,
// not by R.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "situ_math.h"

namespace moe {

__global__ __launch_bounds__(256) void situ_fwd_kernel(const uint16_t* __restrict__ h,
                                                       int64_t R, int H, SituCoef c,
                                                       uint16_t* __restrict__ a) {
  const uint32_t hc = (uint32_t)(H >> 3);                 // 16-byte chunks per half-row
  const int64_t n = R * (int64_t)hc;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / hc;
    const int cc = (int)(i - r * hc);
    const uint16_t* hr = h + r * (2 * (int64_t)H) + 8 * cc;
    const u32x4 g = __builtin_nontemporal_load((const u32x4*)hr);
    const u32x4 l = __builtin_nontemporal_load((const u32x4*)(hr + H));
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = situ_fwd(bf16_lo(g[q]), bf16_lo(l[q]), c);
      const float a1 = situ_fwd(bf16_hi(g[q]), bf16_hi(l[q]), c);
      o[q] = pack_bf16x2(a0, a1);
    }
    __builtin_nontemporal_store(o, (u32x4*)(a + r * (int64_t)H + 8 * cc));
  }
}

__global__ __launch_bounds__(256) void situ_bwd_kernel(const uint16_t* __restrict__ h,
                                                       const uint16_t* __restrict__ da,
                                                       int64_t R, int H, SituCoef c,
                                                       uint16_t* __restrict__ dh) {
  const uint32_t hc = (uint32_t)(H >> 3);
  const int64_t n = R * (int64_t)hc;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / hc;
    const int cc = (int)(i - r * hc);
    const int64_t hoff = r * (2 * (int64_t)H) + 8 * cc;
    const u32x4 g = __builtin_nontemporal_load((const u32x4*)(h + hoff));
    const u32x4 l = __builtin_nontemporal_load((const u32x4*)(h + hoff + H));
    const u32x4 d = __builtin_nontemporal_load((const u32x4*)(da + r * (int64_t)H + 8 * cc));
    u32x4 og, ol;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a0, g0, l0, a1, g1, l1;
      situ_bwd(bf16_lo(g[q]), bf16_lo(l[q]), bf16_lo(d[q]), c, a0, g0, l0);
      situ_bwd(bf16_hi(g[q]), bf16_hi(l[q]), bf16_hi(d[q]), c, a1, g1, l1);
      og[q] = pack_bf16x2(g0, g1);
      ol[q] = pack_bf16x2(l0, l1);
    }
    __builtin_nontemporal_store(og, (u32x4*)(dh + hoff));
    __builtin_nontemporal_store(ol, (u32x4*)(dh + hoff + H));
  }
}

static unsigned situ_grid(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t launch_situ_fwd(const uint16_t* h, int64_t R, int H, SituCoef c, uint16_t* a,
                           hipStream_t s) {
  const int64_t n = R * (int64_t)(H / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(situ_fwd_kernel, dim3(situ_grid(n)), dim3(256), 0, s, h, R, H, c, a);
  return hipGetLastError();
}

hipError_t launch_situ_bwd(const uint16_t* h, const uint16_t* da, int64_t R, int H,
                           SituCoef c, uint16_t* dh, hipStream_t s) {
  const int64_t n = R * (int64_t)(H / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(situ_bwd_kernel, dim3(situ_grid(n)), dim3(256), 0, s, h, da, R, H, c, dh);
  return hipGetLastError();
}

}  // namespace moe
