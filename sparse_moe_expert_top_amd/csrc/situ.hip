// Streaming SiTU-GLU forward and backward (gfx950).
//
// "Frontier-scale RL with Kimi K3", section "Streaming activations": the custom op keeps
// only the bf16 pre-activation h = [g | l] of shape [R, 2H], streams over it with a
// constant-size fp32 working set, and recomputes tanh and sigmoid in the backward; this is
// valid because the activation is elementwise.
//
// Here each lane owns 16-byte chunks (8 columns) of a row: it reads g and l (and da) with
// 16-byte non-temporal loads, keeps all fp32 intermediates in registers and writes the
// bf16 result with 16-byte non-temporal stores. The grid walks row-chunks in a grid-stride
// loop, so the fp32 working set is fixed by the launch, not by R. Measured on MI355X at
// R = 131072, H = 3072: a grid of 256 workgroups per CU (far more than are resident, so
// the dispatcher keeps every CU's queue full as waves retire) with 2 chunks per lane per
// step streams at 5.3-5.6 TB/s, against 4.6-4.9 TB/s for a persistent grid of 8 per CU
// and the same for 1-8 chunks per step; plain (temporal) loads cost 5-10%.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "situ_math.h"

namespace moe {

// Grid-stride walk over (row, 16-byte chunk) pairs without a division per step: the
// stride is added as (dr rows, dc chunks) with a carry. Each thread advances kU strides per
// iteration and issues all kU chunks' loads before any arithmetic, keeping kU x 32 (fwd)
// or kU x 48 (bwd) bytes in flight per lane.
#ifndef MOE_SITU_UNROLL
#define MOE_SITU_UNROLL 2
#endif
#ifndef MOE_SITU_BLOCKS_PER_CU
#define MOE_SITU_BLOCKS_PER_CU 256
#endif
#ifndef MOE_SITU_NT_LOAD
#define MOE_SITU_NT_LOAD 1
#endif
#ifndef MOE_SITU_NT_STORE
#define MOE_SITU_NT_STORE 1
#endif
constexpr int kU = MOE_SITU_UNROLL;

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
#if MOE_SITU_NT_LOAD
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}
__device__ __forceinline__ void st16(u32x4 v, uint16_t* p) {
#if MOE_SITU_NT_STORE
  __builtin_nontemporal_store(v, (u32x4*)p);
#else
  *(u32x4*)p = v;
#endif
}

struct ChunkWalk {
  int64_t r, dr;
  int cc, dc, hc;
  __device__ void init(int64_t i0, int64_t stride, int hc_) {
    hc = hc_;
    dr = stride / hc;
    dc = (int)(stride - dr * hc);
    r = i0 / hc;
    cc = (int)(i0 - r * hc);
  }
  __device__ void step() {
    r += dr;
    cc += dc;
    if (cc >= hc) { cc -= hc; r += 1; }
  }
};

template <bool B4>
__global__ __launch_bounds__(256) void situ_fwd_kernel(const uint16_t* __restrict__ h,
                                                       int64_t R, int H, SituCoef c,
                                                       uint16_t* __restrict__ a) {
  ChunkWalk w;
  w.init((int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x,
         H >> 3);
  while (w.r < R) {
    int64_t ro[kU];
    int co[kU];
    u32x4 g[kU], l[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      ro[u] = w.r;
      co[u] = w.cc;
      if (w.r < R) {
        const uint16_t* hr = h + w.r * (2 * (int64_t)H) + 8 * w.cc;
        g[u] = ld16(hr);
        l[u] = ld16(hr + H);
      }
      w.step();
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ro[u] >= R) break;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a0 = situ_fwd<B4>(bf16_lo(g[u][q]), bf16_lo(l[u][q]), c);
        const float a1 = situ_fwd<B4>(bf16_hi(g[u][q]), bf16_hi(l[u][q]), c);
        o[q] = pack_bf16x2(a0, a1);
      }
      st16(o, a + ro[u] * (int64_t)H + 8 * co[u]);
    }
  }
}

template <bool B4>
__global__ __launch_bounds__(256) void situ_bwd_kernel(const uint16_t* __restrict__ h,
                                                       const uint16_t* __restrict__ da,
                                                       int64_t R, int H, SituCoef c,
                                                       uint16_t* __restrict__ dh) {
  ChunkWalk w;
  w.init((int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x,
         H >> 3);
  while (w.r < R) {
    int64_t ro[kU];
    int co[kU];
    u32x4 g[kU], l[kU], d[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      ro[u] = w.r;
      co[u] = w.cc;
      if (w.r < R) {
        const int64_t hoff = w.r * (2 * (int64_t)H) + 8 * w.cc;
        g[u] = ld16(h + hoff);
        l[u] = ld16(h + hoff + H);
        d[u] = ld16(da + w.r * (int64_t)H + 8 * w.cc);
      }
      w.step();
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ro[u] >= R) break;
      u32x4 og, ol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float g0, l0, g1, l1;
        situ_grad<B4>(bf16_lo(g[u][q]), bf16_lo(l[u][q]), bf16_lo(d[u][q]), c, g0, l0);
        situ_grad<B4>(bf16_hi(g[u][q]), bf16_hi(l[u][q]), bf16_hi(d[u][q]), c, g1, l1);
        og[q] = pack_bf16x2(g0, g1);
        ol[q] = pack_bf16x2(l0, l1);
      }
      const int64_t hoff = ro[u] * (2 * (int64_t)H) + 8 * co[u];
      st16(og, dh + hoff);
      st16(ol, dh + hoff + H);
    }
  }
}

static unsigned situ_grid(int64_t n) {
  int64_t blocks = (n + 256 * kU - 1) / (256 * kU);
  const int64_t cap = (int64_t)device_cu_count() * MOE_SITU_BLOCKS_PER_CU;
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t launch_situ_fwd(const uint16_t* h, int64_t R, int H, SituCoef c, uint16_t* a,
                           hipStream_t s) {
  const int64_t n = R * (int64_t)(H / 8);
  if (n == 0) return hipSuccess;
  if (c.b4) hipLaunchKernelGGL(situ_fwd_kernel<true>, dim3(situ_grid(n)), dim3(256), 0, s, h, R, H, c, a);
  else hipLaunchKernelGGL(situ_fwd_kernel<false>, dim3(situ_grid(n)), dim3(256), 0, s, h, R, H, c, a);
  return hipGetLastError();
}

hipError_t launch_situ_bwd(const uint16_t* h, const uint16_t* da, int64_t R, int H,
                           SituCoef c, uint16_t* dh, hipStream_t s) {
  const int64_t n = R * (int64_t)(H / 8);
  if (n == 0) return hipSuccess;
  if (c.b4) hipLaunchKernelGGL(situ_bwd_kernel<true>, dim3(situ_grid(n)), dim3(256), 0, s, h, da, R, H, c, dh);
  else hipLaunchKernelGGL(situ_bwd_kernel<false>, dim3(situ_grid(n)), dim3(256), 0, s, h, da, R, H, c, dh);
  return hipGetLastError();
}

}  // namespace moe
