// Streaming SiTU-GLU forward and backward (gfx950).
//
// "Frontier-scale RL with Kimi K3", section "Streaming activations": the custom op keeps
// only the bf16 pre-activation h = [g | l] of shape [R, 2H], streams over it with a
// constant-size fp32 working set, and recomputes tanh and sigmoid in the backward; this is
// valid because the activation is elementwise.
//
// Here each lane owns 16-byte chunks (8 columns) of a row: it reads g and l (and da) with
// 16-byte non-temporal loads, keeps all fp32 intermediates in registers and writes the
// bf16 result with 16-byte non-temporal stores. One launch covers every chunk once: a thread
// takes KU chunks 256 apart and finds each chunk's row and column with one 32-bit division
// by the chunks per row, so nothing is set up per thread beyond that. Chunk indices past the
// end are clamped to the last chunk, so every lane loads, computes and stores without a
// branch: the lanes of the last block that run past the end rewrite the last chunk with the
// same bytes its own lane writes. Launches are split by rows so each covers fewer than 2^32
// chunks. No memory beyond the inputs and outputs is used, whatever R. On MI355X at
// R = 131072, H = 3072, a grid-stride walk of 256 workgroups per CU measured 3-6 % slower
// than one launch over every chunk, and plain (temporal) loads 5-10 % slower.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include "common.h"
#include "launch.h"
#include "situ_math.h"

namespace moe {

#ifndef MOE_SITU_NT_LOAD
#define MOE_SITU_NT_LOAD 1
#endif
#ifndef MOE_SITU_NT_STORE
#define MOE_SITU_NT_STORE 1
#endif

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

// Chunks per thread: two for the forward (four 16-byte loads) and two for the backward
// (six). Measured against 1, 4 and 8 on R = 131072, H = 3072: within 1 %, except 8 for the
// forward and 4 for the backward, 3-5 % slower.
#ifndef MOE_SITU_FWD_KU
#define MOE_SITU_FWD_KU 2
#endif
#ifndef MOE_SITU_BWD_KU
#define MOE_SITU_BWD_KU 2
#endif
constexpr int kFwdKU = MOE_SITU_FWD_KU;
constexpr int kBwdKU = MOE_SITU_BWD_KU;

template <bool B4>
__global__ __launch_bounds__(256) void situ_fwd_kernel(const uint16_t* __restrict__ h,
                                                       uint32_t n, uint32_t hc, int H,
                                                       SituCoef c, uint16_t* __restrict__ a) {
  constexpr int KU = kFwdKU;
  const uint32_t i0 = blockIdx.x * (256u * KU) + threadIdx.x;
  u32x4 g[KU], l[KU];
  uint32_t rr[KU], cc[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const uint32_t i = min(i0 + 256u * u, n - 1u);
    rr[u] = i / hc;
    cc[u] = i - rr[u] * hc;
    const uint16_t* hr = h + (int64_t)rr[u] * (2 * H) + 8 * cc[u];
    g[u] = ld16(hr);
    l[u] = ld16(hr + H);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load is issued before the first use
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = situ_fwd<B4>(bf16_lo(g[u][q]), bf16_lo(l[u][q]), c);
      const float a1 = situ_fwd<B4>(bf16_hi(g[u][q]), bf16_hi(l[u][q]), c);
      o[q] = pack_bf16x2(a0, a1);
    }
    st16(o, a + (int64_t)rr[u] * H + 8 * cc[u]);
  }
}

template <bool B4>
__global__ __launch_bounds__(256) void situ_bwd_kernel(const uint16_t* __restrict__ h,
                                                       const uint16_t* __restrict__ da,
                                                       uint32_t n, uint32_t hc, int H,
                                                       SituCoef c, uint16_t* __restrict__ dh) {
  constexpr int KU = kBwdKU;
  const uint32_t i0 = blockIdx.x * (256u * KU) + threadIdx.x;
  u32x4 g[KU], l[KU], d[KU];
  uint32_t rr[KU], cc[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const uint32_t i = min(i0 + 256u * u, n - 1u);
    rr[u] = i / hc;
    cc[u] = i - rr[u] * hc;
    const int64_t hoff = (int64_t)rr[u] * (2 * H) + 8 * cc[u];
    g[u] = ld16(h + hoff);
    l[u] = ld16(h + hoff + H);
    d[u] = ld16(da + (int64_t)rr[u] * H + 8 * cc[u]);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load is issued before the first use
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    u32x4 og, ol;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float g0, l0, g1, l1;
      situ_grad<B4>(bf16_lo(g[u][q]), bf16_lo(l[u][q]), bf16_lo(d[u][q]), c, g0, l0);
      situ_grad<B4>(bf16_hi(g[u][q]), bf16_hi(l[u][q]), bf16_hi(d[u][q]), c, g1, l1);
      og[q] = pack_bf16x2(g0, g1);
      ol[q] = pack_bf16x2(l0, l1);
    }
    const int64_t hoff = (int64_t)rr[u] * (2 * H) + 8 * cc[u];
    st16(og, dh + hoff);
    st16(ol, dh + hoff + H);
  }
}

// Rows per launch: each launch covers fewer than 2^32 chunks (H / 8 per row), with room for
// the last block's overhang. MOE_SITU_ROWS_PER_LAUNCH (environment, read per call) may lower
// it, so the split across launches can be exercised on small inputs.
static int64_t situ_rows_per_launch(int H) {
  int64_t step = (((int64_t)1 << 32) - 4096) / (H / 8);
  if (const char* env = getenv("MOE_SITU_ROWS_PER_LAUNCH")) {
    const long long v = atoll(env);
    if (v > 0 && v < step) step = v;
  }
  return step;
}

hipError_t launch_situ_fwd(const uint16_t* h, int64_t R, int H, SituCoef c, uint16_t* a,
                           hipStream_t s) {
  const uint32_t hc = (uint32_t)(H / 8);
  const int64_t step = situ_rows_per_launch(H);
  for (int64_t r0 = 0; r0 < R; r0 += step) {
    const int64_t rows = (R - r0 < step) ? R - r0 : step;
    const uint32_t n = (uint32_t)(rows * hc);
    const unsigned blocks = (unsigned)((n + 256u * kFwdKU - 1) / (256u * kFwdKU));
    const uint16_t* hp = h + r0 * 2 * H;
    uint16_t* ap = a + r0 * H;
    if (c.b4) hipLaunchKernelGGL(situ_fwd_kernel<true>, dim3(blocks), dim3(256), 0, s, hp, n, hc, H, c, ap);
    else hipLaunchKernelGGL(situ_fwd_kernel<false>, dim3(blocks), dim3(256), 0, s, hp, n, hc, H, c, ap);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_situ_bwd(const uint16_t* h, const uint16_t* da, int64_t R, int H,
                           SituCoef c, uint16_t* dh, hipStream_t s) {
  const uint32_t hc = (uint32_t)(H / 8);
  const int64_t step = situ_rows_per_launch(H);
  for (int64_t r0 = 0; r0 < R; r0 += step) {
    const int64_t rows = (R - r0 < step) ? R - r0 : step;
    const uint32_t n = (uint32_t)(rows * hc);
    const unsigned blocks = (unsigned)((n + 256u * kBwdKU - 1) / (256u * kBwdKU));
    const uint16_t* hp = h + r0 * 2 * H;
    const uint16_t* dap = da + r0 * H;
    uint16_t* dhp = dh + r0 * 2 * H;
    if (c.b4) hipLaunchKernelGGL(situ_bwd_kernel<true>, dim3(blocks), dim3(256), 0, s, hp, dap, n, hc, H, c, dhp);
    else hipLaunchKernelGGL(situ_bwd_kernel<false>, dim3(blocks), dim3(256), 0, s, hp, dap, n, hc, H, c, dhp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
