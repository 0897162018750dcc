// Routing, dispatch metadata, combine and the small reductions of the backward (gfx950).
//
// Routing follows "Inside Kimi K3", section "Idea One" (top-k of the router scores, softmax
// over the kept values). The dispatch metadata is the on-GPU form of the expert-sorted
// token copy of "Kimi K3 ... Memory", section "MoE 反向" (second saving).
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------------------ routing
// One wavefront per token. Each lane holds NV logits (expert e = lane + 64 i). k rounds of
// a wavefront arg-max (value descending, index ascending on ties) pick the slots in order;
// the picked value's owner lane retires it. The softmax runs in fp32 over the k picks.
template <int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ gates_out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwave = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t t = wave; t < T; t += nwave) {
    const float* row = logits + t * (int64_t)E;
    float v[NV];
    uint32_t retired = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? row[e] : 0.0f;
      if (e >= E) retired |= 1u << i;
    }
    float my_v = 0.0f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        // ascending e within the lane, so a strict '>' keeps the lower index on ties
        if (!((retired >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
          bv = v[i];
          bi = lane + 64 * i;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) retired |= 1u << (bi >> 6);
      if (lane == j) {
        my_v = bv;
        my_i = bi;
      }
    }
    const float m = __shfl(my_v, 0, 64);        // first pick is the maximum
    float ex = (lane < k) ? expf(my_v - m) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < k) {
      idx_out[t * k + lane] = my_i;
      gates_out[t * k + lane] = ex / sum;
    }
  }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* idx,
                             float* gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nv = (E + 63) / 64;
  const int64_t waves_needed = T;
  int64_t blocks = (waves_needed + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  dim3 grid((unsigned)blocks), block(256);
  if (nv <= 1) hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, idx, gates);
  else if (nv <= 2) hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, idx, gates);
  else if (nv <= 4) hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, idx, gates);
  else if (nv <= 8) hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, idx, gates);
  else hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, idx, gates);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ permute
// Counting sort of the local routes by expert, stable by token:
//   1. count:   per 256-token block, a histogram over local experts (LDS atomics only add,
//               so the counts do not depend on ordering);
//   2. scan:    one workgroup turns the expert-major [E_loc][nblk] counts into row bases;
//   3. scatter: per block, the rank of a token among the block's tokens that picked the
//               same expert is a popcount over a per-expert token bitmask, so rows follow
//               token order exactly.
constexpr int kPermTok = 256;

int permute_blocks(int64_t T) { return (int)((T + kPermTok - 1) / kPermTok); }

size_t permute_ws_bytes(int64_t T, int E_loc) {
  const size_t n = (size_t)E_loc * (size_t)(permute_blocks(T) > 0 ? permute_blocks(T) : 1);
  return ((n * sizeof(int32_t) + 255) / 256) * 256;
}

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                            int64_t T, int k, int e_lo,
                                                            int E_loc, int nblk,
                                                            int32_t* __restrict__ cnt) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E_loc; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPermTok + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j] - e_lo;
      if ((unsigned)e < (unsigned)E_loc) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E_loc; e += 256) cnt[(int64_t)e * nblk + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* cnt, int n,
                                                            int nblk, int E_loc, int64_t R_cap,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ status) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int seg = (n + 1023) / 1024;
  const int lo = tid * seg;
  const int hi = min(lo + seg, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += cnt[i];
  part[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - local;        // exclusive prefix of this segment
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run;
    run += c;
  }
  __threadfence_block();
  __syncthreads();
  const int total = part[1023];
  for (int e = tid; e < E_loc; e += 1024) {
    const int64_t b = (nblk > 0) ? cnt[(int64_t)e * nblk] : 0;
    offsets[e] = (int32_t)(b < R_cap ? b : R_cap);
  }
  if (tid == 0) {
    offsets[E_loc] = (int32_t)((int64_t)total < R_cap ? (int64_t)total : R_cap);
    status[0] = ((int64_t)total > R_cap) ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gates, int64_t T, int k,
    int e_lo, int E_loc, int nblk, const int32_t* __restrict__ base, int64_t R_cap,
    int32_t* __restrict__ row_token, float* __restrict__ row_gate,
    int32_t* __restrict__ slot_row) {
  __shared__ uint32_t mask[1024 * 8];   // [expert][256 token bits]
  for (int i = threadIdx.x; i < E_loc * 8; i += 256) mask[i] = 0;
  __syncthreads();
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kPermTok + tid;
  const bool valid = t < T;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (valid) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j] - e_lo;
      if ((unsigned)e < (unsigned)E_loc) atomicOr(&mask[e * 8 + w], bit);
    }
  }
  __syncthreads();
  if (!valid) return;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j] - e_lo;
    int32_t row = -1;
    if ((unsigned)e < (unsigned)E_loc) {
      int rank = __popc(mask[e * 8 + w] & (bit - 1u));
      for (int q = 0; q < w; ++q) rank += __popc(mask[e * 8 + q]);
      const int64_t r = (int64_t)base[(int64_t)e * nblk + blockIdx.x] + rank;
      if (r < R_cap) {
        row = (int32_t)r;
        row_token[r] = (int32_t)t;
        row_gate[r] = gates[t * k + j];
      }
    }
    slot_row[t * k + j] = row;
  }
}

hipError_t launch_permute(const int32_t* idx, const float* gates, int64_t T, int k, int e_lo,
                          int E_loc, int64_t R_cap, int32_t* offsets, int32_t* row_token,
                          float* row_gate, int32_t* slot_row, int32_t* status, void* ws,
                          hipStream_t s) {
  const int nblk = permute_blocks(T);
  int32_t* cnt = (int32_t*)ws;
  if (nblk > 0) {
    hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(256), 0, s, idx, T, k, e_lo,
                       E_loc, nblk, cnt);
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, E_loc * nblk, nblk,
                     E_loc, R_cap, offsets, status);
  if (nblk > 0) {
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(256), 0, s, idx, gates, T, k,
                       e_lo, E_loc, nblk, cnt, R_cap, row_token, row_gate, slot_row);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ combine
// out[t] = bf16( sum_j w(r) rows[r] ), r = slot_row[t, j] >= 0, in fp32 and slot order.
// One workgroup per token at a time; each lane owns 8 consecutive columns (16 bytes).
__global__ __launch_bounds__(256) void unpermute_kernel(const uint16_t* __restrict__ rows,
                                                        const int32_t* __restrict__ slot_row,
                                                        const float* __restrict__ w,
                                                        int64_t T, int k, int n,
                                                        uint16_t* __restrict__ out) {
  const int nc = n >> 3;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* sr = slot_row + t * k;
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int r = sr[j];
        if (r < 0) continue;
        const float wt = w ? w[r] : 1.0f;
        const u32x4 v = *(const u32x4*)(rows + (int64_t)r * n + 8 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wt * bf16_lo(v[q]);
          acc[2 * q + 1] += wt * bf16_hi(v[q]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      *(u32x4*)(out + t * n + 8 * c) = o;
    }
  }
}

hipError_t launch_unpermute(const uint16_t* rows, const int32_t* slot_row, const float* w,
                            int64_t T, int k, int n, uint16_t* out, hipStream_t s) {
  if (T == 0 || n == 0) return hipSuccess;
  int64_t blocks = T;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)blocks), dim3(256), 0, s, rows, slot_row,
                     w, T, k, n, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ dp
// dp partials come in [nslots][R_cap] (one slot per (N-tile, wave column) of the dA GEMM).
// Pass 1 sums the slots of each row into slot 0 in a fixed order (coalesced over rows);
// pass 2 scatters rows to (token, slot), zero for non-local slots.
__global__ __launch_bounds__(256) void dp_row_reduce_kernel(float* __restrict__ part,
                                                            int nslots, int64_t R_cap,
                                                            const int32_t* __restrict__ offsets,
                                                            int E_loc) {
  const int64_t R = offsets[E_loc];
  for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < R;
       r += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int q = 0; q < nslots; ++q) s += part[(int64_t)q * R_cap + r];
    part[r] = s;
  }
}

__global__ __launch_bounds__(256) void dp_scatter_kernel(const float* __restrict__ dp_rows,
                                                         const int32_t* __restrict__ slot_row,
                                                         int64_t n, float* __restrict__ dp) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int r = slot_row[i];
    dp[i] = (r >= 0) ? dp_rows[r] : 0.0f;
  }
}

hipError_t launch_dp_reduce_scatter(float* part, int nslots, int64_t R_cap,
                                    const int32_t* offsets, int E_loc,
                                    const int32_t* slot_row, int64_t T, int k, float* dp,
                                    hipStream_t s) {
  const int64_t cap = (int64_t)device_cu_count() * 8;
  int64_t b1 = (R_cap + 255) / 256;
  if (b1 > cap) b1 = cap;
  if (b1 > 0)
    hipLaunchKernelGGL(dp_row_reduce_kernel, dim3((unsigned)b1), dim3(256), 0, s, part, nslots,
                       R_cap, offsets, E_loc);
  const int64_t n = T * k;
  int64_t b2 = (n + 255) / 256;
  if (b2 > cap) b2 = cap;
  if (b2 > 0)
    hipLaunchKernelGGL(dp_scatter_kernel, dim3((unsigned)b2), dim3(256), 0, s, part, slot_row,
                       n, dp);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ router bwd
// dL/dv_j = p_j (g_j - sum_i p_i g_i) for the softmax over the kept logits.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ p,
                                                         const float* __restrict__ g,
                                                         int64_t T, int k,
                                                         float* __restrict__ out) {
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T;
       t += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s += p[t * k + j] * g[t * k + j];
    for (int j = 0; j < k; ++j) out[t * k + j] = p[t * k + j] * (g[t * k + j] - s);
  }
}

hipError_t launch_router_bwd(const float* gates, const float* dp, int64_t T, int k,
                             float* dlogits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int64_t b = (T + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (b > cap) b = cap;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)b), dim3(256), 0, s, gates, dp, T, k,
                     dlogits);
  return hipGetLastError();
}

}  // namespace moe
