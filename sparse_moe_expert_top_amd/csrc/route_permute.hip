// Routing, dispatch metadata, combine and the small reductions of the backward (gfx950).
//
// Routing follows "Inside Kimi K3", section "Idea One" (top-k of the router scores, softmax
// over the kept values). The dispatch metadata is the on-GPU form of the expert-sorted
// token copy of "Kimi K3 ... Memory", section "MoE 反向" (second saving).
#include <hip/hip_runtime.h>

#include <type_traits>
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------------------ routing
// Up to 32 experts, one lane per token (route_topk_lane_kernel below); otherwise one
// wavefront per token, lane l holding the logits of experts l, l+64, ... . Every logit
// becomes a 64-bit key whose order is the routing order: the high word is the fp32 value
// bits mapped to an unsigned order (-0 -> +0 first, so the two zeros tie), the low word is the
// complement of the expert index (equal values: lower index first). Keys are unique, so
// "the k largest keys in descending order" is exactly the slot order.
//
// Selection: thr = the k-th largest of the 64 per-lane maxima, taken over the keys' value
// words by a bitwise radix select (one ballot per bit). At least k logits have a value at
// or above thr, so the top k are among them. When at most 64 pass (the usual case: ~20-30
// of 896 for k = 16), they are compacted through LDS, each one's rank among them is counted
// from broadcast LDS reads, and the k best are placed by rank; lane j then holds slot j.
// Otherwise (many ties) k rounds of a wave arg-max pick them one by one. The softmax runs
// in fp32 over the k picked values.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;                     // -0 -> +0 on the bits (no float op)
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(~e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// NV = ceil(E / 64) exactly (the launcher instantiates 1..16, E <= 1024). Each wavefront
// spends most of a token waiting on dependent steps, so the kernel is compiled for five
// wavefronts per SIMD (at most 96 VGPRs, no spills) rather than the four its free register
// allocation gives.
template <int NV>
__global__ __launch_bounds__(256, 5) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ gates_out) {
  __shared__ uint64_t cand[4][64];
  __shared__ uint64_t sel[4][32];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwave = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t t = wave; t < T; t += nwave) {
    const float* row = logits + t * (int64_t)E;
    // all of the row's loads first, so they are in flight together (a guarded load would be
    // one round trip per 64 logits). NV = ceil(E / 64): only the last group can pass E, and
    // its lanes past E re-read column E-1 (in bounds).
    float val[NV];
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) val[i] = row[lane + 64 * i];
    val[NV - 1] = row[min(lane + 64 * (NV - 1), E - 1)];
    // value words of the keys (the index word of logit i is ~(lane + 64 i)); bit i of
    // `live` marks logit i as present (lane + 64 i < E) and, in the many-ties path, not yet
    // picked. An absent key reads as 0, below every real key.
    uint32_t kv[NV];
    uint32_t live = 0;
    uint32_t lmax = 0;                                // value word of the lane's best key
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      kv[i] = (e < E) ? (uint32_t)(route_key(val[i], e) >> 32) : 0u;
      if (e < E) live |= 1u << i;
      lmax = kv[i] > lmax ? kv[i] : lmax;
    }
    auto key = [&](int i) __attribute__((always_inline)) -> uint64_t {
      return ((live >> i) & 1u) ? (((uint64_t)kv[i] << 32) | (uint32_t)~(lane + 64 * i)) : 0;
    };
    // largest thr with at least k lane maxima >= thr
    uint32_t thr = 0;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = thr | (1u << bit);
      if (__builtin_popcountll(__ballot(lmax >= c)) >= k) thr = c;
    }
    int c = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) c += (((live >> i) & 1u) && kv[i] >= thr) ? 1 : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);
    uint64_t mine = 0;
    if (total <= 64) {
      int pos = incl - c;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (((live >> i) & 1u) && kv[i] >= thr) cand[wv][pos++] = key(i);
      __builtin_amdgcn_wave_barrier();
      const uint64_t my = (lane < total) ? cand[wv][lane] : 0;
      // rank among the candidates: broadcast reads, eight in flight at a time
      int rank = 0;
      int j = 0;
      for (; j + 8 <= total; j += 8) {
        uint64_t cj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cj[u] = cand[wv][j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (cj[u] > my) ? 1 : 0;
      }
      for (; j < total; ++j) rank += (cand[wv][j] > my) ? 1 : 0;
      if (lane < total && rank < k) sel[wv][rank] = my;
      __builtin_amdgcn_wave_barrier();
      if (lane < k) mine = sel[wv][lane];
      __builtin_amdgcn_wave_barrier();
    } else {
      for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) best = key(i) > best ? key(i) : best;
        best = wave_max64(best);
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (key(i) == best) live &= ~(1u << i);      // keys are unique: only the winner
        if (lane == j) mine = best;
      }
    }
    const float v = key_value(mine);
    const float m = __shfl(v, 0, 64);                 // slot 0 holds the maximum
    const float ex = (lane < k) ? expf(v - m) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < k) {
      idx_out[t * k + lane] = key_index(mine);
      gates_out[t * k + lane] = ex / sum;
    }
  }
}

// Routing for E <= EM <= 32, one lane per token: the token's E logits become the same order
// keys as above; a key's slot is the number of the token's keys above it (keys are unique),
// so the k largest go straight to their slots, and the softmax takes its maximum, the value
// of slot 0, from the largest key (keys past E read as 0, below every real key). A block's
// 256 rows of logits, and its [256, k] outputs, are contiguous in memory, so both move
// between HBM and LDS as whole contiguous ranges and each lane works from LDS.
template <int EM>
__global__ __launch_bounds__(256) void route_topk_lane_kernel(const float* __restrict__ logits,
                                                              int64_t T, int E, int k,
                                                              int32_t* __restrict__ idx_out,
                                                              float* __restrict__ gates_out) {
  __shared__ float s_val[256 * EM];
  __shared__ int32_t s_idx[256 * EM];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 256;
  const int rows = (int)min((int64_t)256, T - t0);
  const int n_in = rows * E;
  const float* src = logits + t0 * E;
  // every load issued before any LDS store (a guarded load-store pair per element would wait
  // out one memory round trip each); indices past the block's range re-read its last element
  float in[EM];
#pragma unroll
  for (int j = 0; j < EM; ++j) in[j] = src[min(tid + 256 * j, n_in - 1)];
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    const int i = tid + 256 * j;
    if (i < n_in) s_val[i] = in[j];
  }
  __syncthreads();
  int slot[EM];
  float ex[EM];
  float sum = 0.0f;
  if (tid < rows) {
    uint64_t key[EM];
    uint64_t kmax = 0;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      key[e] = (e < E) ? route_key(s_val[tid * E + e], e) : 0ull;
      kmax = key[e] > kmax ? key[e] : kmax;
    }
    const float m = key_value(kmax);
#pragma unroll
    for (int i = 0; i < EM; ++i) {
      int r = 0;
#pragma unroll
      for (int j = 0; j < EM; ++j) r += (key[j] > key[i]) ? 1 : 0;
      slot[i] = (i < E && r < k) ? r : -1;
      ex[i] = (slot[i] >= 0) ? expf(key_value(key[i]) - m) : 0.0f;
      sum += ex[i];
    }
  }
  __syncthreads();                                   // every lane is done reading the logits
  if (tid < rows) {
#pragma unroll
    for (int i = 0; i < EM; ++i) {
      if (slot[i] >= 0) {
        s_idx[tid * k + slot[i]] = i;
        s_val[tid * k + slot[i]] = ex[i] / sum;
      }
    }
  }
  __syncthreads();
  const int n_out = rows * k;
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    const int i = tid + 256 * j;
    if (i < n_out) {
      idx_out[t0 * k + i] = s_idx[i];
      gates_out[t0 * k + i] = s_val[i];
    }
  }
}

// Launches route_topk_kernel<nv> for the runtime nv in [NV, 16].
template <int NV>
static void route_launch_nv(int nv, dim3 grid, const float* logits, int64_t T, int E, int k,
                            int32_t* idx, float* gates, hipStream_t s) {
  if constexpr (NV <= 16) {
    if (nv == NV)
      hipLaunchKernelGGL(route_topk_kernel<NV>, grid, dim3(256), 0, s, logits, T, E, k, idx, gates);
    else
      route_launch_nv<NV + 1>(nv, grid, logits, T, E, k, idx, gates, s);
  }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* idx,
                             float* gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 32) {
    const dim3 grid((unsigned)((T + 255) / 256));
    if (E <= 8)
      hipLaunchKernelGGL(route_topk_lane_kernel<8>, grid, dim3(256), 0, s, logits, T, E, k, idx, gates);
    else if (E <= 16)
      hipLaunchKernelGGL(route_topk_lane_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, idx, gates);
    else
      hipLaunchKernelGGL(route_topk_lane_kernel<32>, grid, dim3(256), 0, s, logits, T, E, k, idx, gates);
    return hipGetLastError();
  }
  const int nv = (E + 63) / 64;
  const int64_t waves_needed = T;
  int64_t blocks = (waves_needed + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  // NV must equal ceil(E / 64): the kernel reads groups 0 .. NV-2 unguarded
  route_launch_nv<1>(nv, dim3((unsigned)blocks), logits, T, E, k, idx, gates, s);
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
// A token's k expert indices (k <= KM), loaded together: entries past k re-read entry k-1
// (in bounds), so no load is guarded and none waits for the previous one. The kernels are
// instantiated for KM = 16 (k <= 16) and KM = 32.
template <int KM>
__device__ __forceinline__ void load_token_routes(const int32_t* __restrict__ row, int k,
                                                  int (&ev)[KM]) {
#pragma unroll
  for (int j = 0; j < KM; ++j) ev[j] = row[min(j, k - 1)];
}
// A token's KM route entries in 16-byte pieces (k == KM and 16-byte aligned rows).
template <int KM, typename T>
__device__ __forceinline__ void load_row_vec(const T* __restrict__ row, T (&v)[KM]) {
  static_assert(sizeof(T) == 4 && KM % 4 == 0, "16-byte pieces of 4-byte entries");
#pragma unroll
  for (int q = 0; q < KM / 4; ++q) {
    const u32x4 w = *(const u32x4*)(row + 4 * q);
    // (element-wise conversions: a bit cast of one vector element reads element 0 on this
    // compiler)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (std::is_same<T, float>::value) v[4 * q + c] = __uint_as_float(w[c]);
      else v[4 * q + c] = (T)w[c];
    }
  }
}

int permute_blocks(int64_t T) { return (int)((T + kPermTok - 1) / kPermTok); }

size_t permute_ws_bytes(int64_t T, int E_loc) {
  const size_t n = (size_t)E_loc * (size_t)(permute_blocks(T) > 0 ? permute_blocks(T) : 1);
  return ((n * sizeof(int32_t) + 255) / 256) * 256;
}

template <int KM>
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                            int64_t T, int k, int e_lo,
                                                            int E_loc, int nblk,
                                                            int32_t* __restrict__ cnt) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E_loc; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPermTok + threadIdx.x;
  if (t < T) {
    int ev[KM];
    if (k == KM && ((uintptr_t)idx & 15u) == 0) load_row_vec(idx + t * KM, ev);
    else load_token_routes(idx + t * k, k, ev);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = ev[j] - e_lo;
      if (j < k && (unsigned)e < (unsigned)E_loc) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E_loc; e += 256) cnt[(int64_t)e * nblk + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* cnt, int n,
                                                            int nblk, int E_loc, int64_t R_cap,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ status) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int seg = (n + 1023) / 1024;
  const int lo = tid * seg;
  const int hi = min(lo + seg, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += cnt[i];
  // inclusive scan of the segment sums: within each wavefront by shuffles, then over the 16
  // wavefront totals by the first wavefront
  int x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = (lane < 16) ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < 16) wsum[lane] = t;
  }
  __syncthreads();
  int run = (wv ? wsum[wv - 1] : 0) + x - local;     // exclusive prefix of this segment
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run;
    run += c;
  }
  __threadfence_block();
  __syncthreads();
  const int total = wsum[15];
  for (int e = tid; e < E_loc; e += 1024) {
    const int64_t b = (nblk > 0) ? cnt[(int64_t)e * nblk] : 0;
    offsets[e] = (int32_t)(b < R_cap ? b : R_cap);
  }
  if (tid == 0) {
    offsets[E_loc] = (int32_t)((int64_t)total < R_cap ? (int64_t)total : R_cap);
    status[0] = ((int64_t)total > R_cap) ? 1 : 0;
  }
}

template <int KM>
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gates, int64_t T, int k,
    int e_lo, int E_loc, int nblk, const int32_t* __restrict__ base, int64_t R_cap,
    int32_t* __restrict__ row_token, float* __restrict__ row_gate,
    int32_t* __restrict__ slot_row) {
  __shared__ uint32_t mask[1024 * 8];   // [expert][256 token bits]
  __shared__ int first[1024 * 8];       // [expert][wave]: row of the wave's first route there
  for (int i = threadIdx.x; i < E_loc * 8; i += 256) mask[i] = 0;
  __syncthreads();
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kPermTok + tid;
  const bool valid = t < T;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  // whole rows in 16-byte pieces when a token's k entries fill KM and the arrays allow it
  const bool vec = k == KM && (((uintptr_t)idx | (uintptr_t)gates | (uintptr_t)slot_row) & 15u) == 0;
  int ev[KM];
  if (valid) {
    if (vec) load_row_vec(idx + t * KM, ev);
    else load_token_routes(idx + t * k, k, ev);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = ev[j] - e_lo;
      if (j < k && (unsigned)e < (unsigned)E_loc) atomicOr(&mask[e * 8 + w], bit);
    }
  }
  __syncthreads();
  // the block's first row of each expert plus the routes of the earlier wavefronts' tokens
  for (int e = tid; e < E_loc; e += 256) {
    int run = base[(int64_t)e * nblk + blockIdx.x];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      first[e * 8 + q] = run;
      run += __popc(mask[e * 8 + q]);
    }
  }
  __syncthreads();
  if (!valid) return;
  float gv[KM];
  const float* grow = gates + t * k;
  if (vec) {
    load_row_vec(grow, gv);
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j) gv[j] = grow[min(j, k - 1)];
  }
  int32_t srow[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    srow[j] = -1;
    if (j >= k) continue;   // k is uniform; continue (not break) lets the loop unroll fully
    const int e = ev[j] - e_lo;
    if ((unsigned)e < (unsigned)E_loc) {
      const int64_t r = (int64_t)first[e * 8 + w] + __popc(mask[e * 8 + w] & (bit - 1u));
      if (r < R_cap) {
        srow[j] = (int32_t)r;
        row_token[r] = (int32_t)t;
        row_gate[r] = gv[j];
      }
    }
  }
  if (vec) {
#pragma unroll
    for (int q = 0; q < KM / 4; ++q)
      *(u32x4*)(slot_row + t * KM + 4 * q) =
          u32x4{(uint32_t)srow[4 * q], (uint32_t)srow[4 * q + 1], (uint32_t)srow[4 * q + 2],
                (uint32_t)srow[4 * q + 3]};
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) slot_row[t * k + j] = srow[j];
  }
}

hipError_t launch_permute(const int32_t* idx, const float* gates, int64_t T, int k, int e_lo,
                          int E_loc, int64_t R_cap, int32_t* offsets, int32_t* row_token,
                          float* row_gate, int32_t* slot_row, int32_t* status, void* ws,
                          hipStream_t s) {
  const int nblk = permute_blocks(T);
  int32_t* cnt = (int32_t*)ws;
  if (nblk > 0) {
    if (k <= 16)
      hipLaunchKernelGGL(permute_count_kernel<16>, dim3(nblk), dim3(256), 0, s, idx, T, k, e_lo,
                         E_loc, nblk, cnt);
    else
      hipLaunchKernelGGL(permute_count_kernel<32>, dim3(nblk), dim3(256), 0, s, idx, T, k, e_lo,
                         E_loc, nblk, cnt);
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, E_loc * nblk, nblk,
                     E_loc, R_cap, offsets, status);
  if (nblk > 0) {
    if (k <= 16)
      hipLaunchKernelGGL(permute_scatter_kernel<16>, dim3(nblk), dim3(256), 0, s, idx, gates, T,
                         k, e_lo, E_loc, nblk, cnt, R_cap, row_token, row_gate, slot_row);
    else
      hipLaunchKernelGGL(permute_scatter_kernel<32>, dim3(nblk), dim3(256), 0, s, idx, gates, T,
                         k, e_lo, E_loc, nblk, cnt, R_cap, row_token, row_gate, slot_row);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ combine
// out[t] = bf16( sum_j w(r) rows[r] ), r = slot_row[t, j] >= 0, in fp32 and slot order.
// One wavefront per token at a time, so a CU keeps as many tokens in flight as it holds
// wavefronts. The wave loads the token's k slot entries (and their weights) at once, one per
// lane, and walks only the local ones, two at a time; each lane owns CPL units of 8
// consecutive columns per pass (one 16-byte load of bf16 rows, two of fp32 rows), so the
// loads of a pass are in flight together. The output row is written with streaming stores.
constexpr int kCombCPL = 4;
template <typename RowT>
__global__ __launch_bounds__(256) void unpermute_kernel(const RowT* __restrict__ rows,
                                                        int64_t ldr,
                                                        const int32_t* __restrict__ slot_row,
                                                        const float* __restrict__ w,
                                                        int64_t T, int k, int n,
                                                        uint16_t* __restrict__ out,
                                                        int64_t ldo) {
  constexpr int VB = sizeof(RowT) == 2 ? 1 : 2;     // 16-byte loads per 8 columns
  const int nc = n >> 3;
  const int lane = threadIdx.x & 63;
  const int64_t nwave = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < T;
       t += nwave) {
    const int rl = (lane < k) ? slot_row[t * k + lane] : -1;
    const float wl = (rl >= 0 && w) ? w[rl] : 1.0f;
    const uint64_t live = __ballot(rl >= 0);
    for (int c0 = 0; c0 < nc; c0 += 64 * kCombCPL) {
      float acc[kCombCPL][8];
#pragma unroll
      for (int u = 0; u < kCombCPL; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
      uint64_t m = live;
      while (m) {
        int rb[2];
        float wb[2];
        int nb = 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          rb[b] = 0;
          wb[b] = 0.0f;
          if (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            rb[b] = __builtin_amdgcn_readlane(rl, j);
            wb[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
            nb = b + 1;
          }
        }
        u32x4 v[2][kCombCPL][VB];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int u = 0; u < kCombCPL; ++u) {
            const int c = c0 + 64 * u + lane;
            if (b < nb && c < nc) {
              const u32x4* src = (const u32x4*)(rows + (int64_t)rb[b] * ldr + 8 * c);
#pragma unroll
              for (int vb = 0; vb < VB; ++vb) v[b][u][vb] = src[vb];
            }
          }
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int u = 0; u < kCombCPL; ++u) {
            const int c = c0 + 64 * u + lane;
            if (b < nb && c < nc) {
              if constexpr (VB == 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  acc[u][2 * q] += wb[b] * bf16_lo(v[b][u][0][q]);
                  acc[u][2 * q + 1] += wb[b] * bf16_hi(v[b][u][0][q]);
                }
              } else {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                  acc[u][q] += wb[b] * __uint_as_float(v[b][u][q >> 2][q & 3]);
              }
            }
          }
      }
#pragma unroll
      for (int u = 0; u < kCombCPL; ++u) {
        const int c = c0 + 64 * u + lane;
        if (c < nc) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
          __builtin_nontemporal_store(o, (u32x4*)(out + t * ldo + 8 * c));
        }
      }
    }
  }
}

template <typename RowT>
static hipError_t run_unpermute(const RowT* rows, int64_t ldr, const int32_t* slot_row,
                                const float* w, int64_t T, int k, int n, uint16_t* out,
                                int64_t ldo, hipStream_t s) {
  if (T == 0 || n == 0) return hipSuccess;
  int64_t blocks = (T + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(unpermute_kernel<RowT>, dim3((unsigned)blocks), dim3(256), 0, s, rows, ldr,
                     slot_row, w, T, k, n, out, ldo);
  return hipGetLastError();
}

hipError_t launch_unpermute(const uint16_t* rows, int64_t ldr, const int32_t* slot_row,
                            const float* w, int64_t T, int k, int n, uint16_t* out,
                            int64_t ldo, hipStream_t s) {
  return run_unpermute(rows, ldr, slot_row, w, T, k, n, out, ldo, s);
}

hipError_t launch_unpermute_f32(const float* rows, int64_t ldr, const int32_t* slot_row,
                                int64_t T, int k, int n, uint16_t* out, int64_t ldo,
                                hipStream_t s) {
  return run_unpermute(rows, ldr, slot_row, (const float*)nullptr, T, k, n, out, ldo, s);
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
    // loads in batches of 8 (in flight together), added in slot order
    float s = 0.0f;
    int q = 0;
    for (; q + 8 <= nslots; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(q + u) * R_cap + r];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; q < nslots; ++q) s += part[(int64_t)q * R_cap + r];
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
