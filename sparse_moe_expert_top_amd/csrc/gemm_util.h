// Pipeline pieces shared by the grouped GEMMs (bf16 and W4A8): direct-to-LDS loads issued
// from inline assembly, explicit wait counts, a barrier the compiler cannot move memory
// accesses across, compile-time loops, and the per-expert tile list.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"

namespace moe {

// Direct-to-LDS loads (global_load_lds_dwordx4 / _dword): each lane's 16 (4) bytes land at
// LDS byte address M0 + 16 (4) * lane, M0 being wave-uniform. They are issued from inline
// assembly so the compiler does not track them: its waitcnt pass cannot tell ring slots apart
// and would otherwise drain every in-flight load before each LDS read. The kernels order
// these loads themselves (explicit vmcnt waits plus barriers); M0 is saved and restored.
//
// dma_saddr: L 16-byte loads from a wave-uniform 64-bit base plus per-lane 32-bit byte
// offsets; load q lands at lds0 + 1024 q.
template <int L>
__device__ __forceinline__ void dma_saddr(uint32_t lds0_in, const void* sbase,
                                          const uint32_t (&voff)[L]) {
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds0_in);
  uint32_t saved;
  if constexpr (L == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds0), "s"(sbase), "v"(voff[0])
        : "memory");
  } else if constexpr (L == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %4, %3\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %5, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds0), "s"(lds0 + 1024u), "s"(sbase), "v"(voff[0]), "v"(voff[1])
        : "memory");
  } else if constexpr (L > 4) {
    static_assert(L % 4 == 0, "loads per operand per stage");
#pragma unroll
    for (int h = 0; h < L / 4; ++h) {
      const uint32_t part[4] = {voff[4 * h], voff[4 * h + 1], voff[4 * h + 2], voff[4 * h + 3]};
      dma_saddr<4>(lds0 + 4096u * h, sbase, part);
    }
  } else {
    static_assert(L == 4, "loads per operand per stage");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %6, %5\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %7, %5\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %8, %5\n\t"
        "s_mov_b32 m0, %4\n\t"
        "global_load_lds_dwordx4 %9, %5\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds0), "s"(lds0 + 1024u), "s"(lds0 + 2048u), "s"(lds0 + 3072u), "s"(sbase),
          "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3])
        : "memory");
  }
}
// dma_saddr_b32: one 4-byte load per lane from a wave-uniform base plus a per-lane byte
// offset (4-byte aligned); the wave's 256 bytes land at lds0.
__device__ __forceinline__ void dma_saddr_b32(uint32_t lds0_in, const void* sbase, uint32_t voff) {
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds0_in);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %3, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds0), "s"(sbase), "v"(voff)
      : "memory");
}
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t a = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Wait until at most N vector-memory operations of this wave are outstanding, and for all
// of its LDS operations (gfx9 s_waitcnt: vmcnt[3:0,15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that the compiler may not move LDS or global accesses across (the
// builtin alone is not a memory operation for it); emits only s_barrier.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, fully unrolled.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

// Calls f(std::integral_constant<int, n>) for a runtime n in [0, N].
template <int N, class F>
__device__ __forceinline__ void dispatch_count(int n, F&& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N) f(std::integral_constant<int, N>{});
    else dispatch_count<N - 1>(n, f);
  }
}

// Tile list of a row-ragged grouped GEMM, built by all NT threads of the workgroup from the
// device-side group offsets: s_pref[g] = first tile of group g (ceil(rows_g / BM) m-tiles
// times n_tiles each), s_pref[G] = total, which is returned. G <= 1024.
template <int NT, int BM>
__device__ __forceinline__ int build_tile_prefix(const int32_t* offsets, int G, int n_tiles,
                                                 int* s_pref, int* s_scan) {
  constexpr int GPT = (1024 + NT - 1) / NT;         // groups per thread
  const int tid = threadIdx.x;
  int loc[GPT];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    int c = 0;
    if (g < G) {
      const int mg = offsets[g + 1] - offsets[g];
      c = ((mg + BM - 1) / BM) * n_tiles;
    }
    loc[i] = c;
    sum += c;
  }
  s_scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = (tid >= off) ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int run = s_scan[tid] - sum;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    if (g < G) s_pref[g] = run;
    run += loc[i];
  }
  const int total = s_scan[NT - 1];
  if (tid == 0) s_pref[G] = total;
  __syncthreads();
  return total;
}

// Group of a tile id: the last g with s_pref[g] <= tile.
__device__ __forceinline__ int tile_group(const int* s_pref, int G, int tile) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// GROUP_M rasterization of a tile inside its group: super-rows of gm m-tiles, each swept over
// all n-tiles with the m index fastest.
__device__ __forceinline__ void raster_tile(int local, int mtiles, int gm, int n_tiles, int& mt,
                                            int& nt) {
  const int per_super = gm * n_tiles;
  const int sr = local / per_super;
  const int rem = local - sr * per_super;
  const int rows = min(gm, mtiles - sr * gm);
  nt = rem / rows;
  mt = sr * gm + (rem - nt * rows);
}

// First tile of workgroup b in a persistent grid of nblk workgroups: consecutive tile ids go
// to one XCD (workgroup i runs on XCD i mod 8) when the grid is a multiple of 8.
__device__ __forceinline__ int xcd_first_tile(int b, int nblk) {
  return ((nblk & 7) == 0) ? ((b & 7) * (nblk >> 3) + (b >> 3)) : b;
}

// Rows [m0, me) of m-tile mt of a group of mg rows with BM-row tiles: the group's 32-row
// fragments are dealt out evenly over its m-tiles (588 rows: 7, 6 and 6 fragments, not
// 8, 8 and 3), so the m-tiles that share a weight panel do nearly equal MFMA work and stay
// in step over the k-loop; a short last tile would run ahead and lose the panel's L2 lines
// before its siblings read them.
template <int BM>
__device__ __forceinline__ void balanced_rows(int mt, int mg, int& m0, int& me) {
  const int nm = (mg + BM - 1) / BM;
  const int F = (mg + 31) / 32;
  m0 = 32 * ((mt * F) / nm);
  me = min(32 * (((mt + 1) * F) / nm), mg);
}

}  // namespace moe
