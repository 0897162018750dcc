// Grouped bf16 GEMMs of the routed-expert layer on gfx950 MFMA, with fused epilogues.
//
// "Kimi K3 ... Memory", section "MoE 反向": each expert computes a_e = SiTU(W_gate x, W_up x),
// o_e = W_down a_e, y = sum p_e o_e; the backward gets dL/dp_e = <W_down^T dL/dy, a_e> and
// dL/da_e = p_e W_down^T dL/dy, redoing the dispatch from the pre-dispatch input. The six
// contractions below are that layer; every one runs over all local experts in one launch:
//
//   name      C[m][n]                         M        N     K       A kind       B kind
//   gate_up   x[tok(r)] . w_gu[e]^T           rows     2H    d       rows+gather  rows (NT)
//   down      a[r] . w_down[e]^T              rows     d     H       rows         rows (NT)
//   dA        dy[tok(r)] . w_down[e]          rows     H     d       rows+gather  k-outer (NN)
//   dX        dh[r] . w_gu[e]                 rows     d     2H      rows         k-outer (NN)
//   dW_down   sum_r dy[tok(r)]^T pa[r]        d        H     rows    k-outer+g    k-outer (TN)
//   dW_gu     sum_r dh[r]^T x[tok(r)]         2H       d     rows    k-outer      k-outer+g
//
// Design (gfx950):
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators; 4 wavefronts per workgroup in a 2x2 grid,
//    each owning a (BM/2) x (BN/2) block of C.
//  * Operands are staged through LDS as [row][64 k] bf16 tiles (two stages, one barrier per
//    k-step). The 16-byte chunk c of row r sits at chunk position c ^ ((r ^ r>>3) & 7), so
//    the MFMA fragment reads (8 consecutive rows, same chunk) and the transposing stores
//    (rows 8 apart, same chunk) both hit distinct banks.
//  * "rows" operands are K-contiguous in HBM and load 16 bytes per lane, optionally through a
//    row index (the dispatch gather). "k-outer" operands are stored with K as the outer
//    index; each lane loads a (BM/32)-row x 8-column block and transposes it in registers
//    (byte permutes) before the LDS store, so every MFMA reads K-contiguous fragments.
//  * Ragged extents come from the device-side expert offsets: a persistent grid walks a tile
//    list built in LDS from those offsets (no host sync). Consecutive tile ids go to the
//    same XCD (workgroup i runs on XCD i mod 8), so the m-tiles sharing one expert's weight
//    panel run together and share that XCD's L2.
//  * Epilogues: gate_up writes h (bf16) and a = bf16(SiTU-GLU(bf16 h)); down writes
//    bf16(p * o) rows for the combine; dA recomputes a from the saved h, accumulates the
//    per-row <G, a> partials, and writes dh and bf16(p a); dX writes bf16 rows; the weight
//    gradients write fp32 (zeros for experts without rows).
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "situ_math.h"

namespace moe {

constexpr int kBK = 32;              // bf16 elements of K per LDS stage
constexpr int kNS = 4;               // stages in the LDS ring
constexpr int kThreads = 256;

enum BKind { B_ROWS = 0, B_KOUT = 1 };
enum Epi { EPI_GATEUP = 0, EPI_ROWS_SCALED = 1, EPI_ROWS = 2, EPI_DA = 3, EPI_F32 = 4 };

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_gather;
  const uint16_t* B;
  int64_t ldb;
  int64_t b_gstride;
  const int32_t* b_gather;
  const int32_t* offsets;
  int G;
  int M, N, K;       // fixed extents; the ragged one comes from offsets
  int H;             // split of the gate/linear halves (gate_up, dA)
  int n_tiles;       // tiles along N (gate_up: along the H gate/linear column pairs)
  int m_tiles;       // tiles along M (weight gradients)
  uint16_t* o0;
  int64_t ld0;
  uint16_t* o1;
  int64_t ld1;
  float* of;
  int64_t ldf;
  int64_t f_gstride;
  const float* row_scale;
  const uint16_t* hsrc;
  float* dp_part;
  int64_t dp_ld;
  SituCoef sc;
};

// ---------------------------------------------------------------------------- LDS stages
// LDS on gfx950 serves a 16-byte-per-lane read in 256-byte passes (64 banks of 4 bytes), so
// a read is conflict-free when the 16 lanes of a pass hit 16 distinct 16-byte slots of a
// 256-byte window.
// A K-contiguous ("rows") operand stage is [TR][kBK] bf16: 64-byte rows of four 16-byte
// chunks, chunk c of row r at position c ^ ((r >> 2) & 3). Sixteen consecutive rows at one
// logical chunk (an MFMA fragment read) then land in sixteen distinct slots.
// A k-outer operand stage is [kBK][TR] bf16 (k-rows of TR columns), chunk c of k-row k at
// position c ^ (4 (k & 3)): a transposing fragment read covers four consecutive k-rows of
// four chunks per pass, which this maps to sixteen distinct slots.
// Stages are filled by direct-to-LDS loads (global_load_lds_dwordx4): a wave's load writes
// 64 x 16 bytes contiguously, so each lane fetches the global chunk that belongs at its
// position; the swizzle above is realised by that choice.
__device__ __forceinline__ int rswz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int kswz(int k) { return (k & 3) << 2; }

// Source of k-rows past the end of a ragged K extent (must read as zeros).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[256];

// One direct-to-LDS load: this lane's 16 bytes at `src` go to LDS byte address
// lds_base + 16 * lane, lds_base being wave-uniform. Issued from inline assembly so the
// compiler does not track it: its waitcnt pass cannot tell ring slots apart and would
// otherwise drain every in-flight load before each LDS read. The kernel orders these loads
// itself (explicit vmcnt waits plus barriers); M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(const uint16_t* src, const uint16_t* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding, and for all
// of its LDS operations (gfx9 s_waitcnt: vmcnt[3:0,15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group, lane
// i = 4a + b receives element b of the 4-element reads of lanes a, 4+a, 8+a, 12+a. When
// lane s of a group points at k-row k0 + s/4, column m0 + 4 (s % 4) of a k-outer tile,
// lane i receives k-rows k0..k0+3 of column m0 + i.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 ds_read_tr(const uint16_t* lds_src) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)lds_src);
}

template <int BM, int BN, bool KRAG, int BKIND, int EPI>
__global__ __launch_bounds__(kThreads, (BM * BN > 128 * 128) ? 1 : 2) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr bool A_KO = KRAG;                       // A k-outer (weight gradients)
  constexpr bool B_KO = (BKIND == B_KOUT);
  constexpr int LA = BM * kBK * 2 / 1024 / 4;       // direct-to-LDS loads per wave per stage
  constexpr int LB = BN * kBK * 2 / 1024 / 4;
  constexpr int LPS = LA + LB;
  constexpr int NIDX = KRAG ? LPS : 0;              // gather-index loads per wave per stage
  constexpr int KS = kBK / 16;                      // MFMA k-steps per stage
  static_assert(!KRAG || BKIND == B_KOUT, "weight gradients read B k-outer");
  static_assert(EPI != EPI_GATEUP || (FN % 2 == 0), "gate/linear pairs");
  static_assert(LA >= 1 && LB >= 1 && kNS == 4, "stage geometry");

  __shared__ __attribute__((aligned(1024))) uint16_t sA[kNS][BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[kNS][BN * kBK];
  __shared__ int s_pref[1025];
  __shared__ int s_scan[kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------------------- tile list
  int total;
  if constexpr (KRAG) {
    total = p.G * p.m_tiles * p.n_tiles;
  } else {
    int loc[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = tid * 4 + i;
      int c = 0;
      if (g < p.G) {
        const int mg = p.offsets[g + 1] - p.offsets[g];
        c = ((mg + BM - 1) / BM) * p.n_tiles;
      }
      loc[i] = c;
      sum += c;
    }
    s_scan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = (tid >= off) ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int run = s_scan[tid] - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = tid * 4 + i;
      if (g < p.G) s_pref[g] = run;
      run += loc[i];
    }
    total = s_scan[kThreads - 1];
    if (tid == 0) s_pref[p.G] = total;
    __syncthreads();
  }

  // Per-lane fragment offsets inside a stage (element units).
  int offa[KS][FM][2], offb[KS][FN][2];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (!A_KO) {
          const int row = wm * WM + i * 32 + (lane & 31);
          offa[s][i][h] = row * kBK + (((2 * s + (lane >> 5)) ^ rswz(row)) << 3);
        } else {
          const int g16 = lane >> 4, i16 = lane & 15;
          const int kr = s * 16 + 8 * (g16 >> 1) + 4 * h + (i16 >> 2);
          const int col = wm * WM + i * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
          offa[s][i][h] = kr * BM + (((col >> 3) ^ kswz(kr)) << 3) + (col & 7);
        }
      }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (!B_KO) {
          const int row = wn * WN + j * 32 + (lane & 31);
          offb[s][j][h] = row * kBK + (((2 * s + (lane >> 5)) ^ rswz(row)) << 3);
        } else {
          const int g16 = lane >> 4, i16 = lane & 15;
          const int kr = s * 16 + 8 * (g16 >> 1) + 4 * h + (i16 >> 2);
          const int col = wn * WN + j * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
          offb[s][j][h] = kr * BN + (((col >> 3) ^ kswz(kr)) << 3) + (col & 7);
        }
      }
  }

  const int nblk = gridDim.x;
  const int b = blockIdx.x;
  const int first = ((nblk & 7) == 0) ? ((b & 7) * (nblk >> 3) + (b >> 3)) : b;

  for (int tile = first; tile < total; tile += nblk) {
    int g, mt, nt;
    if constexpr (KRAG) {
      const int per = p.m_tiles * p.n_tiles;
      g = tile / per;
      const int rem = tile - g * per;
      nt = rem / p.m_tiles;
      mt = rem - nt * p.m_tiles;
    } else {
      int lo = 0, hi = p.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= tile) lo = mid; else hi = mid;
      }
      g = lo;
      const int mg = p.offsets[g + 1] - p.offsets[g];
      const int mtg = (mg + BM - 1) / BM;
      const int local = tile - s_pref[g];
      nt = local / mtg;
      mt = local - nt * mtg;
    }
    const int r0 = p.offsets[g];
    const int gcount = p.offsets[g + 1] - r0;
    const int Mg = KRAG ? p.M : gcount;
    const int Kg = KRAG ? gcount : p.K;
    const int nk = (Kg + kBK - 1) / kBK;
    const int m0 = mt * BM;
    const int n0 = nt * BN;
    const int j0 = nt * (BN / 2);          // gate_up: first gate/linear column pair
    const uint16_t* Bg = p.B + (int64_t)g * p.b_gstride;

    // ------------------------------------------------------------ load addressing
    // Load q of this wave fills bytes [(wave * L + q) * 1024, +1024) of a stage; lane L
    // writes the 16 bytes at + 16 L.
    const uint16_t* a_src[LA];   // rows: per-stage base (advance kBK per stage)
    int a_kr[LA], a_col[LA];     // k-outer: k-row inside the stage and source column
    const uint16_t* b_src[LB];
    int b_kr[LB], b_col[LB];
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int byte = (wave * LA + q) * 1024 + lane * 16;
      if constexpr (!A_KO) {
        const int row = byte / (kBK * 2);
        const int c = ((byte % (kBK * 2)) >> 4) ^ rswz(row);
        const int m = min(m0 + row, Mg - 1);
        const int srow = p.a_gather ? p.a_gather[r0 + m] : (r0 + m);
        a_src[q] = p.A + (int64_t)srow * p.lda + c * 8;
      } else {
        const int kr = byte / (BM * 2);
        const int c = ((byte % (BM * 2)) >> 4) ^ kswz(kr);
        a_kr[q] = kr;
        a_col[q] = min(m0 + c * 8, p.M - 8);
      }
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int byte = (wave * LB + q) * 1024 + lane * 16;
      if constexpr (!B_KO) {
        const int row = byte / (kBK * 2);
        const int c = ((byte % (kBK * 2)) >> 4) ^ rswz(row);
        int wrow;
        if constexpr (EPI == EPI_GATEUP) {
          const int w = row / WN, qq = row % WN;
          const int jj = min(j0 + w * (WN / 2) + (qq % (WN / 2)), p.H - 1);
          wrow = (qq < WN / 2) ? jj : p.H + jj;
        } else {
          wrow = min(n0 + row, p.N - 1);
        }
        b_src[q] = Bg + (int64_t)wrow * p.ldb + c * 8;
      } else {
        const int kr = byte / (BN * 2);
        const int c = ((byte % (BN * 2)) >> 4) ^ kswz(kr);
        b_kr[q] = kr;
        b_col[q] = min(n0 + c * 8, p.N - 8);
      }
    }

    // Ragged-K operands: storage row of each load's k-row for the next stage to issue
    // (-1 past the group's end), fetched one stage ahead of its use.
    int ia[KRAG ? LA : 1], ib[KRAG ? LB : 1];
    auto fetch_rows = [&](int kt) {
      if constexpr (KRAG) {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
          const int kg = kt * kBK + a_kr[q];
          ia[q] = (kg < Kg) ? (p.a_gather ? p.a_gather[r0 + kg] : (r0 + kg)) : -1;
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
          const int kg = kt * kBK + b_kr[q];
          ib[q] = (kg < Kg) ? (p.b_gather ? p.b_gather[r0 + kg] : (r0 + kg)) : -1;
        }
      }
    };
    auto issue = [&](int kt) {
      const int slot = kt & (kNS - 1);
#pragma unroll
      for (int q = 0; q < LA; ++q) {
        const uint16_t* src;
        if constexpr (!A_KO) src = a_src[q] + kt * kBK;
        else src = (ia[q] >= 0) ? p.A + (int64_t)ia[q] * p.lda + a_col[q] : g_zero_row;
        dma16(src, &sA[slot][(wave * LA + q) * 512]);
      }
#pragma unroll
      for (int q = 0; q < LB; ++q) {
        const uint16_t* src;
        if constexpr (!B_KO) src = b_src[q] + kt * kBK;
        else if constexpr (!KRAG) src = Bg + (int64_t)(kt * kBK + b_kr[q]) * p.ldb + b_col[q];
        else src = (ib[q] >= 0) ? p.B + (int64_t)ib[q] * p.ldb + b_col[q] : g_zero_row;
        dma16(src, &sB[slot][(wave * LB + q) * 512]);
      }
      if (kt + 1 < nk) fetch_rows(kt + 1);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto compute_stage = [&](int slot) {
      bf16x8 af[KS][FM], bfr[KS][FN];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if constexpr (!A_KO) {
            af[s][i] = *(const bf16x8*)&sA[slot][offa[s][i][0]];
          } else {
            const i16x4 lo = ds_read_tr(&sA[slot][offa[s][i][0]]);
            const i16x4 hi = ds_read_tr(&sA[slot][offa[s][i][1]]);
            af[s][i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (!B_KO) {
            bfr[s][j] = *(const bf16x8*)&sB[slot][offb[s][j][0]];
          } else {
            const i16x4 lo = ds_read_tr(&sB[slot][offb[s][j][0]]);
            const i16x4 hi = ds_read_tr(&sB[slot][offb[s][j][1]]);
            bfr[s][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
    };

    // ------------------------------------------------------------ k pipeline
    // kNS-stage ring: stages kt+1 .. kt+kNS-2 stay in flight while stage kt is consumed.
    // Before stage kt is read: this wave's loads for it have landed (vmcnt) and every
    // wave's have (barrier). The same barrier orders the refill of the slot consumed in
    // the previous iteration after every wave's reads of it.
    fetch_rows(0);
#pragma unroll
    for (int st = 0; st < kNS - 1; ++st)
      if (st < nk) issue(st);
    for (int kt = 0; kt < nk; ++kt) {
      const int remaining = nk - 1 - kt;
      if (remaining >= 2) wait_vm_lgkm0<2 * (LPS + NIDX)>();
      else if (remaining == 1) wait_vm_lgkm0<LPS + NIDX>();
      else wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kt + kNS - 1 < nk) issue(kt + kNS - 1);
      compute_stage(kt & (kNS - 1));
    }
    // every wave is done with the ring before the next tile refills it
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // ------------------------------------------------------------ epilogues
    // acc[i][j][v] holds C[row][col] with row = i*32 + 8*(v/4) + 4*(lane/32) + v%4 and
    // col = j*32 + lane%32 inside the wavefront's block.
    const int col_l = lane & 31;
    const int rq = (lane >> 5) * 4;
    if constexpr (EPI == EPI_F32) {
      float* Cg = p.of + (int64_t)g * p.f_gstride;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + col_l;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rq + (v & 3);
            if (row < p.M && col < p.N) Cg[(int64_t)row * p.ldf + col] = acc[i][j][v];
          }
        }
    } else if constexpr (EPI == EPI_ROWS || EPI == EPI_ROWS_SCALED) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rq + (v & 3);
          if (row >= Mg) continue;
          const int64_t r = r0 + row;
          float sc = 1.0f;
          if constexpr (EPI == EPI_ROWS_SCALED) sc = p.row_scale[r];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + col_l;
            if (col < p.N) p.o0[r * p.ld0 + col] = f32_to_bf16(acc[i][j][v] * sc);
          }
        }
    } else if constexpr (EPI == EPI_GATEUP) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rq + (v & 3);
          if (row >= Mg) continue;
          const int64_t r = r0 + row;
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const int jj = j0 + wn * (WN / 2) + j * 32 + col_l;
            if (jj >= p.H) continue;
            const uint16_t hg = f32_to_bf16(acc[i][j][v]);
            const uint16_t hl = f32_to_bf16(acc[i][j + FN / 2][v]);
            p.o0[r * p.ld0 + jj] = hg;
            p.o0[r * p.ld0 + p.H + jj] = hl;
            p.o1[r * p.ld1 + jj] = f32_to_bf16(situ_fwd(bf16_to_f32(hg), bf16_to_f32(hl), p.sc));
          }
        }
    } else if constexpr (EPI == EPI_DA) {
      const int slot = nt * 2 + wn;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rq + (v & 3);
          const bool vr = row < Mg;
          const int64_t r = r0 + (vr ? row : 0);
          const float pr = vr ? p.row_scale[r] : 0.0f;
          float part = 0.0f;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + j * 32 + col_l;
            if (vr && n < p.N) {
              const float gv = acc[i][j][v];
              const uint16_t* hr = p.hsrc + r * (2 * (int64_t)p.H);
              float a, dgv, dlv;
              situ_bwd(bf16_to_f32(hr[n]), bf16_to_f32(hr[p.H + n]), pr * gv, p.sc, a, dgv, dlv);
              const float ab = round_bf16(a);
              part += gv * ab;
              uint16_t* dr = p.o0 + r * p.ld0;
              dr[n] = f32_to_bf16(dgv);
              dr[p.H + n] = f32_to_bf16(dlv);
              p.o1[r * p.ld1 + n] = f32_to_bf16(pr * ab);
            }
          }
          // sum over the 32 lanes that share this row
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
          if (vr && col_l == 0) p.dp_part[(int64_t)slot * p.dp_ld + r] = part;
        }
    }
  }
}

// ---------------------------------------------------------------------------- launchers
template <int BM, int BN, bool KRAG, int BKIND, int EPI>
static hipError_t run_gemm(const GemmArgs& args, int64_t max_tiles, hipStream_t s) {
  auto kern = grouped_gemm_kernel<BM, BN, KRAG, BKIND, EPI>;
  static int occ = -1;                   // workgroups per CU for this instantiation
  if (occ < 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, kThreads, 0) != hipSuccess || o < 1)
      o = 1;
    occ = o;
  }
  int64_t grid = (int64_t)device_cu_count() * occ;
  if (max_tiles < grid) grid = max_tiles;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, args);
  return hipGetLastError();
}

// Tile shapes per contraction (BM x BN); each must be 128 or 256.
#ifndef MOE_TILE_GU
#define MOE_TILE_GU 128, 128
#endif
#ifndef MOE_TILE_DN
#define MOE_TILE_DN 128, 128
#endif
#ifndef MOE_TILE_DA
#define MOE_TILE_DA 128, 128
#endif
#ifndef MOE_TILE_DX
#define MOE_TILE_DX 128, 128
#endif
#ifndef MOE_TILE_WD
#define MOE_TILE_WD 128, 128
#endif
#ifndef MOE_TILE_WG
#define MOE_TILE_WG 128, 128
#endif
struct TileShape { int bm, bn; };
constexpr TileShape kGU{MOE_TILE_GU}, kDN{MOE_TILE_DN}, kDA{MOE_TILE_DA}, kDX{MOE_TILE_DX},
    kWD{MOE_TILE_WD}, kWG{MOE_TILE_WG};

static GemmArgs blank_args() {
  GemmArgs a;
  __builtin_memset(&a, 0, sizeof(a));
  return a;
}

static int64_t mragged_tile_bound(int64_t R_cap, int E_loc, int bm, int n_tiles) {
  return ((R_cap + bm - 1) / bm + E_loc) * (int64_t)n_tiles;
}

hipError_t launch_gemm_gate_up(const uint16_t* x, const int32_t* row_token,
                               const int32_t* offsets, int E_loc, int64_t R_cap, int d, int H,
                               const uint16_t* w_gu, SituCoef c, uint16_t* h, uint16_t* a,
                               hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = x; p.lda = d; p.a_gather = row_token;
  p.B = w_gu; p.ldb = d; p.b_gstride = (int64_t)2 * H * d;
  p.offsets = offsets; p.G = E_loc;
  p.N = 2 * H; p.K = d; p.H = H;
  p.n_tiles = (H + kGU.bn / 2 - 1) / (kGU.bn / 2);
  p.o0 = h; p.ld0 = 2 * H; p.o1 = a; p.ld1 = H;
  p.sc = c;
  return run_gemm<kGU.bm, kGU.bn, false, B_ROWS, EPI_GATEUP>(
      p, mragged_tile_bound(R_cap, E_loc, kGU.bm, p.n_tiles), s);
}

hipError_t launch_gemm_down(const uint16_t* a, const int32_t* offsets, const float* row_gate,
                            int E_loc, int64_t R_cap, int H, int d, const uint16_t* w_down,
                            uint16_t* rows_out, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = a; p.lda = H;
  p.B = w_down; p.ldb = H; p.b_gstride = (int64_t)d * H;
  p.offsets = offsets; p.G = E_loc;
  p.N = d; p.K = H;
  p.n_tiles = (d + kDN.bn - 1) / kDN.bn;
  p.o0 = rows_out; p.ld0 = d; p.row_scale = row_gate;
  return run_gemm<kDN.bm, kDN.bn, false, B_ROWS, EPI_ROWS_SCALED>(
      p, mragged_tile_bound(R_cap, E_loc, kDN.bm, p.n_tiles), s);
}

int gemm_da_slots(int H) { return ((H + kDA.bn - 1) / kDA.bn) * 2; }

hipError_t launch_gemm_da(const uint16_t* dy, const int32_t* row_token, const int32_t* offsets,
                          int E_loc, int64_t R_cap, int d, int H, const uint16_t* w_down,
                          const uint16_t* h, const float* row_gate, SituCoef c, uint16_t* dh,
                          uint16_t* pa, float* dp_part, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dy; p.lda = d; p.a_gather = row_token;
  p.B = w_down; p.ldb = H; p.b_gstride = (int64_t)d * H;      // B(n=j, k) = w_down[e][k][j]
  p.offsets = offsets; p.G = E_loc;
  p.N = H; p.K = d; p.H = H;
  p.n_tiles = (H + kDA.bn - 1) / kDA.bn;
  p.o0 = dh; p.ld0 = 2 * H; p.o1 = pa; p.ld1 = H;
  p.row_scale = row_gate; p.hsrc = h; p.dp_part = dp_part; p.dp_ld = R_cap;
  p.sc = c;
  return run_gemm<kDA.bm, kDA.bn, false, B_KOUT, EPI_DA>(
      p, mragged_tile_bound(R_cap, E_loc, kDA.bm, p.n_tiles), s);
}

hipError_t launch_gemm_dx(const uint16_t* dh, const int32_t* offsets, int E_loc,
                          int64_t R_cap, int d, int H, const uint16_t* w_gu,
                          uint16_t* rows_out, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dh; p.lda = 2 * H;
  p.B = w_gu; p.ldb = d; p.b_gstride = (int64_t)2 * H * d;    // B(n, k) = w_gu[e][k][n]
  p.offsets = offsets; p.G = E_loc;
  p.N = d; p.K = 2 * H;
  p.n_tiles = (d + kDX.bn - 1) / kDX.bn;
  p.o0 = rows_out; p.ld0 = d;
  return run_gemm<kDX.bm, kDX.bn, false, B_KOUT, EPI_ROWS>(
      p, mragged_tile_bound(R_cap, E_loc, kDX.bm, p.n_tiles), s);
}

hipError_t launch_gemm_dw_down(const uint16_t* dy, const int32_t* row_token,
                               const uint16_t* pa, const int32_t* offsets, int E_loc, int d,
                               int H, float* dw_down, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dy; p.lda = d; p.a_gather = row_token;                // A(m, k=r) = dy[tok(r)][m]
  p.B = pa; p.ldb = H;                                        // B(n, k=r) = pa[r][n]
  p.offsets = offsets; p.G = E_loc;
  p.M = d; p.N = H;
  p.m_tiles = (d + kWD.bm - 1) / kWD.bm;
  p.n_tiles = (H + kWD.bn - 1) / kWD.bn;
  p.of = dw_down; p.ldf = H; p.f_gstride = (int64_t)d * H;
  return run_gemm<kWD.bm, kWD.bn, true, B_KOUT, EPI_F32>(
      p, (int64_t)E_loc * p.m_tiles * p.n_tiles, s);
}

hipError_t launch_gemm_dw_gu(const uint16_t* dh, const uint16_t* x, const int32_t* row_token,
                             const int32_t* offsets, int E_loc, int d, int H, float* dw_gu,
                             hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dh; p.lda = 2 * H;                                    // A(m, k=r) = dh[r][m]
  p.B = x; p.ldb = d; p.b_gather = row_token;                 // B(n, k=r) = x[tok(r)][n]
  p.offsets = offsets; p.G = E_loc;
  p.M = 2 * H; p.N = d;
  p.m_tiles = (2 * H + kWG.bm - 1) / kWG.bm;
  p.n_tiles = (d + kWG.bn - 1) / kWG.bn;
  p.of = dw_gu; p.ldf = d; p.f_gstride = (int64_t)2 * H * d;
  return run_gemm<kWG.bm, kWG.bn, true, B_KOUT, EPI_F32>(
      p, (int64_t)E_loc * p.m_tiles * p.n_tiles, s);
}

}  // namespace moe
