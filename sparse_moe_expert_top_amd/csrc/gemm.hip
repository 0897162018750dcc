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
//   dW_gu     sum_r dh[r]^T x[tok(r)]         2H       d     rows    k-outer      k-outer+g (TN)
//
// Design (gfx950):
//  * v_mfma_f32_32x32x16_bf16 with fp32 accumulators. A workgroup of WGM x WGN wavefronts
//    owns a BM x BN tile; each wavefront a (BM/WGM) x (BN/WGN) block of it. The large
//    configuration (256 x 256, 8 wavefronts, two per SIMD) loads 8 bytes per kFLOP.
//  * K advances in stages of BK through an NS-slot LDS ring. Each stage is filled by
//    direct-to-LDS loads (global_load_lds_dwordx4, 1 KiB per wavefront instruction), issued
//    NS-1 stages ahead of its use; one barrier per stage, placed before the stage's last
//    k-step, orders fills after the reads of the slot they overwrite, and the last k-step's
//    MFMAs cover the next stage's first fragment reads. dA and dX use a ping-pong form
//    instead (32-deep stages, 4 slots, the two wavefronts of each SIMD one phase apart).
//  * A wavefront whose 32-row fragments lie wholly past the end of a group's rows skips
//    them (the k-loop is compiled once per count of live fragments), so the last, partly
//    filled tile of each expert costs only the MFMAs of its live rows.
//  * "rows" operands (K contiguous in HBM) stay [row][BK] in LDS, with an XOR swizzle of the
//    16-byte chunks; each lane loads the chunk that belongs at its LDS position, optionally
//    through a row index (the dispatch gather). MFMA fragments are ds_read_b128.
//  * "k-outer" operands (K the outer index in HBM) stay [k][row] in LDS and are read with
//    the transposing ds_read_b64_tr_b16, so no operand is ever transposed in registers.
//    Ragged-K tails read a zero row.
//  * Ragged extents come from the device-side expert offsets: a persistent grid walks a tile
//    list built in LDS from those offsets (no host sync). Inside an expert, tiles go in
//    GROUP_M super-rows (all n-tiles of group_m m-tiles, m fastest), and consecutive tile
//    ids go to one XCD (workgroup i runs on XCD i mod 8), so tiles running together on an
//    XCD share both operand panels in its L2.
//  * Epilogues: gate_up writes h (bf16) and a = bf16(SiTU-GLU(bf16 h)); down writes fp32
//    p * o rows for the combine; dA recomputes a from the saved h, accumulates the per-row
//    <G, a> partials, and writes dh and bf16(p a); dX writes fp32 rows; the weight gradients
//    write fp32 rows (zeros for experts without rows) with streaming stores. down and dX
//    cover a window [c0, c0 + nc) of their output columns per launch, so a caller with a
//    smaller workspace combines the columns in several passes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "gemm_util.h"
#include "launch.h"
#include "mxfp8.h"
#include "situ_math.h"

namespace moe {

enum BKind { B_ROWS = 0, B_KOUT = 1 };
enum Epi {
  EPI_GATEUP = 0, EPI_ROWS_SCALED = 1, EPI_ROWS = 2, EPI_DA = 3, EPI_F32 = 4,
  EPI_GATEUP_MX = 5,   // gate_up storing h as MXFP8 codes + scales
  EPI_DA_MX = 6        // dA reading h from MXFP8 codes + scales
};

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
  int group_m;       // m-tiles per rasterization super-row
  uint16_t* o0;
  int64_t ld0;
  uint16_t* o1;
  int64_t ld1;
  float* of;
  int64_t ldf;
  int64_t f_gstride;
  const float* row_scale;
  const uint16_t* hsrc;
  uint8_t* q0;         // MXFP8 h codes [R, 2H] and scale bytes [R, 2H/32] (gate_up, stored)
  uint8_t* s0;
  const uint8_t* qsrc; // MXFP8 h codes and scales (dA, read)
  const uint8_t* ssrc;
  float* dp_part;
  int64_t dp_ld;
  SituCoef sc;
};

// Tile configuration: BM x BN tile, WGM x WGN wavefronts, BK-deep stages, NS-slot ring,
// WPE = wavefronts per SIMD the kernel is compiled for, PP = ping-pong k-loop (below).
template <int BM_, int BN_, int WGM_, int WGN_, int BK_, int NS_, int WPE_, bool PP_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_, NS = NS_;
  static constexpr int WPE = WPE_;
  static constexpr bool PP = PP_;
  static constexpr int NT = 64 * WGM * WGN;
};
using CfgPP = TileCfg<256, 256, 2, 4, 32, 4, 2, true>;  // 8 waves, 4 x 32 KiB ring, ping-pong
using CfgBig = TileCfg<256, 256, 2, 4, 64, 2, 2>;        // 8 waves, 2 x 64 KiB ring

// ---------------------------------------------------------------------------- LDS stages
// LDS on gfx950 serves a 16-byte-per-lane read in 256-byte passes (64 banks of 4 bytes), so
// a read is conflict-free when the 16 lanes of a pass hit 16 distinct 16-byte slots of a
// 256-byte window.
// A "rows" stage is [TR][BK] bf16. With BK = 64 a row is 128 bytes and chunk c of row r sits
// at position c ^ ((r >> 1) & 7); with BK = 32 a row is 64 bytes and chunk c sits at
// c ^ ((r >> 2) & 3). Sixteen consecutive rows at one logical chunk (a fragment read) then
// land in sixteen distinct slots.
// A "k-outer" stage is [BK][TR] bf16 (k-rows of TR >= 128 columns), chunk c of k-row k at
// position c ^ (4 (k & 3)): a transposing fragment read covers four consecutive k-rows of
// four chunks per pass, which this maps to sixteen distinct slots.
// Direct-to-LDS loads write a wavefront's 64 x 16 bytes contiguously, so the swizzle is
// realised by which global chunk each lane fetches.
template <int BK>
__device__ __forceinline__ int rswz(int row) {
  if constexpr (BK == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
__device__ __forceinline__ int kswz(int k) { return (k & 3) << 2; }

// Source of k-rows past the end of a ragged K extent (must read as zeros).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[256];

// dma_vaddr: one direct-to-LDS load (global_load_lds_dwordx4, issued and ordered like
// dma_saddr) from a per-lane 64-bit address.
__device__ __forceinline__ void dma_vaddr(const uint16_t* src, uint32_t lds_in) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
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

// Output stores of the epilogues; NT marks them streaming so they do not displace the
// operand panels that neighbouring tiles re-read from L2.
#ifndef MOE_NT_F32
#define MOE_NT_F32 1
#endif
#ifndef MOE_NT_ROWS
#define MOE_NT_ROWS 1
#endif
__device__ __forceinline__ void st_f32(float* p, float v) {
#if MOE_NT_F32
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}
#ifndef MOE_NT_F32ROWS
#define MOE_NT_F32ROWS 1
#endif
__device__ __forceinline__ void st_f32x4(float* p, f32x4 v) {
#if MOE_NT_F32ROWS
  __builtin_nontemporal_store(v, (f32x4*)p);
#else
  *(f32x4*)p = v;
#endif
}
__device__ __forceinline__ void st_row16(uint16_t* p, u32x4 v) {
#if MOE_NT_ROWS
  __builtin_nontemporal_store(v, (u32x4*)p);
#else
  *(u32x4*)p = v;
#endif
}

// TAG only tells apart contractions that would otherwise share one instantiation (dW_down and
// dW_gu), so profiles name each kernel.
template <class C, bool KRAG, int BKIND, int EPI, int TAG = 0>
__global__ __launch_bounds__(C::NT, C::WPE) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NS = C::NS, NT = C::NT, NW = NT / 64;
  constexpr int WM = BM / C::WGM, WN = BN / C::WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr bool A_KO = KRAG;                       // A k-outer (weight gradients)
  constexpr bool B_KO = (BKIND == B_KOUT);
  constexpr int LA = BM * BK * 2 / 1024 / NW;       // direct-to-LDS loads per wave per stage
  constexpr int LB = BN * BK * 2 / 1024 / NW;
  constexpr int LPS = LA + LB;
  constexpr int KS = BK / 16;                       // MFMA k-steps per stage
  constexpr int GPT = (1024 + NT - 1) / NT;         // expert offsets per thread in the scan
  static_assert(LA * 1024 * NW == BM * BK * 2 && LB * 1024 * NW == BN * BK * 2, "loads");
  static_assert(LA >= 1 && LB >= 1 && (NS == 2 || NS == 4), "stage geometry");
  static_assert(!KRAG || BKIND == B_KOUT, "weight gradients read B k-outer");
  constexpr bool IS_GU = (EPI == EPI_GATEUP || EPI == EPI_GATEUP_MX);
  constexpr bool IS_DA = (EPI == EPI_DA || EPI == EPI_DA_MX);
  constexpr bool HMX = (EPI == EPI_GATEUP_MX || EPI == EPI_DA_MX);
  static_assert(!IS_GU || (FN % 2 == 0), "gate/linear pairs");
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(!C::PP || (NT == 512 && NS == 4 && BK == 32), "ping-pong geometry");

  // One LDS ring for both operands; after the k-loop it doubles as the epilogue's staging.
  __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * (BM + BN) * BK];
  uint16_t (*sA)[BM * BK] = reinterpret_cast<uint16_t (*)[BM * BK]>(ring);
  uint16_t (*sB)[BN * BK] = reinterpret_cast<uint16_t (*)[BN * BK]>(ring + NS * BM * BK);
  __shared__ int s_pref[1025];
  __shared__ int s_scan[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring);

  // ---------------------------------------------------------------- tile list
  int total;
  if constexpr (KRAG) total = p.G * p.m_tiles * p.n_tiles;
  else total = build_tile_prefix<NT, BM>(p.offsets, p.G, p.n_tiles, s_pref, s_scan);

  // Per-lane fragment offsets inside a stage (element units): offset = base[i] + step[s][h].
  int abase[FM], bbase[FN], astep[KS][2], bstep[KS][2];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (!A_KO) {
        abase[i] = (wm * WM + i * 32 + (lane & 31)) * BK;
      } else {
        const int chunk = (wm * WM + i * 32 + (g16 & 1) * 16) / 8 + ((i16 & 3) >> 1);
        abase[i] = (8 * (g16 >> 1) + (i16 >> 2)) * BM + ((chunk ^ kswz(i16 >> 2)) << 3) +
                   4 * (i16 & 1);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (!B_KO) {
        bbase[j] = (wn * WN + j * 32 + (lane & 31)) * BK;
      } else {
        const int chunk = (wn * WN + j * 32 + (g16 & 1) * 16) / 8 + ((i16 & 3) >> 1);
        bbase[j] = (8 * (g16 >> 1) + (i16 >> 2)) * BN + ((chunk ^ kswz(i16 >> 2)) << 3) +
                   4 * (i16 & 1);
      }
    }
    const int rsw = rswz<BK>(lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        astep[s][h] = A_KO ? (s * 16 + 4 * h) * BM : (((2 * s + (lane >> 5)) ^ rsw) << 3);
        bstep[s][h] = B_KO ? (s * 16 + 4 * h) * BN : (((2 * s + (lane >> 5)) ^ rsw) << 3);
      }
  }

  const int nblk = gridDim.x;
  const int b = blockIdx.x;
#ifndef MOE_XCD_MAP
#define MOE_XCD_MAP 1
#endif
  const int first = MOE_XCD_MAP ? xcd_first_tile(b, nblk) : b;

  for (int tile = first; tile < total; tile += nblk) {
    int g, mt, nt;
    if constexpr (KRAG) {
      const int per = p.m_tiles * p.n_tiles;
      g = tile / per;
      raster_tile(tile - g * per, p.m_tiles, p.group_m, p.n_tiles, mt, nt);
    } else {
      g = tile_group(s_pref, p.G, tile);
      const int mg = p.offsets[g + 1] - p.offsets[g];
      raster_tile(tile - s_pref[g], (mg + BM - 1) / BM, p.group_m, p.n_tiles, mt, nt);
    }
    g = __builtin_amdgcn_readfirstlane(g);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int r0 = p.offsets[g];
    const int gcount = p.offsets[g + 1] - r0;
    const int Mg = KRAG ? p.M : gcount;
    const int Kg = KRAG ? gcount : p.K;
    const int nk = (Kg + BK - 1) / BK;
    int m0 = mt * BM;
    int Me = Mg;                           // end (exclusive) of this tile's rows
    if constexpr (!KRAG) balanced_rows<BM>(mt, Mg, m0, Me);
    const int n0 = nt * BN;
    const int j0 = nt * (BN / 2);          // gate_up: first gate/linear column pair
    const uint16_t* Bg = p.B + (int64_t)g * p.b_gstride;

    // ------------------------------------------------------------ load addressing
    // Load q of this wave fills bytes [(wave * L + q) * 1024, +1024) of a stage; lane L
    // writes the 16 bytes at + 16 L.
    // Rows and fixed-K k-outer operands: wave-uniform base (advanced per stage) plus a
    // per-lane 32-bit byte offset. Ragged-K k-outer operands: k-row and column per load.
    uint32_t a_off[LA], b_off[LB];
    // k-row and column of load q of a k-outer operand with TR columns per k-row (recomputed
    // where needed: only the partial last stage of a ragged-K tile uses them per lane)
    auto kout_kr = [&](int q, int L, int TR) __attribute__((always_inline)) {
      return ((wave * L + q) * 1024 + lane * 16) / (TR * 2);
    };
    auto kout_col = [&](int q, int L, int TR, int t0, int ext) __attribute__((always_inline)) {
      const int byte = (wave * L + q) * 1024 + lane * 16;
      const int kr = byte / (TR * 2);
      const int c = ((byte % (TR * 2)) >> 4) ^ kswz(kr);
      return min(t0 + c * 8, ext - 8);
    };
    // rows of A: gathered rows are addressed from A itself, contiguous rows from row r0
    const uint16_t* a_base = p.a_gather ? p.A : p.A + (int64_t)r0 * p.lda;
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int byte = (wave * LA + q) * 1024 + lane * 16;
      if constexpr (!A_KO) {
        const int row = byte / (BK * 2);
        const int c = ((byte % (BK * 2)) >> 4) ^ rswz<BK>(row);
        const int m = min(m0 + row, Me - 1);
        const int srow = p.a_gather ? p.a_gather[r0 + m] : m;
        a_off[q] = (uint32_t)(((int64_t)srow * p.lda + c * 8) * 2);
      } else {
        const int kr = byte / (BM * 2);
        const int c = ((byte % (BM * 2)) >> 4) ^ kswz(kr);
        const int a_col = min(m0 + c * 8, p.M - 8);
        // full stages: gathered rows add idx * lda at issue; contiguous rows are fixed here
        a_off[q] = (uint32_t)(((p.a_gather ? 0 : (int64_t)kr * p.lda) + a_col) * 2);
      }
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int byte = (wave * LB + q) * 1024 + lane * 16;
      if constexpr (!B_KO) {
        const int row = byte / (BK * 2);
        const int c = ((byte % (BK * 2)) >> 4) ^ rswz<BK>(row);
        int wrow;
        if constexpr (IS_GU) {
          const int w = row / WN, qq = row % WN;
          const int jj = min(j0 + w * (WN / 2) + (qq % (WN / 2)), p.H - 1);
          wrow = (qq < WN / 2) ? jj : p.H + jj;
        } else {
          wrow = min(n0 + row, p.N - 1);
        }
        b_off[q] = (uint32_t)(((int64_t)wrow * p.ldb + c * 8) * 2);
      } else {
        const int kr = byte / (BN * 2);
        const int c = ((byte % (BN * 2)) >> 4) ^ kswz(kr);
        const int b_col = min(n0 + c * 8, p.N - 8);
        b_off[q] = (uint32_t)((((KRAG && p.b_gather) ? 0 : (int64_t)kr * p.ldb) + b_col) * 2);
      }
    }

    // Ragged-K operands. In a full stage this wave's loads cover KPW consecutive k-rows;
    // their storage rows (for a gathered operand) come from one scalar load, issued one
    // stage ahead. Scalar loads are counted by lgkmcnt, so using them never waits for the
    // direct-to-LDS loads in flight (per-lane index loads would: vmcnt retires in order).
    // The partial last stage looks its rows up per lane when it is issued.
    constexpr int KPW = BK / NW;
    static_assert(!KRAG || (BM == 256 && BN == 256 && KPW == 2 * LA && KPW == 2 * LB),
                  "a full-stage load covers two k-rows, one per half-wave");
    typedef int kidx_t __attribute__((ext_vector_type(KPW)));
    typedef __attribute__((address_space(4))) const kidx_t cidx_t;
    kidx_t ga{}, gb{};
    auto fetch_a = [&](int kt) __attribute__((always_inline)) {
      if constexpr (KRAG) {
        if ((kt + 1) * BK <= Kg && p.a_gather)
          ga = *(cidx_t*)(p.a_gather + r0 + kt * BK + wave_u * KPW);
      }
    };
    auto fetch_b = [&](int kt) __attribute__((always_inline)) {
      if constexpr (KRAG) {
        if ((kt + 1) * BK <= Kg && p.b_gather)
          gb = *(cidx_t*)(p.b_gather + r0 + kt * BK + wave_u * KPW);
      }
    };
    // Row index of this lane's k-row in a full stage: lanes 0..31 take the first of the load's
    // two k-rows, lanes 32..63 the second. Both candidates pass through empty asm as scalars,
    // so the compiler selects between two registers instead of indexing the vector with a
    // per-lane index (which it expands into a compare-and-select chain over all KPW entries).
    auto pick_row = [&](const kidx_t& gv, auto qc) __attribute__((always_inline)) -> uint32_t {
      constexpr int Q = decltype(qc)::value;
      uint32_t lo = (uint32_t)gv[2 * Q], hi = (uint32_t)gv[2 * Q + 1];
      asm volatile("" : "+s"(lo), "+s"(hi));
      return (lane < 32) ? lo : hi;
    };
    auto tail_row = [&](const int32_t* gather, int kr) __attribute__((always_inline)) {
      const int kg = kr;
      return (kg < Kg) ? (gather ? gather[r0 + kg] : (r0 + kg)) : -1;
    };
    // A operand of stage kt: direct-to-LDS loads.
    auto issue_a = [&](int kt) __attribute__((always_inline)) {
      const int slot = kt & (NS - 1);
      const uint32_t lds_a = ring_lds + slot * (BM * BK * 2) + wave_u * (LA * 1024);
      if constexpr (!A_KO) {
        dma_saddr<LA>(lds_a, uniform_ptr(a_base + kt * BK), a_off);
      } else if ((kt + 1) * BK <= Kg) {
        // full ragged-K stage: every k-row exists
        uint32_t voff[LA];
        static_for<LA>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          voff[q] = p.a_gather ? pick_row(ga, qc) * (uint32_t)(p.lda * 2) + a_off[q] : a_off[q];
        });
        const uint16_t* base = p.a_gather ? p.A : p.A + (int64_t)(r0 + kt * BK) * p.lda;
        dma_saddr<LA>(lds_a, uniform_ptr(base), voff);
      } else {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
          const int ra = tail_row(p.a_gather, kt * BK + kout_kr(q, LA, BM));
          dma_vaddr((ra >= 0) ? p.A + (int64_t)ra * p.lda + kout_col(q, LA, BM, m0, p.M) : g_zero_row,
                    lds_a + q * 1024);
        }
      }
    };
    // B operand of stage kt: wave-uniform base and per-lane byte offsets (full stages), or
    // the per-lane source row (partial ragged-K stage; nullptr reads as zeros).
    auto b_base = [&](int kt) __attribute__((always_inline)) -> const uint16_t* {
      if constexpr (!B_KO) return Bg + kt * BK;
      else if constexpr (!KRAG) return Bg + (int64_t)kt * BK * p.ldb;
      else return p.b_gather ? p.B : p.B + (int64_t)(r0 + kt * BK) * p.ldb;
    };
    auto b_voff = [&](auto qc) __attribute__((always_inline)) -> uint32_t {
      constexpr int q = decltype(qc)::value;
      if constexpr (KRAG)
        return p.b_gather ? pick_row(gb, qc) * (uint32_t)(p.ldb * 2) + b_off[q] : b_off[q];
      else return b_off[q];
    };
    auto b_full = [&](int kt) __attribute__((always_inline)) {
      return !KRAG || (kt + 1) * BK <= Kg;
    };
    // B operand, direct-to-LDS form.
    auto issue_b = [&](int kt) __attribute__((always_inline)) {
      const int slot = kt & (NS - 1);
      const uint32_t lds_b = ring_lds + NS * (BM * BK * 2) + slot * (BN * BK * 2) + wave_u * (LB * 1024);
      if (b_full(kt)) {
        uint32_t voff[LB];
        static_for<LB>([&](auto qc) __attribute__((always_inline)) {
          voff[decltype(qc)::value] = b_voff(qc);
        });
        dma_saddr<LB>(lds_b, uniform_ptr(b_base(kt)), voff);
      } else {
#pragma unroll
        for (int q = 0; q < LB; ++q) {
          const int rb = tail_row(p.b_gather, kt * BK + kout_kr(q, LB, BN));
          dma_vaddr((rb >= 0) ? p.B + (int64_t)rb * p.ldb + kout_col(q, LB, BN, n0, p.N) : g_zero_row,
                    lds_b + q * 1024);
        }
      }
    };
    auto issue = [&](int kt) __attribute__((always_inline)) {
      issue_a(kt);
      issue_b(kt);
    };
    // Row indices of ragged-K stage kt (scalar loads, counted by lgkmcnt). Scalar loads may
    // return out of order with LDS reads, so while one is pending every wait for fragments
    // has to be lgkmcnt(0): the k-loop fetches stage kt's indices just before the wait that
    // precedes its issue, where they land while the wave waits for the stage in flight
    // (fetched right after an issue, they held up the next fragment wait by their latency).
    auto fetch = [&](int kt) __attribute__((always_inline)) {
      if (kt < nk) {
        fetch_a(kt);
        fetch_b(kt);
      }
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // NF = fragments (32-row blocks) of this wave that hold rows of the group; the rest
    // are neither read nor multiplied.
    auto load_frags = [&](auto nfc, int slot, int s, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN]) __attribute__((always_inline)) {
      constexpr int NF = decltype(nfc)::value;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i >= NF) {
        } else if constexpr (!A_KO) {
          af[i] = *(const bf16x8*)&sA[slot][abase[i] + astep[s][0]];
        } else {
          const i16x4 lo = ds_read_tr(&sA[slot][abase[i] + astep[s][0]]);
          const i16x4 hi = ds_read_tr(&sA[slot][abase[i] + astep[s][1]]);
          af[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (!B_KO) {
          bfr[j] = *(const bf16x8*)&sB[slot][bbase[j] + bstep[s][0]];
        } else {
          const i16x4 lo = ds_read_tr(&sB[slot][bbase[j] + bstep[s][0]]);
          const i16x4 hi = ds_read_tr(&sB[slot][bbase[j] + bstep[s][1]]);
          bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto mfma_step = [&](auto nfc, const bf16x8 (&af)[FM], const bf16x8 (&bfr)[FN]) __attribute__((always_inline)) {
      constexpr int NF = decltype(nfc)::value;
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Waits until this wave's loads of stage `next` have landed, `later` stages being issued
    // after it, and until its own LDS reads are done.
    auto wait_stage = [&](int later) __attribute__((always_inline)) {
      if (later >= 2) wait_vm_lgkm0<2 * LPS>();
      else if (later == 1) wait_vm_lgkm0<LPS>();
      else wait_vm_lgkm0<0>();
    };

    // ------------------------------------------------------------ k pipeline
    // Stages kt+1 .. kt+NS-1 are in flight while stage kt is consumed. Fragments of k-step
    // s+1 are read from LDS while the MFMAs of step s run. The barrier of stage kt sits
    // before its last k-step: by then every wave has read all of stage kt into registers
    // (so slot kt can be refilled with stage kt+NS) and has waited for its own loads of
    // stage kt+1 (so after the barrier all of stage kt+1 is in LDS). The MFMAs of the last
    // k-step then cover the refill's issue and the latency of stage kt+1's first fragment
    // reads, instead of leaving the matrix core idle across the barrier.
    //
    // Ping-pong form (C::PP: 32-deep stages, 4-slot ring, 8 wavefronts). Wavefronts w and
    // w + 4 share a SIMD. The groups {0..3} and {4..7} run one phase apart, so on every SIMD
    // one wavefront issues MFMAs while the other issues loads and LDS reads. A stage j is a
    // memory phase (issue stage j+3's loads, read both k-steps' fragments of stage j) and a
    // math phase (its MFMAs), each ended by a barrier; group 1 starts one barrier late and
    // group 0 ends one barrier late, so both execute the same barriers. The barriers order:
    //  * the refill with stage j+3 after all reads of stage j-1, whose slot it reuses: group
    //    0 read it before its own MFMAs of stage j-1; group 1 read it in the phase just
    //    before and waits for those reads before that phase's barrier;
    //  * the reads of stage j+1 after all of its loads: each wavefront waits for its own
    //    loads of stage j+1 before the barrier that ends group 1's memory phase of stage j.
    static_assert(KS % 2 == 0, "fragment double buffer alternates within a stage");
    static_assert(!(C::PP && KRAG), "the ping-pong k-loop serves fixed-K contractions");
    const int pgrp = C::PP ? (wave_u >> 2) : 0;
    auto kloop_pp = [&](auto nfc) __attribute__((always_inline)) {
      bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
      for (int st = 0; st < 3; ++st)
        if (st < nk) issue(st);
      wait_stage(min(2, nk - 1));
      block_sync();
      if (pgrp) block_sync();
      for (int j = 0; j < nk; ++j) {
        const int slot = j & 3;
        if (j + 3 < nk) issue(j + 3);
        load_frags(nfc, slot, 0, fa[0], fb[0]);
        load_frags(nfc, slot, 1, fa[1], fb[1]);
        if (pgrp) wait_stage(min(2, nk - 2 - j));
        block_sync();
        mfma_step(nfc, fa[0], fb[0]);
        mfma_step(nfc, fa[1], fb[1]);
        if (!pgrp) wait_stage(min(2, nk - 2 - j));
        block_sync();
      }
      if (!pgrp) block_sync();
      // every wave is done with the ring before the epilogue stages through it
      wait_vm_lgkm0<0>();
      block_sync();
    };
    auto kloop_std = [&](auto nfc) __attribute__((always_inline)) {
      bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
      for (int st = 0; st < NS - 1; ++st) {
        fetch(st);
        if (st < nk) issue(st);
      }
      fetch(NS - 1);
      wait_stage(min(NS - 2, nk - 1));
      block_sync();
      if (NS - 1 < nk) issue(NS - 1);
      load_frags(nfc, 0, 0, fa[0], fb[0]);
      // k-steps 0 .. KS-2 of the stage in `slot`; the last one's fragments end in fa[1]
      auto first_steps = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s + 1 < KS; ++s) {
          load_frags(nfc, slot, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
          mfma_step(nfc, fa[s & 1], fb[s & 1]);
        }
      };
      // The last stage is peeled off, so the last k-step's MFMAs of every other stage follow
      // the next stage's first fragment reads on one path only: they use registers read
      // before the barrier and wait for nothing (a join with the last stage's path made the
      // compiler wait for those reads there).
      for (int kt = 0; kt + 1 < nk; ++kt) {
        first_steps(kt & (NS - 1));
        fetch(kt + NS);
        wait_stage(min(NS - 2, nk - 2 - kt));
        block_sync();
        if (kt + NS < nk) issue(kt + NS);
        load_frags(nfc, (kt + 1) & (NS - 1), 0, fa[0], fb[0]);
        mfma_step(nfc, fa[1], fb[1]);
      }
      if (nk > 0) {
        first_steps((nk - 1) & (NS - 1));
        mfma_step(nfc, fa[1], fb[1]);
      }
      // every wave is done with the ring before the epilogue stages through it
      wait_vm_lgkm0<0>();
      block_sync();
    };
    auto kloop = [&](auto nfc) __attribute__((always_inline)) {
      if constexpr (C::PP) kloop_pp(nfc);
      else kloop_std(nfc);
    };
    // Row GEMMs: a tile at the end of a group may hold only a few rows; this wave's
    // fragments wholly past the group's last row are skipped (a wave-uniform count).
    int nfv = FM;
    if constexpr (!KRAG) {
      const int wrow0 = m0 + (wave_u / C::WGN) * WM;
      nfv = max(0, min(FM, (Me - wrow0 + 31) / 32));
    }
    nfv = __builtin_amdgcn_readfirstlane(nfv);
    if constexpr (KRAG) kloop(std::integral_constant<int, FM>{});
    else dispatch_count<FM>(nfv, kloop);

    // ------------------------------------------------------------ epilogues
    // Each wavefront stages one 32-row block of its accumulators at a time in LDS (fp32,
    // row stride EPS = WN + 8 floats, so rows r and r + 4 fall in opposite bank halves), then
    // re-reads it row-major: every lane owns 8 consecutive columns of a row, so global loads
    // and stores are 16 bytes wide. acc[i][j][v] holds row i*32 + 8*(v/4) + 4*(lane/32) +
    // v%4 and column j*32 + lane%32 of the wavefront's block.
    if constexpr (EPI == EPI_F32) {
      // fp32 weight gradients: the 32 lanes of a half-wave write 128 contiguous bytes of a row
      // (one full cache line) per store, so the accumulators go straight to memory.
      float* Cg = p.of + (int64_t)g * p.f_gstride;
      if (m0 + BM <= p.M && n0 + BN <= p.N) {
        // Whole tile in range: a per-lane 32-bit byte offset from the tile origin plus a
        // wave-uniform offset per store (no per-store guard or 64-bit multiply; an expert's
        // block of the output is well under 4 GiB). The offsets are laundered through empty
        // asm each tile so the compiler recomputes them here instead of keeping all 128 live.
        char* Ct = reinterpret_cast<char*>(Cg + (int64_t)m0 * p.ldf + n0);
        uint32_t ld4 = (uint32_t)p.ldf * 4u;
        uint32_t lo4 = ((uint32_t)(wm * WM + (lane >> 5) * 4) * (uint32_t)p.ldf +
                        (uint32_t)(wn * WN + (lane & 31))) * 4u;
        asm volatile("" : "+s"(ld4));
        asm volatile("" : "+v"(lo4));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t o = lo4 + (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * ld4;
#pragma unroll
            for (int j = 0; j < FN; ++j)
              st_f32(reinterpret_cast<float*>(Ct + o + (uint32_t)(j * 128)), acc[i][j][v]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int row = m0 + wm * WM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
              if (row < p.M && col < p.N) st_f32(&Cg[(int64_t)row * p.ldf + col], acc[i][j][v]);
            }
          }
      }
    } else {
    constexpr int EPS = WN + 8;
    static_assert(WN == 64, "epilogue lane mapping assumes 64-column wavefront blocks");
    static_assert(NW * 32 * EPS * 4 <= NS * (BM + BN) * BK * 2, "epilogue staging fits the ring");
    float* st = reinterpret_cast<float*>(ring) + wave * 32 * EPS;
    // down: each block's row scales are loaded before the block is staged, all at once: a
    // load issued between two output stores would wait for the earlier store too
    // (vector-memory operations complete in order), one round trip per 8-row step.
    constexpr bool ROW_SCALE = (EPI == EPI_ROWS_SCALED);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= nfv) break;
      const int rblk = m0 + wm * WM + i * 32;            // tile-relative row of block row 0
      // fp32 row epilogues: lane group lane/8 takes rows 0,4,1,5,2,6,3,7 (+ 8 ps), so each
      // 16-lane LDS read pass covers two rows in opposite bank halves
      const int rl = (((lane >> 3) & 1) << 2) | (lane >> 4);
      float rsc[4];
      if constexpr (ROW_SCALE) {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          const int row = rblk + ps * 8 + rl;
          rsc[ps] = (row < Me) ? p.row_scale[r0 + row] : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          st[((v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * EPS + j * 32 + (lane & 31)] = acc[i][j][v];
      if constexpr (IS_GU) {
        // lane: 8 gate columns (cc) of row (ps*16 + lane/4) and the matching 8 linear columns;
        // the 4 lanes of a row hold 32 consecutive (32-aligned) gate and linear columns each:
        // one MXFP8 block of each
        const int cc = lane & 3;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
          const int row = ps * 16 + (lane >> 2);
          const int jj = j0 + wn * (WN / 2) + cc * 8;
          const f32x4 g0 = *(const f32x4*)&st[row * EPS + cc * 8];
          const f32x4 g1 = *(const f32x4*)&st[row * EPS + cc * 8 + 4];
          const f32x4 l0 = *(const f32x4*)&st[row * EPS + 32 + cc * 8];
          const f32x4 l1 = *(const f32x4*)&st[row * EPS + 32 + cc * 8 + 4];
          if (rblk + row < Me && jj < p.H) {
            const int64_t r = r0 + rblk + row;
            const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
            u32x4 hg, hl, av;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              hg[q] = pack_bf16x2(gv[2 * q], gv[2 * q + 1]);
              hl[q] = pack_bf16x2(lv[2 * q], lv[2 * q + 1]);
            }
            auto act = [&](auto b4) {
              constexpr bool B4 = decltype(b4)::value;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                av[q] = pack_bf16x2(situ_fwd<B4>(bf16_lo(hg[q]), bf16_lo(hl[q]), p.sc),
                                    situ_fwd<B4>(bf16_hi(hg[q]), bf16_hi(hl[q]), p.sc));
            };
            if (p.sc.b4) act(std::true_type{}); else act(std::false_type{});
            if constexpr (HMX) {
              // the stored h is MXFP8 of the bf16 h that `a` was computed from
              float gb[8], lb[8];
              float mg = 0.0f, ml = 0.0f;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                gb[2 * q] = bf16_lo(hg[q]); gb[2 * q + 1] = bf16_hi(hg[q]);
                lb[2 * q] = bf16_lo(hl[q]); lb[2 * q + 1] = bf16_hi(hl[q]);
                mg = fmaxf(mg, fmaxf(fabsf(gb[2 * q]), fabsf(gb[2 * q + 1])));
                ml = fmaxf(ml, fmaxf(fabsf(lb[2 * q]), fabsf(lb[2 * q + 1])));
              }
              const uint32_t sg = mx_scale_byte(mx_amax4(mg));
              const uint32_t sl = mx_scale_byte(mx_amax4(ml));
              uint8_t* qr = p.q0 + r * (2 * (int64_t)p.H);
              *(u32x2*)&qr[jj] = mx_encode8(gb, sg);
              *(u32x2*)&qr[p.H + jj] = mx_encode8(lb, sl);
              if (cc == 0) {
                uint8_t* sr = p.s0 + r * (2 * (int64_t)p.H / kMxBlock);
                sr[jj / kMxBlock] = (uint8_t)sg;
                sr[(p.H + jj) / kMxBlock] = (uint8_t)sl;
              }
            } else {
              st_row16(&p.o0[r * p.ld0 + jj], hg);
              st_row16(&p.o0[r * p.ld0 + p.H + jj], hl);
            }
            st_row16(&p.o1[r * p.ld1 + jj], av);
          }
        }
      } else if constexpr (EPI == EPI_ROWS || EPI == EPI_ROWS_SCALED) {
        // fp32 rows (the combine sums them in fp32 and rounds a token's sum once). The 8
        // lanes of a row hold columns 4 cc .. 4 cc + 3 and 32 + 4 cc .. 32 + 4 cc + 3, so each
        // of the two stores writes whole 128-byte lines of 8 rows.
        const int cc = lane & 7;
        const int col = n0 + wn * WN;                    // N is a multiple of 64
        if (col < p.N) {
#pragma unroll
          for (int ps = 0; ps < 4; ++ps) {
            const int row = ps * 8 + rl;
            const f32x4 c0 = *(const f32x4*)&st[row * EPS + cc * 4];
            const f32x4 c1 = *(const f32x4*)&st[row * EPS + 32 + cc * 4];
            if (rblk + row < Me) {
              float* dst = p.of + (int64_t)(r0 + rblk + row) * p.ldf + col + cc * 4;
              if constexpr (EPI == EPI_ROWS_SCALED) {
                const float sc = rsc[ps];
                st_f32x4(dst, f32x4{c0[0] * sc, c0[1] * sc, c0[2] * sc, c0[3] * sc});
                st_f32x4(dst + 32, f32x4{c1[0] * sc, c1[1] * sc, c1[2] * sc, c1[3] * sc});
              } else {
                st_f32x4(dst, c0);
                st_f32x4(dst + 32, c1);
              }
            }
          }
        }
      } else {
        // lane: columns cc*8 .. cc*8+7 of row ps*8 + lane/8
        const int cc = lane & 7;
        const int col = n0 + wn * WN + cc * 8;
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          const int row = ps * 8 + (lane >> 3);
          const f32x4 c0 = *(const f32x4*)&st[row * EPS + cc * 8];
          const f32x4 c1 = *(const f32x4*)&st[row * EPS + cc * 8 + 4];
          const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          if constexpr (IS_DA) {
            if (rblk + row < Me && col < p.N) {
              const int64_t r = r0 + rblk + row;
              const float pr = p.row_scale[r];
              // the saved pre-activation of these 8 columns (gate half, linear half): bf16
              // pairs, or MXFP8 decoded to fp32
              u32x4 hg = {0u, 0u, 0u, 0u}, hl = {0u, 0u, 0u, 0u};
              u32x2 qg = {0u, 0u}, ql = {0u, 0u};
              int xg = 0, xl = 0;
              if constexpr (HMX) {
                const uint8_t* qr = p.qsrc + r * (2 * (int64_t)p.H);
                const uint8_t* sr = p.ssrc + r * (2 * (int64_t)p.H / kMxBlock);
                qg = *(const u32x2*)&qr[col];
                ql = *(const u32x2*)&qr[p.H + col];
                xg = (int)sr[col / kMxBlock] - 127;
                xl = (int)sr[(p.H + col) / kMxBlock] - 127;
              } else {
                const uint16_t* hr = p.hsrc + r * (2 * (int64_t)p.H);
                hg = *(const u32x4*)&hr[col];
                hl = *(const u32x4*)&hr[p.H + col];
              }
              auto hgv = [&](int i) __attribute__((always_inline)) {
                if constexpr (HMX)
                  return __builtin_amdgcn_ldexpf(e4m3_code(qg[i >> 2], i & 3), xg);
                else return (i & 1) ? bf16_hi(hg[i >> 1]) : bf16_lo(hg[i >> 1]);
              };
              auto hlv = [&](int i) __attribute__((always_inline)) {
                if constexpr (HMX)
                  return __builtin_amdgcn_ldexpf(e4m3_code(ql[i >> 2], i & 3), xl);
                else return (i & 1) ? bf16_hi(hl[i >> 1]) : bf16_lo(hl[i >> 1]);
              };
              u32x4 og, ol, oa;
              float acc_p = 0.0f;
              auto grad = [&](auto b4) {
                constexpr bool B4 = decltype(b4)::value;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  float a0, dg0, dl0, a1, dg1, dl1;
                  situ_bwd<B4>(hgv(2 * q), hlv(2 * q), pr * cv[2 * q], p.sc, a0, dg0, dl0);
                  situ_bwd<B4>(hgv(2 * q + 1), hlv(2 * q + 1), pr * cv[2 * q + 1], p.sc, a1, dg1,
                               dl1);
                  // a0, a1 rounded to bf16 by one packed conversion (the same rounding)
                  const uint32_t aw = pack_bf16x2(a0, a1);
                  const float ab0 = bf16_lo(aw), ab1 = bf16_hi(aw);
                  acc_p = fmaf(cv[2 * q], ab0, acc_p);
                  acc_p = fmaf(cv[2 * q + 1], ab1, acc_p);
                  og[q] = pack_bf16x2(dg0, dg1);
                  ol[q] = pack_bf16x2(dl0, dl1);
                  oa[q] = pack_bf16x2(pr * ab0, pr * ab1);
                }
              };
              if (p.sc.b4) grad(std::true_type{}); else grad(std::false_type{});
              uint16_t* dr = p.o0 + r * p.ld0;
              st_row16(&dr[col], og);
              st_row16(&dr[p.H + col], ol);
              st_row16(&p.o1[r * p.ld1 + col], oa);
              part[ps] = acc_p;
            }
          }
        }
        if constexpr (IS_DA) {
          // <G, a> over this wavefront's 64 columns: sum the 8 lanes that share a row
          const int slot = nt * C::WGN + wn;
#pragma unroll
          for (int ps = 0; ps < 4; ++ps) {
            float v = part[ps];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            const int row = ps * 8 + (lane >> 3);
            if (cc == 0 && rblk + row < Me) p.dp_part[(int64_t)slot * p.dp_ld + r0 + rblk + row] = v;
          }
        }
      }
    }
    }
    // the next tile refills the ring only after every wave has read its staging
    wait_vm_lgkm0<0>();
    block_sync();
  }
}

// ---------------------------------------------------------------------------- launchers
template <class C, bool KRAG, int BKIND, int EPI, int TAG = 0>
static hipError_t run_gemm(const GemmArgs& args, int64_t max_tiles, hipStream_t s) {
  auto kern = grouped_gemm_kernel<C, KRAG, BKIND, EPI, TAG>;
  static int occ = -1;                   // workgroups per CU for this instantiation
  if (occ < 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, C::NT, 0) != hipSuccess || o < 1)
      o = 1;
    occ = o;
  }
  int64_t grid = (int64_t)device_cu_count() * occ;
  if (max_tiles < grid) grid = max_tiles;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, args);
  return hipGetLastError();
}

// Tile configuration per contraction.
#ifndef MOE_CFG_GU
#define MOE_CFG_GU CfgBig
#endif
#ifndef MOE_CFG_DN
#define MOE_CFG_DN CfgBig
#endif
#ifndef MOE_CFG_DA
#define MOE_CFG_DA CfgPP
#endif
#ifndef MOE_CFG_DX
#define MOE_CFG_DX CfgPP
#endif
#ifndef MOE_CFG_WD
#define MOE_CFG_WD CfgBig
#endif
#ifndef MOE_CFG_WG
#define MOE_CFG_WG CfgBig
#endif
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 4
#endif
#ifndef MOE_GROUP_M_W                 // the weight gradients' super-row height
#define MOE_GROUP_M_W 8
#endif
using CGU = MOE_CFG_GU;
using CDN = MOE_CFG_DN;
using CDA = MOE_CFG_DA;
using CDX = MOE_CFG_DX;
using CWD = MOE_CFG_WD;
using CWG = MOE_CFG_WG;

static GemmArgs blank_args() {
  GemmArgs a;
  __builtin_memset(&a, 0, sizeof(a));
  a.group_m = MOE_GROUP_M;
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
  p.n_tiles = (H + CGU::BN / 2 - 1) / (CGU::BN / 2);
  p.o0 = h; p.ld0 = 2 * H; p.o1 = a; p.ld1 = H;
  p.sc = c;
  return run_gemm<CGU, false, B_ROWS, EPI_GATEUP>(
      p, mragged_tile_bound(R_cap, E_loc, CGU::BM, p.n_tiles), s);
}

hipError_t launch_gemm_gate_up_mx(const uint16_t* x, const int32_t* row_token,
                                  const int32_t* offsets, int E_loc, int64_t R_cap, int d,
                                  int H, const uint16_t* w_gu, SituCoef c, uint8_t* h_codes,
                                  uint8_t* h_scales, uint16_t* a, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = x; p.lda = d; p.a_gather = row_token;
  p.B = w_gu; p.ldb = d; p.b_gstride = (int64_t)2 * H * d;
  p.offsets = offsets; p.G = E_loc;
  p.N = 2 * H; p.K = d; p.H = H;
  p.n_tiles = (H + CGU::BN / 2 - 1) / (CGU::BN / 2);
  p.q0 = h_codes; p.s0 = h_scales; p.o1 = a; p.ld1 = H;
  p.sc = c;
  return run_gemm<CGU, false, B_ROWS, EPI_GATEUP_MX>(
      p, mragged_tile_bound(R_cap, E_loc, CGU::BM, p.n_tiles), s);
}

hipError_t launch_gemm_down(const uint16_t* a, const int32_t* offsets, const float* row_gate,
                            int E_loc, int64_t R_cap, int H, int d, int c0, int nc,
                            const uint16_t* w_down, float* rows_out, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = a; p.lda = H;
  p.B = w_down + (int64_t)c0 * H; p.ldb = H; p.b_gstride = (int64_t)d * H;   // rows c0..c0+nc
  p.offsets = offsets; p.G = E_loc;
  p.N = nc; p.K = H;
  p.n_tiles = (nc + CDN::BN - 1) / CDN::BN;
  p.of = rows_out; p.ldf = nc; p.row_scale = row_gate;
  return run_gemm<CDN, false, B_ROWS, EPI_ROWS_SCALED>(
      p, mragged_tile_bound(R_cap, E_loc, CDN::BM, p.n_tiles), s);
}

int gemm_da_slots(int H) { return ((H + CDA::BN - 1) / CDA::BN) * CDA::WGN; }

hipError_t launch_gemm_da(const uint16_t* dy, const int32_t* row_token, const int32_t* offsets,
                          int E_loc, int64_t R_cap, int d, int H, const uint16_t* w_down,
                          const uint16_t* h, const uint8_t* h_codes, const uint8_t* h_scales,
                          const float* row_gate, SituCoef c, uint16_t* dh, uint16_t* pa,
                          float* dp_part, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dy; p.lda = d; p.a_gather = row_token;
  p.B = w_down; p.ldb = H; p.b_gstride = (int64_t)d * H;      // B(n=j, k) = w_down[e][k][j]
  p.offsets = offsets; p.G = E_loc;
  p.N = H; p.K = d; p.H = H;
  p.n_tiles = (H + CDA::BN - 1) / CDA::BN;
  p.o0 = dh; p.ld0 = dh_ld(H); p.o1 = pa; p.ld1 = H;
  p.row_scale = row_gate; p.hsrc = h; p.dp_part = dp_part; p.dp_ld = R_cap;
  p.qsrc = h_codes; p.ssrc = h_scales;
  p.sc = c;
  if (h_codes)
    return run_gemm<CDA, false, B_KOUT, EPI_DA_MX>(
        p, mragged_tile_bound(R_cap, E_loc, CDA::BM, p.n_tiles), s);
  return run_gemm<CDA, false, B_KOUT, EPI_DA>(
      p, mragged_tile_bound(R_cap, E_loc, CDA::BM, p.n_tiles), s);
}

hipError_t launch_gemm_dx(const uint16_t* dh, const int32_t* offsets, int E_loc,
                          int64_t R_cap, int d, int H, int c0, int nc, const uint16_t* w_gu,
                          float* rows_out, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dh; p.lda = dh_ld(H);
  p.B = w_gu + c0; p.ldb = d; p.b_gstride = (int64_t)2 * H * d;   // B(n, k) = w_gu[e][k][c0 + n]
  p.offsets = offsets; p.G = E_loc;
  p.N = nc; p.K = 2 * H;
  p.n_tiles = (nc + CDX::BN - 1) / CDX::BN;
  p.of = rows_out; p.ldf = nc;
  return run_gemm<CDX, false, B_KOUT, EPI_ROWS>(
      p, mragged_tile_bound(R_cap, E_loc, CDX::BM, p.n_tiles), s);
}

hipError_t launch_gemm_dw_down(const uint16_t* dy, const int32_t* row_token,
                               const uint16_t* pa, const int32_t* offsets, int E_loc, int d,
                               int H, float* dw_down, hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dy; p.lda = d; p.a_gather = row_token;                // A(m, k=r) = dy[tok(r)][m]
  p.B = pa; p.ldb = H;                                        // B(n, k=r) = pa[r][n]
  p.group_m = MOE_GROUP_M_W;
  p.offsets = offsets; p.G = E_loc;
  p.M = d; p.N = H;
  p.m_tiles = (d + CWD::BM - 1) / CWD::BM;
  p.n_tiles = (H + CWD::BN - 1) / CWD::BN;
  p.of = dw_down; p.ldf = H; p.f_gstride = (int64_t)d * H;
  return run_gemm<CWD, true, B_KOUT, EPI_F32>(p, (int64_t)E_loc * p.m_tiles * p.n_tiles, s);
}

hipError_t launch_gemm_dw_gu(const uint16_t* dh, const uint16_t* x, const int32_t* row_token,
                             const int32_t* offsets, int E_loc, int d, int H, float* dw_gu,
                             hipStream_t s) {
  GemmArgs p = blank_args();
  p.A = dh; p.lda = dh_ld(H);                                 // A(m, k=r) = dh[r][m]
  p.B = x; p.ldb = d; p.b_gather = row_token;                 // B(n, k=r) = x[tok(r)][n]
  p.group_m = MOE_GROUP_M_W;
  p.offsets = offsets; p.G = E_loc;
  p.M = 2 * H; p.N = d;
  p.m_tiles = (2 * H + CWG::BM - 1) / CWG::BM;
  p.n_tiles = (d + CWG::BN - 1) / CWG::BN;
  p.of = dw_gu; p.ldf = d; p.f_gstride = (int64_t)2 * H * d;
  return run_gemm<CWG, true, B_KOUT, EPI_F32, 1>(p, (int64_t)E_loc * p.m_tiles * p.n_tiles, s);
}

}  // namespace moe
