// W4A8 forward of the routed experts on gfx950 block-scaled MFMA, and the MXFP4 weight
// quantizer.
//
// "Frontier-scale RL with Kimi K3", section "Low precision (MXFP4) rollouts": the rollout
// engine runs the MoE layers with 4-bit weights and 8-bit activations. Both are OCP MX
// formats here: weights MXFP4 (E2M1, mxfp4.h), activations MXFP8 (E4M3, mxfp8.h), each with
// one E8M0 scale per 32 elements along the reduction dimension. The expert is the layer of
// "Kimi K3 ... Memory", section "MoE 反向" (a = SiTU(W_gate x, W_up x), o = W_down a). Two
// contractions, each over all local experts in one launch:
//
//   name      C[m][n]                      M      N    K    A (MXFP8)          B (MXFP4)
//   gate_up   x8[tok(r)] . w4_gu[e]^T     rows   2H   d    x, gathered rows   w_gu rows
//   down      a8[r] . w4_down[e]^T        rows   d    H    a rows             w_down rows
//
// gate_up's epilogue rounds h to bf16, applies SiTU-GLU, rounds a to bf16 and writes it as
// MXFP8 (the down GEMM's A operand); down's writes fp32 p o rows for the combine, over a
// window of its output columns per launch.
//
// Design (gfx950):
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with A = E4M3, B = E2M1 and fp32 accumulators. Operand
//    layout of this instruction (established with single-wave probes against an fp64 model):
//    a k-step's two 32-deep K blocks are the lane halves of the fp4 operand (lane 32b + n
//    holds K [32b, 32b + 32) of column n, low nibble first); the fp8 operand's lane 32h + m
//    holds K [16h, 16h + 16) of row m in bytes 0..15 and K [32 + 16h, +16) in bytes 16..31;
//    the scale of row m (column n) for block b is the op_sel-selected byte of lane 32b + m
//    (32b + n). The instruction's sum of a block's products is not an fp32 round-to-nearest
//    sum of the exact products: it deviated from one by up to 1.6e-4 of the sum of the
//    products' magnitudes on full-range random codes and scales.
//  * 256 x 256 tiles, 8 wavefronts (two per SIMD) of 64 x 128, K stages of 128 filled by
//    direct-to-LDS loads: A [256][128 B] with chunk c of row r at c ^ ((r >> 1) & 7),
//    B [256][64 B] with chunk c at c ^ ((r >> 2) & 3), so sixteen consecutive rows of one
//    logical chunk hit sixteen distinct 16-byte slots. Per stage and wavefront: 4 A and 2 B
//    loads; per k-step and fragment two ds_read_b128 (A) or one (B), and one ds_read_b32 of
//    the scales per stage.
//  * Block scales. Each stage needs 4 scale bytes of each of the tile's 512 rows (A's and
//    B's). When K is a multiple of 512 and at most 3584, a scale block beside a 2-slot ring
//    (96 KiB + 56 KiB) holds them as 16-byte chunks of 4 stages, one 16-byte load per row and
//    chunk, each chunk requested 4 stages before its first read. Otherwise a 3-slot ring
//    (156 KiB) carries each stage's scale bytes in the stage slot, one 4-byte load per row and
//    stage. Fetching a row's 4 bytes once per stage touches 512 cache lines per stage; the
//    chunked block fetches each line a quarter as often.
//  * The pipeline, tile list, balanced row split, XCD-aware order and fragment skipping are
//    those of the bf16 grouped GEMM (gemm.hip, gemm_util.h).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "gemm_util.h"
#include "launch.h"
#include "mxfp4.h"
#include "mxfp8.h"
#include "situ_math.h"

namespace moe {

enum W4Epi { W4_GATEUP = 0, W4_ROWS_SCALED = 1 };

struct W4A8Args {
  const uint8_t* A;          // E4M3 codes, K bytes per row
  const uint8_t* As;         // scale bytes, K/32 per row
  const int32_t* a_gather;   // storage row of each routed row (gate_up), or null (row = r)
  const uint8_t* B;          // E2M1 codes [G][N][K/2]
  const uint8_t* Bs;         // scale bytes [G][N][K/32]
  const int32_t* offsets;
  int G, N, K, H;
  int n_tiles, group_m;
  uint8_t* qa;               // gate_up: a codes [R, H] and scale bytes [R, H/32]
  uint8_t* sa;
  int64_t b_gs, bs_gs;       // per-expert strides of B and Bs (bytes)
  float* o;                  // down: fp32 p o rows [R, N], leading dimension ldo
  int64_t ldo;
  const float* row_scale;
  SituCoef sc;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

#ifndef MOE_W4_NS
#define MOE_W4_NS 3
#endif

// SB selects where a stage's scale bytes come from. false: each stage slot of the ring holds
// them, one 4-byte load per tile row and stage (512 rows: 512 cache lines per stage for 2 KiB).
// true (K a multiple of 512 and at most 3584, scale arrays 16-byte aligned): a scale block
// after a 2-slot ring holds all K / 128 stages of them for every tile row as 16-byte chunks
// of 4 stages, [chunk][512 rows][16 bytes]; one 16-byte load per row fetches a chunk, so the
// scale loads per tile drop from K / 128 to K / 512 per row. Chunk c + 1 is requested with
// stage 4 c's refill, four stages before its first read.
template <int EPI, bool SB>
__global__ __launch_bounds__(512, 2) void w4a8_gemm_kernel(W4A8Args p) {
  constexpr int BM = 256, BN = 256, BK = 128, NS = SB ? 2 : MOE_W4_NS, NT = 512, NW = 8;
  constexpr int WGN = 2, WM = 64, WN = 128, FM = WM / 32, FN = WN / 32;
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK / 2, AS_BYTES = BM * 4, BS_BYTES = BN * 4;
  constexpr int SC_OFF = A_BYTES + B_BYTES;        // A scales, then B scales (SB: unused)
  constexpr int STAGE = A_BYTES + B_BYTES + (SB ? 0 : AS_BYTES + BS_BYTES);
  constexpr int SB_CH = 7;                         // scale block: chunks of 4 stages (K <= 3584)
  constexpr int SB_OFF = NS * STAGE;
  constexpr int SB_BYTES = SB ? SB_CH * 512 * 16 : 0;
  constexpr int LA = A_BYTES / 1024 / NW;          // 16-byte direct loads per wave per stage
  constexpr int LB = B_BYTES / 1024 / NW;
  constexpr int LPS = LA + LB + (SB ? 0 : 1);      // + one 4-byte scale load
  static_assert(LA == 4 && LB == 2 && AS_BYTES / 256 + BS_BYTES / 256 == NW, "stage loads");
  static_assert(NS == 2 || NS == 3, "ring depth");
  static_assert(NW * 64 == 512, "scale block: one row per lane");
  constexpr bool GU = (EPI == W4_GATEUP);

  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE + SB_BYTES];
  __shared__ int s_pref[1025];
  __shared__ int s_scan[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring);

  const int total = build_tile_prefix<NT, BM>(p.offsets, p.G, p.n_tiles, s_pref, s_scan);

  // Fragment byte offsets inside a stage. Fragment rows are 32-aligned, so the swizzle of
  // lane row l32 is the same in every fragment, and the chunk of k-step s (and half t) is
  // the lane's base chunk XOR a constant: A chunk 4s + 2t + hh sits at (4s + 2t) ^ (hh ^ swz),
  // B chunk 2s + hh at 2s ^ (hh ^ swz).
  const int hh = lane >> 5, l32 = lane & 31;
  const uint32_t a_base = (uint32_t)((wm * WM + l32) * BK + ((hh ^ ((l32 >> 1) & 7)) << 4));
  const uint32_t b_base = (uint32_t)(A_BYTES + (wn * WN + l32) * (BK / 2) + ((hh ^ ((l32 >> 2) & 3)) << 4));
  const uint32_t as_base = (uint32_t)(SC_OFF + (wm * WM + l32) * 4);
  const uint32_t bs_base = (uint32_t)(SC_OFF + AS_BYTES + (wn * WN + l32) * 4);
  const uint32_t sb_as_base = (uint32_t)(SB_OFF + (wm * WM + l32) * 16);
  const uint32_t sb_bs_base = (uint32_t)(SB_OFF + (256 + wn * WN + l32) * 16);

  const int nblk = gridDim.x;
  const int nk = p.K / BK;
  const int ks = p.K / 32;                          // scale bytes per row
  for (int tile = xcd_first_tile(blockIdx.x, nblk); tile < total; tile += nblk) {
    int g = tile_group(s_pref, p.G, tile);
    const int mg = p.offsets[g + 1] - p.offsets[g];
    int mt, nt;
    raster_tile(tile - s_pref[g], (mg + BM - 1) / BM, p.group_m, p.n_tiles, mt, nt);
    g = __builtin_amdgcn_readfirstlane(g);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int r0 = p.offsets[g];
    const int Mg = p.offsets[g + 1] - r0;
    int m0, Me;
    balanced_rows<BM>(mt, Mg, m0, Me);
    const int n0 = nt * BN;
    const int j0 = nt * (BN / 2);                  // gate_up: first gate/linear column pair
    const uint8_t* Bg = p.B + (int64_t)g * p.b_gs;
    const uint8_t* Bsg = p.Bs + (int64_t)g * p.bs_gs;

    // weight row of tile row `row` (gate_up interleaves each wavefront's 64 gate rows with
    // the matching 64 linear rows)
    auto w_row = [&](int row) __attribute__((always_inline)) {
      if constexpr (GU) {
        const int w = row / WN, q = row % WN;
        const int jj = min(j0 + w * (WN / 2) + (q % (WN / 2)), p.H - 1);
        return (q < WN / 2) ? jj : p.H + jj;
      } else {
        return min(n0 + row, p.N - 1);
      }
    };
    // A row of tile row `row`: gathered rows are token rows, addressed from A itself (the
    // host keeps T * K below 2^32); contiguous rows are addressed from the tile's first row,
    // so their 32-bit offsets stay below 256 K whatever the row count
    auto a_srow = [&](int row) __attribute__((always_inline)) {
      const int m = min(m0 + row, Me - 1);
      return p.a_gather ? p.a_gather[r0 + m] : m - m0;
    };
    const int64_t a_row0 = p.a_gather ? 0 : (int64_t)r0 + m0;
    const uint8_t* a_tile = p.A + a_row0 * p.K;
    const uint8_t* as_tile = p.As + a_row0 * ks;

    // waves 0..3 load the A scales of rows 64 w .. 64 w + 63, waves 4..7 the B scales
    const bool s_is_a = wave_u < 4;
    const uint8_t* s_src = s_is_a ? as_tile : Bsg;
    // ------------------------------------------------------------ load addressing
    uint32_t a_off[LA], b_off[LB], s_off;
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int byte = (wave * LA + q) * 1024 + lane * 16;
      const int row = byte >> 7;
      const int c = ((byte & 127) >> 4) ^ ((row >> 1) & 7);
      a_off[q] = (uint32_t)a_srow(row) * (uint32_t)p.K + (uint32_t)(c << 4);
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int byte = (wave * LB + q) * 1024 + lane * 16;
      const int row = byte >> 6;
      const int c = ((byte & 63) >> 4) ^ ((row >> 2) & 3);
      b_off[q] = (uint32_t)w_row(row) * (uint32_t)(p.K / 2) + (uint32_t)(c << 4);
    }
    s_off = (uint32_t)(s_is_a ? a_srow(wave * 64 + lane) : w_row((wave - 4) * 64 + lane)) *
            (uint32_t)ks;

    auto issue = [&](int kt) __attribute__((always_inline)) {
      const uint32_t base = ring_lds + (kt % NS) * STAGE;
      dma_saddr<LA>(base + wave_u * (LA * 1024), uniform_ptr(a_tile + kt * BK), a_off);
      dma_saddr<LB>(base + A_BYTES + wave_u * (LB * 1024), uniform_ptr(Bg + kt * (BK / 2)), b_off);
      if constexpr (!SB)
        dma_saddr_b32(base + SC_OFF + wave_u * 256, uniform_ptr(s_src + kt * 4), s_off);
    };
    // SB: chunk c (the scale bytes of stages 4 c .. 4 c + 3) of the wavefront's 64 rows, 16
    // bytes per lane, into [c][row]
    auto issue_chunk = [&](int c) __attribute__((always_inline)) {
      const uint32_t o1[1] = {s_off};
      dma_saddr<1>(ring_lds + SB_OFF + c * (512 * 16) + wave_u * 1024,
                   uniform_ptr(s_src + c * 16), o1);
    };
    auto wait_stage = [&](int later) __attribute__((always_inline)) {
      if (later >= 2) wait_vm_lgkm0<2 * LPS>();
      else if (later == 1) wait_vm_lgkm0<LPS>();
      else wait_vm_lgkm0<0>();
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // The slot and lane bases are passed through empty asm at each use, so the compiler
    // forms each address when it is needed instead of keeping every variant live.
    auto load_frags = [&](auto nfc, int slot, auto sc, i32x8 (&af)[FM], u32x4 (&bfr)[FN])
        __attribute__((always_inline)) {
      constexpr int NF = decltype(nfc)::value;
      constexpr int S = decltype(sc)::value;
      uint32_t ab = a_base + (uint32_t)(slot * STAGE), bb = b_base + (uint32_t)(slot * STAGE);
      asm volatile("" : "+v"(ab));
      asm volatile("" : "+v"(bb));
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i < NF) {
          const uint8_t* r = ring + i * 32 * BK;
          const u32x4 lo = *(const u32x4*)(r + (ab ^ ((4 * S) << 4)));
          const u32x4 hi = *(const u32x4*)(r + (ab ^ ((4 * S + 2) << 4)));
          af[i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const u32x4*)(ring + j * 32 * (BK / 2) + (bb ^ ((2 * S) << 4)));
    };
    // each lane's scale word of the stage holds blocks 0..3 of its row; shifted by 8 hh, its
    // byte 2 s is block 2 s + hh, the block of k-step s that this lane supplies
    // (SB: the word of stage kt in chunk kt / 4 of each fragment row of the scale block)
    auto load_scales = [&](auto nfc, int kt, uint32_t (&sa)[FM], uint32_t (&sb)[FN])
        __attribute__((always_inline)) {
      constexpr int NF = decltype(nfc)::value;
      constexpr int RS = SB ? 32 * 16 : 128;          // bytes from one fragment's rows to the next
      uint32_t ab, bb;
      if constexpr (SB) {
        const uint32_t col = (uint32_t)(kt >> 2) * (512u * 16u) + (uint32_t)(kt & 3) * 4u;
        ab = sb_as_base + col;
        bb = sb_bs_base + col;
      } else {
        ab = as_base + (uint32_t)((kt % NS) * STAGE);
        bb = bs_base + (uint32_t)((kt % NS) * STAGE);
      }
      asm volatile("" : "+v"(ab));
      asm volatile("" : "+v"(bb));
#pragma unroll
      for (int i = 0; i < FM; ++i)
        if (i < NF) sa[i] = *(const uint32_t*)(ring + i * RS + ab) >> (8 * hh);
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j] = *(const uint32_t*)(ring + j * RS + bb) >> (8 * hh);
    };
    auto mfma_step = [&](auto nfc, auto sc, const i32x8 (&af)[FM], const u32x4 (&bfr)[FN],
                         const uint32_t (&sa)[FM], const uint32_t (&sb)[FN])
        __attribute__((always_inline)) {
      constexpr int NF = decltype(nfc)::value;
      constexpr int S = decltype(sc)::value;
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const i32x8 b8 = {(int)bfr[j][0], (int)bfr[j][1], (int)bfr[j][2], (int)bfr[j][3], 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], b8, acc[i][j], 0, 4, 2 * S, (int)sa[i], 2 * S, (int)sb[j]);
        }
    };

    // ------------------------------------------------------------ k pipeline
    // As in the bf16 GEMM: stages kt+1 .. kt+NS-1 are in flight while stage kt is consumed;
    // the barrier of stage kt sits before its second (last) k-step, when every wave has read
    // the whole stage (fragments of both k-steps, and the scales) into registers, and has
    // waited for its own loads of stage kt+1. The next stage's scales are read after the last
    // k-step's MFMAs are issued.
    auto kloop = [&](auto nfc) __attribute__((always_inline)) {
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      i32x8 fa0[FM], fa1[FM];
      u32x4 fb0[FN], fb1[FN];
      uint32_t sa[FM], sb[FN];
      if constexpr (SB) issue_chunk(0);
#pragma unroll
      for (int st = 0; st < NS - 1; ++st)
        if (st < nk) issue(st);
      wait_stage(min(NS - 2, nk - 1));
      block_sync();
      if (NS - 1 < nk) issue(NS - 1);
      load_scales(nfc, 0, sa, sb);
      load_frags(nfc, 0, S0{}, fa0, fb0);
      // the last stage is peeled off, so the last k-step's MFMAs of every other stage follow
      // the next stage's first fragment reads on one path only and wait for nothing
      for (int kt = 0; kt + 1 < nk; ++kt) {
        load_frags(nfc, kt % NS, S1{}, fa1, fb1);
        mfma_step(nfc, S0{}, fa0, fb0, sa, sb);
        wait_stage(min(NS - 2, nk - 2 - kt));
        block_sync();
        // (SB: chunk kt / 4 + 1 is waited for with stage kt + 2 and read from stage kt + 4)
        if (SB && (kt & 3) == 0 && 4 * ((kt >> 2) + 1) < nk) issue_chunk((kt >> 2) + 1);
        if (kt + NS < nk) issue(kt + NS);
        load_frags(nfc, (kt + 1) % NS, S0{}, fa0, fb0);
        mfma_step(nfc, S1{}, fa1, fb1, sa, sb);
        load_scales(nfc, kt + 1, sa, sb);
      }
      if (nk > 0) {
        load_frags(nfc, (nk - 1) % NS, S1{}, fa1, fb1);
        mfma_step(nfc, S0{}, fa0, fb0, sa, sb);
        mfma_step(nfc, S1{}, fa1, fb1, sa, sb);
      }
      wait_vm_lgkm0<0>();
      block_sync();
    };
    int nfv;
    {
      const int wrow0 = m0 + (wave_u / WGN) * WM;
      nfv = max(0, min(FM, (Me - wrow0 + 31) / 32));
    }
    nfv = __builtin_amdgcn_readfirstlane(nfv);
    dispatch_count<FM>(nfv, kloop);

    // ------------------------------------------------------------ epilogues
    // Each wavefront stages a 32-row, 64-column half of its block at a time in LDS (fp32, row
    // stride EPS = 72 floats), then re-reads it row-major. acc[i][j][v] holds row
    // i*32 + 8*(v/4) + 4*(lane/32) + v%4 and column j*32 + lane%32 of the wavefront's block.
    // gate_up's half hf pairs gate fragment hf (columns 32 hf ..) with linear fragment 2 + hf.
    constexpr int EPS = 72;
    static_assert(NW * 32 * EPS * 4 <= NS * STAGE, "epilogue staging fits the ring");
    float* stg = reinterpret_cast<float*>(ring) + wave * 32 * EPS;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= nfv) break;
      const int rblk = m0 + wm * WM + i * 32;
      // down: the block's row scales are loaded before it is staged, all at once (a load
      // issued between two output stores would also wait for the earlier store: vector-memory
      // operations complete in order)
      float rsc[4];
      if constexpr (!GU) {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          const int row = rblk + ps * 8 + (lane >> 3);
          rsc[ps] = (row < Me) ? p.row_scale[r0 + row] : 0.0f;
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int f0 = GU ? hf : 2 * hf, f1 = GU ? 2 + hf : 2 * hf + 1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int srow = ((v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * EPS + (lane & 31);
          stg[srow] = acc[i][f0][v];
          stg[srow + 32] = acc[i][f1][v];
        }
        if constexpr (GU) {
          // lane: 8 gate columns (cc) of row ps*16 + lane/4 and the matching 8 linear columns;
          // the 4 lanes of a row cover one 32-aligned block of a's columns (one MXFP8 block),
          // and all 4 take the same branch
          const int cc = lane & 3;
#pragma unroll
          for (int ps = 0; ps < 2; ++ps) {
            const int row = ps * 16 + (lane >> 2);
            const int jj = j0 + wn * (WN / 2) + hf * 32 + cc * 8;
            const f32x4 g0 = *(const f32x4*)&stg[row * EPS + cc * 8];
            const f32x4 g1 = *(const f32x4*)&stg[row * EPS + cc * 8 + 4];
            const f32x4 l0 = *(const f32x4*)&stg[row * EPS + 32 + cc * 8];
            const f32x4 l1 = *(const f32x4*)&stg[row * EPS + 32 + cc * 8 + 4];
            if (rblk + row < Me && jj < p.H) {
              const int64_t r = r0 + rblk + row;
              const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
              const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
              float av[8];
              float amax = 0.0f;
              auto act = [&](auto b4) {
                constexpr bool B4 = decltype(b4)::value;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                  av[q] = round_bf16(situ_fwd<B4>(round_bf16(gv[q]), round_bf16(lv[q]), p.sc));
                  amax = fmaxf(amax, fabsf(av[q]));
                }
              };
              if (p.sc.b4) act(std::true_type{}); else act(std::false_type{});
              const uint32_t sbyte = mx_scale_byte(mx_amax4(amax));
              *(u32x2*)&p.qa[r * p.H + jj] = mx_encode8(av, sbyte);
              if (cc == 0) p.sa[r * (p.H / kMxBlock) + jj / kMxBlock] = (uint8_t)sbyte;
            }
          }
        } else {
          // lane: columns cc*8 .. cc*8+7 of row ps*8 + lane/8
          const int cc = lane & 7;
          const int col = n0 + wn * WN + hf * 64 + cc * 8;
#pragma unroll
          for (int ps = 0; ps < 4; ++ps) {
            const int row = ps * 8 + (lane >> 3);
            const f32x4 c0 = *(const f32x4*)&stg[row * EPS + cc * 8];
            const f32x4 c1 = *(const f32x4*)&stg[row * EPS + cc * 8 + 4];
            if (rblk + row < Me && col < p.N) {
              const int64_t r = r0 + rblk + row;
              const float sc = rsc[ps];
              float* dst = p.o + r * p.ldo + col;
              *(f32x4*)dst = f32x4{c0[0] * sc, c0[1] * sc, c0[2] * sc, c0[3] * sc};
              *(f32x4*)(dst + 4) = f32x4{c1[0] * sc, c1[1] * sc, c1[2] * sc, c1[3] * sc};
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

template <int EPI, bool SB>
static hipError_t run_w4a8_kernel(const W4A8Args& args, int64_t max_tiles, hipStream_t s) {
  auto kern = w4a8_gemm_kernel<EPI, SB>;
  static int occ = -1;
  if (occ < 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, 512, 0) != hipSuccess || o < 1) o = 1;
    occ = o;
  }
  int64_t grid = (int64_t)device_cu_count() * occ;
  if (max_tiles < grid) grid = max_tiles;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, s, args);
  return hipGetLastError();
}

// The scale-block form needs 16-byte aligned scale rows (K a multiple of 512) and arrays, and
// K <= 3584 (28 stages of scale bytes per row in LDS).
template <int EPI>
static hipError_t run_w4a8(const W4A8Args& args, int64_t max_tiles, hipStream_t s) {
  const bool sb = args.K % 512 == 0 && args.K <= 3584 && (uintptr_t)args.As % 16 == 0 &&
                  (uintptr_t)args.Bs % 16 == 0 && args.bs_gs % 16 == 0;
  return sb ? run_w4a8_kernel<EPI, true>(args, max_tiles, s)
            : run_w4a8_kernel<EPI, false>(args, max_tiles, s);
}

#ifndef MOE_GROUP_M
#define MOE_GROUP_M 4
#endif

static int64_t w4_tile_bound(int64_t R_cap, int E_loc, int n_tiles) {
  return ((R_cap + 255) / 256 + E_loc) * (int64_t)n_tiles;
}

hipError_t launch_w4a8_gate_up(const uint8_t* x_codes, const uint8_t* x_scales,
                               const int32_t* row_token, const int32_t* offsets, int E_loc,
                               int64_t R_cap, int d, int H, const uint8_t* w_codes,
                               const uint8_t* w_scales, SituCoef c, uint8_t* a_codes,
                               uint8_t* a_scales, hipStream_t s) {
  W4A8Args p;
  __builtin_memset(&p, 0, sizeof(p));
  p.A = x_codes; p.As = x_scales; p.a_gather = row_token;
  p.B = w_codes; p.Bs = w_scales; p.offsets = offsets;
  p.G = E_loc; p.N = 2 * H; p.K = d; p.H = H;
  p.b_gs = (int64_t)2 * H * (d / 2); p.bs_gs = (int64_t)2 * H * (d / 32);
  p.n_tiles = (H + 127) / 128; p.group_m = MOE_GROUP_M;
  p.qa = a_codes; p.sa = a_scales; p.sc = c;
  return run_w4a8<W4_GATEUP>(p, w4_tile_bound(R_cap, E_loc, p.n_tiles), s);
}

hipError_t launch_w4a8_down(const uint8_t* a_codes, const uint8_t* a_scales,
                            const int32_t* offsets, const float* row_gate, int E_loc,
                            int64_t R_cap, int H, int d, int c0, int nc,
                            const uint8_t* w_codes, const uint8_t* w_scales, float* rows_out,
                            hipStream_t s) {
  W4A8Args p;
  __builtin_memset(&p, 0, sizeof(p));
  p.A = a_codes; p.As = a_scales;
  // weight rows c0 .. c0 + nc of every expert
  p.B = w_codes + (int64_t)c0 * (H / 2); p.Bs = w_scales + (int64_t)c0 * (H / 32);
  p.b_gs = (int64_t)d * (H / 2); p.bs_gs = (int64_t)d * (H / 32);
  p.offsets = offsets;
  p.G = E_loc; p.N = nc; p.K = H; p.H = H;
  p.n_tiles = (nc + 255) / 256; p.group_m = MOE_GROUP_M;
  p.o = rows_out; p.ldo = nc; p.row_scale = row_gate;
  return run_w4a8<W4_ROWS_SCALED>(p, w4_tile_bound(R_cap, E_loc, p.n_tiles), s);
}

// ---------------------------------------------------------------------------- MXFP4 codec
// Each lane owns 8 consecutive elements (16 bytes of bf16, 4 code bytes); the 4 lanes of a
// 32-element block are consecutive lanes and always active together (chunk counts and the
// grid stride are multiples of 4).
__global__ __launch_bounds__(256) void mx4_quantize_kernel(const uint16_t* __restrict__ v,
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
    const uint32_t sb = mx4_scale_byte(mx_amax4(m));
    *(uint32_t*)(codes + c * 4) = mx4_encode8(f, sb);
    if ((c & 3) == 0) scales[c >> 2] = (uint8_t)sb;
  }
}

__global__ __launch_bounds__(256) void mx4_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             int64_t nchunks,
                                                             uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    float f[8];
    mx4_decode8(*(const uint32_t*)(codes + c * 4), scales[c >> 2], f);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
    *(u32x4*)(out + c * 8) = o;
  }
}

static unsigned mx4_grid(int64_t nchunks) {
  int64_t blocks = (nchunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 64;
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t launch_mx4_quantize(const uint16_t* v, int64_t rows, int n, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  const int64_t nchunks = rows * (int64_t)(n / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx4_quantize_kernel, dim3(mx4_grid(nchunks)), dim3(256), 0, s, v, nchunks,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int n,
                                 uint16_t* out, hipStream_t s) {
  const int64_t nchunks = rows * (int64_t)(n / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx4_dequantize_kernel, dim3(mx4_grid(nchunks)), dim3(256), 0, s, codes,
                     scales, nchunks, out);
  return hipGetLastError();
}

}  // namespace moe
