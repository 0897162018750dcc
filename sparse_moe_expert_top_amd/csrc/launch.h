// Internal launchers behind the C ABI (declared here, defined next to their kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_math.h"

namespace moe {

// Device facts used to size persistent grids (cached per device).
int device_cu_count();

// Leading dimension (elements) of the backward's dh rows [R, 2H] in the workspace: 64
// elements (one cache line) past 2H. The weight gradient dW_gu reads dh a k-row (512 bytes of
// a row) at a time, 64 consecutive rows per stage; with a stride of 2H elements (12 KiB at
// H = 3072) those rows start at the same offset modulo every power of two up to 4 KiB. The
// extra line staggers them: on the large-context workload dW_gu fetched 23 % fewer bytes
// from beyond the L2 and ran 2-4 % faster. (bf16(p a), read the same way by dW_down at a
// 6 KiB stride, measured no faster padded.)
inline int64_t dh_ld(int H) { return 2 * (int64_t)H + 64; }

// Routing and dispatch metadata ("Inside Kimi K3", "Idea One"; "MoE 反向", second saving).
hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* idx,
                             float* gates, hipStream_t s);
int permute_blocks(int64_t T);
size_t permute_ws_bytes(int64_t T, int E_loc);
hipError_t launch_permute(const int32_t* idx, const float* gates, int64_t T, int k, int e_lo,
                          int E_loc, int64_t R_cap, int32_t* offsets, int32_t* row_token,
                          float* row_gate, int32_t* slot_row, int32_t* status, void* ws,
                          hipStream_t s);
// out[t, 0..n) = bf16(sum over local slots of w(r) rows[r, 0..n)), summed in fp32 in slot
// order; rows have leading dimension ldr (elements), out ldo. n a multiple of 8.
hipError_t launch_unpermute(const uint16_t* rows, int64_t ldr, const int32_t* slot_row,
                            const float* w, int64_t T, int k, int n, uint16_t* out,
                            int64_t ldo, hipStream_t s);
hipError_t launch_unpermute_f32(const float* rows, int64_t ldr, const int32_t* slot_row,
                                int64_t T, int k, int n, uint16_t* out, int64_t ldo,
                                hipStream_t s);
hipError_t launch_dp_reduce_scatter(float* part, int nslots, int64_t R_cap,
                                    const int32_t* offsets, int E_loc,
                                    const int32_t* slot_row, int64_t T, int k, float* dp,
                                    hipStream_t s);
hipError_t launch_router_bwd(const float* gates, const float* dp, int64_t T, int k,
                             float* dlogits, hipStream_t s);

// Streaming SiTU-GLU ("Frontier-scale RL with Kimi K3", "Streaming activations").
hipError_t launch_situ_fwd(const uint16_t* h, int64_t R, int H, SituCoef c, uint16_t* a,
                           hipStream_t s);
hipError_t launch_situ_bwd(const uint16_t* h, const uint16_t* da, int64_t R, int H,
                           SituCoef c, uint16_t* dh, hipStream_t s);

// Grouped GEMMs ("MoE 反向": expert forward equation and the rewritten backward).
// Rows of group e are [offsets[e], offsets[e+1]).
hipError_t launch_gemm_gate_up(const uint16_t* x, const int32_t* row_token,
                               const int32_t* offsets, int E_loc, int64_t R_cap, int d, int H,
                               const uint16_t* w_gu, SituCoef c, uint16_t* h, uint16_t* a,
                               hipStream_t s);
// gate_up storing the saved h as MXFP8 (codes [R, 2H], scale bytes [R, 2H/32]).
hipError_t launch_gemm_gate_up_mx(const uint16_t* x, const int32_t* row_token,
                                  const int32_t* offsets, int E_loc, int64_t R_cap, int d,
                                  int H, const uint16_t* w_gu, SituCoef c, uint8_t* h_codes,
                                  uint8_t* h_scales, uint16_t* a, hipStream_t s);
// down: fp32 rows p * o over output columns [c0, c0 + nc): rows_out [R_cap, nc].
hipError_t launch_gemm_down(const uint16_t* a, const int32_t* offsets, const float* row_gate,
                            int E_loc, int64_t R_cap, int H, int d, int c0, int nc,
                            const uint16_t* w_down, float* rows_out, hipStream_t s);
// dA: G = dy[row_token] . w_down[e]; epilogue writes dh, pa = bf16(p a) and dp partials.
int gemm_da_slots(int H);
// The saved h is read from bf16 `h`, or from MXFP8 codes and scales when h_codes != nullptr.
hipError_t launch_gemm_da(const uint16_t* dy, const int32_t* row_token, const int32_t* offsets,
                          int E_loc, int64_t R_cap, int d, int H, const uint16_t* w_down,
                          const uint16_t* h, const uint8_t* h_codes, const uint8_t* h_scales,
                          const float* row_gate, SituCoef c, uint16_t* dh, uint16_t* pa,
                          float* dp_part, hipStream_t s);
// dX rows: dh . w_gu[e] over columns [c0, c0 + nc)  ->  fp32 rows [R_cap, nc]
hipError_t launch_gemm_dx(const uint16_t* dh, const int32_t* offsets, int E_loc,
                          int64_t R_cap, int d, int H, int c0, int nc, const uint16_t* w_gu,
                          float* rows_out, hipStream_t s);
// Weight gradients with ragged K = rows of the expert.
hipError_t launch_gemm_dw_down(const uint16_t* dy, const int32_t* row_token,
                               const uint16_t* pa, const int32_t* offsets, int E_loc, int d,
                               int H, float* dw_down, hipStream_t s);
hipError_t launch_gemm_dw_gu(const uint16_t* dh, const uint16_t* x, const int32_t* row_token,
                             const int32_t* offsets, int E_loc, int d, int H, float* dw_gu,
                             hipStream_t s);

// MXFP8 storage format of the saved pre-activation (mxfp8.h); n a multiple of 32.
hipError_t launch_mx_quantize(const uint16_t* v, int64_t rows, int n, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int n,
                                uint16_t* out, hipStream_t s);

// W4A8 forward ("Frontier-scale RL with Kimi K3", "Low precision (MXFP4) rollouts"): MXFP8
// activations x MXFP4 weights on the block-scaled MFMA; K (d for gate_up, H for down) a
// multiple of 128. gate_up writes a as MXFP8 (codes [R, H], scales [R, H/32]); down writes
// fp32 p o rows [R_cap, nc] for output columns [c0, c0 + nc).
hipError_t launch_w4a8_gate_up(const uint8_t* x_codes, const uint8_t* x_scales,
                               const int32_t* row_token, const int32_t* offsets, int E_loc,
                               int64_t R_cap, int d, int H, const uint8_t* w_codes,
                               const uint8_t* w_scales, SituCoef c, uint8_t* a_codes,
                               uint8_t* a_scales, hipStream_t s);
hipError_t launch_w4a8_down(const uint8_t* a_codes, const uint8_t* a_scales,
                            const int32_t* offsets, const float* row_gate, int E_loc,
                            int64_t R_cap, int H, int d, int c0, int nc,
                            const uint8_t* w_codes, const uint8_t* w_scales, float* rows_out,
                            hipStream_t s);
// MXFP4 format of the W4A8 weights (mxfp4.h); n a multiple of 32.
hipError_t launch_mx4_quantize(const uint16_t* v, int64_t rows, int n, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);
hipError_t launch_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int n,
                                 uint16_t* out, hipStream_t s);

}  // namespace moe
