// extern "C" entry points of libmoe.so: argument validation, workspace layout, launches.
// Declarations and the contract of each call are in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "launch.h"
#include "situ_math.h"

namespace moe {

static thread_local int g_last_hip_error = 0;

int device_cu_count() {
  static int cache[128];                 // per device id; 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128) dev = 0;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v > 0) return v;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cu <= 0)
    cu = 256;
  __atomic_store_n(&cache[dev], cu, __ATOMIC_RELAXED);
  return cu;
}

static inline moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }

static size_t bwd_dh_bytes(int64_t R_cap, int H) { return round256((size_t)R_cap * 2 * H * 2); }
static size_t bwd_ov_bytes(int64_t R_cap, int d, int H) {
  return round256((size_t)R_cap * (size_t)(H > d ? H : d) * 2);
}
static size_t bwd_dp_bytes(int64_t R_cap, int H) {
  return round256((size_t)gemm_da_slots(H) * (size_t)R_cap * 4);
}

static inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The W4A8 GEMMs advance K in stages of 128 (four 32-element scale blocks per row).
static bool w4a8_dims_ok(int d, int H) {
  return d > 0 && H > 0 && d % 128 == 0 && H % 128 == 0 && d <= (1 << 16) && H <= (1 << 16);
}

static bool layer_dims_ok(int d, int H) {
  return d > 0 && H > 0 && d % 64 == 0 && H % 64 == 0 && d <= (1 << 16) && H <= (1 << 16);
}

// The GEMMs address token rows and one expert's rows with 32-bit byte offsets: a [T, d],
// [T, 2H] or [T, H] row block must span less than 4 GiB.
static bool rows_addressable(int64_t T, int d, int H) {
  const int64_t w = (int64_t)(d > 2 * H ? d : 2 * H);
  return T * w * 2 < ((int64_t)1 << 32);
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case MOE_ERR_UNSUPPORTED: return "outside the supported envelope (alignment, d/H multiple of 64, k <= 32, E <= 1024)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_CAPACITY: return "routed rows exceed the row capacity";
    case MOE_ERR_HIP: return "HIP launch failed (see moe_last_hip_error)";
  }
  return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_version(void) { return 100; }   // 0.1.0

moe_status moe_workspace_size(int which, int64_t T, int E_loc, int k, int d, int H,
                              int64_t R_cap, size_t* bytes) {
  (void)k;
  if (!bytes) return MOE_ERR_NULL;
  if (T < 0 || R_cap < 0) return MOE_ERR_SHAPE;
  switch (which) {
    case MOE_WS_PERMUTE:
      if (E_loc < 1 || E_loc > 1024) return MOE_ERR_SHAPE;
      *bytes = permute_ws_bytes(T, E_loc);
      return MOE_OK;
    case MOE_WS_SITU_GLU_FWD:
    case MOE_WS_SITU_GLU_BWD:
      *bytes = 0;
      return MOE_OK;
    case MOE_WS_DOWN_COMBINE:
      if (!layer_dims_ok(d, H)) return MOE_ERR_UNSUPPORTED;
      *bytes = round256((size_t)R_cap * d * 2);
      return MOE_OK;
    case MOE_WS_EXPERT_BWD:
      if (!layer_dims_ok(d, H)) return MOE_ERR_UNSUPPORTED;
      *bytes = bwd_dh_bytes(R_cap, H) + bwd_ov_bytes(R_cap, d, H) + bwd_dp_bytes(R_cap, H);
      return MOE_OK;
  }
  return MOE_ERR_SHAPE;
}

moe_status moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                          float* gates, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
  if (k > 32 || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || T * (int64_t)E >= (int64_t)1 << 40)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !gates) return MOE_ERR_NULL;
  return hip_status(launch_route_topk(logits, T, E, k, topk_idx, gates, stream));
}

moe_status moe_permute(const int32_t* topk_idx, const float* gates, int64_t T, int k,
                       int e_lo, int E_loc, int64_t R_cap, int32_t* expert_offsets,
                       int32_t* row_token, float* row_gate, int32_t* slot_row,
                       int32_t* status_flag, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || e_lo < 0 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || R_cap >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets || !status_flag || !ws) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !gates || !slot_row)) return MOE_ERR_NULL;
  if (R_cap > 0 && (!row_token || !row_gate)) return MOE_ERR_NULL;
  if (ws_bytes < permute_ws_bytes(T, E_loc)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute(topk_idx, gates, T, k, e_lo, E_loc, R_cap, expert_offsets,
                                   row_token, row_gate, slot_row, status_flag, ws, stream));
}

moe_status moe_unpermute(const void* rows, const int32_t* slot_row, const float* row_weight,
                         int64_t T, int k, int n, void* out, hipStream_t stream) {
  if (T < 0 || k < 1 || n < 1) return MOE_ERR_SHAPE;
  if (k > 32 || n % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!rows || !slot_row || !out) return MOE_ERR_NULL;
  if (!aligned16(rows) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_unpermute((const uint16_t*)rows, slot_row, row_weight, T, k, n,
                                     (uint16_t*)out, stream));
}

moe_status moe_grouped_gemm_gate_up(const void* x, const int32_t* row_token,
                                    const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                    int d, int H, const void* w_gu, float beta,
                                    float linear_beta, void* h, void* a, hipStream_t stream) {
  if (E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w_gu) return MOE_ERR_NULL;
  if (R_cap == 0) return MOE_OK;
  if (!x || !row_token || !h || !a) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gu) || !aligned16(h) || !aligned16(a))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_gemm_gate_up((const uint16_t*)x, row_token, expert_offsets, E_loc,
                                        R_cap, d, H, (const uint16_t*)w_gu,
                                        make_situ_coef(beta, linear_beta), (uint16_t*)h,
                                        (uint16_t*)a, stream));
}

moe_status moe_grouped_gemm_gate_up_mx(const void* x, const int32_t* row_token,
                                       const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                       int d, int H, const void* w_gu, float beta,
                                       float linear_beta, void* h_codes, void* h_scales,
                                       void* a, hipStream_t stream) {
  if (E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w_gu) return MOE_ERR_NULL;
  if (R_cap == 0) return MOE_OK;
  if (!x || !row_token || !h_codes || !h_scales || !a) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gu) || !aligned16(h_codes) || !aligned16(a))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_gemm_gate_up_mx((const uint16_t*)x, row_token, expert_offsets, E_loc,
                                           R_cap, d, H, (const uint16_t*)w_gu,
                                           make_situ_coef(beta, linear_beta), (uint8_t*)h_codes,
                                           (uint8_t*)h_scales, (uint16_t*)a, stream));
}

moe_status situ_glu_fwd(const void* h, int64_t R, int H, float beta, float linear_beta,
                        void* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (R < 0 || H < 1) return MOE_ERR_SHAPE;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (R == 0) return MOE_OK;
  if (!h || !a) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(a)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_situ_fwd((const uint16_t*)h, R, H, make_situ_coef(beta, linear_beta),
                                    (uint16_t*)a, stream));
}

moe_status situ_glu_bwd(const void* h, const void* da, int64_t R, int H, float beta,
                        float linear_beta, void* dh, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (R < 0 || H < 1) return MOE_ERR_SHAPE;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (R == 0) return MOE_OK;
  if (!h || !da || !dh) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(da) || !aligned16(dh)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_situ_bwd((const uint16_t*)h, (const uint16_t*)da, R, H,
                                    make_situ_coef(beta, linear_beta), (uint16_t*)dh, stream));
}

moe_status moe_grouped_gemm_down_combine(const void* a, const int32_t* expert_offsets,
                                         const float* row_gate, const int32_t* slot_row,
                                         int64_t T, int k, int E_loc, int64_t R_cap, int H,
                                         int d, const void* w_down, void* y, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || !rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets || !w_down) return MOE_ERR_NULL;
  if (T > 0 && (!slot_row || !y)) return MOE_ERR_NULL;
  if (R_cap > 0 && (!a || !row_gate || !ws)) return MOE_ERR_NULL;
  if (ws_bytes < round256((size_t)R_cap * d * 2)) return MOE_ERR_WORKSPACE;
  if ((a && !aligned16(a)) || !aligned16(w_down) || (y && !aligned16(y)) ||
      (ws && !aligned16(ws)))
    return MOE_ERR_UNSUPPORTED;
  uint16_t* rows = (uint16_t*)ws;
  if (R_cap > 0) {
    hipError_t e = launch_gemm_down((const uint16_t*)a, expert_offsets, row_gate, E_loc, R_cap,
                                    H, d, (const uint16_t*)w_down, rows, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (T == 0) return MOE_OK;
  // rows were already scaled by p in the GEMM epilogue, so the combine is a plain sum
  return hip_status(launch_unpermute(rows, slot_row, nullptr, T, k, d, (uint16_t*)y, stream));
}

static moe_status expert_bwd_impl(const void* dy, const void* x, const void* h,
                                  const void* h_codes, const void* h_scales,
                                  const int32_t* row_token, const float* row_gate,
                                  const int32_t* slot_row, const int32_t* expert_offsets,
                                  int64_t T, int k, int E_loc, int64_t R_cap, int d, int H,
                                  const void* w_gu, const void* w_down, float beta,
                                  float linear_beta, void* dx, float* dw_gu, float* dw_down,
                                  float* dp, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || !rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w_gu || !w_down || !dw_gu || !dw_down) return MOE_ERR_NULL;
  if (T > 0 && (!dy || !x || !slot_row || !dx || !dp)) return MOE_ERR_NULL;
  if (R_cap > 0 && ((!h && !(h_codes && h_scales)) || !row_token || !row_gate || !ws))
    return MOE_ERR_NULL;
  const size_t need = bwd_dh_bytes(R_cap, H) + bwd_ov_bytes(R_cap, d, H) + bwd_dp_bytes(R_cap, H);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const void* ptrs[] = {dy, x, h, h_codes, w_gu, w_down, dx, dw_gu, dw_down, ws};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_UNSUPPORTED;
  const SituCoef c = make_situ_coef(beta, linear_beta);
  uint8_t* base = (uint8_t*)ws;
  uint16_t* dh = (uint16_t*)base;
  uint16_t* ov = (uint16_t*)(base + bwd_dh_bytes(R_cap, H));     // pa, then dx rows
  float* dpp = (float*)(base + bwd_dh_bytes(R_cap, H) + bwd_ov_bytes(R_cap, d, H));
  hipError_t e = hipSuccess;
  if (R_cap > 0) {
    e = launch_gemm_da((const uint16_t*)dy, row_token, expert_offsets, E_loc, R_cap, d, H,
                       (const uint16_t*)w_down, (const uint16_t*)h, (const uint8_t*)h_codes,
                       (const uint8_t*)h_scales, row_gate, c, dh, ov, dpp, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  // weight gradients: every expert's slice is written (zeros when it has no rows)
  e = launch_gemm_dw_down((const uint16_t*)dy, row_token, ov, expert_offsets, E_loc, d, H,
                          dw_down, stream);
  if (e != hipSuccess) return hip_status(e);
  e = launch_gemm_dw_gu(dh, (const uint16_t*)x, row_token, expert_offsets, E_loc, d, H, dw_gu,
                        stream);
  if (e != hipSuccess) return hip_status(e);
  if (R_cap > 0) {
    e = launch_gemm_dx(dh, expert_offsets, E_loc, R_cap, d, H, (const uint16_t*)w_gu, ov,
                       stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (T == 0) return MOE_OK;
  e = launch_unpermute(ov, slot_row, nullptr, T, k, d, (uint16_t*)dx, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_dp_reduce_scatter(dpp, gemm_da_slots(H), R_cap, expert_offsets,
                                             E_loc, slot_row, T, k, dp, stream));
}

moe_status moe_expert_bwd(const void* dy, const void* x, const void* h,
                          const int32_t* row_token, const float* row_gate,
                          const int32_t* slot_row, const int32_t* expert_offsets, int64_t T,
                          int k, int E_loc, int64_t R_cap, int d, int H, const void* w_gu,
                          const void* w_down, float beta, float linear_beta, void* dx,
                          float* dw_gu, float* dw_down, float* dp, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (R_cap > 0 && !h) return MOE_ERR_NULL;
  return expert_bwd_impl(dy, x, h, nullptr, nullptr, row_token, row_gate, slot_row,
                         expert_offsets, T, k, E_loc, R_cap, d, H, w_gu, w_down, beta,
                         linear_beta, dx, dw_gu, dw_down, dp, ws, ws_bytes, stream);
}

moe_status moe_expert_bwd_mx(const void* dy, const void* x, const void* h_codes,
                             const void* h_scales, const int32_t* row_token,
                             const float* row_gate, const int32_t* slot_row,
                             const int32_t* expert_offsets, int64_t T, int k, int E_loc,
                             int64_t R_cap, int d, int H, const void* w_gu, const void* w_down,
                             float beta, float linear_beta, void* dx, float* dw_gu,
                             float* dw_down, float* dp, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  if (R_cap > 0 && (!h_codes || !h_scales)) return MOE_ERR_NULL;
  return expert_bwd_impl(dy, x, nullptr, h_codes, h_scales, row_token, row_gate, slot_row,
                         expert_offsets, T, k, E_loc, R_cap, d, H, w_gu, w_down, beta,
                         linear_beta, dx, dw_gu, dw_down, dp, ws, ws_bytes, stream);
}

moe_status moe_mxfp8_quantize(const void* v, int64_t rows, int n, void* codes, void* scales,
                              hipStream_t stream) {
  if (rows < 0 || n < 1) return MOE_ERR_SHAPE;
  if (n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!v || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(v) || !aligned16(codes)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_mx_quantize((const uint16_t*)v, rows, n, (uint8_t*)codes,
                                       (uint8_t*)scales, stream));
}

moe_status moe_mxfp8_dequantize(const void* codes, const void* scales, int64_t rows, int n,
                                void* out, hipStream_t stream) {
  if (rows < 0 || n < 1) return MOE_ERR_SHAPE;
  if (n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!codes || !scales || !out) return MOE_ERR_NULL;
  if (!aligned16(codes) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_mx_dequantize((const uint8_t*)codes, (const uint8_t*)scales, rows, n,
                                         (uint16_t*)out, stream));
}

moe_status moe_mxfp4_quantize(const void* v, int64_t rows, int n, void* codes, void* scales,
                              hipStream_t stream) {
  if (rows < 0 || n < 1) return MOE_ERR_SHAPE;
  if (n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!v || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(v) || !aligned4(codes)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_mx4_quantize((const uint16_t*)v, rows, n, (uint8_t*)codes,
                                        (uint8_t*)scales, stream));
}

moe_status moe_mxfp4_dequantize(const void* codes, const void* scales, int64_t rows, int n,
                                void* out, hipStream_t stream) {
  if (rows < 0 || n < 1) return MOE_ERR_SHAPE;
  if (n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!codes || !scales || !out) return MOE_ERR_NULL;
  if (!aligned4(codes) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_mx4_dequantize((const uint8_t*)codes, (const uint8_t*)scales, rows, n,
                                          (uint16_t*)out, stream));
}

moe_status moe_grouped_gemm_gate_up_w4a8(const void* x_codes, const void* x_scales, int64_t T,
                                         const int32_t* row_token,
                                         const int32_t* expert_offsets, int E_loc,
                                         int64_t R_cap, int d, int H, const void* w_gu_codes,
                                         const void* w_gu_scales, float beta, float linear_beta,
                                         void* a_codes, void* a_scales, hipStream_t stream) {
  if (T < 0 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (E_loc > 1024 || !w4a8_dims_ok(d, H) || R_cap >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)d >= (int64_t)1 << 32) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w_gu_codes || !w_gu_scales) return MOE_ERR_NULL;
  if (R_cap == 0) return MOE_OK;
  if (!x_codes || !x_scales || !row_token || !a_codes || !a_scales) return MOE_ERR_NULL;
  if (!aligned16(x_codes) || !aligned4(x_scales) || !aligned16(w_gu_codes) ||
      !aligned4(w_gu_scales) || !aligned16(a_codes))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_w4a8_gate_up(
      (const uint8_t*)x_codes, (const uint8_t*)x_scales, row_token, expert_offsets, E_loc, R_cap,
      d, H, (const uint8_t*)w_gu_codes, (const uint8_t*)w_gu_scales,
      make_situ_coef(beta, linear_beta), (uint8_t*)a_codes, (uint8_t*)a_scales, stream));
}

moe_status moe_grouped_gemm_down_combine_w4a8(const void* a_codes, const void* a_scales,
                                              const int32_t* expert_offsets,
                                              const float* row_gate, const int32_t* slot_row,
                                              int64_t T, int k, int E_loc, int64_t R_cap, int H,
                                              int d, const void* w_down_codes,
                                              const void* w_down_scales, void* y, void* ws,
                                              size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024 || !w4a8_dims_ok(d, H) || R_cap >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || !rows_addressable(T, d, H))
    return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets || !w_down_codes || !w_down_scales) return MOE_ERR_NULL;
  if (T > 0 && (!slot_row || !y)) return MOE_ERR_NULL;
  if (R_cap > 0 && (!a_codes || !a_scales || !row_gate || !ws)) return MOE_ERR_NULL;
  if (ws_bytes < round256((size_t)R_cap * d * 2)) return MOE_ERR_WORKSPACE;
  if ((a_codes && !aligned16(a_codes)) || (a_scales && !aligned4(a_scales)) ||
      !aligned16(w_down_codes) || !aligned4(w_down_scales) || (y && !aligned16(y)) ||
      (ws && !aligned16(ws)))
    return MOE_ERR_UNSUPPORTED;
  uint16_t* rows = (uint16_t*)ws;
  if (R_cap > 0) {
    hipError_t e = launch_w4a8_down((const uint8_t*)a_codes, (const uint8_t*)a_scales,
                                    expert_offsets, row_gate, E_loc, R_cap, H, d,
                                    (const uint8_t*)w_down_codes, (const uint8_t*)w_down_scales,
                                    rows, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (T == 0) return MOE_OK;
  // rows were already scaled by p in the GEMM epilogue, so the combine is a plain sum
  return hip_status(launch_unpermute(rows, slot_row, nullptr, T, k, d, (uint16_t*)y, stream));
}

moe_status moe_router_bwd(const float* gates, const float* dp, int64_t T, int k,
                          float* dlogits_kept, hipStream_t stream) {
  if (T < 0 || k < 1) return MOE_ERR_SHAPE;
  if (k > 32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!gates || !dp || !dlogits_kept) return MOE_ERR_NULL;
  return hip_status(launch_router_bwd(gates, dp, T, k, dlogits_kept, stream));
}

}  // extern "C"
