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

// The combines read fp32 rows [R_cap, w] covering w output columns at a time: w = d in one
// pass, or a multiple of 256 columns per pass when the workspace is smaller (each column's
// arithmetic is the same either way, so the results are bit-identical).
static int combine_min_cols(int d) { return d < 256 ? d : 256; }
static size_t rows_bytes(int64_t R_cap, int w) { return round256((size_t)R_cap * (size_t)w * 4); }
// Widest window whose rows fit in `avail` bytes: all d columns, or a multiple of 256 (0 when
// not even the narrowest window fits).
static int combine_cols(int64_t R_cap, int d, size_t avail) {
  if (R_cap == 0) return d;
  const size_t w = avail / ((size_t)R_cap * 4);
  if (w >= (size_t)d) return d;
  return (int)(w / 256 * 256);
}

// Backward workspace: dh [R_cap, 2H] bf16 (row stride dh_ld(H)) | dp partials [slots, R_cap]
// fp32 | overlay of bf16(p a) [R_cap, H] and then the dX rows (fp32, one column window at a
// time).
static size_t bwd_dh_bytes(int64_t R_cap, int H) { return round256((size_t)R_cap * dh_ld(H) * 2); }
static size_t bwd_dp_bytes(int64_t R_cap, int H) {
  return round256((size_t)gemm_da_slots(H) * (size_t)R_cap * 4);
}
static size_t bwd_pa_bytes(int64_t R_cap, int H) { return round256((size_t)R_cap * H * 2); }
static size_t bwd_ws_bytes(int64_t R_cap, int d, int H, int w) {
  const size_t ov = rows_bytes(R_cap, w);
  const size_t pa = bwd_pa_bytes(R_cap, H);
  return bwd_dh_bytes(R_cap, H) + bwd_dp_bytes(R_cap, H) + (ov > pa ? ov : pa);
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

// Scratch of moe_grouped_gemm_down_combine_noalloc: the fp32 rows p o of one column window.
// Each GPU the library runs on holds its own copy until the process ends. In host code the
// name `scratch` is only a stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device and kept.
static __device__ __attribute__((aligned(256))) float scratch[MOE_NOALLOC_SCRATCH_BYTES / 4];
static void* g_scratch_ptr[128];

static hipError_t static_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 128) return hipErrorInvalidDevice;
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
  }
  *out = (float*)p;
  return hipSuccess;
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
    case MOE_WS_EXPERT_BWD:
      return moe_workspace_size_passes(which, T, E_loc, k, d, H, R_cap, 1, bytes);
  }
  return MOE_ERR_SHAPE;
}

moe_status moe_workspace_size_passes(int which, int64_t T, int E_loc, int k, int d, int H,
                                     int64_t R_cap, int passes, size_t* bytes) {
  (void)E_loc;
  (void)k;
  if (!bytes) return MOE_ERR_NULL;
  if (T < 0 || R_cap < 0 || passes < 1) return MOE_ERR_SHAPE;
  if (which != MOE_WS_DOWN_COMBINE && which != MOE_WS_EXPERT_BWD) return MOE_ERR_SHAPE;
  if (!layer_dims_ok(d, H)) return MOE_ERR_UNSUPPORTED;
  int w = (d + passes - 1) / passes;
  w = (w + 255) / 256 * 256;
  if (w > d) w = d;
  *bytes = which == MOE_WS_DOWN_COMBINE ? rows_bytes(R_cap, w) : bwd_ws_bytes(R_cap, d, H, w);
  return MOE_OK;
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
  return hip_status(launch_unpermute((const uint16_t*)rows, n, slot_row, row_weight, T, k, n,
                                     (uint16_t*)out, n, stream));
}

moe_status moe_grouped_gemm_gate_up(const void* x, int64_t T, const int32_t* row_token,
                                    const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                    int d, int H, const void* w_gu, float beta,
                                    float linear_beta, void* h, void* a, hipStream_t stream) {
  if (T < 0 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  // the gather addresses token rows with 32-bit byte offsets, and an expert holds at most T rows
  if (!rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
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

moe_status moe_grouped_gemm_gate_up_mx(const void* x, int64_t T, const int32_t* row_token,
                                       const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                       int d, int H, const void* w_gu, float beta,
                                       float linear_beta, void* h_codes, void* h_scales,
                                       void* a, hipStream_t stream) {
  if (T < 0 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  // the gather addresses token rows with 32-bit byte offsets, and an expert holds at most T rows
  if (!rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
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

// down GEMM + combine with fp32 rows in `rows` (rows_bytes of them): one pass per window of
// output columns that fits.
static moe_status down_combine_impl(const void* a, const int32_t* expert_offsets,
                                    const float* row_gate, const int32_t* slot_row, int64_t T,
                                    int k, int E_loc, int64_t R_cap, int H, int d,
                                    const void* w_down, void* y, float* rows, size_t rows_avail,
                                    hipStream_t stream) {
  if (T < 0 || k < 1 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || !rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets || !w_down) return MOE_ERR_NULL;
  if (T > 0 && (!slot_row || !y)) return MOE_ERR_NULL;
  if (R_cap > 0 && (!a || !row_gate || !rows)) return MOE_ERR_NULL;
  const int w = combine_cols(R_cap, d, rows ? rows_avail : 0);
  if (w < combine_min_cols(d)) return MOE_ERR_WORKSPACE;
  if ((a && !aligned16(a)) || !aligned16(w_down) || (y && !aligned16(y)) ||
      (rows && !aligned16(rows)))
    return MOE_ERR_UNSUPPORTED;
  // one pass per window of w output columns: fp32 rows p o, then their fp32 slot-order sum
  for (int c0 = 0; c0 < d; c0 += w) {
    const int nc = d - c0 < w ? d - c0 : w;
    if (R_cap > 0) {
      hipError_t e = launch_gemm_down((const uint16_t*)a, expert_offsets, row_gate, E_loc, R_cap,
                                      H, d, c0, nc, (const uint16_t*)w_down, rows, stream);
      if (e != hipSuccess) return hip_status(e);
    }
    if (T > 0) {
      hipError_t e = launch_unpermute_f32(rows, nc, slot_row, T, k, nc, (uint16_t*)y + c0, d,
                                          stream);
      if (e != hipSuccess) return hip_status(e);
    }
  }
  return MOE_OK;
}

moe_status moe_grouped_gemm_down_combine(const void* a, const int32_t* expert_offsets,
                                         const float* row_gate, const int32_t* slot_row,
                                         int64_t T, int k, int E_loc, int64_t R_cap, int H,
                                         int d, const void* w_down, void* y, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return down_combine_impl(a, expert_offsets, row_gate, slot_row, T, k, E_loc, R_cap, H, d,
                           w_down, y, (float*)ws, ws_bytes, stream);
}

moe_status moe_grouped_gemm_down_combine_noalloc(const void* a, const int32_t* expert_offsets,
                                                 const float* row_gate,
                                                 const int32_t* slot_row, int64_t T, int k,
                                                 int E_loc, int64_t R_cap, int H, int d,
                                                 const void* w_down, void* y,
                                                 hipStream_t stream) {
  if (R_cap < 0) return MOE_ERR_SHAPE;
  if (R_cap * (int64_t)combine_min_cols(d > 0 ? d : 1) * 4 > (int64_t)MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE;                    // rows beyond what the static scratch holds
  float* rows = nullptr;
  if (R_cap > 0) {
    const hipError_t e = static_scratch(&rows);
    if (e != hipSuccess) return hip_status(e);
  }
  return down_combine_impl(a, expert_offsets, row_gate, slot_row, T, k, E_loc, R_cap, H, d,
                           w_down, y, rows, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

static moe_status expert_bwd_impl(const void* dy, const void* x, const void* h,
                                  const void* h_codes, const void* h_scales,
                                  const int32_t* row_token, const float* row_gate,
                                  const int32_t* slot_row, const int32_t* expert_offsets,
                                  int64_t T, int k, int E_loc, int64_t R_cap, int d, int H,
                                  const void* w_gu, const void* w_down, float beta,
                                  float linear_beta, void* dx, float* dw_gu, float* dw_down,
                                  float* dp, void* ws, size_t ws_bytes, int stages,
                                  hipStream_t stream) {
  if (stages < 1 || stages > MOE_BWD_ALL) return MOE_ERR_SHAPE;
  if (T < 0 || k < 1 || E_loc < 1 || R_cap < 0) return MOE_ERR_SHAPE;
  if (k > 32 || E_loc > 1024 || !layer_dims_ok(d, H) || R_cap >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t)1 << 31 || !rows_addressable(T, d, H)) return MOE_ERR_UNSUPPORTED;
  if (!(beta > 0.0f) || !(linear_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w_gu || !w_down || !dw_gu || !dw_down) return MOE_ERR_NULL;
  if (T > 0 && (!dy || !x || !slot_row || !dx || !dp)) return MOE_ERR_NULL;
  if (R_cap > 0 && ((!h && !(h_codes && h_scales)) || !row_token || !row_gate || !ws))
    return MOE_ERR_NULL;
  const size_t fixed = bwd_dh_bytes(R_cap, H) + bwd_dp_bytes(R_cap, H);
  if (!ws) ws_bytes = 0;
  if (ws_bytes < fixed + bwd_pa_bytes(R_cap, H)) return MOE_ERR_WORKSPACE;
  const int w = combine_cols(R_cap, d, ws_bytes - fixed);
  if (w < combine_min_cols(d)) return MOE_ERR_WORKSPACE;
  const void* ptrs[] = {dy, x, h, h_codes, w_gu, w_down, dx, dw_gu, dw_down, ws};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_UNSUPPORTED;
  const SituCoef c = make_situ_coef(beta, linear_beta);
  uint8_t* base = (uint8_t*)ws;
  uint16_t* dh = (uint16_t*)base;
  float* dpp = (float*)(base + bwd_dh_bytes(R_cap, H));
  uint16_t* ov = (uint16_t*)(base + fixed);        // bf16(p a), then the fp32 dX rows
  hipError_t e = hipSuccess;
  if ((stages & MOE_BWD_DA) && R_cap > 0) {
    e = launch_gemm_da((const uint16_t*)dy, row_token, expert_offsets, E_loc, R_cap, d, H,
                       (const uint16_t*)w_down, (const uint16_t*)h, (const uint8_t*)h_codes,
                       (const uint8_t*)h_scales, row_gate, c, dh, ov, dpp, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  // weight gradients: every expert's slice is written (zeros when it has no rows)
  if (stages & MOE_BWD_DW_DOWN) {
    e = launch_gemm_dw_down((const uint16_t*)dy, row_token, ov, expert_offsets, E_loc, d, H,
                            dw_down, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (stages & MOE_BWD_DW_GU) {
    e = launch_gemm_dw_gu(dh, (const uint16_t*)x, row_token, expert_offsets, E_loc, d, H, dw_gu,
                          stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (stages & MOE_BWD_DX) {
    float* rows = (float*)ov;                    // overwrites bf16(p a): after DW_DOWN
    for (int c0 = 0; c0 < d; c0 += w) {
      const int nc = d - c0 < w ? d - c0 : w;
      if (R_cap > 0) {
        e = launch_gemm_dx(dh, expert_offsets, E_loc, R_cap, d, H, c0, nc,
                           (const uint16_t*)w_gu, rows, stream);
        if (e != hipSuccess) return hip_status(e);
      }
      if (T > 0) {
        e = launch_unpermute_f32(rows, nc, slot_row, T, k, nc, (uint16_t*)dx + c0, d, stream);
        if (e != hipSuccess) return hip_status(e);
      }
    }
  }
  if ((stages & MOE_BWD_DP) && T > 0) {
    e = launch_dp_reduce_scatter(dpp, gemm_da_slots(H), R_cap, expert_offsets, E_loc, slot_row,
                                 T, k, dp, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  return MOE_OK;
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
                         linear_beta, dx, dw_gu, dw_down, dp, ws, ws_bytes, MOE_BWD_ALL,
                         stream);
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
                         linear_beta, dx, dw_gu, dw_down, dp, ws, ws_bytes, MOE_BWD_ALL,
                         stream);
}

moe_status moe_expert_bwd_stages(const void* dy, const void* x, const void* h,
                                 const void* h_codes, const void* h_scales,
                                 const int32_t* row_token, const float* row_gate,
                                 const int32_t* slot_row, const int32_t* expert_offsets,
                                 int64_t T, int k, int E_loc, int64_t R_cap, int d, int H,
                                 const void* w_gu, const void* w_down, float beta,
                                 float linear_beta, void* dx, float* dw_gu, float* dw_down,
                                 float* dp, void* ws, size_t ws_bytes, int stages,
                                 hipStream_t stream) {
  if (h && (h_codes || h_scales)) return MOE_ERR_SHAPE;         // one stored form of h
  if (R_cap > 0 && !h && !(h_codes && h_scales)) return MOE_ERR_NULL;
  return expert_bwd_impl(dy, x, h, h_codes, h_scales, row_token, row_gate, slot_row,
                         expert_offsets, T, k, E_loc, R_cap, d, H, w_gu, w_down, beta,
                         linear_beta, dx, dw_gu, dw_down, dp, ws, ws_bytes, stages, stream);
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
  const int w = combine_cols(R_cap, d, ws ? ws_bytes : 0);
  if (w < combine_min_cols(d)) return MOE_ERR_WORKSPACE;
  if ((a_codes && !aligned16(a_codes)) || (a_scales && !aligned4(a_scales)) ||
      !aligned16(w_down_codes) || !aligned4(w_down_scales) || (y && !aligned16(y)) ||
      (ws && !aligned16(ws)))
    return MOE_ERR_UNSUPPORTED;
  float* rows = (float*)ws;
  for (int c0 = 0; c0 < d; c0 += w) {
    const int nc = d - c0 < w ? d - c0 : w;
    if (R_cap > 0) {
      hipError_t e = launch_w4a8_down((const uint8_t*)a_codes, (const uint8_t*)a_scales,
                                      expert_offsets, row_gate, E_loc, R_cap, H, d, c0, nc,
                                      (const uint8_t*)w_down_codes,
                                      (const uint8_t*)w_down_scales, rows, stream);
      if (e != hipSuccess) return hip_status(e);
    }
    if (T > 0) {
      hipError_t e = launch_unpermute_f32(rows, nc, slot_row, T, k, nc, (uint16_t*)y + c0, d,
                                          stream);
      if (e != hipSuccess) return hip_status(e);
    }
  }
  return MOE_OK;
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
