/*
 * moe.h - C ABI of the MI355X (gfx950) routed-expert layer library `libmoe.so`.
 *
 * The layer is the routed Mixture-of-Experts expert block of a Kimi-K3-style model on one
 * GPU's local share of experts, forward and backward:
 *   - routing: top-k of each token's router logits, softmax over the k kept values
 *     ("Inside Kimi K3", section "Idea One", routing snippet);
 *   - expert forward a_e = SiTU(W_gate x, W_up x), o_e = W_down a_e, y = sum_e p_e o_e and
 *     the backward that takes dL/dp_e as <W_down^T dL/dy, a_e> so o_e is never stored
 *     ("Kimi K3 ... Memory", section "MoE 反向", forward equation and p-gradient rewrite);
 *   - SiTU-GLU: gate' = beta tanh(g/beta) sigmoid(g), lin' = linear_beta tanh(l/linear_beta),
 *     a = gate' lin', gate half first; only the bf16 pre-activation [R, 2H] is kept and tanh
 *     and sigmoid are recomputed in the backward ("Frontier-scale RL with Kimi K3", section
 *     "Streaming activations");
 *   - the backward redoes the dispatch from the pre-dispatch input ("MoE 反向", second saving).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA memory) unless a
 *     comment says otherwise. The caller owns every buffer; the library never allocates.
 *   - Layout is row-major and contiguous. bf16 tensors are passed as `void*` holding IEEE
 *     bfloat16 bit patterns. Weights are [out, in]: w_gu[e] is [2H, d] with the H W_gate rows
 *     first and the H W_up rows second; w_down[e] is [d, H].
 *   - Every call is asynchronous on `stream` (0 = the null stream). Calls are thread-safe:
 *     the library keeps no mutable global state besides a cached device-property table.
 *   - Host-side validation runs before any launch; on error nothing is launched and the
 *     output contents are unchanged. After MOE_ERR_HIP, moe_last_hip_error() gives the
 *     hipError_t of the failed launch on the calling thread.
 *   - Pointers to bf16/fp32 tensors must be 16-byte aligned; d and H must be multiples of
 *     64; k <= 32; E <= 1024; E_loc <= 1024. Token-indexed tensors must span less than
 *     4 GiB per row block: T * max(d, 2H) * 2 < 2^32 (every call that reads token rows
 *     takes T and checks it before any launch).
 *   - Routed rows R are data-dependent and stay on the device in expert_offsets[E_loc].
 *     Buffers indexed by rows are sized by a caller-chosen capacity R_cap (T*k always
 *     suffices). moe_permute clamps the offsets to R_cap and raises *status_flag when the
 *     true row count exceeds it, so the later calls never touch rows >= R_cap.
 *   - y, dx and dp are this GPU's additive partial sums over its local experts (zero for
 *     routes to other GPUs' experts), so summing them over GPUs gives the full layer.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,        /* inconsistent or negative sizes (k > E, e_lo + E_loc > E, ...) */
  MOE_ERR_UNSUPPORTED = 3,  /* outside the supported envelope (alignment, d/H % 64, k > 32) */
  MOE_ERR_WORKSPACE = 4,    /* ws_bytes below moe_workspace_size() */
  MOE_ERR_CAPACITY = 5,     /* reserved: the device-side row overflow is reported by flag */
  MOE_ERR_HIP = 6           /* a HIP launch failed; see moe_last_hip_error() */
} moe_status;

/* Entry-point ids for moe_workspace_size(). */
typedef enum {
  MOE_WS_PERMUTE = 1,
  MOE_WS_SITU_GLU_FWD = 2,
  MOE_WS_SITU_GLU_BWD = 3,
  MOE_WS_DOWN_COMBINE = 4,      /* one combine pass over all d columns (fastest) */
  MOE_WS_EXPERT_BWD = 5         /* one dX combine pass over all d columns (fastest) */
} moe_ws_kind;

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* moe_status_string(moe_status s);

/* hipError_t (as int) of the last MOE_ERR_HIP returned on this thread, 0 if none. */
int moe_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int moe_version(void);

/*
 * moe_route_topk - routing ("Inside Kimi K3", "Idea One"): for each token t, keep the k
 * largest of logits[t, 0..E) and set gates[t, :] = softmax over those k values.
 *   logits    [T, E] fp32, finite (precondition; not checked on the device).
 *   topk_idx  [T, k] int32 out: global expert ids in slot order = value descending, equal
 *             values by lower expert index (-0.0 ties +0.0).
 *   gates     [T, k] fp32 out: exp(v_j - v_0) / sum_i exp(v_i - v_0), computed in fp32.
 * Errors: NULL pointers (when T > 0), T < 0, E < 1, k < 1, k > E, k > 32, E > 1024.
 */
moe_status moe_route_topk(const float* logits, int64_t T, int E, int k,
                          int32_t* topk_idx, float* gates, hipStream_t stream);

/*
 * moe_permute - dispatch metadata on one GPU ("MoE 反向", second saving: the grouped GEMM
 * reads the tokens arranged by expert). Keeps routes to experts e_lo..e_lo+E_loc-1 and
 * sorts them by local expert, stably by token within an expert (a counting sort; no atomic
 * decides an order, so the result is bit-reproducible).
 *   topk_idx, gates  [T, k] from moe_route_topk.
 *   expert_offsets   [E_loc+1] int32 out: row range of local expert e is
 *                    [offsets[e], offsets[e+1]); values clamped to R_cap.
 *   row_token        [R_cap] int32 out: token of each row.
 *   row_gate         [R_cap] fp32 out: gate of each row (not renormalised).
 *   slot_row         [T, k] int32 out: row of route (t, j); -1 for non-local routes and for
 *                    routes dropped because they fall beyond R_cap.
 *   status_flag      device int32 out: 0, or 1 when the local route count exceeds R_cap.
 *   ws, ws_bytes     device scratch of moe_workspace_size(MOE_WS_PERMUTE, ...) bytes.
 * Errors: NULL pointers, e_lo < 0, E_loc < 1, E_loc > 1024, k > 32, R_cap < 0, small ws.
 */
moe_status moe_permute(const int32_t* topk_idx, const float* gates, int64_t T, int k,
                       int e_lo, int E_loc, int64_t R_cap,
                       int32_t* expert_offsets, int32_t* row_token, float* row_gate,
                       int32_t* slot_row, int32_t* status_flag,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_unpermute - combine of expert rows back to tokens: the sum over a token's routes in
 * the forward equation y = sum_e p_e o_e ("Kimi K3 ... Memory", section "MoE 反向"), and
 * the return of the re-dispatched rows to their tokens in the backward (same section,
 * second saving):
 *   out[t, :] = bf16( sum over j with slot_row[t,j] >= 0 of w(r) * rows[r, :] ),
 *   r = slot_row[t, j], w = row_weight[r] or 1 when row_weight is NULL; the sum is taken in
 *   fp32 in slot order. Tokens with no local route get zeros.
 *   rows [R_cap, n] bf16 (caller-owned, read only), slot_row [T, k] int32, row_weight
 *   [R_cap] fp32 or NULL, out [T, n] bf16 (written). n must be a multiple of 8; rows and out
 *   16-byte aligned. Every slot_row entry must be -1 or a row below R_cap (precondition).
 * Errors: T < 0, k < 1, n < 1 (MOE_ERR_SHAPE); k > 32, n % 8, T * k >= 2^31, misaligned
 * pointers (MOE_ERR_UNSUPPORTED); NULL pointers when T > 0 (MOE_ERR_NULL).
 */
moe_status moe_unpermute(const void* rows, const int32_t* slot_row, const float* row_weight,
                         int64_t T, int k, int n, void* out, hipStream_t stream);

/*
 * moe_grouped_gemm_gate_up - the expert forward's first half, a_e = SiTU(W_gate x, W_up x)
 * ("Kimi K3 ... Memory", section "MoE 反向", forward equation), keeping only the bf16
 * pre-activation for the backward ("Frontier-scale RL with Kimi K3", section "Streaming
 * activations": the custom op saves one bf16 [R, 2H] tensor). For every local expert e and
 * its rows r:
 *   h[r, :]  = bf16( x[row_token[r], :] . w_gu[e]^T )           (saved for the backward)
 *   a[r, j]  = bf16( SiTU-GLU(h[r, j], h[r, H + j]) ), j < H      (input of the down GEMM)
 * The dispatch (row gather through row_token) is fused into the operand load; SiTU-GLU is
 * fused into the epilogue and computed in fp32 from the bf16-rounded h.
 *   x [T, d] bf16 (read), row_token [R_cap] and expert_offsets [E_loc+1] (device, from
 *   moe_permute), w_gu [E_loc, 2H, d] bf16 (read), h [R_cap, 2H] bf16 and a [R_cap, H] bf16
 *   (written for rows below expert_offsets[E_loc]; other rows untouched). All caller-owned.
 * Errors: T < 0, E_loc < 1, R_cap < 0, beta or linear_beta not > 0 (MOE_ERR_SHAPE);
 * T * max(d, 2H) * 2 >= 2^32 (the gather addresses token rows with 32-bit offsets), d or H
 * not a multiple of 64, E_loc > 1024, R_cap >= 2^31, misaligned pointers
 * (MOE_ERR_UNSUPPORTED); NULL pointers (MOE_ERR_NULL). Nothing is launched on error.
 */
moe_status moe_grouped_gemm_gate_up(const void* x, int64_t T, const int32_t* row_token,
                                    const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                    int d, int H, const void* w_gu, float beta,
                                    float linear_beta, void* h, void* a, hipStream_t stream);

/*
 * situ_glu_fwd - streaming SiTU-GLU forward, the naive activation's definition in
 * "Frontier-scale RL with Kimi K3", section "Streaming activations": the last dimension of h
 * splits into a gate half g and a linear half l, gate' = beta tanh(g/beta) sigmoid(g),
 * lin' = linear_beta tanh(l/linear_beta), and the product is cast back to the input dtype:
 *   a[r, j] = bf16(gate'(h[r, j]) * lin'(h[r, H + j])).
 *   h [R, 2H] bf16 (read), a [R, H] bf16 (written); caller-owned, 16-byte aligned. fp32
 *   math in registers; the kernel needs no memory beyond its inputs and outputs, so `ws` may
 *   be NULL and moe_workspace_size reports 0 (the constant-size fp32 working set is the
 *   per-wave register tile, independent of R).
 * Errors: R < 0, H < 1, beta or linear_beta not > 0 (MOE_ERR_SHAPE); H % 8, misaligned
 * pointers (MOE_ERR_UNSUPPORTED); NULL h or a when R > 0 (MOE_ERR_NULL).
 */
moe_status situ_glu_fwd(const void* h, int64_t R, int H, float beta, float linear_beta,
                        void* a, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * situ_glu_bwd - dh = [da * lin' * dgate'/dg , da * gate' * dlin'/dl] with tanh and sigmoid
 * recomputed from h ("Streaming activations", custom op item 1).
 *   h [R, 2H] bf16, da [R, H] bf16, dh [R, 2H] bf16 out (may not alias h or da).
 */
moe_status situ_glu_bwd(const void* h, const void* da, int64_t R, int H, float beta,
                        float linear_beta, void* dh, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * moe_grouped_gemm_down_combine - o[r, :] = a[r, :] . w_down[e]^T for the rows of each
 * local expert, then y[t, :] = bf16( sum_j p_j o[slot_row[t, j], :] ) ("MoE 反向", forward
 * equation). o is a transient of this call, never kept: the fp32 rows p o live in `ws`, and
 * the combine adds them in fp32 in slot order, so each element of y is rounded to bf16 once.
 *   a [R_cap, H] bf16, row_gate [R_cap] fp32, slot_row [T, k], w_down [E_loc, d, H] bf16,
 *   y [T, d] bf16 out.
 *   ws: moe_workspace_size(MOE_WS_DOWN_COMBINE, ...) bytes (fp32 rows [R_cap, d]) runs one
 *   pass; a smaller ws (down to moe_workspace_size_passes with passes = d / 256) runs the
 *   GEMM and combine once per window of w output columns, w = the largest multiple of 256
 *   whose fp32 rows [R_cap, w] fit. Results are bit-identical for every ws size.
 * Errors: as moe_expert_bwd for the shared arguments; MOE_ERR_WORKSPACE below the minimum.
 */
moe_status moe_grouped_gemm_down_combine(const void* a, const int32_t* expert_offsets,
                                         const float* row_gate, const int32_t* slot_row,
                                         int64_t T, int k, int E_loc, int64_t R_cap, int H,
                                         int d, const void* w_down, void* y,
                                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_grouped_gemm_down_combine_noalloc - moe_grouped_gemm_down_combine for callers that
 * cannot allocate or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments without ws; the fp32 rows p o live in a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES held by each GPU the library runs on
 * until the process ends, and the combine runs in as many column windows as that requires
 * (results bit-identical to moe_grouped_gemm_down_combine). Nothing is allocated: the array's
 * device address is looked up once per device (hipGetSymbolAddress) on the first call.
 * Every call on one GPU shares its array, so calls that overlap on one GPU (other streams,
 * other threads) race; calls on one stream are ordered and safe. Nothing in the array needs
 * to start at zero: each pass writes every row the combine reads.
 * Errors: as moe_grouped_gemm_down_combine; R_cap * min(d, 256) * 4 > MOE_NOALLOC_SCRATCH_BYTES
 * (more rows than one 256-column window of the array holds: R_cap > 65536 for d >= 256)
 * returns MOE_ERR_WORKSPACE before any launch; a failed symbol lookup returns MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_grouped_gemm_down_combine_noalloc(const void* a, const int32_t* expert_offsets,
                                                 const float* row_gate,
                                                 const int32_t* slot_row, int64_t T, int k,
                                                 int E_loc, int64_t R_cap, int H, int d,
                                                 const void* w_down, void* y,
                                                 hipStream_t stream);

/*
 * moe_expert_bwd - backward of the expert layer with dL/dy = dy ("MoE 反向"):
 *   G      = dy[row_token] . w_down[e]                        (re-dispatch of dy fused)
 *   a      = SiTU-GLU(h) recomputed exactly as in the forward epilogue
 *   dp     = <G, a> per row        (dL/dp_e = <W_down^T dL/dy, a_e>; o_e is never used)
 *   dh     = SiTU-GLU'(h) applied to da = p G                 (bf16, transient in ws)
 *   dw_down[e] = sum_r (p_r dy_r) a_r^T                        fp32, overwritten
 *   dw_gu[e]   = sum_r dh_r x_r^T                              fp32, overwritten
 *   dx[t]  = bf16( sum_j (dh . w_gu[e])[slot_row[t, j]] )
 *   dp[t, j] = dp of row slot_row[t, j], 0 for non-local slots.
 * Experts with no rows get dw = 0.
 *   dy, x [T, d] bf16; h [R_cap, 2H] bf16 (saved by the forward); metadata from
 *   moe_permute; dx [T, d] bf16 out; dw_gu [E_loc, 2H, d] fp32 out; dw_down [E_loc, d, H]
 *   fp32 out; dp [T, k] fp32 out.
 *   ws: dh [R_cap, 2H] bf16 (rows 2H + 64 elements apart), the dp partials and an overlay of
 *   bf16(p a) [R_cap, H] with the fp32 dX rows. moe_workspace_size(MOE_WS_EXPERT_BWD, ...)
 *   bytes combine dx in one pass;
 *   a smaller ws (down to moe_workspace_size_passes with passes = d / 256) runs the dX GEMM
 *   and its combine once per window of output columns (bit-identical results).
 *   dx is summed in fp32 over a token's slots and rounded to bf16 once.
 * Errors: T < 0, k < 1, E_loc < 1, R_cap < 0, beta or linear_beta not > 0 (MOE_ERR_SHAPE);
 * k > 32, E_loc > 1024, d or H not a multiple of 64, R_cap >= 2^31, T * k >= 2^31,
 * T * max(d, 2H) * 2 >= 2^32, misaligned pointers (MOE_ERR_UNSUPPORTED); NULL pointers
 * (MOE_ERR_NULL); ws below the minimum (MOE_ERR_WORKSPACE).
 */
moe_status moe_expert_bwd(const void* dy, const void* x, const void* h,
                          const int32_t* row_token, const float* row_gate,
                          const int32_t* slot_row, const int32_t* expert_offsets,
                          int64_t T, int k, int E_loc, int64_t R_cap, int d, int H,
                          const void* w_gu, const void* w_down, float beta, float linear_beta,
                          void* dx, float* dw_gu, float* dw_down, float* dp,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Stages of the backward, in the order they run (moe_expert_bwd_stages). */
typedef enum {
  MOE_BWD_DA = 1,        /* dA GEMM + SiTU-GLU' + dp partials: writes dh, bf16(p a), partials */
  MOE_BWD_DW_DOWN = 2,   /* dw_down from dy and bf16(p a) */
  MOE_BWD_DW_GU = 4,     /* dw_gu from dh and x */
  MOE_BWD_DX = 8,        /* dX GEMM + combine into dx (reuses the memory of bf16(p a)) */
  MOE_BWD_DP = 16,       /* dp from the partials */
  MOE_BWD_ALL = 31
} moe_bwd_stage;

/*
 * moe_expert_bwd_stages - the stages of moe_expert_bwd selected by the bit mask `stages`,
 * run in the order of moe_bwd_stage. Calls over one backward must pass the same arguments and
 * `ws`; the workspace carries what MOE_BWD_DA writes to the later stages, so DA runs first,
 * and DW_DOWN runs before DX (DX reuses the memory DW_DOWN reads). Running the stages in any
 * grouping, in that order, gives results bit-identical to moe_expert_bwd; a caller may defer
 * the weight-gradient GEMMs or time each stage. The saved h is given either as bf16 `h` or as
 * MXFP8 `h_codes` and `h_scales` (the other form NULL).
 * Errors: as moe_expert_bwd; stages outside 1..MOE_BWD_ALL or both forms of h given
 * (MOE_ERR_SHAPE).
 */
moe_status moe_expert_bwd_stages(const void* dy, const void* x, const void* h,
                                 const void* h_codes, const void* h_scales,
                                 const int32_t* row_token, const float* row_gate,
                                 const int32_t* slot_row, const int32_t* expert_offsets,
                                 int64_t T, int k, int E_loc, int64_t R_cap, int d, int H,
                                 const void* w_gu, const void* w_down, float beta,
                                 float linear_beta, void* dx, float* dw_gu, float* dw_down,
                                 float* dp, void* ws, size_t ws_bytes, int stages,
                                 hipStream_t stream);

/*
 * MXFP8 storage of the saved pre-activation ("Kimi K3 ... Memory", unified activation
 * manager and ledger summary: most saved activations are kept block-wise in FP8, which
 * halves them again). Format (the pages do not fix one; read as OCP Microscaling v1.0
 * MXFP8): rows are cut into blocks of 32 consecutive elements; each block stores a scale
 * byte s = X + 127 with X = floor(log2(max |v|)) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block), and each element the E4M3 code of v / 2^X (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; round to nearest, ties to even; saturate to +-448; the sign is
 * kept when the magnitude rounds to zero). The value read back is E4M3(code) * 2^X.
 * A row of n elements takes n code bytes plus n/32 scale bytes.
 */

/*
 * moe_grouped_gemm_gate_up_mx - moe_grouped_gemm_gate_up with the saved h stored as MXFP8:
 *   h_codes [R_cap, 2H] uint8 out, h_scales [R_cap, 2H/32] uint8 out hold the MXFP8 form of
 *   the bf16 h that `a` is computed from; a [R_cap, H] bf16 out as in the bf16 call.
 * Same arguments, limits and errors otherwise; h_codes must be 16-byte aligned.
 */
moe_status moe_grouped_gemm_gate_up_mx(const void* x, int64_t T, const int32_t* row_token,
                                       const int32_t* expert_offsets, int E_loc, int64_t R_cap,
                                       int d, int H, const void* w_gu, float beta,
                                       float linear_beta, void* h_codes, void* h_scales,
                                       void* a, hipStream_t stream);

/*
 * moe_expert_bwd_mx - moe_expert_bwd reading the saved h from MXFP8 (h_codes [R_cap, 2H],
 * h_scales [R_cap, 2H/32], as written by moe_grouped_gemm_gate_up_mx): a, dp and dh are
 * recomputed from the stored value. Same workspace, outputs and errors as moe_expert_bwd.
 */
moe_status moe_expert_bwd_mx(const void* dy, const void* x, const void* h_codes,
                             const void* h_scales, const int32_t* row_token,
                             const float* row_gate, const int32_t* slot_row,
                             const int32_t* expert_offsets, int64_t T, int k, int E_loc,
                             int64_t R_cap, int d, int H, const void* w_gu, const void* w_down,
                             float beta, float linear_beta, void* dx, float* dw_gu,
                             float* dw_down, float* dp, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * moe_mxfp8_quantize - v [rows, n] bf16 -> codes [rows, n] uint8, scales [rows, n/32] uint8
 * in the format above. moe_mxfp8_dequantize - the inverse, out [rows, n] bf16 (exact for
 * values of magnitude >= 2^-126; E4M3 values carry 4 significant bits).
 * n must be a multiple of 32 (MOE_ERR_UNSUPPORTED otherwise); v, codes and out 16-byte
 * aligned; scales has no alignment requirement.
 */
moe_status moe_mxfp8_quantize(const void* v, int64_t rows, int n, void* codes, void* scales,
                              hipStream_t stream);
moe_status moe_mxfp8_dequantize(const void* codes, const void* scales, int64_t rows, int n,
                                void* out, hipStream_t stream);

/*
 * moe_router_bwd - gradient through the softmax over the kept logits: with p the gates and
 * g = dL/dp, dlogit_kept[t, j] = p_j (g_j - sum_i p_i g_i) (fp32). Logits that were not kept
 * do not reach the output. Only meaningful when all k routes of a token are local (or dp
 * has been summed over GPUs).
 *   gates, dp [T, k] fp32; dlogits_kept [T, k] fp32 out.
 */
moe_status moe_router_bwd(const float* gates, const float* dp, int64_t T, int k,
                          float* dlogits_kept, hipStream_t stream);

/*
 * W4A8 expert forward ("Frontier-scale RL with Kimi K3", section "Low precision (MXFP4)
 * rollouts": the rollout engine runs the MoE layers with 4-bit weights and 8-bit
 * activations; the explainer's "Idea Four": MXFP4 values in small blocks that share one
 * scale). Forward only. The pages fix no formats; this library reads them as OCP
 * Microscaling v1.0:
 *   - MXFP4 row of n elements: n/2 code bytes, E2M1 element 2j in the low nibble of byte j
 *     and 2j+1 in the high nibble (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7,
 *     sign in bit 3), plus n/32 scale bytes X + 127 (block of 32 scaled by 2^X,
 *     X = floor(log2(amax)) - 2 clamped to [-127, 127], -127 for an all-zero block).
 *     Elements round to nearest, ties to even, from v / 2^X and saturate to +-6.
 *   - MXFP8 activations: the format of moe_mxfp8_quantize (E4M3, X = floor(log2 amax) - 8).
 *   - Blocks run along the reduction dimension: x [T, d] and w_gu[e] [2H, d] along d;
 *     a [R, H] and w_down[e] [d, H] along H.
 * The products run on the block-scaled MFMA (fp32 accumulation; its per-block sums are not
 * round-to-nearest fp32 sums: results agree with an exact sum to about 2^-13 of the sum of
 * magnitudes at worst). d and H must be multiples of 128 (MOE_ERR_UNSUPPORTED otherwise).
 * Speed, not results: a GEMM whose reduction length (d for gate/up, H for down) is a multiple
 * of 512 and at most 3584, with both of its scale arrays 16-byte aligned, keeps its block
 * scales in LDS for a whole tile; other shapes and 4-byte aligned scales load them per stage.
 * Both forms give bit-identical results.
 */

/*
 * moe_mxfp4_quantize - v [rows, n] bf16 -> codes [rows, n/2] uint8, scales [rows, n/32]
 * uint8 in the MXFP4 format above. moe_mxfp4_dequantize - the inverse, out [rows, n] bf16
 * (exact: each value is an E2M1 value times a power of two). n must be a multiple of 32
 * (MOE_ERR_UNSUPPORTED otherwise); v and out 16-byte aligned, codes 4-byte aligned.
 */
moe_status moe_mxfp4_quantize(const void* v, int64_t rows, int n, void* codes, void* scales,
                              hipStream_t stream);
moe_status moe_mxfp4_dequantize(const void* codes, const void* scales, int64_t rows, int n,
                                void* out, hipStream_t stream);

/*
 * moe_grouped_gemm_gate_up_w4a8 - for every local expert e and its rows r, with x8 and w4
 * the values of the MXFP8 x and the MXFP4 w_gu:
 *   h[r, :]  = bf16( x8[row_token[r], :] . w4_gu[e]^T )       (not stored)
 *   a[r, j]  = bf16( SiTU-GLU(h[r, j], h[r, H + j]) ), j < H
 *   a_codes, a_scales = MXFP8 of a, blocks of 32 along H: the down GEMM's input.
 * The dispatch (row gather through row_token) is fused into the operand load.
 *   x_codes [T, d] uint8 and x_scales [T, d/32] uint8 (moe_mxfp8_quantize of x);
 *   row_token [R_cap], expert_offsets [E_loc+1] (device) from moe_permute;
 *   w_gu_codes [E_loc, 2H, d/2] and w_gu_scales [E_loc, 2H, d/32] (moe_mxfp4_quantize of
 *   w_gu viewed as [E_loc * 2H, d]); a_codes [R_cap, H] out, a_scales [R_cap, H/32] out.
 * Alignment: x_codes, w_gu_codes, a_codes 16 bytes; x_scales, w_gu_scales 4 bytes.
 * Errors: as moe_grouped_gemm_gate_up, plus T < 0, T * d >= 2^32.
 */
moe_status moe_grouped_gemm_gate_up_w4a8(const void* x_codes, const void* x_scales, int64_t T,
                                         const int32_t* row_token,
                                         const int32_t* expert_offsets, int E_loc,
                                         int64_t R_cap, int d, int H, const void* w_gu_codes,
                                         const void* w_gu_scales, float beta, float linear_beta,
                                         void* a_codes, void* a_scales, hipStream_t stream);

/*
 * moe_grouped_gemm_down_combine_w4a8 - moe_grouped_gemm_down_combine on W4A8 operands:
 * o[r, :] = a8[r, :] . w4_down[e]^T, y[t, :] = bf16( sum_j p_j o[slot_row[t, j], :] ).
 *   a_codes [R_cap, H], a_scales [R_cap, H/32] from moe_grouped_gemm_gate_up_w4a8;
 *   w_down_codes [E_loc, d, H/2], w_down_scales [E_loc, d, H/32] (moe_mxfp4_quantize of
 *   w_down viewed as [E_loc * d, H]); y [T, d] bf16 out; ws as for
 *   moe_grouped_gemm_down_combine (fp32 rows p o, one pass per window of output columns).
 * Alignment: a_codes, w_down_codes, y, ws 16 bytes; a_scales, w_down_scales 4 bytes.
 * Errors: as moe_grouped_gemm_down_combine.
 */
moe_status moe_grouped_gemm_down_combine_w4a8(const void* a_codes, const void* a_scales,
                                              const int32_t* expert_offsets,
                                              const float* row_gate, const int32_t* slot_row,
                                              int64_t T, int k, int E_loc, int64_t R_cap, int H,
                                              int d, const void* w_down_codes,
                                              const void* w_down_scales, void* y, void* ws,
                                              size_t ws_bytes, hipStream_t stream);

/*
 * moe_workspace_size - bytes of `ws` the entry point `which` needs for these sizes
 * (arguments that do not apply are ignored). Host-only; launches nothing.
 */
moe_status moe_workspace_size(int which, int64_t T, int E_loc, int k, int d, int H,
                              int64_t R_cap, size_t* bytes);

/*
 * moe_workspace_size_passes - bytes of `ws` for MOE_WS_DOWN_COMBINE (also the W4A8 down
 * combine) or MOE_WS_EXPERT_BWD (also the MXFP8-store backward) when the combine is to run in
 * `passes` passes over the output columns: windows of w = ceil(d / passes) rounded up to a
 * multiple of 256 (at most d) columns. passes = 1 equals moe_workspace_size; fewer bytes per
 * pass trade fp32 row memory for re-reading the GEMM's row operand once per pass.
 * Errors: passes < 1 or another `which` (MOE_ERR_SHAPE); as moe_workspace_size otherwise.
 */
moe_status moe_workspace_size_passes(int which, int64_t T, int E_loc, int k, int d, int H,
                                     int64_t R_cap, int passes, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
