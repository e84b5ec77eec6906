/*
 * moe_fp8.h -- C ABI of libmoe_fp8.so: the forward pass of one DeepSeekMoE
 * layer on an AMD Instinct MI355X (gfx950), FP8 E4M3 with fine-grained scales.
 *
 * Pages cited (by title and section):
 *   [VE] "DeepSeek-V3, explained." (vibeengines.com): numbered recipe steps
 *        3 (MoE shape), 4 (sigmoid routing with a bias), 5 (no token dropped),
 *        7 (FP8 with 1x128 / 128x128 scales) and the symbol glossary.
 *   [TP] "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
 *        Prediction, and FP8 Training at 671B Scale" (trishampatil.com):
 *        section III (affinity, selection and gate equations; bias thermostat
 *        and its flowchart), section V (FP8: Figure 6, details 1-4).
 *   [DF] "DeepSeek-V3 Technical Report" (deepforge.srivtx.xyz): part 1
 *        "Per-tile FP8 scaling" (scale = 448 / amax, E4M3 rounding).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers on the current HIP device, owned by the
 *     caller, and must stay valid until the work on `stream` completes.  The
 *     library never allocates, never synchronises the host and keeps no
 *     pointer after returning.
 *   - Matrices are row-major.  Both GEMM operands are K-contiguous.  FP8 values
 *     are raw OCP E4M3 ("fn", max 448) byte codes.  bf16 values are raw 16-bit
 *     patterns.  Scales are stored as dequantisation factors d = amax / 448.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *   - Return value: MOE_OK, or an error code.  On any code other than
 *     MOE_ERR_HIP nothing was enqueued.  MOE_ERR_HIP means a HIP launch failed;
 *     moe_last_hip_error() returns the hipError_t of that failure.
 *   - Sizes of zero tokens / rows are valid and enqueue nothing.
 *   - Inputs must be finite; with non-finite inputs output values are
 *     unspecified but every access stays in bounds.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                       */
  MOE_ERR_SHAPE = 2,       /* a size is negative or violates a divisibility rule */
  MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                 */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or too small                   */
  MOE_ERR_DEVICE = 5,      /* the current device is not gfx950                 */
  MOE_ERR_UNSUPPORTED = 6, /* a valid but unsupported combination of arguments */
  MOE_ERR_HIP = 7          /* a HIP call failed; see moe_last_hip_error()      */
} moe_status_t;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype_t;

/* Grouped GEMM epilogues. */
typedef enum {
  MOE_EPI_BF16 = 0,       /* out: bf16 [total_rows, n_out], row stride ldo elements */
  MOE_EPI_SWIGLU_FP8 = 1, /* out: E4M3 [total_rows, n_out/2] (ldo bytes per row),
                             out_d: float [total_rows, n_out/256]                 */
  MOE_EPI_F32 = 2         /* out: float [total_rows, n_out], row stride ldo       */
} moe_epilogue_t;

/*
 * Router and biased top-k ([TP] section III affinity, selection and gate
 * equations; [VE] recipe step 4):
 *   s[t,i]   = sigmoid(sum_h x[t,h] * Wr[i,h])       (bf16 inputs, fp32 math)
 *   chosen   = the k experts with the largest fl32(s[t,i] + bias[i]),
 *              ties to the lower expert index, listed in that order
 *   gate[t,j]= s[t,idx[t,j]] / sum_j' s[t,idx[t,j']]  (the bias never enters)
 * Group-limited selection ([VE] recipe step 5; [DF] "Balancing without a
 * balance loss"; [TP] section V "Custom all-to-all kernels"), on when
 * n_groups > 1: the N experts form n_groups groups of N / n_groups
 * consecutive indices (one per node); a group's score is the float32 sum of
 * its k / topk_groups largest biased keys, added in descending order; only the
 * topk_groups best groups (score descending, group index ascending) are
 * eligible, and the k experts are the best keys among them.  n_groups <= 1
 * turns it off.  Otherwise requires n_groups <= 64, N % n_groups == 0,
 * 1 <= topk_groups <= n_groups, k % topk_groups == 0 and
 * k / topk_groups <= N / n_groups (MOE_ERR_SHAPE).
 * x_bf16 [T,H], w_router_bf16 [N,H] (row i is expert i's centroid), bias [N]
 * float.  scores [T,N] float is written when non-NULL.  topk_idx int32 [T,k],
 * topk_gate float [T,k].  The sum over h is split into slices whose float
 * partial sums are added in slice order (deterministic); ws is device scratch
 * of at least moe_route_workspace_bytes(T, H, N) bytes, 16-byte aligned
 * (MOE_ERR_WORKSPACE otherwise).
 * Requires H % 128 == 0, 16 <= N <= 256, N % 16 == 0, 1 <= k <= min(N, 32),
 * T * H * 2 < 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 */
size_t moe_route_workspace_bytes(int T, int H, int N);
moe_status_t moe_route_topk(const void* x_bf16, const void* w_router_bf16, const float* bias,
                            int T, int H, int N, int k, int n_groups, int topk_groups,
                            float* scores, int32_t* topk_idx, float* topk_gate, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * moe_route_topk plus the 1x128 activation quantisation of x ([TP] section
 * V, FP8 detail 1 and Figure 6; [DF] part 1, "Per-tile FP8 scaling"), taken
 * from the same read of x: the scores, top_idx and topk_gate of
 * moe_route_topk, and x_q uint8 [T,H] (dense, E4M3 codes) with x_d float
 * [T,H/128], equal bit for bit to fp8_quant_1x128(x_bf16, MOE_BF16, T, H, H,
 * x_q, x_d).  Same arguments, workspace, limits and errors as moe_route_topk;
 * x_q (16-byte aligned) and x_d (4-byte aligned) must not be NULL when
 * T > 0 (MOE_ERR_NULL) and must not overlap x or the workspace.
 */
moe_status_t moe_route_topk_quant_x(const void* x_bf16, const void* w_router_bf16,
                                    const float* bias, int T, int H, int N, int k, int n_groups,
                                    int topk_groups, float* scores, int32_t* topk_idx,
                                    float* topk_gate, uint8_t* x_q, float* x_d, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/*
 * Opt-in FP8 router: the same scores, selection and gates as moe_route_topk,
 * but the logits come from block-scaled FP8 operands (the product of [TP]
 * section V, FP8 details 1-2, applied to the gating GEMM, which detail 4
 * keeps in higher precision; hence opt-in, and its routing can differ from
 * the bf16 router's on tokens whose k-th and (k+1)-th keys are close):
 *   z[t,i] = sum_c d_x[t,c] * d_W[i/128,c] * sum_{h in block c} q_x[t,h] q_W[i,h]
 * x_q E4M3 [T,H] with x_d float [T,H/128] (fp8_quant_1x128 output);
 * w_router_q E4M3 [N,H] with w_router_d float [N/128,H/128]
 * (fp8_quant_128x128 output).  Each block product is formed by the MFMA in
 * float and scaled with one FMA; blocks are added in order within an H slice
 * and the slices in slice order.  ws as for moe_route_topk (the same size
 * suffices).  Requires H % 128 == 0, N % 128 == 0, 128 <= N <= 256,
 * 1 <= k <= min(N, 32), T * H < 2^31 (MOE_ERR_UNSUPPORTED otherwise); x_q,
 * w_router_q and ws 16-byte aligned, the scale arrays 4-byte aligned.
 */
moe_status_t moe_route_topk_fp8(const uint8_t* x_q, const float* x_d, const uint8_t* w_router_q,
                                const float* w_router_d, const float* bias, int T, int H, int N,
                                int k, int n_groups, int topk_groups, float* scores,
                                int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * The selection and gate steps alone, from a given float score tensor
 * scores [T,N] (same definitions as moe_route_topk, group-limited selection
 * included).  Requires 1 <= N <= 1024, 1 <= k <= min(N, 32).
 */
moe_status_t moe_topk_from_scores(const float* scores, const float* bias, int T, int N, int k,
                                  int n_groups, int topk_groups, int32_t* topk_idx,
                                  float* topk_gate, hipStream_t stream);

/*
 * Per-expert token counts and the token permutation.  Every (token, slot)
 * assignment gets a row; nothing is dropped ([VE] recipe step 5).  The counts
 * feed the bias update ([TP] section III flowchart, "token counts").
 *   counts[e]     = #{(t,j): idx[t,j] = e}                       int32 [N]
 *   offsets[e]    = sum_{e'<e} counts[e'], offsets[N] = T*k,
 *                   offsets[N+1] = T*k + T if with_shared else T*k   int32 [N+2]
 *   row_of[t,j]   = offsets[e] + rank of (t,j) among the assignments of e in
 *                   (token, slot) order                            int32 [T,k]
 *   token_of[row] = token of that row; with_shared appends group N with rows
 *                   T*k + t -> t                          int32 [T*k (+T)]
 * Deterministic (no atomics decide any order).  idx entries must lie in
 * [0, N) (entries outside are clamped into range).  ws: device scratch of at
 * least moe_permute_workspace_bytes(T, N, k) bytes.
 * Requires 1 <= N <= 1024, 1 <= k <= 32.
 */
size_t moe_permute_workspace_bytes(int T, int N, int k);
moe_status_t moe_permute(const int32_t* topk_idx, int T, int N, int k, int with_shared,
                         int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_permute without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as moe_permute
 * minus ws/ws_bytes.  Its scratch (the per-block counts of the counting sort,
 * moe_permute_workspace_bytes(T, N, k) bytes) lives in a device array of the
 * library of moe_permute_noalloc_max_scratch_bytes() bytes (1 MiB), which
 * each GPU the library runs on holds until the process ends; larger problems
 * (e.g. T > 65536 at N = 1024, T > 262144 at N = 256) return
 * MOE_ERR_UNSUPPORTED and enqueue nothing.  The call allocates nothing; every
 * call on one GPU shares that GPU's array, so calls that may overlap on one
 * GPU (on different streams, or from different threads) race and must be
 * ordered by the caller.  Nothing in the array needs clearing between calls.
 */
size_t moe_permute_noalloc_max_scratch_bytes(void);
moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int N, int k, int with_shared,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of,
                                 int32_t* token_of, hipStream_t stream);

/*
 * 1x128 activation quantiser ([TP] section V FP8 detail 1; [DF] "Per-tile FP8
 * scaling").  For each row r and 128-column tile j of x [rows, cols] (row
 * stride ld elements, dtype dt):
 *   amax = max |x|;  m = fl32(448 / amax);  d[r,j] = fl32(amax / 448);
 *   q[r,c] = E4M3_RNE_saturating(fl32(x[r,c] * m))    (sign kept)
 * A tile with amax == 0, or whose m overflows, stores 0x00 codes and d = 1.
 * q uint8 [rows, cols] (dense), d float [rows, cols/128].
 * Requires cols % 128 == 0, ld >= cols, ld % 8 == 0.
 */
moe_status_t fp8_quant_1x128(const void* x, moe_dtype_t dt, int rows, int cols, int ld,
                             uint8_t* q, float* d, hipStream_t stream);

/*
 * 128x128 weight quantiser (same rule per 128x128 block; [VE] recipe step 7).
 * w_bf16 [batch, rows, cols] -> q uint8 [batch, rows, cols],
 * d float [batch, rows/128, cols/128].  With interleave_gate_up (for
 * W1 = [W_gate; W_up], rows = 2I) the output row blocks are reordered so that
 * output block 2j is gate block j and output block 2j+1 is up block j (d
 * follows the same order).  Requires rows % 128 == 0, cols % 128 == 0, and
 * rows % 256 == 0 with interleave_gate_up.
 */
moe_status_t fp8_quant_128x128(const void* w_bf16, int batch, int rows, int cols,
                               int interleave_gate_up, uint8_t* q, float* d, hipStream_t stream);

/*
 * Grouped block-scaled FP8 GEMM ([TP] section V Figure 6: FP8 inputs, FP32
 * accumulation, BF16 output; FP8 detail 2: the scales change every 128
 * elements of K, so each 128-deep block's product is scaled on its own):
 *   C[r,c] = sum_kb (sum_{h in kb} A[src(r),h] B[g,c,h]) * a_d[src(r),kb] * b_d[g,c/128,kb]
 * for every row r of group g, i.e. group_offsets[g] <= r < group_offsets[g+1].
 * src(r) = a_row_index[r] when a_row_index is non-NULL (fused gather), else r.
 * Epilogues:
 *   MOE_EPI_BF16        out[r,c] = bf16(C[r,c] * (row_scale ? row_scale[r] : 1))
 *   MOE_EPI_F32         out[r,c] = C[r,c]
 *   MOE_EPI_SWIGLU_FP8  B holds W1 with gate/up 128-row blocks interleaved
 *                       (fp8_quant_128x128 with interleave_gate_up); for h
 *                       column c' = 128 j + i:  h = SiLU(C[r, 256j+i]) * C[r, 256j+128+i]
 *                       in float, then 1x128-quantised as fp8_quant_1x128 does:
 *                       out (E4M3) [r, c'], out_d [r, j].
 * a_q [a_rows, lda] (lda >= k_dim bytes), a_d [a_rows, k_dim/128]; b_q [G, n_out, k_dim],
 * b_d [G, n_out/128, k_dim/128]; group_offsets int32 [G+1] on the device,
 * non-decreasing, group_offsets[0] = 0, group_offsets[G] = total_rows (values
 * outside [0, total_rows] are clamped).  1 <= num_groups <= 1025, k_dim <= 16384,
 * a_rows * lda < 2^31, and with MOE_EPI_BF16 ldo <= 2^22 (MOE_ERR_UNSUPPORTED
 * otherwise).
 * Requires k_dim % 128 == 0, n_out % 128 == 0 (% 256 with MOE_EPI_SWIGLU_FP8),
 * lda % 16 == 0, ldo % 8 == 0 elements (% 16 bytes for SWIGLU_FP8), 16-byte
 * aligned a_q, b_q and out.
 */
typedef struct {
  const uint8_t* a_q;
  const float* a_d;
  int lda;
  int a_rows;                   /* rows of a_q / a_d; gathered indices are clamped to it */
  const int32_t* a_row_index;
  const uint8_t* b_q;
  const float* b_d;
  const int32_t* group_offsets;
  int num_groups;
  int total_rows;
  int n_out;
  int k_dim;
  int epilogue;
  void* out;
  float* out_d;
  int ldo;
  const float* row_scale;
} moe_gemm_fp8_args;

moe_status_t moe_grouped_gemm_fp8(const moe_gemm_fp8_args* args, hipStream_t stream);

/*
 * The same product with the row tile chosen by the caller (same passages as
 * above; the result does not depend on the tile: every output is the same
 * sequence of per-block products and fused multiply-adds).  tile_rows:
 *   0    as moe_grouped_gemm_fp8: 256-row tiles when total_rows >= 128 *
 *        num_groups for MOE_EPI_SWIGLU_FP8, and for MOE_EPI_BF16 when also
 *        n_out % 256 == 0 and ldo <= 2^21; else 128-row tiles;
 *   128  128-row tiles (every epilogue);
 *   256  256-row tiles (MOE_EPI_SWIGLU_FP8; MOE_EPI_BF16 with n_out % 256 == 0
 *        and ldo <= 2^21).
 * Any other value, or 256 where it is not allowed, returns
 * MOE_ERR_UNSUPPORTED before anything is launched.  Arguments, layouts and the other errors are
 * those of moe_grouped_gemm_fp8.
 */
moe_status_t moe_grouped_gemm_fp8_tiles(const moe_gemm_fp8_args* args, int tile_rows,
                                        hipStream_t stream);

/*
 * Gate-weighted combine ([VE] glossary: routed weights sum to 1 and the shared
 * expert is added at full weight; [TP] Figure 2, outputs "summed into the
 * block output"):
 *   y[t,:] = bf16( residual[t,:] (if non-NULL) + out[shared_row0 + t,:]
 *                  + sum_{j=0..k-1} gate[t,j] * out[row_of[t,j],:] )
 * accumulated in float, in that order, one fused multiply-add per slot.
 * shared_row0 < 0 means no shared expert.  out_rows_bf16 [*, H],
 * gate float [T,k], row_of int32 [T,k], residual/y bf16 [T,H].
 * Requires H % 8 == 0.
 */
moe_status_t moe_combine(const void* out_rows_bf16, const float* gate, const int32_t* row_of,
                         int shared_row0, int T, int H, int k, const void* residual_bf16,
                         void* y_bf16, hipStream_t stream);

/*
 * Sign-based bias update ([TP] section III, "How the bias is set"; [VE]
 * recipe step 4): target = T*k/N; overloaded (N*c > T*k) -> b -= gamma,
 * underloaded (N*c < T*k) -> b += gamma, on target -> unchanged; one float
 * add of fl32(gamma).  bias float [N] updated in place, counts int32 [N].
 */
moe_status_t moe_bias_update(float* bias, const int32_t* counts, int N, int T, int k, float gamma,
                             hipStream_t stream);

/*
 * Sequence-wise balance statistic ([TP] section III, "The one small loss that
 * remains"; [VE] recipe step 4): for each sequence s (tokens seq_offsets[s] ..
 * seq_offsets[s+1]-1, T_s of them, clamped into [0, T]),
 *   loss[s] = alpha * sum_i f_i P_i,  f_i = N / (k T_s) * #{(t,j): idx = i},
 *   P_i = (1 / T_s) * sum of the gates expert i received;
 * 0 for an empty sequence.  topk_idx int32 [T,k] and topk_gate float [T,k] as
 * moe_route_topk writes them (idx entries outside [0, N) are clamped),
 * seq_offsets int32 [n_seq + 1] device, loss float [n_seq].  Gates are summed
 * in units of 2^-32 and the result is formed in double, so it is
 * deterministic.  Requires 1 <= N <= 1024, 1 <= k <= 32.
 */
moe_status_t moe_seq_balance_loss(const int32_t* topk_idx, const float* topk_gate,
                                  const int32_t* seq_offsets, int n_seq, int T, int N, int k,
                                  float alpha, float* loss, hipStream_t stream);

/*
 * FP8 backward GEMMs of a linear layer Y = X W^T ([TP] section V, Figure 6:
 * the input-gradient and weight-gradient GEMMs also take FP8 inputs and
 * accumulate in FP32; detail 3: E4M3 on every tensor; detail 4 and [DF] part 1
 * "FP8 training, from first principles": gradients kept in higher precision).
 *
 * Dgrad, dX = dY W, is moe_grouped_gemm_fp8 with a_q/a_d = fp8_quant_1x128 of
 * dY (tokens x output channels, grouped like the forward rows) and b_q/b_d =
 * the transposed weight codes and scales written by fp8_transpose_128x128.
 *
 * fp8_transpose_128x128: exact transpose of 128x128 block-quantised weights,
 * w_q E4M3 [batch, rows, cols] with w_d float [batch, rows/128, cols/128] ->
 * wt_q [batch, cols, rows], wt_d [batch, cols/128, rows/128] (a block's codes
 * transposed, its scale unchanged).  Requires rows % 128 == 0,
 * cols % 128 == 0; code pointers 16-byte aligned.
 */
moe_status_t fp8_transpose_128x128(const uint8_t* w_q, const float* w_d, int batch, int rows,
                                   int cols, uint8_t* wt_q, float* wt_d, hipStream_t stream);

/*
 * Token-tile quantiser for Wgrad (the contraction runs over tokens, so each
 * operand gets one scale per 128 consecutive tokens of one channel; a tile
 * never spans two experts).  x [rows, cols] (bf16 or float, row stride ldx
 * elements) in expert-grouped row order, group g = rows group_offsets[g] ..
 * group_offsets[g+1]-1 (device int32 [num_groups + 1], clamped into
 * [0, rows]).  Writes pad_offsets int32 [num_groups + 1] (group g's first
 * padded token column, P_g = sum over earlier groups of 128 * ceil(rows_g /
 * 128); pad_offsets[G] = the padded length) and, transposed, xt_q E4M3
 * [cols, ldt] (column P_g + j of channel c = token group_offsets[g] + j) and
 * xt_d float [cols, ldt/128].  A group's last tile covers its remaining
 * tokens only: its amax is over them and the other positions are code 0.
 * Per tile: m = fl32(448/amax), d = fl32(amax/448), code = E4M3(x*m) (zero
 * tile: codes 0, d = 1).  Columns past pad_offsets[G] are not written.
 * Requires cols % 64 == 0, ldt % 128 == 0, ldt >= rows + 127 * num_groups,
 * 1 <= num_groups <= 1025, ceil(rows/128) + num_groups <= 65535
 * (MOE_ERR_UNSUPPORTED otherwise); x and xt_q 16-byte aligned.
 */
moe_status_t fp8_quant_tokens_128(const void* x, moe_dtype_t dtype, int rows, int cols,
                                  long long ldx, const int32_t* group_offsets, int num_groups,
                                  uint8_t* xt_q, float* xt_d, long long ldt, int32_t* pad_offsets,
                                  hipStream_t stream);

/*
 * Wgrad grouped GEMM: for every expert g,
 *   out[g][n][k] = sum over the 128-token tiles c of group g of
 *                  d_A[n, c] d_B[k, c] sum_{j in c} q_A[n, j] q_B[k, j]
 * i.e. dW_g = dY_g^T X_g from the token-tile operands of
 * fp8_quant_tokens_128: a_q [n_rows, lda] / a_d [n_rows, lda/128] (dY^T),
 * b_q [k_rows, ldb] / b_d [k_rows, ldb/128] (X^T), pad_offsets int32
 * [num_groups + 1] (device, multiples of 128, clamped to the operands'
 * width).  out float [num_groups, n_rows, k_rows]; an empty expert gets zeros.
 * Each tile product comes from the FP8 MFMA in float and is scaled and added
 * with float multiplies and fused multiply-adds, tiles in token order.
 * Requires n_rows % 128 == 0, k_rows % 128 == 0, lda and ldb multiples of 128,
 * n_rows * lda < 2^31 and k_rows * ldb < 2^31 (MOE_ERR_UNSUPPORTED); code
 * pointers and out 16-byte aligned.
 */
moe_status_t moe_grouped_wgrad_fp8(const uint8_t* a_q, const float* a_d, long long lda,
                                   int n_rows, const uint8_t* b_q, const float* b_d,
                                   long long ldb, int k_rows, const int32_t* pad_offsets,
                                   int num_groups, float* out, hipStream_t stream);

/*
 * Diagnostic, not a step of the layer: the attainable rate of the FP8 matrix
 * instruction the grouped GEMMs use (v_mfma_f32_16x16x128_f8f6f4), so that a
 * GEMM's throughput can be stated against a measured peak beside the published
 * one.  Enqueues `blocks` workgroups of 4 waves; every wave issues
 * iters * 16 of these MFMAs (16 independent accumulators, no memory traffic
 * in the loop), i.e. blocks * 4 * iters * 16 * 65536 flops in all, and writes
 * blocks * 256 floats to `sink` (device, caller-owned).  The caller times it
 * (events on `stream`).  1 <= blocks <= 2^20, iters >= 1 (MOE_ERR_SHAPE).
 */
moe_status_t moe_probe_fp8_mfma(int blocks, int iters, float* sink, hipStream_t stream);

/*
 * Diagnostic, not a step of the layer: the attainable HBM read and write
 * rates, so that each bandwidth-bound step can be stated against what the
 * device delivers for its own mix of reads and writes as well as against the
 * published peak.  Modes 0 and 2 read all `bytes` of `buf` with 16-byte
 * loads (0: eight non-temporal loads in flight per lane; 2: four ordinary
 * ones) and XOR-fold them into *sink (device, caller-owned, one unsigned);
 * modes 1 and 3 write all `bytes` of `buf` with 16-byte stores (1:
 * non-temporal; 3: ordinary; sink unused, may be NULL).  The caller times it
 * (events on `stream`) and takes the faster mode of each kind.  Requires
 * 0 <= mode <= 3 and bytes % 16 == 0 (MOE_ERR_SHAPE), buf 16-byte aligned
 * (MOE_ERR_ALIGN), buf non-NULL and, for the read modes, sink non-NULL
 * (MOE_ERR_NULL).
 */
moe_status_t moe_probe_hbm(int mode, void* buf, size_t bytes, unsigned* sink, hipStream_t stream);

/*
 * The whole forward pass of one layer in one call ([TP] section III flowchart
 * and Figure 2; [VE] recipe steps 4-7), enqueued on `stream` in this order:
 *   FP8 router only: fp8_quant_1x128(x) ahead of the routing;
 *   moe_route_topk (or moe_route_topk_fp8 when router_fp8) -> idx, gate;
 *   moe_permute (counts, offsets, row_of, token_of; with_shared appends the
 *     shared expert as group N);
 *   bf16 router: fp8_quant_1x128(x);
 *   moe_grouped_gemm_fp8 with MOE_EPI_SWIGLU_FP8 over the G = N (+1) groups,
 *     A = the quantised x gathered through token_of, B = W1 -> h codes/scales;
 *   moe_grouped_gemm_fp8 with MOE_EPI_BF16, A = h, B = W2 -> expert rows;
 *   moe_combine (shared row T*k + t when with_shared) -> y;
 *   moe_bias_update(bias, counts) when update_bias.
 * Each step computes exactly what its own entry point computes, so the
 * results are bit-identical to calling the steps one by one.
 * Operands (device pointers; shapes with R = T*k + (with_shared ? T : 0)):
 *   x bf16 [T,H]; w_router bf16 [N,H] (bf16 router) or w_router_q E4M3 [N,H]
 *   with w_router_d float [N/128,H/128] (router_fp8); bias float [N], updated
 *   in place when update_bias; w1_q E4M3 [G,2I,H] gate/up interleaved with
 *   w1_d float [G,2I/128,H/128] (fp8_quant_128x128 with interleave_gate_up);
 *   w2_q E4M3 [G,H,I] with w2_d float [G,H/128,I/128]; residual bf16 [T,H]
 *   or NULL; y bf16 [T,H] (written).  Optional outputs, each NULL to skip:
 *   scores float [T,N], topk_idx int32 [T,k], topk_gate float [T,k],
 *   counts int32 [N] (when NULL these live in the workspace).
 * ws: device scratch of at least moe_layer_workspace_bytes(T, H, N, k, I,
 * with_shared) bytes, 256-byte aligned (MOE_ERR_WORKSPACE / MOE_ERR_ALIGN);
 * it holds every intermediate (about R * (H * 2 + I + I / 32) + T * H bytes),
 * so the call allocates nothing and may be captured in a HIP graph.  Calls
 * that share a workspace must be ordered on one stream.
 * Requires H % 128 == 0, I % 128 == 0, H, I <= 16384, 16 <= N <= 256,
 * N % 16 == 0 (N % 128 == 0 and N >= 128 with router_fp8), 1 <= k <= min(N, 32),
 * the group conditions of moe_route_topk (MOE_ERR_SHAPE); T * H * 2 and R * I
 * below 2^31 (MOE_ERR_UNSUPPORTED; at the DeepSeek-V3 shape, T up to 116508
 * tokens).  Every check runs before the
 * first launch.
 */
typedef struct {
  const void* x;
  const void* w_router;
  const uint8_t* w_router_q;
  const float* w_router_d;
  float* bias;
  const uint8_t* w1_q;
  const float* w1_d;
  const uint8_t* w2_q;
  const float* w2_d;
  int T, H, N, k, I;
  int with_shared;              /* nonzero: expert N is the shared expert */
  int n_groups, topk_groups;    /* group-limited selection when n_groups > 1 */
  int router_fp8;               /* nonzero: the opt-in FP8 router */
  int update_bias;              /* nonzero: sign update of bias after combine */
  float gamma;                  /* bias update speed */
  const void* residual;
  void* y;
  float* scores;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
} moe_layer_args;

size_t moe_layer_workspace_bytes(int T, int H, int N, int k, int I, int with_shared);
moe_status_t moe_layer_forward(const moe_layer_args* args, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status_t status);
/* hipError_t of the most recent MOE_ERR_HIP on this thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
