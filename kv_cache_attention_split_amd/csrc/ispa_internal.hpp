// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP kernel files.
// Nothing here is part of the public ABI (include/ispa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace ispa {

// ------------------------------------------------------------------------------------------------
// Attention
// ------------------------------------------------------------------------------------------------
struct AttnArgs {
  const void *q;
  int64_t q_stride;                 // elements between query tokens
  const void *sink_k, *sink_v;
  int64_t sink_n, sink_stride;
  const void *cur_k, *cur_v;
  int64_t cur_n, cur_stride;
  const void *hist_k, *hist_v;
  int64_t hist_n, hist_stride;      // hist_n is 0 when only the local branch is wanted
  void *a_loc, *a_full;
  float *lse_loc, *lse_hist, *lse_full;
  int32_t n_q, n_heads;
  float scale_log2;                 // softmax_scale * log2(e)
  // Optional per-key additive logit bias, natural-log units, one pointer per segment (NULL = zero):
  // key j of segment S in head h gets S_b[h * S_bhs + j]. bias_to_score = 1 / softmax_scale
  // turns it into raw-score units, so that (q.k + b / tau) * tau = tau q.k + b.
  const float *sink_b, *cur_b, *hist_b;
  int64_t sink_bhs, cur_bhs, hist_bhs;
  float bias_to_score;
  // FP8 scores: q and the keys as OCP e4m3 bytes with one scale per head each (device [H])
  const float *q_scale, *k_scale;
  // FP8 value product (with FP8 scores): the values as e4m3 bytes with one scale per head (device [H]);
  // NULL = bf16 values
  const float *v_scale;
  // log-sum-exp-only form: the keys are split into lse_splits ranges per (head, query tile); each writes
  // its (running max in log2 units, exp-sum) to lse_part[(split * n_heads + head) * n_q + query]
  float *lse_part;
  int lse_splits;
  // balanced schedule (launch_attn_bf16_balanced): per-segment state slots and per-unit counters
  float *split_ws;
  int *split_count;
};

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t s);
// Balanced schedule of the bf16 head_dim-128 kernel (no bias): `grid` workgroups share the tiles of
// all (head, query tile) units equally; cut units merge their segments' partial states through `ws`
// (attn_balanced_ws_bytes bytes, 256-byte aligned). attn_balanced_grid gives 0 where the plain launch
// already fills the compute units (then no workspace is needed).
int attn_balanced_grid(int64_t n_q, int n_heads, int64_t n_keys_loc, int64_t n_keys_hist, int cus);
size_t attn_balanced_ws_bytes(int64_t n_q, int n_heads, int grid);
hipError_t launch_attn_bf16_balanced(const AttnArgs &a, int head_dim, int grid, void *ws, hipStream_t s);
// Log-sum-exp rows only (a.a_loc and a.a_full must be NULL, no bias): no value copies or products.
// For head_dim 128 the keys are split over lse_splits_for(n_q, n_heads) workgroups per query tile and
// a.lse_part must hold that many [n_heads, n_q] float2 partial states; a.lse_full receives the merge.
int lse_splits_for(int64_t n_q, int n_heads);
hipError_t launch_attn_lse_bf16(const AttnArgs &a, int head_dim, hipStream_t s);
// Future-query importance: score[h][j] = (1/n_p) sum_i exp(tau q_i . k_j - lse[h][i]) over the keys
// of three segments in cache order (bf16 keys and proxies, head_dim 64 or 128).
hipError_t launch_future_colsum_bf16(const uint16_t *q, int64_t q_stride, int64_t n_p, const float *lse,
                                     const uint16_t *k0, int64_t s0, int64_t n0, const uint16_t *k1,
                                     int64_t s1, int64_t n1, const uint16_t *k2, int64_t s2, int64_t n2,
                                     int n_heads, int head_dim, float scale_log2, float *scores,
                                     int64_t scores_hs, hipStream_t s);
hipError_t launch_token_scores(const float *scores, int64_t hs, int n_heads, int64_t n, float lambda,
                               const float *hist, float *token, hipStream_t s);
// TempCache merge: per group, mean key and value rows (fp32 sums in member order) and ln(count).
hipError_t launch_kv_merge(bool bf16, int width, const void *k, const void *v, int64_t n, int64_t in_stride,
                           const int32_t *offsets, const int32_t *members, int64_t n_groups, void *k_out,
                           void *v_out, int64_t out_stride, float *bias_out, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, int head_dim, hipStream_t s);
// e4m3 q and keys (scores on the FP8 matrix cores), bf16 values and outputs; head_dim 128.
hipError_t launch_attn_fp8(const AttnArgs &a, int head_dim, hipStream_t s);
// Per-head absmax / 448 of [n, H, d] rows (bf16 or fp32); quantisation to e4m3 with per-head scales.
hipError_t launch_fp8_head_scales(bool bf16, const void *x, int64_t n, int n_heads, int head_dim, int64_t stride,
                                  float *scales, hipStream_t s);
hipError_t launch_fp8_quantize(bool bf16, const void *x, int64_t n, int n_heads, int head_dim, int64_t stride,
                               const float *scales, uint8_t *out, int64_t out_stride, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Gram accumulation (bf16 rows, fp32 sums)
// ------------------------------------------------------------------------------------------------
hipError_t launch_gram_bf16(int64_t n_rows, int d, const uint16_t *a_loc, const uint16_t *a_full,
                            float *G, float *X, float *F, hipStream_t s);
// The same for `batch` layers with the same n_rows and d (per-layer pointers; F NULL for none): one
// launch per 48 layers, 256 x 256 tiles when the launch has enough of them, else 128 x 128.
hipError_t launch_gram_bf16_batch(int64_t n_rows, int d, int batch, const uint16_t *const *a_loc,
                                  const uint16_t *const *a_full, float *const *G, float *const *X,
                                  float *const *F, hipStream_t s);
// e4m3 rows [n, d] with per-head scales (d / head_dim of each); same sums of the dequantised rows.
hipError_t launch_gram_fp8(int64_t n_rows, int d, int head_dim, const uint8_t *a_loc, const float *s_loc,
                           const uint8_t *a_full, const float *s_full, float *G, float *X, float *F, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// fp32 batched GEMM on MFMA:  C[i][j] = alpha * sum_k opA[i][k] opB[k][j] + beta * C[i][j]
//   ta = 0: opA[i][k] = A[i*lda + k]        ta = 1: opA[i][k] = A[k*lda + i]
//   tb = 0: opB[k][j] = B[k*ldb + j]        tb = 1: opB[k][j] = B[j*ldb + k]
//   a2 != NULL (ta = 0 only): opA = A - A2 elementwise (same lda)
//   lower: skip 128x128 output tiles lying strictly above the diagonal (col0 > row0 + 127)
//   dot mode (E != NULL): instead of storing C, write per-tile partial sums
//     sum_{tile} E[i*lde + j] * (alpha * (AB)[i][j]) in fp64 to part[p * tiles + tile]
//   sym (dot mode, AB and E both symmetric): tiles above the diagonal are skipped (their partial
//     is 0) and strictly-lower tiles count twice, so the partials still sum to <E, AB>
//   dot = 2: a second matrix E2 (same lde) is reduced against the same product tile, its partials
//     written to part2 (same layout); with sym, E2 must be symmetric too
//   inplace: C is also the A or B operand, and the product only mixes elements within 128 rows (C = A)
//     or 128 columns (C = B) of it. Such a launch keeps 128 x 128 tiles whatever its size: a workgroup
//     then reads everything its own tile depends on before it writes, and no other workgroup reads
//     what it writes. (With 64 x 64 tiles two workgroups would share those 128 rows or columns, and
//     one could read what the other has already overwritten.)
// ------------------------------------------------------------------------------------------------
constexpr int kMaxGemmBatch = 48;

struct GemmBatch {
  const float *A[kMaxGemmBatch];
  const float *A2[kMaxGemmBatch];
  const float *B[kMaxGemmBatch];
  float *C[kMaxGemmBatch];
  const float *E[kMaxGemmBatch];
  const float *E2[kMaxGemmBatch];
  double *P2[kMaxGemmBatch];     // set by launch_gemm_f32 from part2
};

struct GemmShape {
  int M, N, K;
  int lda, ldb, ldc, lde;
  int ta, tb, lower, sub, dot;
  int sym;        // dot mode with a symmetric product and E: lower tiles only, off-diagonal ones x2
  int hform;      // dot mode: E = (E2 + A2) - (X + X^T) with X = E, formed in fp64 per element
  int inplace;    // C aliases an operand within one 128-row or 128-column extent: 128 tiles only
  float alpha, beta;
};

// Launch one batched GEMM of `count` problems (count <= kMaxGemmBatch). `part` is required in dot mode,
// `part2` when dot = 2.
hipError_t launch_gemm_f32(const GemmBatch &b, int count, const GemmShape &sh, double *part,
                           int64_t part_stride, hipStream_t s, double *part2 = nullptr);
int gemm_tiles(int M, int N);     // number of output tiles (partials per problem in dot mode)

// Sum the dot partials per problem in a fixed order (deterministic), over `terms` groups:
//   out[p] = sum_g coef[g] * sum_{t < tiles} part[(g * count + p) * stride + t]
// With `info` (device int32 [count]), problems whose info is nonzero get NaN instead.
hipError_t launch_reduce_partials(const double *part, int count, int64_t stride, int tiles, int terms,
                                  const double *coef /* host, terms <= 4 */, double *out,
                                  hipStream_t s, const int32_t *info = nullptr);
// Per 128 x 128 tile of a d x d matrix (the tiles of gemm_tiles(d, d), same order): the sum of
// squares in fp64, a fixed order within the tile -> part[p * stride + tile]
hipError_t launch_sumsq_tiles(const float *base, int64_t layer_stride, int d, int count, double *part,
                              int64_t stride, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Blocked Cholesky building blocks
// ------------------------------------------------------------------------------------------------
constexpr int kMaxBatch = 48;
struct PtrBatch {
  float *p[kMaxBatch];
};
struct CPtrBatch {
  const float *p[kMaxBatch];
};

// L = G + lambda I (full copy) for each layer
hipError_t launch_shift_copy(const CPtrBatch &G, float *L, int64_t L_stride, int d, float lambda,
                             int count, hipStream_t s);
// Factor the nb x nb diagonal block at (k0, k0) of each L in place (lower Cholesky) and write its
// inverse to Linv (nb x nb, row-major). info[layer] records the first failing column (1-based).
hipError_t launch_potrf_diag(float *L, int64_t L_stride, int d, int k0, int nb, float *Linv,
                             int64_t Linv_stride, int32_t *info, int count, hipStream_t s);
// out = in^T for d x d matrices (batch, per-layer pointers)
hipError_t launch_transpose(const CPtrBatch &in, const PtrBatch &out, int d, int count, hipStream_t s);
// out = a + b, out = a - b (elementwise, d x d)
hipError_t launch_add(const CPtrBatch &a, const CPtrBatch &b, const PtrBatch &out, int d, int count,
                      hipStream_t s);
hipError_t launch_sub(const CPtrBatch &a, const CPtrBatch &b, const PtrBatch &out, int d, int count,
                      hipStream_t s);
hipError_t launch_copy(const CPtrBatch &in, const PtrBatch &out, int d, int count, hipStream_t s);
// H = (F + G) - (X + X^T) elementwise (exactly symmetric when F and G are), d x d
hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// L-Layer steady state
// ------------------------------------------------------------------------------------------------
// out [d_out, d_in] bf16 = W + dW (fp32 sum, round to nearest even); W, dW are [d_out, d_in] when
// linear != 0, else [d_in, d_out] (transposed on the way)
hipError_t launch_apply_delta(const float *W, const float *dW, int d_in, int d_out, int linear,
                              uint16_t *out, hipStream_t s);
// y [n, d_out] (row stride ldy) = a [n, d_in] (row stride lda) . w^T, w [d_out, d_in]; all bf16,
// fp32 accumulation; d_in % 32 == 0
hipError_t launch_project_bf16(int64_t n, int d_in, int d_out, const uint16_t *a, int64_t lda,
                               const uint16_t *w, uint16_t *y, int64_t ldy, hipStream_t s);

}  // namespace ispa
