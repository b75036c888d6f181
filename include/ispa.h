/*
 * ispa.h - C ABI of the ISPA hot path on AMD Instinct MI355X (gfx950).
 *
 * ISPA ("Instance-Specific Parametric Absorption", technical summary pages on gist.science, Italian
 * and Japanese editions) compresses the KV cache of a streaming autoregressive video model: during a
 * warmup every layer produces a full-context and a local-context attention output, the gap between
 * them is absorbed into the output projection by a closed-form ridge solve, and the layers where that
 * works best drop their history cache. This library implements that path's device work.
 *
 * Conventions (all entry points):
 *  - Tensors are caller-owned device memory (allocated by the caller, e.g. PyTorch). The library
 *    never allocates or frees device memory and keeps no state between calls. Scratch memory is
 *    passed in through (ws, ws_bytes); the matching *_workspace() function gives the size needed.
 *    One exception: ispa_future_scores_noalloc takes no workspace and uses a fixed-size library array
 *    on each GPU instead (see its declaration).
 *  - Every call validates its arguments on the host first, enqueues its kernels on `stream`
 *    (a hipStream_t; NULL is the default stream) and returns without waiting. An argument error
 *    returns before anything is enqueued. Nothing throws across the ABI.
 *  - Layouts are row-major. Token-major activations: Q, K, V are [n, H, d_h] with a row stride (in
 *    elements) between tokens of at least H*d_h; A outputs are [n_q, H*d_h] with heads concatenated
 *    (column h*d_h + c). LSE outputs are [H, n_q] fp32, natural log.
 *  - Device pointers must be 16-byte aligned; bf16 row strides must be multiples of 8 elements and
 *    fp32 row strides multiples of 4.
 *  - Status codes: ISPA_OK, ISPA_E_ARG (bad pointer, size or alignment), ISPA_E_UNSUPPORTED (valid but
 *    not implemented: head_dim, dtype), ISPA_E_WORKSPACE (ws too small), ISPA_E_HIP (a HIP launch
 *    failed; hipGetLastError is cleared).
 */
#ifndef ISPA_H
#define ISPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ISPA_OK = 0,
  ISPA_E_ARG = -1,
  ISPA_E_UNSUPPORTED = -2,
  ISPA_E_WORKSPACE = -3,
  ISPA_E_HIP = -4
} ispa_status;

typedef enum { ISPA_F32 = 0, ISPA_BF16 = 1 } ispa_dtype;

/* One KV-cache segment of a layer: keys and values [n, H, d_h] in the call's dtype.
 * row_stride (elements) is the distance between consecutive tokens, >= H*d_h and < 2^23 (larger
 * strides return ISPA_E_UNSUPPORTED). n may be 0 (then k and
 * v may be NULL). */
typedef struct {
  const void *k;
  const void *v;
  int64_t n;
  int64_t row_stride;
} ispa_kv_segment;

/* ---------------------------------------------------------------------------------------------
 * Dual-stream attention (ISPA page, section 2 "Framework Core", stage 1 "Dual-Stream Warmup", and
 * its Decomposable Attention paragraph).
 *
 * For every head h and query i (the current-chunk tokens):
 *   A_loc   = softmax attention of q_i over the local keys  L = sink U cur
 *   A_full  = softmax attention of q_i over all keys        U = sink U cur U hist
 *   lse_X   = log sum_{j in X} exp(softmax_scale * q_i . k_j)   for X = L, hist, U
 * Both outputs come from one pass over the cache: the local keys are visited first and their
 * normalised output and LSE are stored, then the same running softmax state continues over the
 * history keys. No mask: every query sees every key of the three segments.
 *
 *   dt            ISPA_BF16 (bf16 in, fp32 accumulate, bf16 out) or ISPA_F32 (fp32 throughout)
 *   n_heads       H >= 1; head_dim d_h in {64, 128}
 *   softmax_scale tau > 0 (1/sqrt(d_h) in the usual case)
 *   q             [n_q, H, d_h], row stride q_row_stride; n_q >= 0 (0 is a no-op)
 *   sink, cur     local segments; sink.n + cur.n >= 1 (an empty local context is an argument error)
 *   hist          history segment; hist.n may be 0: then a_full is bitwise a_loc, lse_hist = -inf
 *                 and lse_full = lse_loc
 *   a_loc         out [n_q, H*d_h] dtype dt, row stride H*d_h
 *   a_full        out, same shape; NULL computes only the local branch (history is then ignored)
 *   lse_loc       out [H, n_q] fp32 (may be NULL); lse_hist, lse_full likewise (NULL = not stored)
 * ------------------------------------------------------------------------------------------- */
ispa_status ispa_attn_dual(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                           const void *q, int64_t n_q, int64_t q_row_stride,
                           ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                           void *a_loc, void *a_full,
                           float *lse_loc, float *lse_hist, float *lse_full,
                           void *stream);

/* ---------------------------------------------------------------------------------------------
 * ispa_attn_dual with a balanced schedule over the compute units (same passage; the merge of key-range
 * partial states is the page's log-sum-exp decomposition applied within a branch). When the
 * (head, 256-query tile) units would leave a tenth or more of the GPU's compute units idle and fill at
 * least half of each XCD's (128 <= units < 230 on 256 compute units; 12 heads x 19 query tiles is 228),
 * one workgroup per compute unit runs: each unit keeps a workgroup for its first key tiles and the
 * spare workgroups of the same XCD share the units' remaining tiles. Cut units' partial online-softmax
 * states (accumulator, running maximum, local and history exp-sums) go to `ws`, and the workgroup that
 * completes a unit's last piece merges the pieces in key order. Otherwise the call is ispa_attn_dual
 * and `ws` is not touched.
 *
 *   arguments, outputs and errors as for ispa_attn_dual, plus
 *   ws, ws_bytes  device scratch of at least ispa_attn_dual_balanced_workspace(...) bytes, 256-byte
 *                 aligned (may be NULL when that size is 0); its contents need no clearing and are
 *                 scratch after the call. Too small or misaligned: ISPA_E_WORKSPACE.
 * Results are within the attention tolerances of ispa_attn_dual and identical from call to call
 * (ranges are merged in a fixed order, whichever workgroup finishes last); they are not bitwise
 * those of ispa_attn_dual, whose single pass adds the same terms in another order. Speed: on MI355X
 * at 12 heads x 4680 queries x 18,720 keys this schedule takes 0.62 ms against 0.59 ms for
 * ispa_attn_dual on the same GPU: storing and merging the partial states costs about as much as the
 * idle compute units it puts to work.
 * ispa_attn_dual_balanced_workspace: bytes for a call with these sizes on the current device (0 when
 * the plain schedule is used: dt other than ISPA_BF16, head_dim other than 128, fewer than 16 key
 * tiles of 64, or a unit count outside the range above); n_local_keys = sink.n + cur.n, n_hist_keys =
 * hist.n (0 for a local-only call). 557,056 bytes per unit (4 state slots) and a counter.
 * ------------------------------------------------------------------------------------------- */
size_t ispa_attn_dual_balanced_workspace(ispa_dtype dt, int32_t n_heads, int32_t head_dim, int64_t n_q,
                                         int64_t n_local_keys, int64_t n_hist_keys);
ispa_status ispa_attn_dual_balanced(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                    const void *q, int64_t n_q, int64_t q_row_stride,
                                    ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                                    void *a_loc, void *a_full,
                                    float *lse_loc, float *lse_hist, float *lse_full,
                                    void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Dual-stream attention with a per-key additive logit bias (FAST-AR summary page, section 2 part A
 * "TempCache", Lemma 5.1: a group of m identical keys is replaced by one key whose value is the
 * group's mean value and whose logit is raised by ln m, with no change to the attention output or
 * its LSE). The logit of key j of a segment S in head h becomes
 *   softmax_scale * q_i . k_j + b_S[h * head_stride + j]
 * in every sum above (outputs and all three LSEs), so a cache merged by ispa_kv_merge, with its
 * ln(count) as the bias, gives the same A_loc, A_full and LSEs as the unmerged cache.
 *
 *   bias          NULL = no bias (the call is then ispa_attn_dual); otherwise
 *     .sink, .cur, .hist   device fp32 per segment, 4-byte aligned, or NULL (zero bias for that
 *                          segment); natural-log units; values must be finite with |b| <= 1e30
 *                          (a large negative value such as -1e30 masks a key)
 *     .*_head_stride       per segment: 0 = one bias per key shared by all heads ([n]); > 0 =
 *                          elements between heads ([H, head_stride], head_stride >= n)
 * Other arguments, outputs and errors as for ispa_attn_dual; a bad bias (misaligned pointer,
 * negative or too small head stride) is ISPA_E_ARG.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
  const float *sink;
  const float *cur;
  const float *hist;
  int64_t sink_head_stride;
  int64_t cur_head_stride;
  int64_t hist_head_stride;
} ispa_kv_bias;

ispa_status ispa_attn_dual_biased(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                  const void *q, int64_t n_q, int64_t q_row_stride,
                                  ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                                  const ispa_kv_bias *bias,
                                  void *a_loc, void *a_full,
                                  float *lse_loc, float *lse_hist, float *lse_full,
                                  void *stream);

/* ---------------------------------------------------------------------------------------------
 * TempCache exact merge of one cache segment (FAST-AR summary page, section 2 part A "TempCache",
 * Lemma 5.1). Groups of token rows become single rows: for group g with members
 * members[offsets[g]], .., members[offsets[g+1] - 1] (token indices into the segment),
 *   k_out[g] = mean of the members' key rows,   v_out[g] = mean of their value rows,
 *   bias_out[g] = ln(offsets[g+1] - offsets[g])
 * over all H*d_h columns; sums in fp32 in member order, one correctly rounded division, one rounding
 * to dt (nearest even for bf16). With the merged rows as a segment and bias_out as its bias,
 * ispa_attn_dual_biased reproduces attention over the original rows exactly when every group's keys
 * are identical (the lemma), and approximately for near-identical keys. Finding the groups (the
 * page's similarity search) is the caller's.
 *
 *   dt          ISPA_BF16 or ISPA_F32 (type of k, v, k_out, v_out)
 *   width       elements per token row, H*d_h; a multiple of 8 (else ISPA_E_UNSUPPORTED)
 *   k, v        device [n, width] rows, row stride in_stride (>= width, multiple of 8), 16-byte aligned
 *   n           rows of the input segment (>= 0)
 *   offsets     device int32 [n_groups + 1], non-decreasing, offsets[0] = 0
 *   members     device int32 [offsets[n_groups]], each in [0, n)
 *   n_groups    0 .. 2^26 (0 is a no-op)
 *   k_out, v_out  device out [n_groups, width], row stride out_stride (>= width, multiple of 8),
 *               16-byte aligned; must not overlap k, v
 *   bias_out    device fp32 out [n_groups], or NULL
 * The device arrays offsets and members are not read on the host: a member outside [0, n) is skipped
 * (contributes zero, never read), and a group with no members gets zero rows and bias -inf (which the biased attention
 * does not accept). Errors: ISPA_E_ARG (sizes, NULL or misaligned pointers), ISPA_E_UNSUPPORTED,
 * ISPA_E_HIP.
 * ------------------------------------------------------------------------------------------- */
ispa_status ispa_kv_merge(ispa_dtype dt, int32_t width, const void *k, const void *v, int64_t n,
                          int64_t in_stride, const int32_t *offsets, const int32_t *members,
                          int64_t n_groups, void *k_out, void *v_out, int64_t out_stride,
                          float *bias_out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * FP8 attention scores (ISPA page, section 4 "Experimental Results": ISPA is paired with W8A8
 * quantisation for its largest speed-up; the page gives no recipe). Queries and keys are stored as
 * OCP FP8 E4M3 bytes with one fp32 scale per head (scale = absmax / 448, value = e4m3 * scale); the
 * scores run on the FP8 matrix cores with fp32 accumulation, values, probabilities and outputs stay
 * bf16. Otherwise exactly ispa_attn_dual: A_loc, A_full and the three LSE rows of the dequantised
 * queries and keys.
 *
 * ispa_fp8_head_scales: scales[h] = max over rows and channels of |x[:, h, :]| / 448 (1 if all zero).
 * ispa_fp8_quantize:   out[r][h*d_h + c] = e4m3(fp32(x[r][h][c] * fp32(1 / scales[h]))), round to
 *                      nearest even, magnitudes beyond 448 saturate.
 *   dt             ISPA_BF16 or ISPA_F32 (type of x); x [n, H, d_h] row stride row_stride (>= H*d_h,
 *                  multiple of 8 elements), 16-byte aligned; n >= 0; d_h in {64, 128}
 *   scales         device fp32 [H] (out for head_scales, in for quantize)
 *   out            device uint8 [n, out_row_stride], out_row_stride >= H*d_h, multiple of 8
 *
 * ispa_attn_dual_fp8: as ispa_attn_dual with dt = ISPA_BF16 except
 *   q              e4m3 bytes [n_q, H, d_h], row stride q_row_stride (bytes, multiple of 16)
 *   q_scale, k_scale  device fp32 [H]: the scales of q and of every key of the cache
 *   sink, cur, hist  .k e4m3 bytes, .v bf16, both with row stride .row_stride (in elements of each,
 *                  multiple of 16, < 2^23)
 *   head_dim       128 only (else ISPA_E_UNSUPPORTED)
 * Errors as for ispa_attn_dual.
 *
 * ispa_attn_dual_fp8_pv: as ispa_attn_dual_fp8, with the value product in FP8 as well (same W8A8 passage;
 * the recipe is a reading, the page gives none):
 *   sink, cur, hist  .k and .v e4m3 bytes, one row stride .row_stride in bytes (multiple of 16, < 2^23)
 *   v_scale        device fp32 [H]: one scale per head for every value row of the cache (absmax / 448,
 *                  as ispa_fp8_head_scales gives); values are e4m3_value * v_scale
 *   Each probability exp(s - m) of the online softmax (m: its running maximum, never below the max by
 *   more than 8 in log2 units, so p <= 256) is rounded to e4m3 (nearest even) for the value product;
 *   the exp-sum that normalises the rows and the log-sum-exp outputs use the unrounded probabilities.
 *   So A_loc and A_full differ from attention on the dequantised values by the probability rounding
 *   (relative 2^-4 at most per normal probability) besides the bf16 output rounding; LSE rows are those
 *   of ispa_attn_dual_fp8.
 * Errors as for ispa_attn_dual (v_scale NULL or misaligned: ISPA_E_ARG).
 * ------------------------------------------------------------------------------------------- */
ispa_status ispa_fp8_head_scales(ispa_dtype dt, const void *x, int64_t n, int32_t n_heads, int32_t head_dim,
                                 int64_t row_stride, float *scales, void *stream);
ispa_status ispa_fp8_quantize(ispa_dtype dt, const void *x, int64_t n, int32_t n_heads, int32_t head_dim,
                              int64_t row_stride, const float *scales, uint8_t *out, int64_t out_row_stride,
                              void *stream);
ispa_status ispa_attn_dual_fp8(int32_t n_heads, int32_t head_dim, float softmax_scale,
                               const uint8_t *q, int64_t n_q, int64_t q_row_stride, const float *q_scale,
                               ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                               const float *k_scale, void *a_loc, void *a_full,
                               float *lse_loc, float *lse_hist, float *lse_full, void *stream);
ispa_status ispa_attn_dual_fp8_pv(int32_t n_heads, int32_t head_dim, float softmax_scale,
                                  const uint8_t *q, int64_t n_q, int64_t q_row_stride, const float *q_scale,
                                  ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                                  const float *k_scale, const float *v_scale, void *a_loc, void *a_full,
                                  float *lse_loc, float *lse_hist, float *lse_full, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Future-query importance of cached keys (Future Forcing summary page, "Componenti Algorithmiche",
 * module 1: keys are scored by the attention weight that proxies of future queries are predicted to
 * give them, mixed with a historical score by a weight lambda; implementation detail 3: computed
 * without the full Q K^T matrix). For head h and key j of the cache (sink, then current, then history):
 *   scores[h * scores_head_stride + j] = (1/n_p) sum_i softmax_j(softmax_scale * q~_i . k_j)
 * the mean over the n_p proxy queries of the weight each gives key j (a head's scores sum to 1).
 * Two passes, no score matrix stored: the log-sum-exp of every proxy over all keys (for d_h = 128 the
 * keys are split over up to 16 workgroups per query tile when the proxy tiles alone would leave compute
 * units idle; their partial (max, sum) states are merged in split order, so the result does not depend
 * on scheduling), then per-key sums of exp(softmax_scale * q~_i . k_j - lse_i). Optionally, per token:
 *   token_score[j] = lambda * mean_h scores[h][j] + (1 - lambda) * hist_token_score[j]
 * Building the proxies (rotary positions of future frames applied to the mean of past pre-rotary
 * queries) is the caller's.
 *
 *   dt             ISPA_BF16 only (else ISPA_E_UNSUPPORTED)
 *   n_heads        H >= 1; head_dim d_h in {64, 128}; softmax_scale tau > 0
 *   q_proxy        [n_p, H, d_h] row stride q_row_stride (>= H*d_h, multiple of 8); n_p >= 1
 *   sink, cur, hist  key segments as for ispa_attn_dual (only .k, .n, .row_stride are read; .v may be
 *                  NULL); together at least one key
 *   scores         out fp32 [H, scores_head_stride], scores_head_stride >= total keys
 *   lambda, hist_token_score, token_score   token_score (fp32 [total keys]) may be NULL: then no
 *                  token scores; hist_token_score may be NULL (historical score 0)
 *   ws             device scratch of at least ispa_future_scores_workspace(H, n_p) bytes: the
 *                  proxies' log-sum-exp rows, then the partial states of the split key ranges
 * Errors: ISPA_E_ARG (sizes, NULL or misaligned pointers, lambda not finite), ISPA_E_UNSUPPORTED,
 * ISPA_E_WORKSPACE, ISPA_E_HIP.
 * ------------------------------------------------------------------------------------------- */
size_t ispa_future_scores_workspace(int32_t n_heads, int64_t n_p);
ispa_status ispa_future_scores(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                               const void *q_proxy, int64_t n_p, int64_t q_row_stride,
                               ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                               float *scores, int64_t scores_head_stride,
                               float lambda, const float *hist_token_score, float *token_score,
                               void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * ispa_future_scores without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Arguments,
 * results and errors are those of ispa_future_scores (the same kernels run); the scratch lives in a
 * library array of ISPA_NOALLOC_SCRATCH_BYTES on each GPU, held until the process ends, and the call
 * allocates and frees nothing.
 *  - Limit: a call needs ispa_future_scores_workspace(n_heads, n_p) bytes of it (0.7 MB for 12 heads x
 *    4680 proxies); larger calls return ISPA_E_WORKSPACE before any GPU work.
 *  - The array belongs to the device current on the calling thread, which must be the device of
 *    `stream`. Its address is looked up on the first call on each device (ISPA_E_HIP if that fails).
 *  - Every call on one GPU uses the same array: calls that overlap on one GPU (other streams, other
 *    threads, a replayed graph beside an eager call) race and must be serialised by the caller.
 *    Nothing in the array needs clearing: each call writes every word it reads.
 * ------------------------------------------------------------------------------------------- */
#define ISPA_NOALLOC_SCRATCH_BYTES (16u << 20)
ispa_status ispa_future_scores_noalloc(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                       const void *q_proxy, int64_t n_p, int64_t q_row_stride,
                                       ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                                       float *scores, int64_t scores_head_stride,
                                       float lambda, const float *hist_token_score, float *token_score,
                                       void *stream);

/* ---------------------------------------------------------------------------------------------
 * Warmup statistics (ISPA page, section 2 stage 2 "Layer Absorb": the closed form needs
 * A_loc^T A_loc and A_loc^T (A_full - A_loc) over the warmup rows; stage 1 says these rows are the
 * warmup chunks' attention outputs).
 *
 * Adds one chunk of rows to the layer's running sums (fp32, no 1/N scaling):
 *   G += A_loc^T A_loc      X += A_loc^T A_full      F += A_full^T A_full   (each [d, d])
 * so that C = X - G = A_loc^T (A_full - A_loc) and H = F - X - X^T + G = D^T D with
 * D = A_full - A_loc. The products only ever multiply exact input values (D is never rounded).
 * G and F are exactly symmetric. The caller zeroes G, X, F before the first chunk; the sums are
 * deterministic (no atomics) and can be saved and restored between chunks.
 *
 *   dt        ISPA_BF16 or ISPA_F32 (type of a_loc / a_full)
 *   n_rows    rows in this chunk (>= 0); d = H*d_h (>= 1)
 *   a_loc, a_full   [n_rows, d] row-major (row stride d)
 *   G, X      [d, d] fp32, accumulated in place; F may be NULL when the error is not needed
 *   ws        unused by the current kernels (ispa_absorb_accumulate_workspace returns 0)
 * ------------------------------------------------------------------------------------------- */
size_t ispa_absorb_accumulate_workspace(int64_t n_rows, int32_t d);
ispa_status ispa_absorb_accumulate(ispa_dtype dt, int64_t n_rows, int32_t d,
                                   const void *a_loc, const void *a_full,
                                   float *G, float *X, float *F,
                                   void *ws, size_t ws_bytes, void *stream);

/* The statistics of several layers' chunks in one call (all with the same n_rows and d), for each
 * layer l:  G[l] += A_loc[l]^T A_loc[l],  X[l] += A_loc[l]^T A_full[l],  F[l] += A_full[l]^T A_full[l].
 * For a model whose layers' attention outputs of a warmup chunk are kept until the chunk ends. The
 * sums are bitwise those of `batch` ispa_absorb_accumulate calls (every output element is a fixed-order
 * sum of exact products); one launch holds the tiles of up to 48 layers, so the GPU stays full at any d.
 *   a_loc, a_full   host arrays of `batch` device pointers to [n_rows, d] rows (row stride d, 16-byte
 *                   aligned), type dt
 *   G, X, F         host arrays of `batch` device pointers to [d, d] fp32 sums (F may be NULL: no F for
 *                   any layer)
 * Errors as for ispa_absorb_accumulate; batch >= 0 (0 is a no-op). */
ispa_status ispa_absorb_accumulate_batched(ispa_dtype dt, int64_t n_rows, int32_t d, int32_t batch,
                                           const void *const *a_loc, const void *const *a_full,
                                           float *const *G, float *const *X, float *const *F, void *stream);

/* FP8 statistics (ISPA page, section 4: ISPA with W8A8): the same sums over rows stored as OCP e4m3
 * bytes with one scale per head (rows quantised by ispa_fp8_quantize with scales from
 * ispa_fp8_head_scales): G += A_loc^T A_loc etc. of the dequantised rows e4m3 * scale, exact products
 * on the FP8 matrix cores, fp32 sums.
 *   a_loc, a_full  device uint8 [n_rows, d] (row stride d), 16-byte aligned
 *   s_loc, s_full  device fp32 [d / head_dim] per-head scales; head_dim in {64, 128}, d % 64 == 0,
 *                  d % head_dim == 0
 *   G, X, F, ws    as for ispa_absorb_accumulate (ws unused)
 */
ispa_status ispa_absorb_accumulate_fp8(int64_t n_rows, int32_t d, int32_t head_dim,
                                       const uint8_t *a_loc, const float *s_loc,
                                       const uint8_t *a_full, const float *s_full,
                                       float *G, float *X, float *F,
                                       void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Closed-form absorb update (ISPA page, section 2 stage 2 "Layer Absorb", second display equation):
 *   dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W = (G + lambda I)^-1 (X - G) W
 * the minimiser of || A_loc (W + dW) - A_full W ||_F^2 + lambda || dW ||_F^2 (first display equation).
 * Solved per layer by a blocked fp32 Cholesky factorisation G + lambda I = L L^T and two blocked
 * triangular solves; batched over layers.
 *
 *   d          matrix size (>= 1); batch = number of layers (>= 0)
 *   lambda     ridge weight (>= 0; 0 only if G is positive definite)
 *   G, X       host arrays of `batch` device pointers to [d, d] fp32 statistics
 *   W          host array of device pointers to [d, d] fp32: W[d_in, d_out] with y = A W, or, if
 *              w_is_linear_weight, an nn.Linear weight [d_out, d_in] (y = A W^T)
 *   dW         host array of device pointers, out [d, d] fp32 in the same orientation as W
 *   info       device int32 [batch], out: 0 = ok, k > 0 = the leading minor of order k of
 *              G + lambda I is not positive (dW of that layer is then undefined)
 *   ws         device scratch of at least ispa_absorb_solve_workspace(d, batch) bytes
 * ------------------------------------------------------------------------------------------- */
size_t ispa_absorb_solve_workspace(int32_t d, int32_t batch);
ispa_status ispa_absorb_solve(int32_t d, int32_t batch, float lambda,
                              const float *const *G, const float *const *X,
                              const float *const *W, int32_t w_is_linear_weight,
                              float *const *dW, int32_t *info,
                              void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Closed-form absorb update and the layer's reconstruction error at it, in one call (ISPA page, section
 * 2 stage 2 "Layer Absorb", both display equations, and "Dynamic Layer Selection"). dW and info are
 * exactly those of ispa_absorb_solve (the same kernels in the same order: identical bits). At the
 * optimum (G + lambda I) dW = C W =: B, so the objective's data term reduces to
 *   eps = <W, H W> - <dW, B> - lambda ||dW||_F^2,   H = (F + G) - (X + X^T) = D^T D,
 * and with L L^T = G + lambda I and Y = L^-1 B (the forward sweep), <dW, B> = ||Y||_F^2. The only d^3
 * term left is W W^T (lower tiles), reduced against H and F in fp64: about d^3 FLOP per layer instead of
 * ispa_layer_error's 4 d^3. ref = <F, W W^T> = ||A_full W||_F^2.
 *
 *   G, X, F, W, dW, info, lambda, w_is_linear_weight   as for ispa_absorb_solve / ispa_layer_error
 *   eps        device double [batch], out; NaN for a layer whose info is nonzero
 *   ref        device double [batch], out (may be NULL)
 *   ws         device scratch of at least ispa_absorb_solve_eps_workspace(d, batch) bytes, 256-byte
 *              aligned
 * For a dW that is not this call's optimum (e.g. rounded or edited weights) use ispa_layer_error.
 * ------------------------------------------------------------------------------------------- */
size_t ispa_absorb_solve_eps_workspace(int32_t d, int32_t batch);
ispa_status ispa_absorb_solve_eps(int32_t d, int32_t batch, float lambda,
                                  const float *const *G, const float *const *X, const float *const *F,
                                  const float *const *W, int32_t w_is_linear_weight,
                                  float *const *dW, int32_t *info, double *eps, double *ref,
                                  void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Reconstruction error per layer (ISPA page, section 2 "Dynamic Layer Selection": layers are ranked
 * by their reconstruction error after the warmup). For the given dW (any dW, not only the optimum):
 *   eps = || A_loc (W + dW) - A_full W ||_F^2
 *       = <W, F W> - 2 <W + dW, X W> + <W + dW, G (W + dW)>      (sums over the warmup rows)
 *   ref = || A_full W ||_F^2 = <W, F W>
 * from the statistics of ispa_absorb_accumulate. Products in fp32, inner products in fp64.
 *
 *   G, X, F, W, dW   host arrays of `batch` device pointers ([d, d] fp32; W, dW oriented as in
 *                    ispa_absorb_solve)
 *   eps        device double [batch], out
 *   ref        device double [batch], out (may be NULL)
 *   ws         device scratch of at least ispa_layer_error_workspace(d, batch) bytes
 * ------------------------------------------------------------------------------------------- */
size_t ispa_layer_error_workspace(int32_t d, int32_t batch);
ispa_status ispa_layer_error(int32_t d, int32_t batch,
                             const float *const *G, const float *const *X, const float *const *F,
                             const float *const *W, int32_t w_is_linear_weight,
                             const float *const *dW, double *eps, double *ref,
                             void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Layer selection (ISPA page, section 2 "Dynamic Layer Selection" and stage 3 "Memory-Efficient
 * Inference": the K layers with the lowest error become L-Layers, the other N - K stay F-Layers).
 * Host-only, no GPU work. Ascending eps, ties to the lower layer index, NaN ranks last.
 *
 *   eps         host double [n_layers]
 *   k           0 <= k <= n_layers
 *   selected    host int32 [k], out: chosen layers in ascending-eps order (may be NULL if k == 0)
 *   is_l_layer  host uint8 [n_layers], out: 1 for chosen layers (may be NULL)
 * ------------------------------------------------------------------------------------------- */
ispa_status ispa_rank_layers(const double *eps, int32_t n_layers, int32_t k,
                             int32_t *selected, uint8_t *is_l_layer);

/* ---------------------------------------------------------------------------------------------
 * L-Layer steady state (ISPA page, section 2 stage 3 "Memory-Efficient Inference": after the warmup
 * the selected layers drop their history keys and values, attend to the sink tokens and the current
 * chunk only, and project with the updated weights W_new = W + dW; the other layers keep the full
 * cache and W). The attention of an L-Layer is ispa_attn_dual with an empty history and
 * a_full = NULL; the three calls below are the weight update, the projection and the eviction plan.
 * ------------------------------------------------------------------------------------------- */

/* W_new = W + dW as bf16 in nn.Linear orientation.
 *
 *   d_in, d_out  matrix sizes (>= 1)
 *   W, dW        device fp32, both [d_in, d_out] (y = A W) or, with w_is_linear_weight, both
 *                [d_out, d_in] (y = A W^T); dense, 16-byte aligned
 *   w_new        device bf16 [d_out, d_in], out: round-to-nearest-even of the fp32 sum W + dW
 *                (one fp32 addition per element), always in the nn.Linear orientation
 * Asynchronous on `stream`; argument errors are returned before any GPU work. */
ispa_status ispa_apply_delta(int32_t d_in, int32_t d_out, const float *W, const float *dW,
                             int32_t w_is_linear_weight, void *w_new, void *stream);

/* Output projection y = A W^T of one chunk (bf16 in, fp32 accumulation, bf16 out).
 *
 *   n            rows (tokens, >= 0; 0 is a no-op)
 *   d_in, d_out  d_in a multiple of 32, d_out a multiple of 8
 *   a            device bf16 [n, d_in], row stride lda elements (lda >= d_in, multiple of 8)
 *   w            device bf16 [d_out, d_in] dense (nn.Linear orientation, e.g. from ispa_apply_delta)
 *   y            device bf16 [n, d_out], out, row stride ldy elements (ldy >= d_out, multiple of 8)
 * All pointers 16-byte aligned. Asynchronous on `stream`. */
ispa_status ispa_project(int64_t n, int32_t d_in, int32_t d_out, const void *a, int64_t lda,
                         const void *w, void *y, int64_t ldy, void *stream);

/* History kept by every layer after the warmup (host-only, no GPU work). With the cache laid out
 * [sink | history | current], an L-Layer keeps 0 history tokens and an F-Layer n_hist.
 *
 *   is_l_layer      host uint8 [n_layers] (e.g. from ispa_rank_layers)
 *   hist_kept       host int64 [n_layers], out
 *   evicted_tokens  host int64, out: key/value tokens freed over all layers (may be NULL)
 * Negative counts are ISPA_E_ARG. */
ispa_status ispa_kv_plan(int32_t n_layers, const uint8_t *is_l_layer, int64_t n_sink, int64_t n_hist,
                         int64_t n_cur, int64_t *hist_kept, int64_t *evicted_tokens);

/* Human-readable name of a status code (static storage). */
const char *ispa_status_string(ispa_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t ispa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ISPA_H */
