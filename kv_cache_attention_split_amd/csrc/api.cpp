// C ABI of the ISPA hot path (declared in include/ispa.h): argument validation, workspace layout,
// and the launch sequences. Validation runs before any HIP call, so argument errors are reported
// without touching the GPU.
#include "ispa.h"
#include "ispa_internal.hpp"

#include <algorithm>
#include <functional>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

using namespace ispa;

namespace {

constexpr int32_t kVersion = 100;   // 0.1.0

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline ispa_status hip_status(hipError_t e) { return e == hipSuccess ? ISPA_OK : ISPA_E_HIP; }

#define ISPA_TRY(expr)                             \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return ISPA_E_HIP;       \
  } while (0)

ispa_status check_segment(const ispa_kv_segment &s, int64_t min_stride, int64_t align_elems) {
  if (s.n < 0) return ISPA_E_ARG;
  if (s.n == 0) return ISPA_OK;
  if (s.k == nullptr || s.v == nullptr) return ISPA_E_ARG;
  if (!aligned16(s.k) || !aligned16(s.v)) return ISPA_E_ARG;
  if (s.row_stride < min_stride || s.row_stride % align_elems != 0) return ISPA_E_ARG;
  if (s.row_stride >= (int64_t(1) << 23)) return ISPA_E_UNSUPPORTED;   // 24-bit in-tile row offsets
  return ISPA_OK;
}

// ---- workspace layouts ---------------------------------------------------------------------------
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int solve_nb(int d) { return (d % 128 == 0) ? 128 : 64; }

struct SolveLayout {
  size_t mat;            // bytes of one d x d fp32 matrix (padded)
  size_t linv;           // bytes of one layer's diagonal-block inverses
  size_t per_layer;
  size_t total(int batch) const { return per_layer * (size_t)batch; }
};
SolveLayout solve_layout(int d) {
  SolveLayout s;
  const int nb = solve_nb(d);
  const int nt = (d + nb - 1) / nb;
  s.mat = round_up((size_t)d * d * sizeof(float), 256);
  s.linv = round_up((size_t)nt * nb * nb * sizeof(float), 256);
  s.per_layer = 3 * s.mat + s.linv;     // L, B, W (standard orientation), Linv blocks
  return s;
}

struct ErrLayout {
  size_t mat, part;
  int tiles;
  size_t total(int batch) const { return (2 * mat + 3 * part) * (size_t)batch; }
};
ErrLayout err_layout(int d) {
  ErrLayout e;
  e.mat = round_up((size_t)d * d * sizeof(float), 256);
  e.tiles = gemm_tiles(d, d);
  e.part = round_up((size_t)e.tiles * sizeof(double), 256);
  return e;
}

ispa_status check_square_batch(int32_t d, int32_t batch) {
  if (d <= 0 || batch < 0) return ISPA_E_ARG;
  if (d % 64 != 0) return ISPA_E_UNSUPPORTED;
  return ISPA_OK;
}

ispa_status check_ptr_array(const float *const *a, int32_t batch) {
  if (batch == 0) return ISPA_OK;
  if (a == nullptr) return ISPA_E_ARG;
  for (int32_t i = 0; i < batch; ++i)
    if (a[i] == nullptr || !aligned16(a[i])) return ISPA_E_ARG;
  return ISPA_OK;
}

}  // namespace

extern "C" {

int32_t ispa_version(void) { return kVersion; }

const char *ispa_status_string(ispa_status s) {
  switch (s) {
    case ISPA_OK: return "ISPA_OK";
    case ISPA_E_ARG: return "ISPA_E_ARG: invalid argument (pointer, size, stride or alignment)";
    case ISPA_E_UNSUPPORTED: return "ISPA_E_UNSUPPORTED: valid but not implemented (dtype, head_dim, d)";
    case ISPA_E_WORKSPACE: return "ISPA_E_WORKSPACE: workspace too small";
    case ISPA_E_HIP: return "ISPA_E_HIP: a HIP call failed";
  }
  return "ISPA: unknown status";
}

// ------------------------------------------------------------------------------------------------
namespace {

bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

ispa_status check_bias(const float *b, int64_t n, int64_t head_stride) {
  if (b == nullptr || n == 0) return ISPA_OK;
  if (!aligned4(b)) return ISPA_E_ARG;
  if (head_stride < 0 || (head_stride != 0 && head_stride < n)) return ISPA_E_ARG;
  return ISPA_OK;
}

// compute units of the current device (cached per device); 0 if it cannot be read
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

// the balanced schedule's grid for this call (0: the plain launch)
int balanced_grid(ispa_dtype dt, int32_t head_dim, int32_t n_heads, int64_t n_q, const ispa_kv_segment &sink,
                  const ispa_kv_segment &cur, const ispa_kv_segment &hist, bool want_full) {
  if (dt != ISPA_BF16 || head_dim != 128 || n_heads <= 0 || n_q <= 0) return 0;
  return attn_balanced_grid(n_q, n_heads, sink.n + cur.n, want_full ? hist.n : 0, device_cus());
}

ispa_status attn_dual_impl(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                           const void *q, int64_t n_q, int64_t q_row_stride, ispa_kv_segment sink,
                           ispa_kv_segment cur, ispa_kv_segment hist, const ispa_kv_bias *bias,
                           void *a_loc, void *a_full, float *lse_loc, float *lse_hist, float *lse_full,
                           void *stream, bool balanced = false, void *ws = nullptr, size_t ws_bytes = 0) {
  if (dt != ISPA_BF16 && dt != ISPA_F32) return ISPA_E_UNSUPPORTED;
  if (n_heads <= 0 || n_q < 0) return ISPA_E_ARG;
  if (head_dim != 64 && head_dim != 128) return ISPA_E_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return ISPA_E_ARG;
  if (n_q > INT32_MAX / 2) return ISPA_E_ARG;
  const int64_t width = (int64_t)n_heads * head_dim;
  const int64_t align_elems = dt == ISPA_BF16 ? 8 : 4;
  if (sink.n < 0 || cur.n < 0 || hist.n < 0) return ISPA_E_ARG;
  if (sink.n + cur.n < 1) return ISPA_E_ARG;
  ispa_status st;
  if ((st = check_segment(sink, width, align_elems)) != ISPA_OK) return st;
  if ((st = check_segment(cur, width, align_elems)) != ISPA_OK) return st;
  if (a_full != nullptr && (st = check_segment(hist, width, align_elems)) != ISPA_OK) return st;
  if (bias != nullptr) {
    if ((st = check_bias(bias->sink, sink.n, bias->sink_head_stride)) != ISPA_OK) return st;
    if ((st = check_bias(bias->cur, cur.n, bias->cur_head_stride)) != ISPA_OK) return st;
    if (a_full != nullptr && (st = check_bias(bias->hist, hist.n, bias->hist_head_stride)) != ISPA_OK)
      return st;
  }
  if (n_q == 0) return ISPA_OK;
  if (q == nullptr || !aligned16(q) || q_row_stride < width || q_row_stride % align_elems != 0)
    return ISPA_E_ARG;
  if (a_loc == nullptr || !aligned16(a_loc)) return ISPA_E_ARG;
  if (a_full != nullptr && !aligned16(a_full)) return ISPA_E_ARG;

  int grid = 0;
  if (balanced) {
    grid = balanced_grid(dt, head_dim, n_heads, n_q, sink, cur, hist, a_full != nullptr);
    const size_t need = attn_balanced_ws_bytes(n_q, n_heads, grid);
    if (need > 0 && (ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 255) != 0)) return ISPA_E_WORKSPACE;
  }
  AttnArgs a{};
  a.q = q;
  a.q_stride = q_row_stride;
  a.sink_k = sink.k;
  a.sink_v = sink.v;
  a.sink_n = sink.n;
  a.sink_stride = sink.row_stride;
  a.cur_k = cur.k;
  a.cur_v = cur.v;
  a.cur_n = cur.n;
  a.cur_stride = cur.row_stride;
  const bool want_full = a_full != nullptr;
  a.hist_k = want_full ? hist.k : nullptr;
  a.hist_v = want_full ? hist.v : nullptr;
  a.hist_n = want_full ? hist.n : 0;
  a.hist_stride = want_full ? hist.row_stride : 0;
  a.a_loc = a_loc;
  a.a_full = a_full;
  a.lse_loc = lse_loc;
  a.lse_hist = want_full ? lse_hist : nullptr;
  a.lse_full = want_full ? lse_full : nullptr;
  a.n_q = (int32_t)n_q;
  a.n_heads = n_heads;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.sink_b = bias != nullptr && sink.n > 0 ? bias->sink : nullptr;
  a.cur_b = bias != nullptr && cur.n > 0 ? bias->cur : nullptr;
  a.hist_b = bias != nullptr && want_full && hist.n > 0 ? bias->hist : nullptr;
  a.sink_bhs = bias != nullptr ? bias->sink_head_stride : 0;
  a.cur_bhs = bias != nullptr ? bias->cur_head_stride : 0;
  a.hist_bhs = bias != nullptr ? bias->hist_head_stride : 0;
  a.bias_to_score = 1.0f / softmax_scale;
  hipStream_t s = (hipStream_t)stream;
  if (grid > 0) return hip_status(launch_attn_bf16_balanced(a, head_dim, grid, ws, s));
  const hipError_t e = dt == ISPA_BF16 ? launch_attn_bf16(a, head_dim, s) : launch_attn_f32(a, head_dim, s);
  return hip_status(e);
}

}  // namespace

ispa_status ispa_attn_dual(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                           const void *q, int64_t n_q, int64_t q_row_stride, ispa_kv_segment sink,
                           ispa_kv_segment cur, ispa_kv_segment hist, void *a_loc, void *a_full,
                           float *lse_loc, float *lse_hist, float *lse_full, void *stream) {
  return attn_dual_impl(dt, n_heads, head_dim, softmax_scale, q, n_q, q_row_stride, sink, cur, hist,
                        nullptr, a_loc, a_full, lse_loc, lse_hist, lse_full, stream);
}

size_t ispa_attn_dual_balanced_workspace(ispa_dtype dt, int32_t n_heads, int32_t head_dim, int64_t n_q,
                                         int64_t n_local_keys, int64_t n_hist_keys) {
  if (n_local_keys < 0 || n_hist_keys < 0) return 0;
  const ispa_kv_segment none{nullptr, nullptr, 0, 0};
  const ispa_kv_segment loc{nullptr, nullptr, n_local_keys, 0};
  const ispa_kv_segment hist{nullptr, nullptr, n_hist_keys, 0};
  const int grid = balanced_grid(dt, head_dim, n_heads, n_q, none, loc, hist, true);
  return attn_balanced_ws_bytes(n_q, n_heads, grid);
}

ispa_status ispa_attn_dual_balanced(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                    const void *q, int64_t n_q, int64_t q_row_stride, ispa_kv_segment sink,
                                    ispa_kv_segment cur, ispa_kv_segment hist, void *a_loc, void *a_full,
                                    float *lse_loc, float *lse_hist, float *lse_full, void *ws, size_t ws_bytes,
                                    void *stream) {
  return attn_dual_impl(dt, n_heads, head_dim, softmax_scale, q, n_q, q_row_stride, sink, cur, hist,
                        nullptr, a_loc, a_full, lse_loc, lse_hist, lse_full, stream, true, ws, ws_bytes);
}

ispa_status ispa_attn_dual_biased(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                  const void *q, int64_t n_q, int64_t q_row_stride, ispa_kv_segment sink,
                                  ispa_kv_segment cur, ispa_kv_segment hist, const ispa_kv_bias *bias,
                                  void *a_loc, void *a_full, float *lse_loc, float *lse_hist,
                                  float *lse_full, void *stream) {
  return attn_dual_impl(dt, n_heads, head_dim, softmax_scale, q, n_q, q_row_stride, sink, cur, hist,
                        bias, a_loc, a_full, lse_loc, lse_hist, lse_full, stream);
}

// ------------------------------------------------------------------------------------------------
namespace {
ispa_status check_fp8_rows(ispa_dtype dt, const void *x, int64_t n, int32_t n_heads, int32_t head_dim,
                           int64_t row_stride) {
  if (dt != ISPA_BF16 && dt != ISPA_F32) return ISPA_E_UNSUPPORTED;
  if (n < 0 || n_heads <= 0) return ISPA_E_ARG;
  if (head_dim != 64 && head_dim != 128) return ISPA_E_UNSUPPORTED;
  if (n > 0 && (x == nullptr || !aligned16(x) || row_stride < (int64_t)n_heads * head_dim || row_stride % 8 != 0))
    return ISPA_E_ARG;
  if (n > INT32_MAX) return ISPA_E_ARG;
  return ISPA_OK;
}
}  // namespace

ispa_status ispa_fp8_head_scales(ispa_dtype dt, const void *x, int64_t n, int32_t n_heads, int32_t head_dim,
                                 int64_t row_stride, float *scales, void *stream) {
  ispa_status st = check_fp8_rows(dt, x, n, n_heads, head_dim, row_stride);
  if (st != ISPA_OK) return st;
  if (scales == nullptr || !aligned4(scales)) return ISPA_E_ARG;
  return hip_status(launch_fp8_head_scales(dt == ISPA_BF16, x, n, n_heads, head_dim, row_stride, scales,
                                           (hipStream_t)stream));
}

ispa_status ispa_fp8_quantize(ispa_dtype dt, const void *x, int64_t n, int32_t n_heads, int32_t head_dim,
                              int64_t row_stride, const float *scales, uint8_t *out, int64_t out_row_stride,
                              void *stream) {
  ispa_status st = check_fp8_rows(dt, x, n, n_heads, head_dim, row_stride);
  if (st != ISPA_OK) return st;
  if (n == 0) return ISPA_OK;
  if (scales == nullptr || !aligned4(scales)) return ISPA_E_ARG;
  if (out == nullptr || ((uintptr_t)out & 7) != 0 || out_row_stride < (int64_t)n_heads * head_dim ||
      out_row_stride % 8 != 0)
    return ISPA_E_ARG;
  return hip_status(launch_fp8_quantize(dt == ISPA_BF16, x, n, n_heads, head_dim, row_stride, scales, out,
                                        out_row_stride, (hipStream_t)stream));
}

namespace {
// FP8 attention: e4m3 q and keys; values bf16 (v_scale NULL) or e4m3 with per-head scales
ispa_status attn_fp8_impl(int32_t n_heads, int32_t head_dim, float softmax_scale, const uint8_t *q, int64_t n_q,
                          int64_t q_row_stride, const float *q_scale, ispa_kv_segment sink, ispa_kv_segment cur,
                          ispa_kv_segment hist, const float *k_scale, const float *v_scale, void *a_loc,
                          void *a_full, float *lse_loc, float *lse_hist, float *lse_full, void *stream) {
  if (n_heads <= 0 || n_q < 0) return ISPA_E_ARG;
  if (head_dim != 128) return ISPA_E_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return ISPA_E_ARG;
  if (n_q > INT32_MAX / 2) return ISPA_E_ARG;
  const int64_t width = (int64_t)n_heads * head_dim;
  if (sink.n < 0 || cur.n < 0 || hist.n < 0) return ISPA_E_ARG;
  if (sink.n + cur.n < 1) return ISPA_E_ARG;
  const bool want_full = a_full != nullptr;
  ispa_kv_segment segs[3] = {sink, cur, hist};
  for (int i = 0; i < 3; ++i) {
    const ispa_kv_segment &sg = segs[i];
    if (i == 2 && !want_full) break;
    if (sg.n == 0) continue;
    if (sg.k == nullptr || sg.v == nullptr || !aligned16(sg.k) || !aligned16(sg.v)) return ISPA_E_ARG;
    if (sg.row_stride < width || sg.row_stride % 16 != 0) return ISPA_E_ARG;
    if (sg.row_stride >= ((int64_t)1 << 23)) return ISPA_E_UNSUPPORTED;
  }
  if (n_q == 0) return ISPA_OK;
  if (q == nullptr || !aligned16(q) || q_row_stride < width || q_row_stride % 16 != 0) return ISPA_E_ARG;
  if (q_scale == nullptr || k_scale == nullptr || !aligned4(q_scale) || !aligned4(k_scale)) return ISPA_E_ARG;
  if (a_loc == nullptr || !aligned16(a_loc)) return ISPA_E_ARG;
  if (a_full != nullptr && !aligned16(a_full)) return ISPA_E_ARG;
  AttnArgs a{};
  a.q = q;
  a.q_stride = q_row_stride;
  a.sink_k = sink.k;
  a.sink_v = sink.v;
  a.sink_n = sink.n;
  a.sink_stride = sink.row_stride;
  a.cur_k = cur.k;
  a.cur_v = cur.v;
  a.cur_n = cur.n;
  a.cur_stride = cur.row_stride;
  a.hist_k = want_full ? hist.k : nullptr;
  a.hist_v = want_full ? hist.v : nullptr;
  a.hist_n = want_full ? hist.n : 0;
  a.hist_stride = want_full ? hist.row_stride : 0;
  a.a_loc = a_loc;
  a.a_full = a_full;
  a.lse_loc = lse_loc;
  a.lse_hist = want_full ? lse_hist : nullptr;
  a.lse_full = want_full ? lse_full : nullptr;
  a.n_q = (int32_t)n_q;
  a.n_heads = n_heads;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.bias_to_score = 1.0f / softmax_scale;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return hip_status(launch_attn_fp8(a, head_dim, (hipStream_t)stream));
}
}  // namespace

ispa_status ispa_attn_dual_fp8(int32_t n_heads, int32_t head_dim, float softmax_scale, const uint8_t *q, int64_t n_q,
                               int64_t q_row_stride, const float *q_scale, ispa_kv_segment sink, ispa_kv_segment cur,
                               ispa_kv_segment hist, const float *k_scale, void *a_loc, void *a_full,
                               float *lse_loc, float *lse_hist, float *lse_full, void *stream) {
  return attn_fp8_impl(n_heads, head_dim, softmax_scale, q, n_q, q_row_stride, q_scale, sink, cur, hist, k_scale,
                       nullptr, a_loc, a_full, lse_loc, lse_hist, lse_full, stream);
}

ispa_status ispa_attn_dual_fp8_pv(int32_t n_heads, int32_t head_dim, float softmax_scale, const uint8_t *q,
                                  int64_t n_q, int64_t q_row_stride, const float *q_scale, ispa_kv_segment sink,
                                  ispa_kv_segment cur, ispa_kv_segment hist, const float *k_scale,
                                  const float *v_scale, void *a_loc, void *a_full, float *lse_loc, float *lse_hist,
                                  float *lse_full, void *stream) {
  if (v_scale == nullptr || !aligned4(v_scale)) return ISPA_E_ARG;
  return attn_fp8_impl(n_heads, head_dim, softmax_scale, q, n_q, q_row_stride, q_scale, sink, cur, hist, k_scale,
                       v_scale, a_loc, a_full, lse_loc, lse_hist, lse_full, stream);
}

// ------------------------------------------------------------------------------------------------
// [lse: H x n_p fp32 | partial (max, sum) states of the key ranges: splits x H x n_p float pairs]
size_t ispa_future_scores_workspace(int32_t n_heads, int64_t n_p) {
  if (n_heads <= 0 || n_p <= 0) return 0;
  const size_t lse = round_up((size_t)n_heads * (size_t)n_p * sizeof(float), 256);
  const size_t part = (size_t)lse_splits_for(n_p, n_heads) * (size_t)n_heads * (size_t)n_p * 2 * sizeof(float);
  return lse + round_up(part, 256);
}

namespace {

// Argument checks of ispa_future_scores (all but the workspace); `total` receives the number of keys.
ispa_status future_scores_check(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                const void *q_proxy, int64_t n_p, int64_t q_row_stride, const ispa_kv_segment *segs,
                                const float *scores, int64_t scores_head_stride, float lambda,
                                const float *hist_token_score, const float *token_score, int64_t *total_out) {
  if (dt != ISPA_BF16) return ISPA_E_UNSUPPORTED;
  if (n_heads <= 0 || n_p <= 0 || n_p > INT32_MAX / 2) return ISPA_E_ARG;
  if (head_dim != 64 && head_dim != 128) return ISPA_E_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale) || !std::isfinite(lambda)) return ISPA_E_ARG;
  const int64_t width = (int64_t)n_heads * head_dim;
  int64_t total = 0;
  for (int i = 0; i < 3; ++i) {
    const ispa_kv_segment &sg = segs[i];
    if (sg.n < 0) return ISPA_E_ARG;
    if (sg.n == 0) continue;
    if (sg.k == nullptr || !aligned16(sg.k)) return ISPA_E_ARG;
    if (sg.row_stride < width || sg.row_stride % 8 != 0) return ISPA_E_ARG;
    if (sg.row_stride >= ((int64_t)1 << 23)) return ISPA_E_UNSUPPORTED;
    total += sg.n;
  }
  if (total < 1 || total > INT32_MAX) return ISPA_E_ARG;
  if (q_proxy == nullptr || !aligned16(q_proxy) || q_row_stride < width || q_row_stride % 8 != 0)
    return ISPA_E_ARG;
  if (scores == nullptr || !aligned4(scores) || scores_head_stride < total) return ISPA_E_ARG;
  if (token_score != nullptr && !aligned4(token_score)) return ISPA_E_ARG;
  if (hist_token_score != nullptr && !aligned4(hist_token_score)) return ISPA_E_ARG;
  *total_out = total;
  return ISPA_OK;
}

// The two passes of ispa_future_scores on checked arguments, with scratch at ws (16-byte aligned, at
// least ispa_future_scores_workspace(n_heads, n_p) bytes).
ispa_status future_scores_run(int32_t n_heads, int32_t head_dim, float softmax_scale, const void *q_proxy,
                              int64_t n_p, int64_t q_row_stride, ispa_kv_segment sink, ispa_kv_segment cur,
                              ispa_kv_segment hist, int64_t total, float *scores, int64_t scores_head_stride,
                              float lambda, const float *hist_token_score, float *token_score, void *ws,
                              hipStream_t s) {
  float *lse = (float *)ws;
  // pass 1: log-sum-exp of every proxy over all keys (values are not read; the key pointers stand in)
  AttnArgs a{};
  const bool local_empty = sink.n + cur.n == 0;
  a.q = q_proxy;
  a.q_stride = q_row_stride;
  a.sink_k = a.sink_v = sink.k;
  a.sink_n = sink.n;
  a.sink_stride = sink.row_stride;
  a.cur_k = a.cur_v = local_empty ? hist.k : cur.k;
  a.cur_n = local_empty ? hist.n : cur.n;
  a.cur_stride = local_empty ? hist.row_stride : cur.row_stride;
  a.hist_k = a.hist_v = local_empty ? nullptr : hist.k;
  a.hist_n = local_empty ? 0 : hist.n;
  a.hist_stride = local_empty ? 0 : hist.row_stride;
  a.lse_full = lse;
  a.lse_part = (float *)((uint8_t *)ws + round_up((size_t)n_heads * (size_t)n_p * sizeof(float), 256));
  a.lse_splits = lse_splits_for(n_p, n_heads);
  a.n_q = (int32_t)n_p;
  a.n_heads = n_heads;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.bias_to_score = 1.0f / softmax_scale;
  hipError_t e = launch_attn_lse_bf16(a, head_dim, s);
  if (e != hipSuccess) return hip_status(e);
  // pass 2: per-key sums of the proxies' weights
  e = launch_future_colsum_bf16((const uint16_t *)q_proxy, q_row_stride, n_p, lse, (const uint16_t *)sink.k,
                                sink.row_stride, sink.n, (const uint16_t *)cur.k, cur.row_stride, cur.n,
                                (const uint16_t *)hist.k, hist.row_stride, hist.n, n_heads, head_dim,
                                a.scale_log2, scores, scores_head_stride, s);
  if (e != hipSuccess) return hip_status(e);
  if (token_score != nullptr)
    e = launch_token_scores(scores, scores_head_stride, n_heads, total, lambda, hist_token_score, token_score, s);
  return hip_status(e);
}

}  // namespace

ispa_status ispa_future_scores(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                               const void *q_proxy, int64_t n_p, int64_t q_row_stride,
                               ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                               float *scores, int64_t scores_head_stride, float lambda,
                               const float *hist_token_score, float *token_score, void *ws,
                               size_t ws_bytes, void *stream) {
  const ispa_kv_segment segs[3] = {sink, cur, hist};
  int64_t total = 0;
  ispa_status st = future_scores_check(dt, n_heads, head_dim, softmax_scale, q_proxy, n_p, q_row_stride, segs,
                                       scores, scores_head_stride, lambda, hist_token_score, token_score, &total);
  if (st != ISPA_OK) return st;
  if (ws == nullptr || ws_bytes < ispa_future_scores_workspace(n_heads, n_p)) return ISPA_E_WORKSPACE;
  if (!aligned16(ws)) return ISPA_E_ARG;
  return future_scores_run(n_heads, head_dim, softmax_scale, q_proxy, n_p, q_row_stride, sink, cur, hist, total,
                           scores, scores_head_stride, lambda, hist_token_score, token_score, ws,
                           (hipStream_t)stream);
}

// ------------------------------------------------------------------------------------------------
// Scratch of ispa_future_scores_noalloc: one array per GPU, held until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
}  // extern "C"

static __device__ __align__(256) uint8_t scratch[ISPA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

ispa_status scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ISPA_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ISPA_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ISPA_OK;
}
}  // namespace

extern "C" {

ispa_status ispa_future_scores_noalloc(ispa_dtype dt, int32_t n_heads, int32_t head_dim, float softmax_scale,
                                       const void *q_proxy, int64_t n_p, int64_t q_row_stride,
                                       ispa_kv_segment sink, ispa_kv_segment cur, ispa_kv_segment hist,
                                       float *scores, int64_t scores_head_stride, float lambda,
                                       const float *hist_token_score, float *token_score, void *stream) {
  const ispa_kv_segment segs[3] = {sink, cur, hist};
  int64_t total = 0;
  ispa_status st = future_scores_check(dt, n_heads, head_dim, softmax_scale, q_proxy, n_p, q_row_stride, segs,
                                       scores, scores_head_stride, lambda, hist_token_score, token_score, &total);
  if (st != ISPA_OK) return st;
  if (ispa_future_scores_workspace(n_heads, n_p) > (size_t)ISPA_NOALLOC_SCRATCH_BYTES) return ISPA_E_WORKSPACE;
  void *ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != ISPA_OK) return st;
  // every word of the scratch that a pass reads is written earlier in the same call (the per-split
  // states by pass 1's workgroups, the merged log-sum-exp rows by its merge), so nothing is cleared
  return future_scores_run(n_heads, head_dim, softmax_scale, q_proxy, n_p, q_row_stride, sink, cur, hist, total,
                           scores, scores_head_stride, lambda, hist_token_score, token_score, ws,
                           (hipStream_t)stream);
}

// ------------------------------------------------------------------------------------------------
ispa_status ispa_kv_merge(ispa_dtype dt, int32_t width, const void *k, const void *v, int64_t n,
                          int64_t in_stride, const int32_t *offsets, const int32_t *members,
                          int64_t n_groups, void *k_out, void *v_out, int64_t out_stride,
                          float *bias_out, void *stream) {
  if (dt != ISPA_BF16 && dt != ISPA_F32) return ISPA_E_UNSUPPORTED;
  if (width <= 0 || n < 0 || n_groups < 0) return ISPA_E_ARG;
  if (width % 8 != 0) return ISPA_E_UNSUPPORTED;
  if (n_groups > (int64_t)1 << 26 || n > INT32_MAX) return ISPA_E_ARG;   // grid of 64 threads per group
  if (n_groups == 0) return ISPA_OK;
  if (offsets == nullptr || ((uintptr_t)offsets & 3) != 0) return ISPA_E_ARG;
  if (n > 0 && (k == nullptr || v == nullptr || !aligned16(k) || !aligned16(v))) return ISPA_E_ARG;
  if (n > 0 && (members == nullptr || ((uintptr_t)members & 3) != 0)) return ISPA_E_ARG;
  if (n > 0 && (in_stride < width || in_stride % 8 != 0)) return ISPA_E_ARG;
  if (k_out == nullptr || v_out == nullptr || !aligned16(k_out) || !aligned16(v_out)) return ISPA_E_ARG;
  if (out_stride < width || out_stride % 8 != 0) return ISPA_E_ARG;
  if (bias_out != nullptr && ((uintptr_t)bias_out & 3) != 0) return ISPA_E_ARG;
  return hip_status(launch_kv_merge(dt == ISPA_BF16, width, k, v, n, in_stride, offsets, members,
                                    n_groups, k_out, v_out, out_stride, bias_out, (hipStream_t)stream));
}

// ------------------------------------------------------------------------------------------------
size_t ispa_absorb_accumulate_workspace(int64_t n_rows, int32_t d) {
  (void)n_rows;
  (void)d;
  return 0;
}

ispa_status ispa_absorb_accumulate(ispa_dtype dt, int64_t n_rows, int32_t d, const void *a_loc,
                                   const void *a_full, float *G, float *X, float *F, void *ws,
                                   size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (dt != ISPA_BF16 && dt != ISPA_F32) return ISPA_E_UNSUPPORTED;
  if (n_rows < 0 || d <= 0) return ISPA_E_ARG;
  if (d % 64 != 0) return ISPA_E_UNSUPPORTED;
  if (G == nullptr || X == nullptr || !aligned16(G) || !aligned16(X)) return ISPA_E_ARG;
  if (F != nullptr && !aligned16(F)) return ISPA_E_ARG;
  if (n_rows == 0) return ISPA_OK;
  if (a_loc == nullptr || a_full == nullptr || !aligned16(a_loc) || !aligned16(a_full)) return ISPA_E_ARG;
  if (n_rows > INT32_MAX) return ISPA_E_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dt == ISPA_BF16)
    return hip_status(launch_gram_bf16(n_rows, d, (const uint16_t *)a_loc, (const uint16_t *)a_full,
                                       G, X, F, s));
  // fp32 rows: three GEMMs  G += A_loc^T A_loc, X += A_loc^T A_full, F += A_full^T A_full
  GemmShape sh{};
  sh.M = d;
  sh.N = d;
  sh.K = (int)n_rows;
  sh.lda = d;
  sh.ldb = d;
  sh.ldc = d;
  sh.ta = 1;
  sh.tb = 0;
  sh.alpha = 1.f;
  sh.beta = 1.f;
  GemmBatch b{};
  const float *al = (const float *)a_loc, *af = (const float *)a_full;
  int cnt = 0;
  b.A[cnt] = al; b.B[cnt] = al; b.C[cnt] = G; ++cnt;
  b.A[cnt] = al; b.B[cnt] = af; b.C[cnt] = X; ++cnt;
  if (F != nullptr) { b.A[cnt] = af; b.B[cnt] = af; b.C[cnt] = F; ++cnt; }
  return hip_status(launch_gemm_f32(b, cnt, sh, nullptr, 0, s));
}

// ------------------------------------------------------------------------------------------------
ispa_status ispa_absorb_accumulate_batched(ispa_dtype dt, int64_t n_rows, int32_t d, int32_t batch,
                                           const void *const *a_loc, const void *const *a_full, float *const *G,
                                           float *const *X, float *const *F, void *stream) {
  if (dt != ISPA_BF16 && dt != ISPA_F32) return ISPA_E_UNSUPPORTED;
  if (n_rows < 0 || d <= 0 || batch < 0) return ISPA_E_ARG;
  if (d % 64 != 0) return ISPA_E_UNSUPPORTED;
  if (n_rows > INT32_MAX) return ISPA_E_ARG;
  if (batch == 0) return ISPA_OK;
  ispa_status st;
  if ((st = check_ptr_array(G, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(X, batch)) != ISPA_OK) return st;
  if (F != nullptr && (st = check_ptr_array(F, batch)) != ISPA_OK) return st;
  if (n_rows == 0) return ISPA_OK;
  if (a_loc == nullptr || a_full == nullptr) return ISPA_E_ARG;
  for (int32_t i = 0; i < batch; ++i)
    if (a_loc[i] == nullptr || a_full[i] == nullptr || !aligned16(a_loc[i]) || !aligned16(a_full[i]))
      return ISPA_E_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dt == ISPA_BF16)
    return hip_status(launch_gram_bf16_batch(n_rows, d, batch, (const uint16_t *const *)a_loc,
                                             (const uint16_t *const *)a_full, G, X, F, s));
  for (int32_t i = 0; i < batch; ++i) {
    st = ispa_absorb_accumulate(dt, n_rows, d, a_loc[i], a_full[i], G[i], X[i], F != nullptr ? F[i] : nullptr,
                                nullptr, 0, stream);
    if (st != ISPA_OK) return st;
  }
  return ISPA_OK;
}

// ------------------------------------------------------------------------------------------------
ispa_status ispa_absorb_accumulate_fp8(int64_t n_rows, int32_t d, int32_t head_dim, const uint8_t *a_loc,
                                       const float *s_loc, const uint8_t *a_full, const float *s_full, float *G,
                                       float *X, float *F, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (n_rows < 0 || d <= 0) return ISPA_E_ARG;
  if (head_dim != 64 && head_dim != 128) return ISPA_E_UNSUPPORTED;
  if (d % 64 != 0 || d % head_dim != 0) return ISPA_E_UNSUPPORTED;
  if (G == nullptr || X == nullptr || !aligned16(G) || !aligned16(X)) return ISPA_E_ARG;
  if (F != nullptr && !aligned16(F)) return ISPA_E_ARG;
  if (n_rows == 0) return ISPA_OK;
  if (a_loc == nullptr || a_full == nullptr || !aligned16(a_loc) || !aligned16(a_full)) return ISPA_E_ARG;
  if (s_loc == nullptr || s_full == nullptr || !aligned4(s_loc) || !aligned4(s_full)) return ISPA_E_ARG;
  if (n_rows > INT32_MAX) return ISPA_E_ARG;
  return hip_status(launch_gram_fp8(n_rows, d, head_dim, a_loc, s_loc, a_full, s_full, G, X, F,
                                    (hipStream_t)stream));
}

size_t ispa_absorb_solve_workspace(int32_t d, int32_t batch) {
  if (d <= 0 || batch <= 0) return 0;
  return solve_layout(d).total(batch);
}

namespace {

// The error at the optimum, requested from the solve: F per layer, outputs, and the partial sums'
// region (4 terms x batch x stride doubles: <H, W W^T>, <F, W W^T>, ||Y||^2, ||dW||^2 per tile).
struct EpsRequest {
  const float *const *F;
  double *eps, *ref;
  double *part;
  int64_t stride;
};

// A second stream per device for work that runs beside the caller's stream inside one call (created
// once, default priority, non-blocking; the call forks to it and joins back through events).
hipError_t side_stream(hipStream_t *out) {
  static std::mutex mu;
  static std::vector<hipStream_t> streams;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)streams.size() <= dev) streams.resize(dev + 1, nullptr);
  if (streams[dev] == nullptr) {
    e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (e != hipSuccess) {
      streams[dev] = nullptr;
      return e;
    }
  }
  *out = streams[dev];
  return hipSuccess;
}
// Two events of one call (no timing), destroyed when the call returns (a recorded event may be
// destroyed before it completes).
struct EventPair {
  hipEvent_t e[2] = {nullptr, nullptr};
  hipError_t create() {
    for (auto &x : e) {
      const hipError_t r = hipEventCreateWithFlags(&x, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  ~EventPair() {
    for (auto &x : e)
      if (x != nullptr) (void)hipEventDestroy(x);
  }
};

ispa_status solve_impl(int32_t d, int32_t batch, float lambda, const float *const *G, const float *const *X,
                       const float *const *W, int32_t w_is_linear_weight, float *const *dW, int32_t *info,
                       void *ws, const EpsRequest *er, hipStream_t s) {
  const SolveLayout lay = solve_layout(d);

  const int nb = solve_nb(d);
  const int nt = (d + nb - 1) / nb;
  const int64_t mat_f = (int64_t)(lay.mat / sizeof(float));
  const int64_t per_f = (int64_t)(lay.per_layer / sizeof(float));

  const int tiles = gemm_tiles(d, d);
  auto term = [&](int g, int layer) { return er->part + ((int64_t)g * batch + layer) * er->stride; };
  // the error at the optimum runs on a second stream of this device (fork and join through events)
  hipStream_t side = nullptr;
  EventPair ev;
  if (er != nullptr) {
    if (side_stream(&side) != hipSuccess || ev.create() != hipSuccess) return ISPA_E_HIP;
  }
  hipEvent_t side_ready = ev.e[0], side_done = ev.e[1];
  for (int p0 = 0; p0 < batch; p0 += kMaxBatch) {
    const int cnt = std::min(batch - p0, kMaxBatch);
    float *base = (float *)ws + (int64_t)p0 * per_f;
    // per-layer regions: [L | B | Wn | Linv], stride per_f
    auto Lp = [&](int i) { return base + (int64_t)i * per_f; };
    auto Bp = [&](int i) { return base + (int64_t)i * per_f + mat_f; };
    auto Wp = [&](int i) { return base + (int64_t)i * per_f + 2 * mat_f; };
    auto Vp = [&](int i) { return base + (int64_t)i * per_f + 3 * mat_f; };
    const int64_t linv_blk = (int64_t)nb * nb;

    ISPA_TRY(launch_zero_i32(info + p0, cnt, s));
    CPtrBatch g{};
    for (int i = 0; i < cnt; ++i) g.p[i] = G[p0 + i];

    // W in the standard orientation (y = A W)
    const float *Wuse[kMaxBatch];
    if (w_is_linear_weight) {
      CPtrBatch in{};
      PtrBatch out{};
      for (int i = 0; i < cnt; ++i) {
        in.p[i] = W[p0 + i];
        out.p[i] = Wp(i);
        Wuse[i] = Wp(i);
      }
      ISPA_TRY(launch_transpose(in, out, d, cnt, s));
    } else {
      for (int i = 0; i < cnt; ++i) Wuse[i] = W[p0 + i];
    }

    // B = (X - G) W: C = X - G goes to the factor's region first (a plain GEMM then reads one operand
    // instead of subtracting two in its inner loop), and G + lambda I overwrites it afterwards
    {
      CPtrBatch x{};
      PtrBatch c{};
      for (int i = 0; i < cnt; ++i) {
        x.p[i] = X[p0 + i];
        c.p[i] = Lp(i);
      }
      ISPA_TRY(launch_sub(x, g, c, d, cnt, s));
      GemmBatch b{};
      GemmShape sh{};
      sh.M = d; sh.N = d; sh.K = d;
      sh.lda = d; sh.ldb = d; sh.ldc = d;
      sh.ta = 0; sh.tb = 0;
      sh.alpha = 1.f; sh.beta = 0.f;
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Lp(i);
        b.B[i] = Wuse[i];
        b.C[i] = Bp(i);
      }
      ISPA_TRY(launch_gemm_f32(b, cnt, sh, nullptr, 0, s));
    }
    if (er != nullptr) {
      // eps = <W, H W> - <dW, B> - lambda ||dW||^2 with H = (F + G) - (X + X^T): one product W W^T, lower
      // tiles only, whose epilogue forms H element by element in fp64 from F, G and X (and X's mirror
      // element) and reduces the product against H and against F (<F, W W^T> = ||A_full W||^2 is the
      // reference). It depends on W and the statistics only, so it runs on a second stream beside the
      // factorisation (whose diagonal blocks occupy 30 workgroups), joined before the reduction.
      ISPA_TRY(hipEventRecord(side_ready, s));
      ISPA_TRY(hipStreamWaitEvent(side, side_ready, 0));
      GemmBatch b{};
      GemmShape sh{};
      sh.M = d; sh.N = d; sh.K = d;
      sh.lda = d; sh.ldb = d; sh.ldc = d; sh.lde = d;
      sh.ta = 0; sh.tb = 1; sh.dot = 2; sh.sym = 1; sh.hform = 1;
      sh.alpha = 1.f; sh.beta = 0.f;
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Wuse[i];
        b.B[i] = Wuse[i];
        b.E[i] = X[p0 + i];
        b.A2[i] = G[p0 + i];
        b.E2[i] = er->F[p0 + i];
      }
      ISPA_TRY(launch_gemm_f32(b, cnt, sh, term(0, p0), er->stride, side, term(1, p0)));
      ISPA_TRY(hipEventRecord(side_done, side));
    }
    ISPA_TRY(launch_shift_copy(g, Lp(0), per_f, d, lambda, cnt, s));

    // Cholesky L L^T = G + lambda I, recursive over block columns: factor the leading half, form the
    // panel below it (a triangular solve from the right, itself recursive: its single block columns
    // are products with a diagonal block's inverse, in place), remove the panel's contribution from
    // the trailing half with one lower-tile product whose depth is the whole leading half, then
    // factor the trailing half. The same products as the block-column-by-block-column form, in fewer
    // and deeper GEMMs. A single block is the diagonal-block kernel (factor and inverse).
    auto panel = [&](int r0, int r1, int j) -> hipError_t {   // L[r0:r1, j] = A[r0:r1, j] Linv_j^T
      GemmBatch b{};
      GemmShape sh{};
      sh.M = (r1 - r0) * nb; sh.N = nb; sh.K = nb;
      sh.lda = d; sh.ldb = nb; sh.ldc = d;
      sh.ta = 0; sh.tb = 1;
      sh.alpha = 1.f; sh.beta = 0.f;
      sh.inplace = 1;                        // C = A: each row's nb columns in one workgroup
      for (int i = 0; i < cnt; ++i) {
        float *pnl = Lp(i) + (int64_t)(r0 * nb) * d + j * nb;
        b.A[i] = pnl;
        b.B[i] = Vp(i) + j * linv_blk;
        b.C[i] = pnl;
      }
      return launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
    };
    // L[r0:r1, c0:c1] = A[r0:r1, c0:c1] L[c0:c1, c0:c1]^-T, over the block columns c0 .. c1
    std::function<hipError_t(int, int, int, int)> trsm = [&](int r0, int r1, int c0, int c1) -> hipError_t {
      if (c1 - c0 == 1) return panel(r0, r1, c0);
      const int cm = c0 + (c1 - c0) / 2;
      hipError_t e = trsm(r0, r1, c0, cm);
      if (e != hipSuccess) return e;
      GemmBatch b{};
      GemmShape sh{};
      sh.M = (r1 - r0) * nb; sh.N = (c1 - cm) * nb; sh.K = (cm - c0) * nb;
      sh.lda = d; sh.ldb = d; sh.ldc = d;
      sh.ta = 0; sh.tb = 1;
      sh.alpha = -1.f; sh.beta = 1.f;
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Lp(i) + (int64_t)(r0 * nb) * d + c0 * nb;   // L[r0:r1, c0:cm]
        b.B[i] = Lp(i) + (int64_t)(cm * nb) * d + c0 * nb;   // L[cm:c1, c0:cm] (transposed)
        b.C[i] = Lp(i) + (int64_t)(r0 * nb) * d + cm * nb;   // A[r0:r1, cm:c1]
      }
      e = launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
      return e != hipSuccess ? e : trsm(r0, r1, cm, c1);
    };
    std::function<hipError_t(int, int)> chol = [&](int k0, int k1) -> hipError_t {
      if (k1 - k0 == 1)
        return launch_potrf_diag(Lp(0), per_f, d, k0 * nb, nb, Vp(0) + k0 * linv_blk, per_f, info + p0, cnt, s);
      const int km = k0 + (k1 - k0) / 2;
      hipError_t e = chol(k0, km);
      if (e == hipSuccess) e = trsm(km, k1, k0, km);
      if (e != hipSuccess) return e;
      // trailing half: A[km:k1, km:k1] -= L[km:k1, k0:km] L[km:k1, k0:km]^T (lower tiles)
      GemmBatch b{};
      GemmShape sh{};
      sh.M = (k1 - km) * nb; sh.N = sh.M; sh.K = (km - k0) * nb;
      sh.lda = d; sh.ldb = d; sh.ldc = d;
      sh.ta = 0; sh.tb = 1; sh.lower = 1;
      sh.alpha = -1.f; sh.beta = 1.f;
      for (int i = 0; i < cnt; ++i) {
        const float *pnl = Lp(i) + (int64_t)(km * nb) * d + k0 * nb;
        b.A[i] = pnl;
        b.B[i] = pnl;
        b.C[i] = Lp(i) + (int64_t)(km * nb) * d + km * nb;
      }
      e = launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
      return e != hipSuccess ? e : chol(km, k1);
    };
    {
      const hipError_t e = chol(0, nt);
      if (e != hipSuccess) return ISPA_E_HIP;
    }

    // Triangular sweeps, recursive over block rows: a range of block rows is split in two halves; the
    // first half is solved, its contribution to the second half is one GEMM over the whole half, then
    // the second half is solved. The same products as a block-row-by-block-row sweep, in fewer and
    // larger GEMMs (the top split of d = 1536 is 768 x 1536 x 768 per layer). A single block row is
    // the product with the diagonal block's inverse, in place.
    auto leaf = [&](int k, bool trans) -> hipError_t {
      const int k0 = k * nb;
      GemmBatch b{};
      GemmShape sh{};
      sh.M = nb; sh.N = d; sh.K = nb;
      sh.lda = nb; sh.ldb = d; sh.ldc = d;
      sh.ta = trans ? 1 : 0; sh.tb = 0;
      sh.alpha = 1.f; sh.beta = 0.f;
      sh.inplace = 1;                        // C = B: each column's nb rows in one workgroup
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Vp(i) + k * linv_blk;
        b.B[i] = Bp(i) + (int64_t)k0 * d;
        b.C[i] = Bp(i) + (int64_t)k0 * d;
      }
      return launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
    };
    // forward, L Y = B on block rows [k0, k1): Y_hi -= L[hi, lo] Y_lo between the halves
    std::function<hipError_t(int, int)> fwd = [&](int k0, int k1) -> hipError_t {
      if (k1 - k0 == 1) return leaf(k0, false);
      const int km = k0 + (k1 - k0) / 2;
      hipError_t e = fwd(k0, km);
      if (e != hipSuccess) return e;
      GemmBatch b{};
      GemmShape sh{};
      sh.M = (k1 - km) * nb; sh.N = d; sh.K = (km - k0) * nb;
      sh.lda = d; sh.ldb = d; sh.ldc = d;
      sh.ta = 0; sh.tb = 0;
      sh.alpha = -1.f; sh.beta = 1.f;
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Lp(i) + (int64_t)(km * nb) * d + k0 * nb;   // L[hi rows][lo columns]
        b.B[i] = Bp(i) + (int64_t)(k0 * nb) * d;             // Y[lo rows]
        b.C[i] = Bp(i) + (int64_t)(km * nb) * d;
      }
      e = launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
      return e != hipSuccess ? e : fwd(km, k1);
    };
    // back, L^T X = Y on block rows [k0, k1): Y_lo -= L[hi, lo]^T X_hi between the halves
    std::function<hipError_t(int, int)> back = [&](int k0, int k1) -> hipError_t {
      if (k1 - k0 == 1) return leaf(k0, true);
      const int km = k0 + (k1 - k0) / 2;
      hipError_t e = back(km, k1);
      if (e != hipSuccess) return e;
      GemmBatch b{};
      GemmShape sh{};
      sh.M = (km - k0) * nb; sh.N = d; sh.K = (k1 - km) * nb;
      sh.lda = d; sh.ldb = d; sh.ldc = d;
      sh.ta = 1; sh.tb = 0;
      sh.alpha = -1.f; sh.beta = 1.f;
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = Lp(i) + (int64_t)(km * nb) * d + k0 * nb;   // opA[r][kk] = L[km nb + kk][k0 nb + r]
        b.B[i] = Bp(i) + (int64_t)(km * nb) * d;             // X[hi rows]
        b.C[i] = Bp(i) + (int64_t)(k0 * nb) * d;
      }
      e = launch_gemm_f32(b, cnt, sh, nullptr, 0, s);
      return e != hipSuccess ? e : back(k0, km);
    };
    ISPA_TRY(fwd(0, nt));
    // ||Y||^2 = <dW, B> at the optimum (B^T (L L^T)^-1 B), before the back sweep overwrites Y
    if (er != nullptr) ISPA_TRY(launch_sumsq_tiles(Bp(0), per_f, d, cnt, term(2, p0), er->stride, s));
    ISPA_TRY(back(0, nt));
    if (er != nullptr) {
      ISPA_TRY(launch_sumsq_tiles(Bp(0), per_f, d, cnt, term(3, p0), er->stride, s));
      // the error product ran beside the factorisation: its partials are complete before the reduction
      ISPA_TRY(hipStreamWaitEvent(s, side_done, 0));
    }
    // dW in the caller's orientation
    CPtrBatch in{};
    PtrBatch out{};
    for (int i = 0; i < cnt; ++i) {
      in.p[i] = Bp(i);
      out.p[i] = dW[p0 + i];
    }
    if (w_is_linear_weight)
      ISPA_TRY(launch_transpose(in, out, d, cnt, s));
    else
      ISPA_TRY(launch_copy(in, out, d, cnt, s));
  }
  if (er != nullptr) {
    const double coef_eps[4] = {1.0, 0.0, -1.0, -(double)lambda};
    ISPA_TRY(launch_reduce_partials(er->part, batch, er->stride, tiles, 4, coef_eps, er->eps, s, info));
    if (er->ref != nullptr) {
      const double coef_ref[1] = {1.0};
      ISPA_TRY(launch_reduce_partials(term(1, 0), batch, er->stride, tiles, 1, coef_ref, er->ref, s));
    }
  }
  return ISPA_OK;
}

ispa_status check_solve_args(int32_t d, int32_t batch, float lambda, const float *const *G, const float *const *X,
                             const float *const *W, float *const *dW, const int32_t *info) {
  ispa_status st = check_square_batch(d, batch);
  if (st != ISPA_OK) return st;
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return ISPA_E_ARG;
  if (batch == 0) return ISPA_OK;
  if ((st = check_ptr_array(G, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(X, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(W, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array((const float *const *)dW, batch)) != ISPA_OK) return st;
  if (info == nullptr) return ISPA_E_ARG;
  return ISPA_OK;
}

// doubles per (term, layer) of the error's partial sums: one per 128 x 128 tile, 256-byte rounded
int64_t eps_part_stride(int d) { return (int64_t)round_up((size_t)gemm_tiles(d, d), 32); }

}  // namespace

ispa_status ispa_absorb_solve(int32_t d, int32_t batch, float lambda, const float *const *G,
                              const float *const *X, const float *const *W, int32_t w_is_linear_weight,
                              float *const *dW, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  ispa_status st = check_solve_args(d, batch, lambda, G, X, W, dW, info);
  if (st != ISPA_OK || batch == 0) return st;
  const size_t need = solve_layout(d).total(batch);
  if (ws == nullptr || ws_bytes < need) return ISPA_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ISPA_E_ARG;
  return solve_impl(d, batch, lambda, G, X, W, w_is_linear_weight, dW, info, ws, nullptr, (hipStream_t)stream);
}

size_t ispa_absorb_solve_eps_workspace(int32_t d, int32_t batch) {
  if (d <= 0 || batch <= 0) return 0;
  return solve_layout(d).total(batch) + 4 * (size_t)batch * (size_t)eps_part_stride(d) * sizeof(double);
}

ispa_status ispa_absorb_solve_eps(int32_t d, int32_t batch, float lambda, const float *const *G,
                                  const float *const *X, const float *const *F, const float *const *W,
                                  int32_t w_is_linear_weight, float *const *dW, int32_t *info, double *eps,
                                  double *ref, void *ws, size_t ws_bytes, void *stream) {
  ispa_status st = check_solve_args(d, batch, lambda, G, X, W, dW, info);
  if (st != ISPA_OK || batch == 0) return st;
  if ((st = check_ptr_array(F, batch)) != ISPA_OK) return st;
  if (eps == nullptr || ((uintptr_t)eps & 7) != 0 || ((uintptr_t)ref & 7) != 0) return ISPA_E_ARG;
  const size_t need = ispa_absorb_solve_eps_workspace(d, batch);
  if (ws == nullptr || ws_bytes < need) return ISPA_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ISPA_E_ARG;
  EpsRequest er;
  er.F = F;
  er.eps = eps;
  er.ref = ref;
  er.part = (double *)((uint8_t *)ws + solve_layout(d).total(batch));
  er.stride = eps_part_stride(d);
  return solve_impl(d, batch, lambda, G, X, W, w_is_linear_weight, dW, info, ws, &er, (hipStream_t)stream);
}


// ------------------------------------------------------------------------------------------------
size_t ispa_layer_error_workspace(int32_t d, int32_t batch) {
  if (d <= 0 || batch <= 0) return 0;
  return err_layout(d).total(batch);
}

ispa_status ispa_layer_error(int32_t d, int32_t batch, const float *const *G, const float *const *X,
                             const float *const *F, const float *const *W, int32_t w_is_linear_weight,
                             const float *const *dW, double *eps, double *ref, void *ws, size_t ws_bytes,
                             void *stream) {
  ispa_status st = check_square_batch(d, batch);
  if (st != ISPA_OK) return st;
  if (batch == 0) return ISPA_OK;
  if ((st = check_ptr_array(G, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(X, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(F, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(W, batch)) != ISPA_OK) return st;
  if ((st = check_ptr_array(dW, batch)) != ISPA_OK) return st;
  if (eps == nullptr) return ISPA_E_ARG;
  const ErrLayout lay = err_layout(d);
  if (ws == nullptr || ws_bytes < lay.total(batch)) return ISPA_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ISPA_E_ARG;

  hipStream_t s = (hipStream_t)stream;
  const int64_t mat_f = (int64_t)(lay.mat / sizeof(float));
  float *mats = (float *)ws;                                        // [batch][2][mat]
  double *part = (double *)((char *)ws + 2 * lay.mat * (size_t)batch);   // [3][batch][part]
  const int64_t part_d = (int64_t)(lay.part / sizeof(double));

  for (int p0 = 0; p0 < batch; p0 += kMaxBatch) {
    const int cnt = std::min(batch - p0, kMaxBatch);
    auto Wn = [&](int i) { return mats + (int64_t)(p0 + i) * 2 * mat_f; };
    auto Wp = [&](int i) { return mats + (int64_t)(p0 + i) * 2 * mat_f + mat_f; };
    const float *Wuse[kMaxBatch];
    if (w_is_linear_weight) {
      CPtrBatch in{}, in2{}, a{}, b{};
      PtrBatch out{}, out2{}, o{};
      for (int i = 0; i < cnt; ++i) {
        in.p[i] = W[p0 + i];
        out.p[i] = Wn(i);
        in2.p[i] = dW[p0 + i];
        out2.p[i] = Wp(i);
        a.p[i] = Wn(i);
        b.p[i] = Wp(i);
        o.p[i] = Wp(i);
        Wuse[i] = Wn(i);
      }
      ISPA_TRY(launch_transpose(in, out, d, cnt, s));
      ISPA_TRY(launch_transpose(in2, out2, d, cnt, s));
      ISPA_TRY(launch_add(a, b, o, d, cnt, s));
    } else {
      CPtrBatch a{}, b{};
      PtrBatch o{};
      for (int i = 0; i < cnt; ++i) {
        a.p[i] = W[p0 + i];
        b.p[i] = dW[p0 + i];
        o.p[i] = Wp(i);
        Wuse[i] = W[p0 + i];
      }
      ISPA_TRY(launch_add(a, b, o, d, cnt, s));
    }
    // eps = <F, W W^T> - 2 <X, W' W^T> + <G, W' W'^T>  (W' = W + dW; each <., .> equals the
    // corresponding <W_a, S W_b> of the residual expansion). The first and last products are
    // symmetric, so only their lower tiles are formed.
    for (int term = 0; term < 3; ++term) {
      GemmShape sh{};
      sh.M = d; sh.N = d; sh.K = d;
      sh.lda = d; sh.ldb = d; sh.ldc = d; sh.lde = d;
      sh.ta = 0; sh.tb = 1; sh.dot = 1;
      sh.sym = term != 1;
      sh.alpha = 1.f; sh.beta = 0.f;
      GemmBatch b{};
      for (int i = 0; i < cnt; ++i) {
        b.A[i] = term == 0 ? Wuse[i] : Wp(i);
        b.B[i] = term == 2 ? Wp(i) : Wuse[i];
        b.E[i] = term == 0 ? F[p0 + i] : term == 1 ? X[p0 + i] : G[p0 + i];
      }
      ISPA_TRY(launch_gemm_f32(b, cnt, sh, part + ((int64_t)term * batch + p0) * part_d, part_d, s));
    }
  }
  const double coef_eps[3] = {1.0, -2.0, 1.0};
  ISPA_TRY(launch_reduce_partials(part, batch, part_d, lay.tiles, 3, coef_eps, eps, s));
  if (ref != nullptr) {
    const double coef_ref[1] = {1.0};
    ISPA_TRY(launch_reduce_partials(part, batch, part_d, lay.tiles, 1, coef_ref, ref, s));
  }
  return ISPA_OK;
}

// ------------------------------------------------------------------------------------------------
ispa_status ispa_rank_layers(const double *eps, int32_t n_layers, int32_t k, int32_t *selected,
                             uint8_t *is_l_layer) {
  if (n_layers < 0 || k < 0 || k > n_layers) return ISPA_E_ARG;
  if (n_layers > 0 && eps == nullptr) return ISPA_E_ARG;
  if (k > 0 && selected == nullptr) return ISPA_E_ARG;
  std::vector<int32_t> order(n_layers);
  std::iota(order.begin(), order.end(), 0);
  auto key = [&](int32_t i) { return std::isnan(eps[i]) ? INFINITY : eps[i]; };
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return key(a) < key(b); });
  for (int32_t i = 0; i < k; ++i) selected[i] = order[i];
  if (is_l_layer != nullptr) {
    std::memset(is_l_layer, 0, (size_t)n_layers);
    for (int32_t i = 0; i < k; ++i) is_l_layer[order[i]] = 1;
  }
  return ISPA_OK;
}

// ------------------------------------------------------------------------------------------------
ispa_status ispa_apply_delta(int32_t d_in, int32_t d_out, const float *W, const float *dW,
                             int32_t w_is_linear_weight, void *w_new, void *stream) {
  if (d_in <= 0 || d_out <= 0) return ISPA_E_ARG;
  if (W == nullptr || dW == nullptr || w_new == nullptr) return ISPA_E_ARG;
  if (!aligned16(W) || !aligned16(dW) || !aligned16(w_new)) return ISPA_E_ARG;
  return hip_status(launch_apply_delta(W, dW, d_in, d_out, w_is_linear_weight ? 1 : 0,
                                       (uint16_t *)w_new, (hipStream_t)stream));
}

ispa_status ispa_project(int64_t n, int32_t d_in, int32_t d_out, const void *a, int64_t lda,
                         const void *w, void *y, int64_t ldy, void *stream) {
  if (n < 0 || d_in <= 0 || d_out <= 0) return ISPA_E_ARG;
  if (d_in % 32 != 0 || d_out % 8 != 0) return ISPA_E_UNSUPPORTED;
  if (n == 0) return ISPA_OK;
  if (a == nullptr || w == nullptr || y == nullptr) return ISPA_E_ARG;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y)) return ISPA_E_ARG;
  if (lda < d_in || lda % 8 != 0 || ldy < d_out || ldy % 8 != 0) return ISPA_E_ARG;
  if ((n + 127) / 128 * ((d_out + 127) / 128) > INT32_MAX) return ISPA_E_UNSUPPORTED;
  return hip_status(launch_project_bf16(n, d_in, d_out, (const uint16_t *)a, lda, (const uint16_t *)w,
                                        (uint16_t *)y, ldy, (hipStream_t)stream));
}

ispa_status ispa_kv_plan(int32_t n_layers, const uint8_t *is_l_layer, int64_t n_sink, int64_t n_hist,
                         int64_t n_cur, int64_t *hist_kept, int64_t *evicted_tokens) {
  if (n_layers < 0 || n_sink < 0 || n_hist < 0 || n_cur < 0) return ISPA_E_ARG;
  if (n_layers > 0 && (is_l_layer == nullptr || hist_kept == nullptr)) return ISPA_E_ARG;
  int64_t evicted = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    hist_kept[i] = is_l_layer[i] ? 0 : n_hist;
    if (is_l_layer[i]) evicted += n_hist;
  }
  if (evicted_tokens != nullptr) *evicted_tokens = evicted;
  return ISPA_OK;
}

}  // extern "C"
