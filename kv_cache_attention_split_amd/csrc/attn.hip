// Dual-stream attention for gfx950 (ISPA page, section 2 "Framework Core", stage 1 "Dual-Stream
// Warmup" and its Decomposable Attention paragraph).
//
// One workgroup owns one (head, query tile) and walks the layer's cache once: first the local keys
// (sink tokens, then the current chunk), then the history keys. A single online-softmax state runs
// through both. When the local keys are exhausted the normalised output and log-sum-exp of the local
// branch are stored (A_loc, lse_loc); the running state then continues over the history, with the
// history's own exp-sum kept apart so that lse_hist is available too, and the final state gives
// A_full and lse_full. This is the page's local/historical split with the merge done in registers:
// the merged result is exactly the single-pass softmax over all keys, and no key is visited twice.
//
// bf16 kernel: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulate);
// the query index runs along the MFMA column, so each lane holds whole softmax rows' statistics and
// the row max / row sum need only one exchange between the two wave halves. K tiles sit in LDS in
// row-major [key][d]; V tiles are transposed into [d][key] while staging, with the keys of every
// 16-key group permuted so that one 16-byte LDS read yields exactly the 8 keys a lane needs for the
// P^T operand that the previous MFMA left in its registers. The running max is updated lazily: the
// accumulator is rescaled only when the max grows by more than 2^8, so exp2 values stay <= 256.
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr float kRescaleThreshold = 8.0f;   // log2 units

// Store one normalised 32-query block of the O^T accumulator as bf16 rows of A. Lane (l32, hf)
// holds query l32 and, per 32-wide column block db, columns 8g + 4hf + {0..3}.
template <int D>
__device__ __forceinline__ void write_rows(const f32x16 (&o)[D / 32], float inv, void *out, int qi,
                                           int n_q, int out_stride, int head_off, int hf) {
  if (out == nullptr || qi >= n_q) return;
  uint16_t *dst = (uint16_t *)out + (int64_t)qi * out_stride + head_off + 4 * hf;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      pk[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2 *)(dst + 32 * db + 8 * g) = pk;
    }
}

__device__ __forceinline__ void write_lse(float *out, float val, int head, int qi, int n_q, int hf) {
  if (out != nullptr && hf == 0 && qi < n_q) out[(int64_t)head * n_q + qi] = val;
}

// Key/value rows of one segment run. The local run is the sink followed by the current chunk (two
// pointers, split at the sink length); the history run is one pointer. All fields are uniform.
struct SegRun {
  const uint16_t *k0, *v0, *k1, *v1;
  int64_t s0, s1, split, n;
};

__device__ __forceinline__ SegRun seg_run(const AttnArgs &a, bool hist) {
  SegRun r;
  const uint16_t *sk = (const uint16_t *)a.sink_k, *sv = (const uint16_t *)a.sink_v;
  const uint16_t *ck = (const uint16_t *)a.cur_k, *cv = (const uint16_t *)a.cur_v;
  const uint16_t *hk = (const uint16_t *)a.hist_k, *hv = (const uint16_t *)a.hist_v;
  r.k0 = hist ? hk : sk;
  r.v0 = hist ? hv : sv;
  r.s0 = hist ? a.hist_stride : a.sink_stride;
  r.k1 = hist ? hk : ck;
  r.v1 = hist ? hv : cv;
  r.s1 = hist ? a.hist_stride : a.cur_stride;
  r.n = hist ? a.hist_n : a.sink_n + a.cur_n;
  r.split = hist ? r.n : a.sink_n;
  return r;
}

// Element offset of key row j of a run (rows past the end are clamped to the last row; their scores
// are masked, so they only need to be readable).
template <bool VALUE>
__device__ __forceinline__ const uint16_t *run_row(const SegRun &r, int64_t j, int head_off) {
  j = j < r.n ? j : r.n - 1;
  const bool second = j >= r.split;
  const int64_t jj = second ? j - r.split : j;
  const uint16_t *base = VALUE ? (second ? r.v1 : r.v0) : (second ? r.k1 : r.k0);
  const int64_t st = second ? r.s1 : r.s0;
  return base + jj * st + head_off;
}

// Global -> register prefetch of key/value tile t (t < nt_loc: local run, else history run).
// Common case: the tile lies inside one sub-run (sink, current or history) and needs no clamping;
// then one uniform base pointer and a 32-bit row offset address every row. Tiles that cross the
// sink/current split or the end of a run take the per-row path.
template <int D, int BK>
__device__ __forceinline__ void load_tile(const AttnArgs &a, int t, int nt_loc, int tid, int head_off,
                                          int vg, int vc, u32x4 (&kreg)[BK * D / 8 / kThreads],
                                          u32x4 (&vreg)[4]) {
  constexpr int CPR = D / 8;
  constexpr int KLD = BK * CPR / kThreads;
  constexpr int VPAIRS = (BK / 4) * CPR;
  const bool hist = t >= nt_loc;
  const SegRun run = seg_run(a, hist);
  const int64_t j0 = (int64_t)(hist ? t - nt_loc : t) * BK;
  const int64_t j1 = j0 + BK;
  const bool in_first = j1 <= run.split && j1 <= run.n;
  const bool in_second = j0 >= run.split && j1 <= run.n;
  if (in_first || in_second) {
    const uint16_t *kb = in_first ? run.k0 + j0 * run.s0 : run.k1 + (j0 - run.split) * run.s1;
    const uint16_t *vb = in_first ? run.v0 + j0 * run.s0 : run.v1 + (j0 - run.split) * run.s1;
    const int st = (int)(in_first ? run.s0 : run.s1);
    kb += head_off;
    vb += head_off;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / CPR, c = idx % CPR;
      kreg[i] = *(const u32x4 *)(kb + (row * st + 8 * c));
    }
    if (tid < VPAIRS) {
#pragma unroll
      for (int e = 0; e < 4; ++e) vreg[e] = *(const u32x4 *)(vb + ((4 * vg + e) * st + 8 * vc));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < KLD; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / CPR, c = idx % CPR;
    kreg[i] = *(const u32x4 *)(run_row<false>(run, j0 + row, head_off) + 8 * c);
  }
  if (tid < VPAIRS) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vreg[e] = *(const u32x4 *)(run_row<true>(run, j0 + 4 * vg + e, head_off) + 8 * vc);
  }
}

// Register -> LDS: K row-major [key][d]; V transposed to [d][key position] (4-key groups of each
// 16-key run at positions {0,2,1,3}, see the kernel comment).
template <int D, int BK, int KST, int VST>
__device__ __forceinline__ void store_tile(uint16_t *k_lds, uint16_t *v_lds, int tid, int vc, int vpos,
                                           const u32x4 (&kreg)[BK * D / 8 / kThreads],
                                           const u32x4 (&vreg)[4]) {
  constexpr int CPR = D / 8;
  constexpr int KLD = BK * CPR / kThreads;
  constexpr int VPAIRS = (BK / 4) * CPR;
#pragma unroll
  for (int i = 0; i < KLD; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / CPR, c = idx % CPR;
    *(u32x4 *)&k_lds[row * KST + 8 * c] = kreg[i];
  }
  if (tid < VPAIRS) {
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const uint32_t x0 = u4_get(vreg[0], mm), x1 = u4_get(vreg[1], mm);
      const uint32_t x2 = u4_get(vreg[2], mm), x3 = u4_get(vreg[3], mm);
      u32x2 lo, hi;
      lo[0] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(x3, x2, 0x05040100u);
      hi[0] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
      hi[1] = __builtin_amdgcn_perm(x3, x2, 0x07060302u);
      const int d0 = 8 * vc + 2 * mm;
      *(u32x2 *)&v_lds[d0 * VST + vpos] = lo;
      *(u32x2 *)&v_lds[(d0 + 1) * VST + vpos] = hi;
    }
  }
}

template <int D, int QB>
__global__ void __launch_bounds__(kThreads, QB == 1 ? 2 : 1) attn_dual_bf16_kernel(AttnArgs a, int n_qt) {
  constexpr int BK = 64;             // keys per tile
  constexpr int KST = D + 8;         // K tile row stride (elements), padded against bank conflicts
  constexpr int VST = BK + 8;        // V^T tile row stride
  constexpr int BQ = 4 * 32 * QB;    // queries per workgroup
  constexpr int NKK = D / 16;        // MFMA k-steps of Q.K
  constexpr int NDB = D / 32;        // 32-wide output column blocks
  constexpr int NB = BK / 32;        // 32-key blocks per tile
  constexpr int CPR = D / 8;         // 16-byte chunks per key row
  constexpr int KLD = BK * CPR / kThreads;
  constexpr int VPAIRS = (BK / 4) * CPR;   // (4-key group, chunk) pairs per V tile
  static_assert(KLD >= 1 && VPAIRS <= kThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * KST];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VST];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int vid = xcd_remap(blockIdx.x, n_qt * a.n_heads);
  const int head = vid / n_qt, qt = vid % n_qt;
  const int head_off = head * D;
  const int qrow0 = qt * BQ + w * 32 * QB;
  const int n_q = a.n_q;
  const int out_stride = a.n_heads * D;
  const float sl2 = a.scale_log2;

  // Q^T operand, kept in registers for the whole pass: lane holds query l32, d = 16kk + 8hf .. +8.
  bf16x8 qr[QB][NKK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qrow0 + qb * 32 + l32;
    const bool ok = qi < n_q;
    const uint16_t *src = (const uint16_t *)a.q + (int64_t)(ok ? qi : 0) * a.q_stride + head_off + hf * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = *(const u32x4 *)(src + kk * 16);
      if (!ok) x = u32x4{0u, 0u, 0u, 0u};
      qr[qb][kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t n_loc = a.sink_n + a.cur_n;
  const int nt_loc = (int)((n_loc + BK - 1) / BK);
  const int nt_hist = (int)((a.hist_n + BK - 1) / BK);
  const int nt = nt_loc + nt_hist;

  f32x16 o[QB][NDB];
  float m[QB], l[QB], l_loc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
    l_loc[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[qb][db][v] = 0.f;
  }

  u32x4 kreg[KLD];
  u32x4 vreg[4];
  const int vg = tid % (BK / 4);     // 4-key group handled by this thread (V staging)
  const int vc = tid / (BK / 4);     // 16-byte chunk along d (V staging)
  // position of this thread's key group inside its 16-key run: groups {0,1,2,3} -> {0,2,1,3}
  const int vg3 = vg & 3;
  const int vpos = 4 * ((vg & ~3) | ((vg3 == 1) ? 2 : (vg3 == 2) ? 1 : vg3));

  // ---- main pass -------------------------------------------------------------------------------
  load_tile<D, BK>(a, 0, nt_loc, tid, head_off, vg, vc, kreg, vreg);
  store_tile<D, BK, KST, VST>(k_lds[0], v_lds[0], tid, vc, vpos, kreg, vreg);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) load_tile<D, BK>(a, t + 1, nt_loc, tid, head_off, vg, vc, kreg, vreg);
    const bool in_hist = t >= nt_loc;
    const int64_t j0 = (int64_t)(in_hist ? t - nt_loc : t) * BK;
    const int64_t nseg = in_hist ? a.hist_n : n_loc;
    const int n_valid = (int)((nseg - j0) < BK ? (nseg - j0) : BK);

    // S^T[key][query] = K Q^T
    f32x16 s[QB][NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[qb][b][v] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kop = *(const bf16x8 *)&k_lds[buf][(32 * b + l32) * KST + 16 * kk + 8 * hf];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][b] = mfma_bf16_32x32x16(kop, qr[qb][kk], s[qb][b]);
      }
    if (n_valid < BK) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 32 * b + 8 * (v >> 2) + 4 * hf + (v & 3);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][b][v] = key < n_valid ? s[qb][b][v] : -INFINITY;
        }
    }
    // online softmax (log2 domain, lazy max update)
    bf16x8 pk[QB][NB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[qb][b][v]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = mx * sl2;
      const bool need = mnew > m[qb] + kRescaleThreshold;
      if (__ballot(need) != 0ull) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m[qb] - mnew) : 1.0f;
        m[qb] = need ? mnew : m[qb];
        l[qb] *= alpha;
        l_loc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[qb][db][v] *= alpha;
      }
      const float mneg = -m[qb];
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][8 * h2 + e], sl2, mneg));
            sum += p[e];
          }
          u32x4 u;
          u[0] = pack_bf16x2(p[0], p[1]);
          u[1] = pack_bf16x2(p[2], p[3]);
          u[2] = pack_bf16x2(p[4], p[5]);
          u[3] = pack_bf16x2(p[6], p[7]);
          pk[qb][b][h2] = __builtin_bit_cast(bf16x8, u);
        }
      }
      l[qb] += sum;
    }
    // O^T[d][query] += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 vop =
              *(const bf16x8 *)&v_lds[buf][(32 * db + l32) * VST + 32 * b + 16 * h2 + 8 * hf];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma_bf16_32x32x16(vop, pk[qb][b][h2], o[qb][db]);
        }

    if (t == nt_loc - 1) {
      // local branch complete: store A_loc / lse_loc, then keep the local exp-sum apart.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float tot = l[qb] + swap_halves(l[qb]);
        const float inv = 1.0f / tot;
        const float lse = (m[qb] + __log2f(tot)) * kLn2;
        const int qi = qrow0 + qb * 32 + l32;
        write_rows<D>(o[qb], inv, a.a_loc, qi, n_q, out_stride, head_off, hf);
        write_lse(a.lse_loc, lse, head, qi, n_q, hf);
        if (nt_hist == 0) {
          write_rows<D>(o[qb], inv, a.a_full, qi, n_q, out_stride, head_off, hf);
          write_lse(a.lse_full, lse, head, qi, n_q, hf);
          write_lse(a.lse_hist, -INFINITY, head, qi, n_q, hf);
        }
        l_loc[qb] = l[qb];
        l[qb] = 0.f;
      }
    }
    if (t + 1 < nt) store_tile<D, BK, KST, VST>(k_lds[buf ^ 1], v_lds[buf ^ 1], tid, vc, vpos, kreg, vreg);
    __syncthreads();
  }
  if (nt_hist > 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float th = l[qb] + swap_halves(l[qb]);
      const float tl = l_loc[qb] + swap_halves(l_loc[qb]);
      const float tot = th + tl;
      const int qi = qrow0 + qb * 32 + l32;
      write_rows<D>(o[qb], 1.0f / tot, a.a_full, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_full, (m[qb] + __log2f(tot)) * kLn2, head, qi, n_q, hf);
      write_lse(a.lse_hist, th > 0.f ? (m[qb] + __log2f(th)) * kLn2 : -INFINITY, head, qi, n_q, hf);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// fp32 kernel: VALU, one query per thread. Same single pass and the same local/history split.
// ------------------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(128) attn_dual_f32_kernel(AttnArgs a, int n_qt) {
  constexpr int BK = 32;
  constexpr int NT = 128;
  __shared__ float k_lds[BK][D];
  __shared__ float v_lds[BK][D];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int qi = qt * NT + tid;
  const bool qok = qi < a.n_q;
  const int head_off = head * D;

  float q[D], o[D];
  const float *qsrc = (const float *)a.q + (int64_t)(qok ? qi : 0) * a.q_stride + head_off;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qok ? qsrc[c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f, l_loc = 0.f;
  const int64_t n_loc = a.sink_n + a.cur_n;
  const int nt_loc = (int)((n_loc + BK - 1) / BK);
  const int nt_hist = (int)((a.hist_n + BK - 1) / BK);
  const int nt = nt_loc + nt_hist;

  auto row_ptr = [&](bool hist, int64_t j, bool value) -> const float * {
    if (hist) return (const float *)(value ? a.hist_v : a.hist_k) + j * a.hist_stride + head_off;
    if (j < a.sink_n) return (const float *)(value ? a.sink_v : a.sink_k) + j * a.sink_stride + head_off;
    j -= a.sink_n;
    return (const float *)(value ? a.cur_v : a.cur_k) + j * a.cur_stride + head_off;
  };
  auto store_out = [&](void *out, float inv) {
    if (!qok || out == nullptr) return;
    float *dst = (float *)out + (int64_t)qi * (a.n_heads * D) + head_off;
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = o[c] * inv;
  };
  auto store_lse = [&](float *out, float val) {
    if (qok && out != nullptr) out[(int64_t)head * a.n_q + qi] = val;
  };

  for (int t = 0; t < nt; ++t) {
    const bool hist = t >= nt_loc;
    const int64_t j0 = (int64_t)(hist ? t - nt_loc : t) * BK;
    const int64_t nseg = hist ? a.hist_n : n_loc;
    const int n_valid = (int)((nseg - j0) < BK ? (nseg - j0) : BK);
    __syncthreads();
    for (int idx = tid; idx < BK * D; idx += NT) {
      const int r = idx / D, c = idx % D;
      int64_t j = j0 + r;
      j = j < nseg ? j : nseg - 1;
      k_lds[r][c] = row_ptr(hist, j, false)[c];
      v_lds[r][c] = row_ptr(hist, j, true)[c];
    }
    __syncthreads();
    float s[BK];
    float mx = -INFINITY;
    for (int r = 0; r < BK; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], k_lds[r][c], acc);
      s[r] = r < n_valid ? acc * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    if (mx > m) {
      const float alpha = exp2f(m - mx);
      m = mx;
      l *= alpha;
      l_loc *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
    }
    for (int r = 0; r < BK; ++r) {
      const float p = exp2f(s[r] - m);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, v_lds[r][c], o[c]);
    }
    if (t == nt_loc - 1) {
      const float inv = 1.0f / l;
      const float lse = (m + log2f(l)) * kLn2;
      store_out(a.a_loc, inv);
      store_lse(a.lse_loc, lse);
      if (nt_hist == 0) {
        store_out(a.a_full, inv);
        store_lse(a.lse_full, lse);
        store_lse(a.lse_hist, -INFINITY);
      }
      l_loc = l;
      l = 0.f;
    }
  }
  if (nt_hist > 0) {
    const float tot = l + l_loc;
    store_out(a.a_full, 1.0f / tot);
    store_lse(a.lse_full, (m + log2f(tot)) * kLn2);
    store_lse(a.lse_hist, l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY);
  }
}

}  // namespace

// Queries per workgroup of the bf16 kernel: 128 * QB.
#ifndef ISPA_ATTN_QB
#define ISPA_ATTN_QB 1
#endif

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t s) {
  constexpr int QB = ISPA_ATTN_QB;
  const int bq = 128 * QB;
  const int n_qt = (a.n_q + bq - 1) / bq;
  const int grid = n_qt * a.n_heads;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_dual_bf16_kernel<128, QB>), dim3(grid), dim3(kThreads), 0, s, a, n_qt);
  else
    hipLaunchKernelGGL((attn_dual_bf16_kernel<64, QB>), dim3(grid), dim3(kThreads), 0, s, a, n_qt);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs &a, int head_dim, hipStream_t s) {
  const int n_qt = (a.n_q + 127) / 128;
  const int grid = n_qt * a.n_heads;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_dual_f32_kernel<128>), dim3(grid), dim3(128), 0, s, a, n_qt);
  else
    hipLaunchKernelGGL((attn_dual_f32_kernel<64>), dim3(grid), dim3(128), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace ispa
