// Future-query importance of cached keys (Future Forcing summary page, "Componenti Algorithmiche",
// module 1: every cached key is scored by the attention weight that proxies of future queries are
// predicted to give it; implementation detail 3: without forming the full Q K^T matrix).
//
// Two passes over the cache per head:
//   1. lse_i = log sum_j exp(tau q~_i . k_j) for every proxy query i: the attention kernel's
//      log-sum-exp-only form (launch_attn_lse_bf16), no values;
//   2. future_colsum_kernel: score_j = (1/n_p) sum_i exp(tau q~_i . k_j - lse_i).
// Neither pass stores a score matrix: pass 2 recomputes each 32x32 block of Q~ K^T on the matrix
// cores and folds it into per-key sums at once.
//
// future_colsum_kernel: a workgroup owns 256 keys of one head (8 waves x 32 keys, the keys' B operands
// held in registers for the whole pass) and walks all proxy queries in stages of 64. A stage (the
// proxies' rows and their lse) reaches LDS by global_load_lds through a ring of three stages, one
// LDS array per slot (the loop is unrolled by the ring depth so the compiler sees which slot a read
// touches). With the proxies along the MFMA rows and the keys along its columns, each lane holds one
// key and 16 proxy rows of a block, so the sum over proxies stays in the lane (plus one exchange
// between the two wave halves at the end). Sums are in a fixed order: deterministic.
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int QT = 64;    // proxy queries per stage
constexpr int NS = 3;     // stages in the ring
constexpr int KT = 32 * kWaves;   // keys per workgroup: one 32-key block per wave

static __device__ float g_pos_inf = INFINITY;

#define ISPA_FS_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
#define ISPA_FS_LDS_BARRIER()            \
  do {                                   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_waitcnt(0xc07f);  \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  } while (0)

struct ScoreArgs {
  const uint16_t *q;                    // proxies [n_p, q_stride], head h at columns h*D
  int64_t q_stride, n_p;
  const float *lse;                     // [H, n_p], natural log
  const uint16_t *k0, *k1, *k2;         // sink, current, history keys
  int64_t s0, s1, s2, n0, n1, n2;       // row strides and lengths
  float *scores;                        // [H, scores_hs], keys in cache order
  int64_t scores_hs;
  float scale_log2;                     // tau * log2(e)
  int n_heads, n_kt;
};

// 16-byte chunk c of row r of a [QT][D] stage is stored at chunk c ^ swz(r): the 16 rows of one
// operand read (same chunk) land on 16 different positions.
template <int D>
__device__ __forceinline__ int q_off(int r, int col) {
  const int swz = D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
  return r * (D * 2) + ((((col >> 3) ^ swz)) << 4) + ((col & 7) << 1);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 1) future_colsum_kernel(ScoreArgs a) {
  constexpr int TB = QT * D * 2;              // bytes of a stage's proxy rows
  constexpr int NKK = D / 16;                 // MFMA k-steps
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int NC = TB / 1024 / kWaves;      // 1 KB copy instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t qs0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qs1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qs2[TB];
  __shared__ __attribute__((aligned(256))) float ls0[QT];
  __shared__ __attribute__((aligned(256))) float ls1[QT];
  __shared__ __attribute__((aligned(256))) float ls2[QT];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int vid = xcd_remap(blockIdx.x, a.n_kt * a.n_heads);
  const int head = vid / a.n_kt, kt = vid % a.n_kt;
  const int head_off = head * D;
  const int64_t n_keys = a.n0 + a.n1 + a.n2;

  // this lane's key and its B operands
  bf16x8 kop[NKK];
  {
    int64_t j = (int64_t)kt * KT + w * 32 + l32;
    j = j < n_keys ? j : n_keys - 1;
    const uint16_t *row = j < a.n0 ? a.k0 + j * a.s0
                        : j < a.n0 + a.n1 ? a.k1 + (j - a.n0) * a.s1
                                          : a.k2 + (j - a.n0 - a.n1) * a.s2;
    row += head_off + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kop[kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(row + 16 * kk));
  }

  // copy geometry: instruction ii of wave w fills 1 KB block w + 8 ii, lane l lands at row
  // r = block * (1024 / (2D)) + l / CPR, stored chunk l % CPR, which holds source chunk (l % CPR) ^ swz(r)
  int crow[NC], ccol[NC];
#pragma unroll
  for (int ii = 0; ii < NC; ++ii) {
    const int r = (w + kWaves * ii) * (1024 / (2 * D)) + lane / CPR;
    crow[ii] = r;
    const int swz = D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
    ccol[ii] = 8 * ((lane % CPR) ^ swz);
  }
  uint64_t zinf = (uint64_t)(uintptr_t)&g_pos_inf;
  asm volatile("" : "+s"(zinf));
  const int n_st = (int)((a.n_p + QT - 1) / QT);
  const float *lse_h = a.lse + (int64_t)head * a.n_p;

  // Rows past the last proxy repeat the last proxy (finite scores) and get lse = +inf (weight 0).
  // The stage's first row is kept opaque so that the addresses are formed anew per stage instead of
  // being carried as per-lane pointers for every slot of the ring.
  auto copy_stage = [&](int s, uint8_t *qs, float *ls) {
    int64_t row0 = (int64_t)s * QT;
    asm volatile("" : "+s"(row0));
#pragma unroll
    for (int ii = 0; ii < NC; ++ii) {
      int64_t i = row0 + crow[ii];
      i = i < a.n_p ? i : a.n_p - 1;
      const uint16_t *src = a.q + i * a.q_stride + head_off + ccol[ii];
      copy_to_lds<16>(src, qs + 1024 * (w + kWaves * ii));
    }
    if (w == 0) {
      const int64_t i = row0 + lane;
      const float *src = i < a.n_p ? lse_h + i : (const float *)(uintptr_t)zinf;
      copy_to_lds<4>(src, ls);
    }
  };

  float col = 0.f;
  const float sl2 = a.scale_log2;
  auto compute = [&](const uint8_t *qs, const float *ls) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      bf16x8 qop[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qop[kk] = *(const bf16x8 *)(qs + q_off<D>(32 * qb + l32, 16 * kk + 8 * hf));
      // -lse * log2(e) of the 16 proxy rows of this lane: rows 32qb + 8(v/4) + 4hf + v%4
      float nl[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = *(const f32x4 *)(ls + 32 * qb + 8 * q4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) nl[4 * q4 + e] = -x[e] * kLog2e;
      }
      f32x16 s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s = mfma_bf16_32x32x16(qop[kk], kop[kk], s);
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], sl2, nl[v]));
      col += sum;
      __builtin_amdgcn_sched_barrier(0);   // one 32-proxy block at a time: bounded registers
    }
  };

  // Stage s: wait for its copies (this wave's stage s+1 copies may still be in flight: NC of them,
  // one more for wave 0, which also copies the lse), then refill the slot of stage s-1, read
  // completely before this barrier, with stage s+2. The loop always runs whole turns of the ring:
  // stages past the end hold zero rows with lse = +inf and add exact zeros.
  auto stage = [&](int s, const uint8_t *qs, const float *ls, uint8_t *qn, float *ln) {
    if (w == 0) ISPA_FS_WAIT_VMCNT(NC + 1);
    else ISPA_FS_WAIT_VMCNT(NC);
    ISPA_FS_LDS_BARRIER();
    copy_stage(s + NS - 1, qn, ln);
    compute(qs, ls);
  };

  copy_stage(0, qs0, ls0);
  copy_stage(1, qs1, ls1);
  for (int s = 0; s < n_st; s += NS) {
    stage(s, qs0, ls0, qs2, ls2);
    stage(s + 1, qs1, ls1, qs0, ls0);
    stage(s + 2, qs2, ls2, qs1, ls1);
  }
  ISPA_FS_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended

  const float tot = halves_sum(col);
  const int64_t j = (int64_t)kt * KT + w * 32 + l32;
  if (hf == 0 && j < n_keys) a.scores[(int64_t)head * a.scores_hs + j] = tot / (float)a.n_p;
}

// token[j] = lambda * mean_h scores[h][j] + (1 - lambda) * hist[j] (hist may be NULL: 0)
__global__ void __launch_bounds__(256) token_score_kernel(const float *scores, int64_t hs, int n_heads,
                                                          int64_t n, float lambda, const float *hist,
                                                          float *token) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int h = 0; h < n_heads; ++h) s += scores[(int64_t)h * hs + j];
  const float f = s / (float)n_heads;
  token[j] = hist != nullptr ? lambda * f + (1.0f - lambda) * hist[j] : lambda * f;
}

}  // namespace

hipError_t launch_future_colsum_bf16(const uint16_t *q, int64_t q_stride, int64_t n_p, const float *lse,
                                     const uint16_t *k0, int64_t s0, int64_t n0, const uint16_t *k1,
                                     int64_t s1, int64_t n1, const uint16_t *k2, int64_t s2, int64_t n2,
                                     int n_heads, int head_dim, float scale_log2, float *scores,
                                     int64_t scores_hs, hipStream_t s) {
  ScoreArgs a;
  a.q = q;
  a.q_stride = q_stride;
  a.n_p = n_p;
  a.lse = lse;
  a.k0 = k0;
  a.k1 = k1;
  a.k2 = k2;
  a.s0 = s0;
  a.s1 = s1;
  a.s2 = s2;
  a.n0 = n0;
  a.n1 = n1;
  a.n2 = n2;
  a.scores = scores;
  a.scores_hs = scores_hs;
  a.scale_log2 = scale_log2;
  a.n_heads = n_heads;
  const int64_t n_keys = n0 + n1 + n2;
  a.n_kt = (int)((n_keys + KT - 1) / KT);
  const int64_t grid = (int64_t)a.n_kt * n_heads;
  if (grid == 0 || n_p == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(future_colsum_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(future_colsum_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_token_scores(const float *scores, int64_t hs, int n_heads, int64_t n, float lambda,
                               const float *hist, float *token, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(token_score_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, scores, hs,
                     n_heads, n, lambda, hist, token);
  return hipGetLastError();
}

}  // namespace ispa
