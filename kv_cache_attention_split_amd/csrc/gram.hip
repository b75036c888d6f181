// Warmup statistics for Layer Absorb (ISPA page, section 2 stage 2: the closed form is built from
// A_loc^T A_loc and A_loc^T (A_full - A_loc), summed over the warmup rows).
//
// The three products G = A_loc^T A_loc, X = A_loc^T A_full and F = A_full^T A_full are the blocks of
// the Gram matrix of the stacked rows Z = [A_loc | A_full]; one launch computes all of them from the
// exact bf16 inputs on v_mfma_f32_32x32x16_bf16. G and F are symmetric: only their upper 128x128
// tiles are computed and each is added to both its own position and its mirror, so G and F stay
// exactly symmetric. X is computed in full. Each output element is owned by one workgroup, which
// reduces over all rows of the chunk in a fixed order and adds its result to the running sum with a
// plain read-modify-write: no atomics, so the sums are deterministic.
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr int BT = 128;          // output tile
constexpr int BR = 64;           // rows per stage
constexpr int ST = BR + 8;       // LDS row stride (elements) of the transposed operand tiles

struct GramArgs {
  const uint16_t *a_loc, *a_full;
  float *G, *X, *F;
  int64_t n_rows;
  int d, T, n_upper, with_f;
};

__device__ __forceinline__ void tri_decode(int idx, int T, int &ti, int &tj) {
  // idx enumerates pairs ti <= tj row by row
  int r = 0;
  while (idx >= T - r) {
    idx -= T - r;
    ++r;
  }
  ti = r;
  tj = r + idx;
}

__global__ void __launch_bounds__(kThreads) gram_bf16_kernel(GramArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BT * ST];   // [buf][operand]

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  int n_tiles = g.n_upper * (g.with_f ? 2 : 1) + g.T * g.T;
  int idx = xcd_remap(blockIdx.x, n_tiles);
  int mat, ti, tj;   // mat: 0 = G, 1 = F, 2 = X
  if (idx < g.n_upper) {
    mat = 0;
    tri_decode(idx, g.T, ti, tj);
  } else if (g.with_f && idx < 2 * g.n_upper) {
    mat = 1;
    tri_decode(idx - g.n_upper, g.T, ti, tj);
  } else {
    mat = 2;
    idx -= g.n_upper * (g.with_f ? 2 : 1);
    ti = idx / g.T;
    tj = idx % g.T;
  }
  const uint16_t *P = (mat == 1) ? g.a_full : g.a_loc;   // rows of the left factor
  const uint16_t *Q = (mat == 0) ? g.a_loc : g.a_full;   // rows of the right factor
  float *out = (mat == 0) ? g.G : (mat == 1) ? g.F : g.X;
  const int i0 = ti * BT, j0 = tj * BT;
  const int d = g.d;

  // staging: each thread owns two (4-row group, 8-column chunk) pairs; threads 0..127 stage the
  // left operand, 128..255 the right one.
  const int op = tid >> 7;
  const int sid = tid & 127;
  const uint16_t *src = op ? Q : P;
  const int col0 = op ? j0 : i0;
  u32x4 r[2][4];
  auto load = [&](int64_t n0) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int pair = sid + 128 * pp;
      const int grp = pair & 15, ch = pair >> 4;
      const int col = col0 + 8 * ch;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t n = n0 + 4 * grp + e;
        if (n < g.n_rows && col < d)
          r[pp][e] = *(const u32x4 *)(src + n * d + col);
        else
          r[pp][e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int buf) {
    uint16_t *dst = lds[buf][op];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int pair = sid + 128 * pp;
      const int grp = pair & 15, ch = pair >> 4;
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const uint32_t x0 = u4_get(r[pp][0], mm), x1 = u4_get(r[pp][1], mm);
        const uint32_t x2 = u4_get(r[pp][2], mm), x3 = u4_get(r[pp][3], mm);
        u32x2 lo, hi;
        lo[0] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        lo[1] = __builtin_amdgcn_perm(x3, x2, 0x05040100u);
        hi[0] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
        hi[1] = __builtin_amdgcn_perm(x3, x2, 0x07060302u);
        const int c = 8 * ch + 2 * mm;
        *(u32x2 *)&dst[c * ST + 4 * grp] = lo;
        *(u32x2 *)&dst[(c + 1) * ST + 4 * grp] = hi;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  const int nst = (int)((g.n_rows + BR - 1) / BR);
  if (nst > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load((int64_t)(st + 1) * BR);
    const uint16_t *As = lds[buf][0];
    const uint16_t *Bs = lds[buf][1];
#pragma unroll
    for (int t = 0; t < BR / 16; ++t) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        av[bi] = *(const bf16x8 *)&As[(wm * 64 + bi * 32 + l32) * ST + 16 * t + 8 * hf];
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        bv[bj] = *(const bf16x8 *)&Bs[(wn * 64 + bj * 32 + l32) * ST + 16 * t + 8 * hf];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma_bf16_32x32x16(av[bi], bv[bj], acc[bi][bj]);
    }
    if (st + 1 < nst) store(buf ^ 1);
    __syncthreads();
  }

  // Stage the 128x128 result in LDS (reusing the operand buffers), then add it to the running sums
  // with coalesced accesses: the tile itself, and for off-diagonal symmetric tiles its mirror.
  float *cs = (float *)&lds[0][0][0];
  constexpr int CST = BT + 1;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int cc = wn * 64 + bj * 32 + l32;
        cs[rr * CST + cc] = acc[bi][bj][v];
      }
  __syncthreads();
  for (int e = tid; e < BT * BT; e += kThreads) {
    const int rr = e >> 7, cc = e & 127;
    const int gr = i0 + rr, gc = j0 + cc;
    if (gr < d && gc < d) out[(int64_t)gr * d + gc] += cs[rr * CST + cc];
  }
  if (mat != 2 && ti != tj) {
    for (int e = tid; e < BT * BT; e += kThreads) {
      const int rr = e >> 7, cc = e & 127;     // mirror position (j0 + rr, i0 + cc) = tile (cc, rr)
      const int gr = j0 + rr, gc = i0 + cc;
      if (gr < d && gc < d) out[(int64_t)gr * d + gc] += cs[cc * CST + rr];
    }
  }
}

}  // namespace

hipError_t launch_gram_bf16(int64_t n_rows, int d, const uint16_t *a_loc, const uint16_t *a_full,
                            float *G, float *X, float *F, hipStream_t s) {
  GramArgs g;
  g.a_loc = a_loc;
  g.a_full = a_full;
  g.G = G;
  g.X = X;
  g.F = F;
  g.n_rows = n_rows;
  g.d = d;
  g.T = (d + BT - 1) / BT;
  g.n_upper = g.T * (g.T + 1) / 2;
  g.with_f = F != nullptr;
  const int n_tiles = g.n_upper * (g.with_f ? 2 : 1) + g.T * g.T;
  if (n_rows == 0 || n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gram_bf16_kernel, dim3(n_tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace ispa
