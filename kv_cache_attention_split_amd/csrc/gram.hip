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
#ifndef ISPA_GRAM_BR
#define ISPA_GRAM_BR 32
#endif
constexpr int BR = ISPA_GRAM_BR;  // rows per stage
constexpr int RB = BT * 2;       // bytes of one tile row (128 bf16)

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

// Operand tiles are kept row-major in LDS ([row of the chunk][128 columns], 256 bytes per row) with
// the 16-byte chunks of row r stored at position c ^ (4 (r mod 4)). ds_read_b64_tr_b16 then yields
// MFMA operands directly: in each 16-lane group, source lane s addresses row k0 + s/4, columns
// n0 + 4 (s mod 4) .. +3, and result lane i receives column n0 + i of rows k0 .. k0+3. The swizzle
// spreads the 4 rows of one read over distinct banks.
__device__ __forceinline__ int swz_off(int r, int col) {   // byte offset of (r, col) in a tile
  const int c = col >> 3;
  return r * RB + (((c ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 read_operand(const uint8_t *tile, int cb, int kb, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int n0 = cb + 16 * (g & 1);
  const int k0 = kb + 8 * (g >> 1);
  const int col = n0 + 4 * (s & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(tile + swz_off(k0 + (s >> 2), col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(tile + swz_off(k0 + 4 + (s >> 2), col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__global__ void __launch_bounds__(kThreads, 2) gram_bf16_kernel(GramArgs g) {
  // [buf][operand] tiles of BR x 128 bf16; after the main loop the same space holds the fp32 result
  // tile (128 x 129 floats)
  constexpr int kTileBytes = BR * RB;
  constexpr int kLdsBytes = BT * (BT + 1) * 4 > 4 * kTileBytes ? BT * (BT + 1) * 4 : 4 * kTileBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  auto tile_ptr = [&](int buf, int op) { return smem + (2 * buf + op) * kTileBytes; };

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
  const int64_t last_row = g.n_rows - 1;

  // staging: thread handles 16-byte chunks e = tid + 256 q (q < NQ) of each operand tile:
  // row r = e / 16, chunk c = e % 16. Columns past d are clamped (their outputs are not stored).
  constexpr int NQ = BR * 16 / kThreads;
  int srow[NQ], scol_p[NQ], scol_q[NQ], soff[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = tid + kThreads * q;
    const int r = e >> 4, c = e & 15;
    srow[q] = r;
    const int cp = i0 + 8 * c, cq = j0 + 8 * c;
    scol_p[q] = cp < d ? cp : d - 8;
    scol_q[q] = cq < d ? cq : d - 8;
    soff[q] = r * RB + ((c ^ (4 * (r & 3))) << 4);
  }
  u32x4 ra[2 * NQ], rb[2 * NQ];   // [operand * NQ + q]
  auto load = [&](u32x4 (&r)[2 * NQ], int64_t n0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      int64_t n = n0 + srow[q];
      n = n < last_row ? n : last_row;
      r[q] = *(const u32x4 *)(P + n * d + scol_p[q]);
      r[NQ + q] = *(const u32x4 *)(Q + n * d + scol_q[q]);
    }
  };
  auto store = [&](const u32x4 (&r)[2 * NQ], int buf, int64_t n0) {
    if (n0 + BR - 1 <= last_row) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        *(u32x4 *)(tile_ptr(buf, 0) + soff[q]) = r[q];
        *(u32x4 *)(tile_ptr(buf, 1) + soff[q]) = r[NQ + q];
      }
    } else {   // tail stage: rows past the chunk end contribute zeros
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const bool ok = n0 + srow[q] <= last_row;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4 *)(tile_ptr(buf, 0) + soff[q]) = ok ? r[q] : z;
        *(u32x4 *)(tile_ptr(buf, 1) + soff[q]) = ok ? r[NQ + q] : z;
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

  auto compute = [&](int buf) {
    const uint8_t *As = tile_ptr(buf, 0);
    const uint8_t *Bs = tile_ptr(buf, 1);
#pragma unroll
    for (int t = 0; t < BR / 16; ++t) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) av[bi] = read_operand(As, wm * 64 + bi * 32, 16 * t, lane);
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) bv[bj] = read_operand(Bs, wn * 64 + bj * 32, 16 * t, lane);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma_bf16_32x32x16(av[bi], bv[bj], acc[bi][bj]);
    }
  };

  // Two stages of global loads stay in flight: while stage s is multiplied out of LDS, stage s+1
  // sits in one register set and stage s+2 is being fetched into the other. Loads are issued
  // unconditionally (clamped rows), so no branch separates them from their use.
  const int nst = (int)((g.n_rows + BR - 1) / BR);
  load(ra, 0);
  load(rb, BR);
  store(ra, 0, 0);
  __syncthreads();
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    load(ra, (int64_t)(st + 2) * BR);
    compute(0);
    store(rb, 1, (int64_t)(st + 1) * BR);
    __syncthreads();
    load(rb, (int64_t)(st + 3) * BR);
    compute(1);
    if (st + 2 < nst) store(ra, 0, (int64_t)(st + 2) * BR);
    __syncthreads();
  }
  if (st < nst) compute(0);
  __syncthreads();

  // Stage the 128x128 result in LDS (reusing the operand buffers), then add it to the running sums
  // with coalesced 16-byte read-modify-writes: the tile itself, and for off-diagonal symmetric tiles
  // its mirror. Each thread issues all of its loads before any add, so the round trips overlap.
  float *cs = (float *)smem;
  constexpr int CST = BT + 1;   // odd stride: both row-wise and column-wise reads spread over banks
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
  // thread -> (row rr = e / 32, 4-column group c4 = e % 32) for e = tid + 256 k, k < 16
  constexpr int NV = BT * BT / 4 / kThreads;   // 16 float4 per thread
  const int c4 = tid & 31;
  const int rbase = tid >> 5;                  // 0..7; rows rbase + 8k
  {
    f32x4 cur[NV];
    const int gc = j0 + 4 * c4;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int gr = i0 + rbase + 8 * k;
      const int grc = gr < d ? gr : d - 1;
      const int gcc = gc < d ? gc : d - 4;
      cur[k] = *(const f32x4 *)&out[(int64_t)grc * d + gcc];
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int rr = rbase + 8 * k;
      const int gr = i0 + rr;
      f32x4 add;
#pragma unroll
      for (int q = 0; q < 4; ++q) add[q] = cs[rr * CST + 4 * c4 + q];
      if (gr < d && gc < d) *(f32x4 *)&out[(int64_t)gr * d + gc] = cur[k] + add;
    }
  }
  if (mat != 2 && ti != tj) {
    // mirror: out[j0 + rr][i0 + cc] += tile[cc][rr]
    f32x4 cur[NV];
    const int gc = i0 + 4 * c4;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int gr = j0 + rbase + 8 * k;
      const int grc = gr < d ? gr : d - 1;
      const int gcc = gc < d ? gc : d - 4;
      cur[k] = *(const f32x4 *)&out[(int64_t)grc * d + gcc];
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int rr = rbase + 8 * k;
      const int gr = j0 + rr;
      f32x4 add;
#pragma unroll
      for (int q = 0; q < 4; ++q) add[q] = cs[(4 * c4 + q) * CST + rr];
      if (gr < d && gc < d) *(f32x4 *)&out[(int64_t)gr * d + gc] = cur[k] + add;
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
