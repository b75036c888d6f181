// fp32 dense linear algebra for the Layer Absorb solve and the reconstruction error (ISPA page,
// section 2 stage 2 "Layer Absorb", closed form dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full -
// A_loc) W; "Dynamic Layer Selection" for the error).
//
//  * gemm_f32_kernel: batched C = alpha op(A) op(B) + beta C on v_mfma_f32_32x32x2f32 (fp32 in, fp32
//    accumulate), 128x128 tiles, optional A - A2 operand, optional lower-triangle tile skipping, and a
//    "dot" epilogue that reduces <E, alpha op(A) op(B)> per tile in fp64 instead of storing.
//  * potrf_diag_kernel: Cholesky factor of one nb x nb diagonal block and its triangular inverse, in
//    LDS, one workgroup per layer. The blocked right-looking factorisation and both triangular solves
//    are then plain GEMMs against these inverses.
//  * small elementwise kernels (shifted copy, transpose, add, copy) and a fixed-order reduction of the
//    dot partials.
#include "ispa_internal.hpp"
#include "device_common.hpp"

// Wait until at most n of this wave's vector-memory operations are in flight (n < 64).
#define ISPA_LINALG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
// Workgroup barrier that waits for this wave's LDS operations but not for its copies in flight (those
// are waited for explicitly before it); the empty asm statements keep memory accesses on their side.
#define ISPA_LINALG_LDS_BARRIER()        \
  do {                                   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_waitcnt(0xc07f);  \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  } while (0)

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr int GT = 128;        // GEMM output tile of the wide launches (and of the dot partials)

// GEMM tile GTT x GTT, k step GK per stage; 4 waves, each a (GTT/2)^2 quarter. GTT = 128 with
// GK = 16 for wide launches; GTT = 64 with GK = 32 when a launch has too few 128-tiles to fill the
// chip (4x the workgroups, same staging shape).
// Epilogue of a GEMM tile held as NBK x NBK 32x32 MFMA blocks per wave (wave (wm, wn) of a 2 x 2 grid,
// WT x WT each): C = alpha AB + beta C, or in dot mode the tile's sum of E .* (alpha AB) (and E2 .*)
// in fp64, written to the problem's partials at `tile`.
template <int NBK, int WT>
__device__ __forceinline__ void gemm_epilogue(const GemmBatch &bt, const GemmShape &sh, int p, int tile, bool diag,
                                              int m0, int n0, int wm, int wn, int tid, f32x16 (&acc)[NBK][NBK]) {
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  if (!sh.dot) {
    float *C = bt.C[p];
#pragma unroll
    for (int bi = 0; bi < NBK; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBK; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WT + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          const int col = n0 + wn * WT + bj * 32 + l32;
          if (row < sh.M && col < sh.N) {
            float *c = C + (int64_t)row * sh.ldc + col;
            float val = sh.alpha * acc[bi][bj][v];
            if (sh.beta != 0.f) val = fmaf(sh.beta, *c, val);
            *c = val;
          }
        }
    return;
  }
  // dot epilogue: sum E .* (alpha AB) (and E2 .* (alpha AB)) over this tile in fp64; with hform the
  // weight is (E2 + A2) - (E + E^T) element by element
  const float *E = bt.E[p];
  const float *E2 = bt.E2[p];
  const float *A2 = bt.A2[p];
  const bool two = sh.dot == 2;
  double s = 0.0, s2 = 0.0;
#pragma unroll
  for (int bi = 0; bi < NBK; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WT + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int col = n0 + wn * WT + bj * 32 + l32;
        if (row < sh.M && col < sh.N) {
          const double prod = (double)(sh.alpha * acc[bi][bj][v]);
          const int64_t rc = (int64_t)row * sh.lde + col;
          double e = (double)E[rc];
          if (sh.hform) e = ((double)E2[rc] + (double)A2[rc]) - (e + (double)E[(int64_t)col * sh.lde + row]);
          s += e * prod;
          if (two) s2 += (double)E2[rc] * prod;
        }
      }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off, 64);
    s2 += __shfl_xor(s2, off, 64);
  }
  __shared__ double wsum[2][4];
  if (lane == 0) {
    wsum[0][w] = s;
    wsum[1][w] = s2;
  }
  __syncthreads();
  if (tid == 0) {
    double *part = (double *)bt.C[p];   // dot mode: C holds this problem's partial array
    const double wgt = (sh.sym && !diag) ? 2.0 : 1.0;
    part[tile] = wgt * (((wsum[0][0] + wsum[0][1]) + wsum[0][2]) + wsum[0][3]);
    if (two) bt.P2[p][tile] = wgt * (((wsum[1][0] + wsum[1][1]) + wsum[1][2]) + wsum[1][3]);
  }
}

template <int GTT, int GK>
__global__ void __launch_bounds__(kThreads) gemm_f32_kernel(GemmBatch bt, GemmShape sh) {
  constexpr int GST = GK + 4;    // LDS row stride (floats): rows of 16-byte reads spread over the banks
  constexpr int WT = GTT / 2;    // wave tile
  constexpr int NBK = WT / 32;   // 32x32 blocks per wave dimension
  constexpr int KPL = GK / 2;    // k values per lane per stage
  __shared__ __attribute__((aligned(16))) float lds[2][2][GTT * GST];   // [buf][A/B][row][k]
  const int p = blockIdx.y;
  const int tn = (sh.N + GTT - 1) / GTT;
  const int tile = blockIdx.x;
  const int ti = tile / tn, tj = tile % tn;
  const int m0 = ti * GTT, n0 = tj * GTT;
  if (sh.dot && sh.sym && tj > ti) {
    if (threadIdx.x == 0) {
      ((double *)bt.C[blockIdx.y])[tile] = 0.0;
      if (sh.dot == 2) bt.P2[blockIdx.y][tile] = 0.0;
    }
    return;
  }
  if (sh.lower && n0 > m0 + GTT - 1) return;
  const float *A = bt.A[p];
  const float *A2 = bt.A2[p];
  const float *B = bt.B[p];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // Staging: waves 0-1 stage the A tile, waves 2-3 the B tile. Each thread owns one 4 x 4 block
  // (4 rows of the tile x 4 k) per stage. A row-major operand ([row][k]) is loaded as 4 float4 along
  // k; a transposed one ([k][row]) as 4 float4 along rows and transposed in registers. Either way
  // the LDS tile is [row][k] and is written with 16-byte stores; lanes 4q..4q+3 cover one row's
  // 16 k, so a 16-lane group writes 256 distinct bytes.
  const int sop = tid >> 7;                 // 0: A, 1: B
  const int st_t = tid & 127;
  const int kblk = st_t % (GK / 4), rblk = st_t / (GK / 4);   // GTT/4 x GK/4 blocks = 128
  const bool s_trans = sop == 0 ? (sh.ta != 0) : (sh.tb == 0);
  const float *s_src = sop == 0 ? A : B;
  const float *s_src2 = sop == 0 ? A2 : nullptr;
  const int s_ld = sop == 0 ? sh.lda : sh.ldb;
  const int s_rows = sop == 0 ? sh.M : sh.N;
  const int s_r0 = (sop == 0 ? m0 : n0) + 4 * rblk;
  const bool s_sub = sop == 0 && sh.sub;
  f32x4 rg[4];
  auto load = [&](int k0) {
    const int kc = k0 + 4 * kblk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!s_trans) {
        const int r = s_r0 + e;
        if (r < s_rows && kc < sh.K) {
          x = *(const f32x4 *)(s_src + (int64_t)r * s_ld + kc);
          if (s_sub) x -= *(const f32x4 *)(s_src2 + (int64_t)r * s_ld + kc);
        }
      } else {
        const int k = kc + e;
        if (s_r0 < s_rows && k < sh.K) x = *(const f32x4 *)(s_src + (int64_t)k * s_ld + s_r0);
      }
      rg[e] = x;
    }
  };
  auto store = [&](int buf) {
    float *S = lds[buf][sop];
    if (!s_trans) {
#pragma unroll
      for (int e = 0; e < 4; ++e) *(f32x4 *)&S[(4 * rblk + e) * GST + 4 * kblk] = rg[e];
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        f32x4 y;
        y[0] = rg[0][f];
        y[1] = rg[1][f];
        y[2] = rg[2][f];
        y[3] = rg[3][f];
        *(f32x4 *)&S[(4 * rblk + f) * GST + 4 * kblk] = y;
      }
    }
  };

  f32x16 acc[NBK][NBK];
#pragma unroll
  for (int bi = 0; bi < NBK; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  const int nst = (sh.K + GK - 1) / GK;
  if (nst > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load((st + 1) * GK);
    const float *As = lds[buf][0];
    const float *Bs = lds[buf][1];
    // k slot mapping inside a stage: MFMA s, wave half hf -> k = KPL hf + s
    f32x4 av[NBK][KPL / 4], bv[NBK][KPL / 4];
#pragma unroll
    for (int bi = 0; bi < NBK; ++bi) {
      const float *r = &As[(wm * WT + bi * 32 + l32) * GST + KPL * hf];
#pragma unroll
      for (int q = 0; q < KPL / 4; ++q) av[bi][q] = *(const f32x4 *)(r + 4 * q);
    }
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj) {
      const float *r = &Bs[(wn * WT + bj * 32 + l32) * GST + KPL * hf];
#pragma unroll
      for (int q = 0; q < KPL / 4; ++q) bv[bj][q] = *(const f32x4 *)(r + 4 * q);
    }
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
#pragma unroll
      for (int bi = 0; bi < NBK; ++bi) {
        const f32x4 &a4 = av[bi][s >> 2];
        const float a = a4[s & 3];
#pragma unroll
        for (int bj = 0; bj < NBK; ++bj) {
          const f32x4 &b4 = bv[bj][s >> 2];
          const float b = b4[s & 3];
          acc[bi][bj] = mfma_f32_32x32x2(a, b, acc[bi][bj]);
        }
      }
    }
    if (st + 1 < nst) store(buf ^ 1);
    __syncthreads();
  }

  gemm_epilogue<NBK, WT>(bt, sh, p, tile, ti == tj, m0, n0, wm, wn, tid, acc);
}

// ------------------------------------------------------------------------------------------------
// GEMM with direct global -> LDS copies (global_load_lds, no staging registers) into a ring of four
// 16-deep k stages, so that three stages are in flight while one is multiplied. 128 x 128 tiles, four
// waves of 64 x 64 (2 x 2 blocks of v_mfma_f32_32x32x2f32), 64 KB of LDS: two workgroups per CU. Each
// operand's stage takes the layout its copy gives: an operand whose memory rows run along k (A, or B^T)
// lands as 128 rows of 16 k (64 B, the four 16-byte chunks of a row XOR-swizzled by row / 4) and is read
// with 16-byte reads; one whose rows run along the output index (A^T, or B) lands as 16 rows of 128
// (512 B) and is read with 4-byte reads, consecutive lanes on consecutive addresses. MFMA s takes
// k = 8 hf + s from lane half hf on both operands. Needs M, N multiples of 16, K a multiple of 64 (whole
// turns of the ring), leading dimensions multiples of 4 and 16-byte aligned operands (the host checks);
// rows past M or N are clamped (their outputs are not stored). Tiles are ordered XCD-aware over
// (problem, tile).
// ------------------------------------------------------------------------------------------------
constexpr int DlT = 128, DlK = 16, DlStage = DlT * DlK;   // tile, stage depth, floats per operand stage

// one operand's share of a stage copy: 8 KB = 8 wave instructions, two per wave
template <bool KROWS>
struct DlCopy {
  const float *src[2];
};
template <bool KROWS>
__device__ __forceinline__ DlCopy<KROWS> dl_copy_setup(const float *base, int ld, int i0, int n_idx, int w,
                                                        int lane) {
  DlCopy<KROWS> c;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ii = w + 4 * h;   // instruction: 1 KB block ii of the stage
    if constexpr (KROWS) {
      // memory rows along k: block ii = index rows 16 ii .. +15, lane -> row 16 ii + lane / 4,
      // stored chunk lane % 4 holding source chunk (lane % 4) ^ ((row / 4) % 4)
      const int r = 16 * ii + (lane >> 2);
      const int ch = (lane & 3) ^ ((r >> 2) & 3);
      const int rc = i0 + r < n_idx ? i0 + r : n_idx - 1;
      c.src[h] = base + (int64_t)rc * ld + 4 * ch;
    } else {
      // memory rows along the index: block ii = k rows 2 ii, 2 ii + 1, lane -> 4 consecutive indices
      const int k = 2 * ii + (lane >> 5);
      int col = i0 + 4 * (lane & 31);
      col = col + 4 <= n_idx ? col : n_idx - 4;
      c.src[h] = base + (int64_t)k * ld + col;
    }
  }
  return c;
}

template <bool TA, bool TB>
__global__ void __launch_bounds__(kThreads, 2) gemm_f32_dl_kernel(GemmBatch bt, GemmShape sh, int tiles) {
  constexpr bool AK = !TA, BK = TB;   // operand memory rows along k
  // four ring slots, each the A stage then the B stage (one array per slot: the compiler then tells a
  // slot's reads from the copies in flight into the others and waits only where they may meet)
  __shared__ __attribute__((aligned(1024))) float ring0[2 * DlStage], ring1[2 * DlStage], ring2[2 * DlStage],
      ring3[2 * DlStage];
  // the symmetric dot mode runs the lower tiles only (`tiles` = T (T + 1) / 2 per problem, T = tn),
  // each zeroing the partial of its mirror tile; otherwise every tile of the grid (`tiles` = T_m T_n)
  const bool tri = sh.dot && sh.sym;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int p = lin / tiles, t = lin % tiles;
  const int tn = (sh.N + DlT - 1) / DlT;
  int ti, tj;
  if (tri) {
    ti = (int)((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
    while (ti * (ti + 1) / 2 > t) --ti;
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    tj = t - ti * (ti + 1) / 2;
    if (ti != tj && threadIdx.x == 0) {
      ((double *)bt.C[p])[tj * tn + ti] = 0.0;
      if (sh.dot == 2) bt.P2[p][tj * tn + ti] = 0.0;
    }
  } else {
    ti = t / tn;
    tj = t % tn;
  }
  const int tile = ti * tn + tj;
  const int m0 = ti * DlT, n0 = tj * DlT;
  if (sh.dot && sh.sym && tj > ti) {   // (not reached in the triangular grid)
    if (threadIdx.x == 0) {
      ((double *)bt.C[p])[tile] = 0.0;
      if (sh.dot == 2) bt.P2[p][tile] = 0.0;
    }
    return;
  }
  if (sh.lower && n0 > m0 + DlT - 1) return;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // A stage: op(A)[m0 + i][k0 + k]; B stage: op(B)[k0 + k][n0 + j]
  const DlCopy<AK> ca = dl_copy_setup<AK>(bt.A[p], sh.lda, m0, sh.M, w, lane);
  const DlCopy<BK> cb = dl_copy_setup<BK>(bt.B[p], sh.ldb, n0, sh.N, w, lane);
  // source advance per stage: 16 k along a row, or 16 memory rows
  const int64_t adv_a = AK ? DlK : (int64_t)DlK * sh.lda;
  const int64_t adv_b = BK ? DlK : (int64_t)DlK * sh.ldb;
  auto copy_stage = [&](int st, float *slot) {
#pragma unroll
    for (int h = 0; h < 2; ++h) copy_to_lds<16>(ca.src[h] + st * adv_a, slot + 256 * (w + 4 * h));
#pragma unroll
    for (int h = 0; h < 2; ++h) copy_to_lds<16>(cb.src[h] + st * adv_b, slot + DlStage + 256 * (w + 4 * h));
  };

  // operand of block b (0, 1) of this wave for MFMA s: index wbase + 32 b + l32, k = 8 hf + s
  auto read_ops = [&](const float *sa, const float *sb, float (&av)[2][8], float (&bv)[2][8]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int ia = wm * 64 + 32 * b + l32, jb = wn * 64 + 32 * b + l32;
      if constexpr (AK) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 x = *(const f32x4 *)(sa + ia * DlK + 4 * ((2 * hf + q) ^ ((ia >> 2) & 3)));
#pragma unroll
          for (int e = 0; e < 4; ++e) av[b][4 * q + e] = x[e];
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) av[b][s] = sa[(8 * hf + s) * DlT + ia];
      }
      if constexpr (BK) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 x = *(const f32x4 *)(sb + jb * DlK + 4 * ((2 * hf + q) ^ ((jb >> 2) & 3)));
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[b][4 * q + e] = x[e];
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) bv[b][s] = sb[(8 * hf + s) * DlT + jb];
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

  const int nst = sh.K / DlK;
  // stage st from slot `cur`; the slot read in the previous stage (`fill`) is refilled with st + 3. Every
  // stage issues its four copies (past the last stage the last one again, into a slot nobody reads), so
  // the wait is the same everywhere: the compiler then sees no branch-dependent count and adds no wait
  // of its own before the reads.
  auto stage = [&](int st, const float *cur, float *fill) {
    ISPA_LINALG_WAIT_VMCNT(8);   // this wave's copies of stage st have landed (st + 1, st + 2 may fly)
    ISPA_LINALG_LDS_BARRIER();   // everyone's; and every wave is done with the slot refilled below
    copy_stage(st + 3 < nst ? st + 3 : nst - 1, fill);
    float av[2][8], bv[2][8];
    read_ops(cur, cur + DlStage, av, bv);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma_f32_32x32x2(av[bi][s], bv[bj][s], acc[bi][bj]);
  };
  if (nst > 0) {
    copy_stage(0, ring0);
    copy_stage(nst > 1 ? 1 : 0, ring1);
    copy_stage(nst > 2 ? 2 : nst - 1, ring2);
  }
  for (int st = 0; st < nst; st += 4) {
    stage(st, ring0, ring3);
    stage(st + 1, ring1, ring0);
    stage(st + 2, ring2, ring1);
    stage(st + 3, ring3, ring2);
  }
  ISPA_LINALG_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended
  gemm_epilogue<2, 64>(bt, sh, p, tile, ti == tj, m0, n0, wm, wn, tid, acc);
}

// ------------------------------------------------------------------------------------------------
// Diagonal block: Cholesky factor and its inverse (one workgroup per layer).
// ------------------------------------------------------------------------------------------------

// Orders a wave's own LDS writes before its later LDS reads (a wave's LDS operations complete in
// order; the fences keep the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 32 x 32 blocks of LDS arrays with row stride SS, in the layout of the 32x32 fp32 MFMA: register v of
// lane (l32, hf) is row 8 (v / 4) + 4 hf + v % 4, column l32.
template <int SS>
__device__ __forceinline__ f32x16 blk_load(const float *C, int l32, int hf) {
  f32x16 v;
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = C[(8 * (r >> 2) + 4 * hf + (r & 3)) * SS + l32];
  return v;
}
template <int SS>
__device__ __forceinline__ void blk_store(float *C, const f32x16 &v, int l32, int hf) {
#pragma unroll
  for (int r = 0; r < 16; ++r) C[(8 * (r >> 2) + 4 * hf + (r & 3)) * SS + l32] = v[r];
}
// acc += sgn A op(B), op(B) = B^T when TB; k = 16 hf + s in MFMA s. With an odd stride SS both a row
// (A, B^T) and a column (B) of a block are conflict-free reads.
template <int SS, bool TB>
__device__ __forceinline__ void blk_mma(f32x16 &acc, const float *A, const float *B, float sgn, int l32, int hf) {
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int k = 16 * hf + s;
    const float a = sgn * A[l32 * SS + k];
    const float b = TB ? B[l32 * SS + k] : B[k * SS + l32];
    acc = mfma_f32_32x32x2(a, b, acc);
  }
}

// One wave factors a 32 x 32 diagonal block in registers (lane (c, h) holds rows 16 h .. 16 h + 15 of
// column c) and forms the inverse of its factor in the same sweep. Step j: the owners of column j
// publish it through LDS (the only cross-lane exchange that needs memory), every lane applies
// A[r][c] -= A[r][j] A[c][j] / A[j][j] (r, c > j) and, for the inverse of the unit-lower factor U
// (U[r][j] = A[r][j] / A[j][j]), Y[r][c] -= U[r][j] Y[j][c] (r > j), Y[j][c] coming from the lane of
// the other half with a half swap. At the end L = U D^1/2 and L^-1 = D^-1/2 Y are written to the
// blocks Sb and Xb (row stride SS, zeros above the diagonal). Returns 1 + the first non-positive pivot
// (0 if none); such a pivot is replaced by 1 to keep the rest finite.
template <int SS>
__device__ __forceinline__ int leaf_factor(float *Sb, float *Xb, float *colbuf, int l32_in, int hf_in) {
  // lane coordinates made opaque here, so that the per-step lane masks are formed inside the sweep
  // instead of being hoisted out of the caller's loop (hundreds of live 64-bit masks)
  int c = l32_in, h = hf_in;
  asm volatile("" : "+v"(c));
  asm volatile("" : "+v"(h));
  const bool up = h != 0;
  float a[16], y[16], pr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = Sb[(16 * h + i) * SS + c];
    y[i] = (16 * h + i == c) ? 1.f : 0.f;
    pr[i] = 1.f;
  }
  float pc = 1.f;
  int lbad = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float *cb = colbuf + 32 * (j & 1);   // two buffers: step j's reads and step j+1's writes never share one
    if (c == j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *(f32x4 *)&cb[16 * h + 4 * q] = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
    }
    wave_lds_sync();
    f32x4 v4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v4[q] = *(const f32x4 *)&cb[16 * h + 4 * q];
    float p = cb[j];
    const float vc = cb[c];
    if (!(p > 0.f)) {
      lbad = lbad ? lbad : j + 1;
      p = 1.f;
    }
    const float ip = __builtin_amdgcn_rcpf(p);   // v_rcp_f32 (1 ulp): the division sat on the step chain
    const float ca = (c > j) ? vc * ip : 0.f;    // A[c][j] / A[j][j] for the columns still to come
    float ylo, yhi;
    halves_pair(y[j & 15], ylo, yhi);
    const float cy = ((j < 16) ? ylo : yhi) * ip; // Y[j][c] / A[j][j]
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // A[r][j] for the rows below the pivot (r = 16 h + i > j), zero above
      const float x = v4[i >> 2][i & 3];
      const float v = (i > j) ? x : ((16 + i > j) ? (up ? x : 0.f) : 0.f);
      a[i] = fmaf(-v, ca, a[i]);
      y[i] = fmaf(-v, cy, y[i]);
    }
    if (c == j) pc = p;
    if (j < 16) pr[j & 15] = up ? pr[j & 15] : p;
    else pr[j & 15] = up ? p : pr[j & 15];
  }
  const float sc = sqrtf(pc);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * h + i;
    Sb[r * SS + c] = r > c ? a[i] / sc : (r == c ? sc : 0.f);
    Xb[r * SS + c] = y[i] * (1.f / sqrtf(pr[i]));
  }
  return lbad;
}

// Blocked over 32 x 32 leaves with the block and its inverse in LDS (row stride NB + 1). Per leaf
// column jb: wave 0 factors the leaf (after applying the previous column's update to it) while the
// other waves apply the previous column's update to the rest of the trailing blocks and form the
// previous row of L^-1 (X_ij = -L_ii^-1 sum_{k=j..i-1} L_ik X_kj); then the panel L_ij = A_ij L_jj^-T.
// Every product is 32 x 32 x 32 on the fp32 MFMA. Nine workgroup barriers for nb = 128.
template <int NB>
__global__ void __launch_bounds__(kThreads) potrf_diag_kernel(float *Lbase, int64_t L_stride, int d,
                                                              int k0, float *Linv_base,
                                                              int64_t Linv_stride, int32_t *info) {
  constexpr int NL = NB / 32;
  constexpr int SS = NB + 1;
  extern __shared__ float smem[];
  float *S = smem;               // [NB][SS]: the block, then L in place (lower blocks)
  float *X = smem + NB * SS;     // [NB][SS]: L^-1 (lower blocks); upper blocks (0, 1 + t) hold products
  __shared__ __attribute__((aligned(16))) float colbuf[64];
  __shared__ int bad;
  const int layer = blockIdx.x;
  float *L = Lbase + layer * L_stride;
  float *Linv = Linv_base + layer * Linv_stride;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  if (tid == 0) bad = 0;
  for (int e = tid; e < NB * NB; e += kThreads) {
    const int r = e / NB, c = e % NB;
    S[r * SS + c] = L[(int64_t)(k0 + r) * d + k0 + c];
  }
  __syncthreads();
  auto SB = [&](int i, int k) { return S + 32 * i * SS + 32 * k; };
  auto XB = [&](int i, int k) { return X + 32 * i * SS + 32 * k; };
  // A_ik -= L_ij L_kj^T
  auto trailing = [&](int i, int k, int j) {
    f32x16 acc = blk_load<SS>(SB(i, k), l32, hf);
    blk_mma<SS, true>(acc, SB(i, j), SB(k, j), -1.f, l32, hf);
    blk_store<SS>(SB(i, k), acc, l32, hf);
  };
  // X_ij = -L_ii^-1 (sum_{k=j..i-1} L_ik X_kj), the sum staged in upper block (0, 1 + slot) of X
  auto xblock = [&](int i, int j, int slot) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll 1
    for (int k = j; k < i; ++k) blk_mma<SS, false>(acc, SB(i, k), XB(k, j), 1.f, l32, hf);
    float *T = XB(0, 1 + slot);
    blk_store<SS>(T, acc, l32, hf);
    wave_lds_sync();
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    blk_mma<SS, false>(acc, XB(i, i), T, -1.f, l32, hf);
    blk_store<SS>(XB(i, j), acc, l32, hf);
  };
#pragma unroll 1
  for (int jb = 0; jb < NL; ++jb) {
    if (w == 0) {
      if (jb > 0) {
        trailing(jb, jb, jb - 1);
        wave_lds_sync();
      }
      const int lb = leaf_factor<SS>(SB(jb, jb), XB(jb, jb), colbuf, l32, hf);
      if (lb && lane == 0 && bad == 0) bad = 32 * jb + lb;
    } else if (jb > 0) {
      int t = 0;
#pragma unroll 1
      for (int k = jb; k < NL; ++k)
#pragma unroll 1
        for (int i = k; i < NL; ++i) {
          if (i == jb && k == jb) continue;
          if (t++ % 3 == w - 1) trailing(i, k, jb - 1);
        }
#pragma unroll 1
      for (int j = 0; j < jb - 1; ++j)
        if (t++ % 3 == w - 1) xblock(jb - 1, j, j);
    }
    __syncthreads();
    if (jb + 1 < NL) {
#pragma unroll 1
      for (int i = jb + 1; i < NL; ++i)
        if (w == (i - jb - 1) % 4) {
          f32x16 acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = 0.f;
          blk_mma<SS, true>(acc, SB(i, jb), XB(jb, jb), 1.f, l32, hf);   // A_ij L_jj^-T
          blk_store<SS>(SB(i, jb), acc, l32, hf);
        }
      __syncthreads();
    }
  }
#pragma unroll 1
  for (int j = 0; j < NL - 1; ++j)
    if (w == j % 4) xblock(NL - 1, j, j);
  __syncthreads();
  for (int e = tid; e < NB * NB; e += kThreads) {
    const int r = e / NB, c = e % NB;
    if (c <= r) L[(int64_t)(k0 + r) * d + k0 + c] = S[r * SS + c];
    Linv[r * NB + c] = c <= r ? X[r * SS + c] : 0.f;
  }
  if (tid == 0 && bad != 0 && info[layer] == 0) info[layer] = k0 + bad;
}

__global__ void shift_copy_kernel(CPtrBatch G, float *L, int64_t L_stride, int d, float lambda) {
  const int layer = blockIdx.y;
  const int64_t n4 = (int64_t)d * d / 4;
  const float *g = G.p[layer];
  float *l = L + layer * L_stride;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    f32x4 x = ((const f32x4 *)g)[e];
    const int64_t base = e * 4;
    const int r = (int)(base / d), c = (int)(base % d);
    if (r >= c && r < c + 4) x[r - c] += lambda;
    ((f32x4 *)l)[e] = x;
  }
}

__global__ void transpose_kernel(CPtrBatch in, PtrBatch out, int d) {
  __shared__ float t[32][33];
  const int layer = blockIdx.z;
  const float *src = in.p[layer];
  float *dst = out.p[layer];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x, ty = threadIdx.y;   // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int gr = by + r, gc = bx + tx;
    if (gr < d && gc < d) t[r][tx] = src[(int64_t)gr * d + gc];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int gr = bx + r, gc = by + tx;
    if (gr < d && gc < d) dst[(int64_t)gr * d + gc] = t[tx][r];
  }
}

template <bool SUB>
__global__ void add_kernel(CPtrBatch a, CPtrBatch b, PtrBatch out, int d) {
  const int layer = blockIdx.y;
  const int64_t n4 = (int64_t)d * d / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const f32x4 x = ((const f32x4 *)a.p[layer])[e];
    const f32x4 y = ((const f32x4 *)b.p[layer])[e];
    ((f32x4 *)out.p[layer])[e] = SUB ? x - y : x + y;
  }
}

__global__ void copy_kernel(CPtrBatch a, PtrBatch out, int d) {
  const int layer = blockIdx.y;
  const int64_t n4 = (int64_t)d * d / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x)
    ((f32x4 *)out.p[layer])[e] = ((const f32x4 *)a.p[layer])[e];
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

struct Coef {
  double c[4];
};

__global__ void reduce_partials_kernel(const double *part, int count, int64_t stride, int tiles,
                                       int terms, Coef coef, double *out, const int32_t *info) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= count) return;
  double tot = 0.0;
  for (int g = 0; g < terms; ++g) {
    const double *pp = part + ((int64_t)g * count + p) * stride;
    double s = 0.0;
    for (int t = 0; t < tiles; ++t) s += pp[t];
    tot += coef.c[g] * s;
  }
  out[p] = (info != nullptr && info[p] != 0) ? __builtin_nan("") : tot;
}

// Sum of squares of one 128 x 128 tile of layer blockIdx.y's d x d matrix, in fp64: each thread sums
// its column pairs of every row in row order, then a fixed tree over the threads.
__global__ void __launch_bounds__(256) sumsq_tiles_kernel(const float *base, int64_t layer_stride, int d,
                                                          double *part, int64_t stride) {
  const int tile = blockIdx.x, layer = blockIdx.y;
  const int tn = (d + GT - 1) / GT;
  const int r0 = (tile / tn) * GT, c0 = (tile % tn) * GT;
  const float *m = base + layer * layer_stride;
  const int tid = threadIdx.x;
  const int c = c0 + (tid & 63) * 2;   // two columns per thread
  const int rq = tid >> 6;             // rows rq, rq + 4, ...
  double s = 0.0;
  for (int r = r0 + rq; r < r0 + GT && r < d; r += 4)
    for (int e = 0; e < 2; ++e)
      if (c + e < d) {
        const double x = m[(int64_t)r * d + c + e];
        s += x * x;
      }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  __shared__ double ws[4];
  if ((tid & 63) == 0) ws[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) part[layer * stride + tile] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
}

inline int grid_for(int64_t n4) {
  int64_t g = (n4 + kThreads - 1) / kThreads;
  return (int)(g < 1024 ? (g < 1 ? 1 : g) : 1024);
}

}  // namespace

int gemm_tiles(int M, int N) { return ((M + GT - 1) / GT) * ((N + GT - 1) / GT); }

hipError_t launch_gemm_f32(const GemmBatch &b, int count, const GemmShape &sh, double *part,
                           int64_t part_stride, hipStream_t s, double *part2) {
  if (count <= 0 || sh.M <= 0 || sh.N <= 0) return hipSuccess;
  if (sh.dot == 2 && part2 == nullptr) return hipErrorInvalidValue;
  GemmBatch bb = b;
  if (sh.dot) {
    for (int p = 0; p < count; ++p) bb.C[p] = (float *)(part + (int64_t)p * part_stride);
    if (sh.dot == 2)
      for (int p = 0; p < count; ++p) bb.P2[p] = part2 + (int64_t)p * part_stride;
  }
  // fewer than two 128-tiles per CU: 64-tiles (dot launches keep 128-tiles: their partial
  // count is gemm_tiles; in-place launches too, so that one workgroup owns each 128 extent)
  const int t128 = gemm_tiles(sh.M, sh.N);
  // the direct-copy kernel: M, N in 16s, K in 64s, 16-byte rows and operands, no operand subtraction;
  // lower-tile products only with K of at least 256 (with 8 stages of 16 and half the workgroups
  // returning at once, the register-staged kernel, three workgroups per CU, hides the load latency
  // better: 189 against 251 us for the largest K = 128 Cholesky update at d = 1536; full-tile K = 128
  // products, such as the sweeps' short splits, run faster here: solve 0.2435 against 0.2478 ms per
  // layer, and the in-place products with a diagonal inverse 24 against 34 us)
  bool dl = !sh.sub && sh.M % 16 == 0 && sh.N % 16 == 0 && sh.K % 64 == 0 && sh.lda % 4 == 0 &&
            sh.ldb % 4 == 0 && (sh.K >= 256 || sh.inplace || !sh.lower) && (!(sh.dot && sh.sym) || sh.M == sh.N) &&
            ((int64_t)t128 * count >= 512 || sh.dot || sh.inplace);
  for (int q = 0; q < count && dl; ++q)
    dl = ((uintptr_t)bb.A[q] % 16 == 0) && ((uintptr_t)bb.B[q] % 16 == 0);
  if (dl) {
    // symmetric dot mode: lower tiles only (M = N)
    const int tn = (sh.N + GT - 1) / GT;
    const int tiles = (sh.dot && sh.sym) ? tn * (tn + 1) / 2 : t128;
    const dim3 grid((unsigned)(tiles * count));
    if (sh.ta == 0 && sh.tb == 0)
      hipLaunchKernelGGL((gemm_f32_dl_kernel<false, false>), grid, dim3(kThreads), 0, s, bb, sh, tiles);
    else if (sh.ta == 0)
      hipLaunchKernelGGL((gemm_f32_dl_kernel<false, true>), grid, dim3(kThreads), 0, s, bb, sh, tiles);
    else if (sh.tb == 0)
      hipLaunchKernelGGL((gemm_f32_dl_kernel<true, false>), grid, dim3(kThreads), 0, s, bb, sh, tiles);
    else
      hipLaunchKernelGGL((gemm_f32_dl_kernel<true, true>), grid, dim3(kThreads), 0, s, bb, sh, tiles);
  } else if (!sh.dot && !sh.inplace && (int64_t)t128 * count < 512) {
    dim3 grid(((sh.M + 63) / 64) * ((sh.N + 63) / 64), count);
    hipLaunchKernelGGL((gemm_f32_kernel<64, 32>), grid, dim3(kThreads), 0, s, bb, sh);
  } else {
    dim3 grid(t128, count);
    hipLaunchKernelGGL((gemm_f32_kernel<128, 16>), grid, dim3(kThreads), 0, s, bb, sh);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const double *part, int count, int64_t stride, int tiles, int terms,
                                  const double *coef, double *out, hipStream_t s, const int32_t *info) {
  Coef c = {{0, 0, 0, 0}};
  for (int g = 0; g < terms && g < 4; ++g) c.c[g] = coef[g];
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((count + 63) / 64), dim3(64), 0, s, part, count,
                     stride, tiles, terms, c, out, info);
  return hipGetLastError();
}

hipError_t launch_sumsq_tiles(const float *base, int64_t layer_stride, int d, int count, double *part,
                              int64_t stride, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(sumsq_tiles_kernel, dim3(gemm_tiles(d, d), count), dim3(256), 0, s, base, layer_stride, d,
                     part, stride);
  return hipGetLastError();
}

hipError_t launch_shift_copy(const CPtrBatch &G, float *L, int64_t L_stride, int d, float lambda,
                             int count, hipStream_t s) {
  hipLaunchKernelGGL(shift_copy_kernel, dim3(grid_for((int64_t)d * d / 4), count), dim3(kThreads), 0, s,
                     G, L, L_stride, d, lambda);
  return hipGetLastError();
}

hipError_t launch_potrf_diag(float *L, int64_t L_stride, int d, int k0, int nb, float *Linv,
                             int64_t Linv_stride, int32_t *info, int count, hipStream_t s) {
  const size_t shmem = 2 * (size_t)nb * (nb + 1) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)potrf_diag_kernel<128>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * 128 * 129 * (int)sizeof(float));
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)potrf_diag_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              2 * 64 * 65 * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (nb == 128)
    hipLaunchKernelGGL(potrf_diag_kernel<128>, dim3(count), dim3(kThreads), shmem, s, L, L_stride, d, k0,
                       Linv, Linv_stride, info);
  else
    hipLaunchKernelGGL(potrf_diag_kernel<64>, dim3(count), dim3(kThreads), shmem, s, L, L_stride, d, k0,
                       Linv, Linv_stride, info);
  return hipGetLastError();
}

hipError_t launch_transpose(const CPtrBatch &in, const PtrBatch &out, int d, int count, hipStream_t s) {
  dim3 grid((d + 31) / 32, (d + 31) / 32, count);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(32, 8), 0, s, in, out, d);
  return hipGetLastError();
}

hipError_t launch_add(const CPtrBatch &a, const CPtrBatch &b, const PtrBatch &out, int d, int count,
                      hipStream_t s) {
  hipLaunchKernelGGL(add_kernel<false>, dim3(grid_for((int64_t)d * d / 4), count), dim3(kThreads), 0, s, a, b,
                     out, d);
  return hipGetLastError();
}

hipError_t launch_sub(const CPtrBatch &a, const CPtrBatch &b, const PtrBatch &out, int d, int count,
                      hipStream_t s) {
  hipLaunchKernelGGL(add_kernel<true>, dim3(grid_for((int64_t)d * d / 4), count), dim3(kThreads), 0, s, a, b,
                     out, d);
  return hipGetLastError();
}

hipError_t launch_copy(const CPtrBatch &in, const PtrBatch &out, int d, int count, hipStream_t s) {
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for((int64_t)d * d / 4), count), dim3(kThreads), 0, s, in,
                     out, d);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace ispa
