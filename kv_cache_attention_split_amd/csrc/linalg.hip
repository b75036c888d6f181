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

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr int GT = 128;        // GEMM output tile of the wide launches (and of the dot partials)

// GEMM tile GTT x GTT, k step GK per stage; 4 waves, each a (GTT/2)^2 quarter. GTT = 128 with
// GK = 16 for wide launches; GTT = 64 with GK = 32 when a launch has too few 128-tiles to fill the
// chip (4x the workgroups, same staging shape).
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
    if (threadIdx.x == 0) ((double *)bt.C[blockIdx.y])[tile] = 0.0;
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
  // dot epilogue: sum E .* (alpha AB) over this tile in fp64
  const float *E = bt.E[p];
  double s = 0.0;
#pragma unroll
  for (int bi = 0; bi < NBK; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WT + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int col = n0 + wn * WT + bj * 32 + l32;
        if (row < sh.M && col < sh.N)
          s += (double)E[(int64_t)row * sh.lde + col] * (double)(sh.alpha * acc[bi][bj][v]);
      }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  __shared__ double wsum[4];
  if (lane == 0) wsum[w] = s;
  __syncthreads();
  if (tid == 0) {
    double *part = (double *)bt.C[p];   // dot mode: C holds this problem's partial array
    const double wgt = (sh.sym && ti != tj) ? 2.0 : 1.0;
    part[tile] = wgt * (((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]);
  }
}

// ------------------------------------------------------------------------------------------------
// Diagonal block: Cholesky factor and its inverse (one workgroup per layer).
// ------------------------------------------------------------------------------------------------

// Register-blocked: a 16 x 16 grid of threads, thread (ty, tx) owning the R x R sub-block at rows
// ty*R.., columns tx*R.. (R = nb / 16). Each elimination step publishes one column (factorisation)
// or one row (inverse) through LDS, then every thread updates its own sub-block in registers: one
// barrier per step and no dependent LDS chains.
template <int NB>
__global__ void __launch_bounds__(kThreads) potrf_diag_kernel(float *Lbase, int64_t L_stride, int d,
                                                              int k0, float *Linv_base,
                                                              int64_t Linv_stride, int32_t *info) {
  constexpr int R = NB / 16;
  extern __shared__ float smem[];
  float *colst = smem;              // [NB][NB]: column j of the updated block at step j (col-major)
  float *rowst = smem + NB * NB;    // [NB][NB]: row j of U^-1 at step j
  __shared__ int bad;
  const int layer = blockIdx.x;
  float *L = Lbase + layer * L_stride;
  float *Linv = Linv_base + layer * Linv_stride;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int r0 = ty * R, c0 = tx * R;
  if (tid == 0) bad = 0;
  float a[R][R];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int k = 0; k < R; ++k) a[i][k] = L[(int64_t)(k0 + r0 + i) * d + k0 + c0 + k];

  // R consecutive floats of LDS (R-aligned) as vector reads
  auto lds_row = [&](const float *p, float (&v)[R]) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const f32x4 x = ((const f32x4 *)p)[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  };
  auto lds_store_row = [&](float *p, const float (&v)[R]) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v[4 * q + e];
      ((f32x4 *)p)[q] = x;
    }
  };

  // factorisation: at step j every thread applies A[r][c] -= A[r][j] A[c][j] / A[j][j] to its
  // sub-block (entries of rows / columns <= j get a zero factor, so they stay unchanged; the upper
  // triangle is updated too, harmlessly, since only the lower is read). Look-ahead: the owners of
  // column j+1 update that column first and publish it to LDS before the rest of the update, so
  // that the LDS write is in flight while the other FMAs run and one barrier per step suffices
  // (each column has its own LDS row). The step loop is unrolled by R so that column j is the
  // fixed register j mod R of its owners.
  if (tx == 0) {
    float col[R];
#pragma unroll
    for (int i = 0; i < R; ++i) col[i] = a[i][0];
    lds_store_row(&colst[r0], col);
  }
  for (int jb = 0; jb < NB; jb += R)
#pragma unroll
  for (int kk = 0; kk < R; ++kk) {
    const int j = jb + kk;
    __syncthreads();   // column j is in LDS
    float cr[R], cc[R];
    lds_row(&colst[j * NB + r0], cr);
    lds_row(&colst[j * NB + c0], cc);
    float piv = colst[j * NB + j];
    if (!(piv > 0.f)) piv = 1.f;   // recorded below; keeps the rest finite
    const float ip = 1.f / piv;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      cr[i] = (r0 + i > j) ? cr[i] * ip : 0.f;
      cc[i] = (c0 + i > j) ? cc[i] : 0.f;
    }
    const int kn = (kk + 1) % R;                          // register of column j+1 (constant once unrolled)
    const bool own_next = (tx == (j + 1) / R) && (j + 1 < NB);
    if (own_next) {
      float col[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        a[i][kn] = fmaf(-cr[i], cc[kn], a[i][kn]);
        col[i] = a[i][kn];
      }
      lds_store_row(&colst[(j + 1) * NB + r0], col);
    }
    cc[kn] = own_next ? 0.f : cc[kn];                    // that column is done
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int k = 0; k < R; ++k) a[i][k] = fmaf(-cr[i], cc[k], a[i][k]);
  }
  __syncthreads();
  if (tid == 0) {
    for (int j = 0; j < NB; ++j)
      if (!(colst[j * NB + j] > 0.f)) {
        bad = j + 1;
        break;
      }
  }
  // inverse of the unit-lower factor U[r][j] = colst[j][r] / piv_j by a forward sweep:
  // Y = I; for each j, rows i > j: Y[i][c] -= U[i][j] Y[j][c]. Same look-ahead: the owners of
  // row j+1 of Y update and publish it first.
  float y[R][R];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int k = 0; k < R; ++k) y[i][k] = (r0 + i == c0 + k) ? 1.f : 0.f;
  if (ty == 0) {
    float row[R];
#pragma unroll
    for (int k = 0; k < R; ++k) row[k] = y[0][k];
    lds_store_row(&rowst[c0], row);
  }
  for (int jb = 0; jb < NB; jb += R)
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    const int j = jb + ii;
    if (j == NB - 1) break;     // uniform: the last row has nothing below it
    __syncthreads();            // row j of Y is in LDS
    // row j of Y is zero beyond column j (Y is lower triangular); rows <= j get u = 0
    float u[R], yr[R];
    lds_row(&colst[j * NB + r0], u);
    lds_row(&rowst[j * NB + c0], yr);
    float piv = colst[j * NB + j];
    if (!(piv > 0.f)) piv = 1.f;
    const float ip = 1.f / piv;
#pragma unroll
    for (int i = 0; i < R; ++i) u[i] = (r0 + i > j) ? u[i] * ip : 0.f;
    const int in = (ii + 1) % R;                          // register row of row j+1 (constant once unrolled)
    const bool own_next = (ty == (j + 1) / R) && (j + 1 < NB - 1);
    if (own_next) {
      float row[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        y[in][k] = fmaf(-u[in], yr[k], y[in][k]);
        row[k] = y[in][k];
      }
      lds_store_row(&rowst[(j + 1) * NB + c0], row);
    }
    u[in] = own_next ? 0.f : u[in];                      // that row is done
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int k = 0; k < R; ++k) y[i][k] = fmaf(-u[i], yr[k], y[i][k]);
  }
  // L = U D^1/2 (lower part of the block), Linv = D^-1/2 Y
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = r0 + i;
    float pr = colst[r * NB + r];
    if (!(pr > 0.f)) pr = 1.f;
    const float isr = 1.f / sqrtf(pr);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int c = c0 + k;
      Linv[r * NB + c] = y[i][k] * isr;
      float pc = colst[c * NB + c];
      if (!(pc > 0.f)) pc = 1.f;
      if (c < r) L[(int64_t)(k0 + r) * d + k0 + c] = colst[c * NB + r] / sqrtf(pc);
      else if (c == r) L[(int64_t)(k0 + r) * d + k0 + c] = sqrtf(pr);
    }
  }
  __syncthreads();
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
                                       int terms, Coef coef, double *out) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= count) return;
  double tot = 0.0;
  for (int g = 0; g < terms; ++g) {
    const double *pp = part + ((int64_t)g * count + p) * stride;
    double s = 0.0;
    for (int t = 0; t < tiles; ++t) s += pp[t];
    tot += coef.c[g] * s;
  }
  out[p] = tot;
}

inline int grid_for(int64_t n4) {
  int64_t g = (n4 + kThreads - 1) / kThreads;
  return (int)(g < 1024 ? (g < 1 ? 1 : g) : 1024);
}

}  // namespace

int gemm_tiles(int M, int N) { return ((M + GT - 1) / GT) * ((N + GT - 1) / GT); }

hipError_t launch_gemm_f32(const GemmBatch &b, int count, const GemmShape &sh, double *part,
                           int64_t part_stride, hipStream_t s) {
  if (count <= 0 || sh.M <= 0 || sh.N <= 0) return hipSuccess;
  GemmBatch bb = b;
  if (sh.dot) {
    for (int p = 0; p < count; ++p) bb.C[p] = (float *)(part + (int64_t)p * part_stride);
  }
  // fewer than two 128-tiles per CU: 64-tiles (dot launches keep 128-tiles: their partial
  // count is gemm_tiles; in-place launches too, so that one workgroup owns each 128 extent)
  const int t128 = gemm_tiles(sh.M, sh.N);
  if (!sh.dot && !sh.inplace && (int64_t)t128 * count < 512) {
    dim3 grid(((sh.M + 63) / 64) * ((sh.N + 63) / 64), count);
    hipLaunchKernelGGL((gemm_f32_kernel<64, 32>), grid, dim3(kThreads), 0, s, bb, sh);
  } else {
    dim3 grid(t128, count);
    hipLaunchKernelGGL((gemm_f32_kernel<128, 16>), grid, dim3(kThreads), 0, s, bb, sh);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const double *part, int count, int64_t stride, int tiles, int terms,
                                  const double *coef, double *out, hipStream_t s) {
  Coef c = {{0, 0, 0, 0}};
  for (int g = 0; g < terms && g < 4; ++g) c.c[g] = coef[g];
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((count + 63) / 64), dim3(64), 0, s, part, count,
                     stride, tiles, terms, c, out);
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
  const size_t shmem = 2 * (size_t)nb * nb * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void *)potrf_diag_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        2 * 128 * 128 * (int)sizeof(float));
    hipFuncSetAttribute((const void *)potrf_diag_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        2 * 64 * 64 * (int)sizeof(float));
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
