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
constexpr int GT = 128;        // GEMM output tile
constexpr int GK = 16;         // GEMM k per stage
constexpr int GST = GK + 4;    // LDS row stride (floats): 16 rows x 16 B reads hit all 64 banks once

__global__ void __launch_bounds__(kThreads) gemm_f32_kernel(GemmBatch bt, GemmShape sh) {
  __shared__ __attribute__((aligned(16))) float lds[2][2][GT * GST];   // [buf][A/B][row][k]
  const int p = blockIdx.y;
  const int tn = (sh.N + GT - 1) / GT;
  const int tile = blockIdx.x;
  const int ti = tile / tn, tj = tile % tn;
  const int m0 = ti * GT, n0 = tj * GT;
  if (sh.lower && n0 > m0 + GT - 1) return;
  const float *A = bt.A[p];
  const float *A2 = bt.A2[p];
  const float *B = bt.B[p];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  f32x4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + kThreads * q;
      // A operand
      if (!sh.ta) {
        const int row = idx >> 2, kq = idx & 3;
        const int gi = m0 + row, gk = k0 + 4 * kq;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gi < sh.M && gk < sh.K) {
          x = *(const f32x4 *)(A + (int64_t)gi * sh.lda + gk);
          if (sh.sub) {
            const f32x4 y = *(const f32x4 *)(A2 + (int64_t)gi * sh.lda + gk);
            x -= y;
          }
        }
        ra[q] = x;
      } else {
        const int kr = idx >> 5, iq = idx & 31;
        const int gi = m0 + 4 * iq, gk = k0 + kr;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gi < sh.M && gk < sh.K) x = *(const f32x4 *)(A + (int64_t)gk * sh.lda + gi);
        ra[q] = x;
      }
      // B operand
      if (sh.tb) {
        const int row = idx >> 2, kq = idx & 3;
        const int gj = n0 + row, gk = k0 + 4 * kq;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gj < sh.N && gk < sh.K) x = *(const f32x4 *)(B + (int64_t)gj * sh.ldb + gk);
        rb[q] = x;
      } else {
        const int kr = idx >> 5, jq = idx & 31;
        const int gj = n0 + 4 * jq, gk = k0 + kr;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gj < sh.N && gk < sh.K) x = *(const f32x4 *)(B + (int64_t)gk * sh.ldb + gj);
        rb[q] = x;
      }
    }
  };
  auto store = [&](int buf) {
    float *As = lds[buf][0];
    float *Bs = lds[buf][1];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + kThreads * q;
      if (!sh.ta) {
        const int row = idx >> 2, kq = idx & 3;
        *(f32x4 *)&As[row * GST + 4 * kq] = ra[q];
      } else {
        const int kr = idx >> 5, iq = idx & 31;
        As[(4 * iq + 0) * GST + kr] = ra[q][0];
        As[(4 * iq + 1) * GST + kr] = ra[q][1];
        As[(4 * iq + 2) * GST + kr] = ra[q][2];
        As[(4 * iq + 3) * GST + kr] = ra[q][3];
      }
      if (sh.tb) {
        const int row = idx >> 2, kq = idx & 3;
        *(f32x4 *)&Bs[row * GST + 4 * kq] = rb[q];
      } else {
        const int kr = idx >> 5, jq = idx & 31;
        Bs[(4 * jq + 0) * GST + kr] = rb[q][0];
        Bs[(4 * jq + 1) * GST + kr] = rb[q][1];
        Bs[(4 * jq + 2) * GST + kr] = rb[q][2];
        Bs[(4 * jq + 3) * GST + kr] = rb[q][3];
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
    // k slot mapping inside a stage: MFMA s, wave half hf -> k = 8 hf + s
    f32x4 av[2][2], bv[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const float *r = &As[(wm * 64 + bi * 32 + l32) * GST + 8 * hf];
      av[bi][0] = *(const f32x4 *)r;
      av[bi][1] = *(const f32x4 *)(r + 4);
    }
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const float *r = &Bs[(wn * 64 + bj * 32 + l32) * GST + 8 * hf];
      bv[bj][0] = *(const f32x4 *)r;
      bv[bj][1] = *(const f32x4 *)(r + 4);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const f32x4 &a4 = av[bi][s >> 2];
        const float a = a4[s & 3];
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
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
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          const int col = n0 + wn * 64 + bj * 32 + l32;
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
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int col = n0 + wn * 64 + bj * 32 + l32;
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
    part[tile] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

// ------------------------------------------------------------------------------------------------
// Diagonal block: Cholesky factor and its inverse (one workgroup per layer).
// ------------------------------------------------------------------------------------------------
constexpr int kMaxNb = 128;

__global__ void __launch_bounds__(kThreads) potrf_diag_kernel(float *Lbase, int64_t L_stride, int d,
                                                              int k0, int nb, float *Linv_base,
                                                              int64_t Linv_stride, int32_t *info) {
  extern __shared__ float smem[];
  const int ld = nb + 1;
  float *A = smem;              // nb x ld
  float *Xi = smem + nb * ld;   // nb x ld
  __shared__ int bad;
  const int layer = blockIdx.x;
  float *L = Lbase + layer * L_stride;
  float *Linv = Linv_base + layer * Linv_stride;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  for (int e = tid; e < nb * nb; e += kThreads) {
    const int r = e / nb, c = e % nb;
    A[r * ld + c] = L[(int64_t)(k0 + r) * d + k0 + c];
    Xi[r * ld + c] = (r == c) ? 1.f : 0.f;
  }
  __syncthreads();
  // right-looking unblocked Cholesky of the block (lower triangle)
  for (int j = 0; j < nb; ++j) {
    float piv = A[j * ld + j];
    if (!(piv > 0.f)) {
      piv = 1.f;
      if (tid == 0 && bad == 0) bad = j + 1;
    }
    const float ljj = sqrtf(piv);
    const float inv = 1.f / ljj;
    __syncthreads();
    if (tid == 0) A[j * ld + j] = ljj;
    for (int i = j + 1 + tid; i < nb; i += kThreads) A[i * ld + j] *= inv;
    __syncthreads();
    const int rem = nb - j - 1;
    for (int e = tid; e < rem * rem; e += kThreads) {
      const int r = j + 1 + e / rem, c = j + 1 + e % rem;
      if (c <= r) A[r * ld + c] -= A[r * ld + j] * A[c * ld + j];
    }
    __syncthreads();
  }
  // inverse of the lower factor by a row sweep: L X = I
  for (int j = 0; j < nb; ++j) {
    const float inv = 1.f / A[j * ld + j];
    for (int c = tid; c <= j; c += kThreads) Xi[j * ld + c] *= inv;
    __syncthreads();
    const int cols = j + 1, rows = nb - j - 1;
    for (int e = tid; e < rows * cols; e += kThreads) {
      const int i = j + 1 + e / cols, c = e % cols;
      Xi[i * ld + c] -= A[i * ld + j] * Xi[j * ld + c];
    }
    __syncthreads();
  }
  for (int e = tid; e < nb * nb; e += kThreads) {
    const int r = e / nb, c = e % nb;
    Linv[r * nb + c] = Xi[r * ld + c];
    if (c <= r) L[(int64_t)(k0 + r) * d + k0 + c] = A[r * ld + c];
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

__global__ void add_kernel(CPtrBatch a, CPtrBatch b, PtrBatch out, int d) {
  const int layer = blockIdx.y;
  const int64_t n4 = (int64_t)d * d / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const f32x4 x = ((const f32x4 *)a.p[layer])[e];
    const f32x4 y = ((const f32x4 *)b.p[layer])[e];
    ((f32x4 *)out.p[layer])[e] = x + y;
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
  dim3 grid(gemm_tiles(sh.M, sh.N), count);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s, bb, sh);
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
  const size_t shmem = 2 * (size_t)nb * (nb + 1) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void *)potrf_diag_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        2 * kMaxNb * (kMaxNb + 1) * (int)sizeof(float));
    attr_set = true;
  }
  hipLaunchKernelGGL(potrf_diag_kernel, dim3(count), dim3(kThreads), shmem, s, L, L_stride, d, k0, nb,
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
  hipLaunchKernelGGL(add_kernel, dim3(grid_for((int64_t)d * d / 4), count), dim3(kThreads), 0, s, a, b,
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
