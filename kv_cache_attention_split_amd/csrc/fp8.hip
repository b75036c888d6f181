// FP8 (OCP E4M3) inputs of the attention scores (ISPA page, section 4 "Experimental Results": ISPA is
// paired with W8A8 quantisation; the page gives no recipe, the one here is per-head absmax scaling).
//
//  * fp8_absmax_kernel + fp8_scale_kernel: scale[h] = max |x[:, h, :]| / 448 (1 for an all-zero head).
//    The maximum is taken with atomicMax on the bit patterns of non-negative floats, which order like
//    the values; a maximum does not depend on the order of its operands, so the result is exact and
//    deterministic.
//  * fp8_quantize_kernel: code = e4m3(fp32(x * fp32(1 / scale[h]))), round to nearest even on the
//    hardware conversion, magnitudes clamped to 448 first (saturation).
// Both are single passes over the rows: HBM-bound.
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kRows = 64;   // rows per absmax workgroup (x 16 chunk lanes per row pass)

template <bool BF16>
__device__ __forceinline__ void load8f(const void *base, int64_t elem, float (&x)[8]) {
  if constexpr (BF16) {
    const u32x4 u = *(const u32x4 *)((const uint16_t *)base + elem);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __builtin_bit_cast(float, u[e] << 16);
      x[2 * e + 1] = __builtin_bit_cast(float, u[e] & 0xffff0000u);
    }
  } else {
    const f32x4 a = *(const f32x4 *)((const float *)base + elem);
    const f32x4 b = *(const f32x4 *)((const float *)base + elem + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
}

__global__ void __launch_bounds__(64) fp8_zero_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// grid (row blocks, heads); 256 threads = 16 rows x 16 chunks of 8 elements per pass (head_dim <= 128)
template <bool BF16>
__global__ void __launch_bounds__(256) fp8_absmax_kernel(const void *x, int64_t n, int head_dim, int64_t stride,
                                                         uint32_t *amax) {
  __shared__ float red[4];
  const int h = blockIdx.y;
  const int cpr = head_dim / 8;                 // chunks per head row
  const int tid = threadIdx.x;
  const int rpp = 256 / cpr;                    // rows per pass
  const int c = tid % cpr, rr = tid / cpr;
  float m = 0.f;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  for (int r = rr; r < kRows; r += rpp) {
    const int64_t row = r0 + r;
    if (row >= n) break;
    float v[8];
    load8f<BF16>(x, row * stride + (int64_t)h * head_dim + 8 * c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    const float b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&amax[h], __builtin_bit_cast(uint32_t, b));
  }
}

__global__ void __launch_bounds__(64) fp8_scale_kernel(uint32_t *amax_then_scale, int n_heads) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= n_heads) return;
  const float a = __builtin_bit_cast(float, amax_then_scale[h]);
  const float s = a > 0.f ? a / 448.0f : 1.0f;
  amax_then_scale[h] = __builtin_bit_cast(uint32_t, s);
}

// one thread per 8 elements of a row; rows x (width / 8) threads
template <bool BF16>
__global__ void __launch_bounds__(256) fp8_quantize_kernel(const void *x, int64_t n, int n_heads, int head_dim,
                                                           int64_t stride, const float *scales, uint8_t *out,
                                                           int64_t out_stride) {
  const int cpr = n_heads * head_dim / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * cpr) return;
  const int64_t row = t / cpr;
  const int c = (int)(t % cpr);
  const int h = (8 * c) / head_dim;
  const float inv = 1.0f / scales[h];
  float v[8];
  load8f<BF16>(x, row * stride + 8 * c, v);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = v[e] * inv;
    y[e] = t != t ? t : fminf(fmaxf(t, -448.0f), 448.0f);
  }
  // two codes into the low, then the high half of each word
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  *(u32x2 *)(out + row * out_stride + 8 * c) = u32x2{(uint32_t)w0, (uint32_t)w1};
}

}  // namespace

hipError_t launch_fp8_head_scales(bool bf16, const void *x, int64_t n, int n_heads, int head_dim, int64_t stride,
                                  float *scales, hipStream_t s) {
  uint32_t *bits = (uint32_t *)scales;
  hipLaunchKernelGGL(fp8_zero_kernel, dim3((n_heads + 63) / 64), dim3(64), 0, s, bits, n_heads);
  if (n > 0) {
    const dim3 grid((unsigned)((n + kRows - 1) / kRows), (unsigned)n_heads);
    if (bf16)
      hipLaunchKernelGGL(fp8_absmax_kernel<true>, grid, dim3(256), 0, s, x, n, head_dim, stride, bits);
    else
      hipLaunchKernelGGL(fp8_absmax_kernel<false>, grid, dim3(256), 0, s, x, n, head_dim, stride, bits);
  }
  hipLaunchKernelGGL(fp8_scale_kernel, dim3((n_heads + 63) / 64), dim3(64), 0, s, bits, n_heads);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(bool bf16, const void *x, int64_t n, int n_heads, int head_dim, int64_t stride,
                               const float *scales, uint8_t *out, int64_t out_stride, hipStream_t s) {
  const int64_t threads = n * (int64_t)(n_heads * head_dim / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(fp8_quantize_kernel<true>, grid, dim3(256), 0, s, x, n, n_heads, head_dim, stride, scales,
                       out, out_stride);
  else
    hipLaunchKernelGGL(fp8_quantize_kernel<false>, grid, dim3(256), 0, s, x, n, n_heads, head_dim, stride, scales,
                       out, out_stride);
  return hipGetLastError();
}

}  // namespace ispa
