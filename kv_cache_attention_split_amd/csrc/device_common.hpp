// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ispa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Native 128-bit vector (HIP's uint4 is a struct; arrays of it defeat register promotion).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs (each with its own L2).
// Map the hardware id to a logical id so that each XCD receives a contiguous range of logical ids:
// neighbouring logical tiles (which share operands) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd;
  const int rem = total % kXcd;
  const int x = bid % kXcd;
  const int slot = bid / kXcd;
  return x * per + (x < rem ? x : rem) + slot;
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32 e4m3 values per lane (OCP FP8 E4M3): lane l holds row (column) l % 32 and k = 32 (l / 32) + byte j
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_e4m3_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);   // formats 0: e4m3
}

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Pack two floats into two bf16 (round to nearest even) in one 32-bit word: lo = a, hi = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

__device__ __forceinline__ uint32_t u4_get(const u32x4 &v, int i) { return v[i]; }

// Lanes l and l^32 exchange a value (the two halves of a wave hold the same MFMA column).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

}  // namespace ispa
