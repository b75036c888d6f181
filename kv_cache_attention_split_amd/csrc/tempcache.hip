// TempCache exact merge of a cache segment (FAST-AR summary page, section 2 part A "TempCache",
// Lemma 5.1: a group of identical keys becomes one key whose value is the group's mean value and
// whose logit is raised by the log of the group size; attention is then unchanged).
//
// kv_merge_kernel: one wave per group. The wave walks the group's member rows in the given order
// (indices read 64 at a time and broadcast from lane to wave) and each lane accumulates 8 columns of
// the key row and 8 of the value row per pass in fp32, 16-byte loads and stores; the mean is one
// division, rounded once to the output type. The merged rows are written densely in group order, and
// the group's log-count goes to the bias output that the biased attention reads.
//
// The work is a gather of whole rows: bound by HBM bandwidth (every member row read once, every
// merged row written once), no reuse to stage in LDS.
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kWaves = 4;

struct MergeArgs {
  const void *k, *v;
  int64_t n, in_stride;
  const int32_t *offsets, *members;
  int64_t n_groups;
  void *k_out, *v_out;
  int64_t out_stride;
  float *bias_out;
  int width;   // elements per row, multiple of 8
};

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t elem, float (&x)[8]) {
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

template <bool BF16>
__device__ __forceinline__ void store8(void *base, int64_t elem, const float (&x)[8]) {
  if constexpr (BF16) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    *(u32x4 *)((uint16_t *)base + elem) = u;
  } else {
    *(f32x4 *)((float *)base + elem) = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4 *)((float *)base + elem + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
}

// P column passes (8 columns x 64 lanes each) are accumulated together, so one member row costs
// 2P loads in flight per lane; P = min(4, passes per row) is chosen on the host.
template <bool BF16, int P>
__global__ void __launch_bounds__(64 * kWaves) kv_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
  if (g >= a.n_groups) return;
  const int32_t m0 = a.offsets[g], m1 = a.offsets[g + 1];
  const int count = m1 > m0 ? m1 - m0 : 0;
  if (lane == 0 && a.bias_out != nullptr) a.bias_out[g] = count > 0 ? logf((float)count) : -INFINITY;
  const float fc = (float)count;
  // The pass loop is wave-uniform: every lane runs every pass, also lanes whose columns lie past the
  // row end (width < 512 P), because the member indices below are loaded one per lane and broadcast
  // with readlane, which must read a lane that has executed the load.
  for (int cb = 0; cb < a.width; cb += 8 * 64 * P) {
    const int c0 = cb + 8 * lane;
    float sk[P][8], sv[P][8];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) sk[p][e] = sv[p][e] = 0.f;
    // member indices 64 at a time, one per lane, then broadcast to the wave; two member rows are
    // loaded before either is added (a member outside [0, n) reads row 0 with weight 0, so there is
    // no branch; the sums keep member order)
    auto load_row = [&](int32_t row, float (&xk)[P][8], float (&xv)[P][8]) -> float {
      const bool ok = row >= 0 && row < a.n;
      const int64_t base = (int64_t)(ok ? row : 0) * a.in_stride;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int c = c0 + 8 * 64 * p;
        const int cc = c < a.width ? c : 0;    // lanes past the row end reload column 0 (not stored)
        load8<BF16>(a.k, base + cc, xk[p]);
        load8<BF16>(a.v, base + cc, xv[p]);
      }
      return ok ? 1.f : 0.f;
    };
    auto add_row = [&](float w, const float (&xk)[P][8], const float (&xv)[P][8]) {
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sk[p][e] = __builtin_fmaf(w, xk[p][e], sk[p][e]);
          sv[p][e] = __builtin_fmaf(w, xv[p][e], sv[p][e]);
        }
    };
    for (int32_t mb = m0; mb < m1 && a.n > 0; mb += 64) {
      const int32_t mine = mb + lane < m1 ? a.members[mb + lane] : -1;
      const int nm = m1 - mb < 64 ? m1 - mb : 64;
      int j = 0;
      for (; j + 1 < nm; j += 2) {
        float ak[P][8], av[P][8], bk[P][8], bv[P][8];
        const float wa = load_row(__builtin_amdgcn_readlane(mine, j), ak, av);
        const float wb = load_row(__builtin_amdgcn_readlane(mine, j + 1), bk, bv);
        add_row(wa, ak, av);
        add_row(wb, bk, bv);
      }
      if (j < nm) {
        float ak[P][8], av[P][8];
        const float wa = load_row(__builtin_amdgcn_readlane(mine, j), ak, av);
        add_row(wa, ak, av);
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + 8 * 64 * p;
      if (c >= a.width) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sk[p][e] = count > 0 ? sk[p][e] / fc : 0.f;
        sv[p][e] = count > 0 ? sv[p][e] / fc : 0.f;
      }
      store8<BF16>(a.k_out, g * a.out_stride + c, sk[p]);
      store8<BF16>(a.v_out, g * a.out_stride + c, sv[p]);
    }
  }
}

}  // namespace

hipError_t launch_kv_merge(bool bf16, int width, const void *k, const void *v, int64_t n, int64_t in_stride,
                           const int32_t *offsets, const int32_t *members, int64_t n_groups, void *k_out,
                           void *v_out, int64_t out_stride, float *bias_out, hipStream_t s) {
  MergeArgs a;
  a.k = k;
  a.v = v;
  a.n = n;
  a.in_stride = in_stride;
  a.offsets = offsets;
  a.members = members;
  a.n_groups = n_groups;
  a.k_out = k_out;
  a.v_out = v_out;
  a.out_stride = out_stride;
  a.bias_out = bias_out;
  a.width = width;
  if (n_groups == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_groups + kWaves - 1) / kWaves)), block(64 * kWaves);
  const int passes = (width + 8 * 64 - 1) / (8 * 64);
#define ISPA_MERGE_LAUNCH(P)                                                                     \
  do {                                                                                           \
    if (bf16)                                                                                    \
      hipLaunchKernelGGL((kv_merge_kernel<true, P>), grid, block, 0, s, a);                     \
    else                                                                                         \
      hipLaunchKernelGGL((kv_merge_kernel<false, P>), grid, block, 0, s, a);                    \
  } while (0)
  switch (passes) {
    case 1: ISPA_MERGE_LAUNCH(1); break;
    case 2: ISPA_MERGE_LAUNCH(2); break;
    case 3: ISPA_MERGE_LAUNCH(3); break;
    default: ISPA_MERGE_LAUNCH(4); break;
  }
#undef ISPA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace ispa
