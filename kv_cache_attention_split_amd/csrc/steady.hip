// L-Layer steady state (ISPA page, section 2 stage 3 "Memory-Efficient Inference": after the warmup a
// converted layer attends to its local context only and projects with the updated weights
// W_new = W + dW).
//
//  * apply_delta_kernel: W_new = W + dW summed in fp32 and rounded to bf16 (nearest, ties to even),
//    written in nn.Linear orientation [d_out, d_in]; from the [d_in, d_out] orientation the sum is
//    transposed through LDS.
//  * proj_bf16_kernel: y = A W_new^T on v_mfma_f32_32x32x16_bf16, A [n, d_in] and W_new [d_out, d_in]
//    both k-contiguous, fp32 accumulation, bf16 output. 128x128 output tiles, 4 waves of 64x64, a ring
//    of four 32-k stages filled by global_load_lds (the Gram kernel's scheme with k-contiguous
//    operands: each 64-byte tile row holds 32 k, read back as 16-byte MFMA operands).
#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

// ---- weight update -------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) apply_delta_kernel(const float *W, const float *dW, int d_in,
                                                          int d_out, int linear, uint16_t *out) {
  __shared__ float t[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  if (linear) {
    // same orientation: out[r][c] = bf16(W[r][c] + dW[r][c]), r < d_out, c < d_in
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
      const int r = by + ty + k, c = bx + tx;
      if (r < d_out && c < d_in) {
        const float s = W[(int64_t)r * d_in + c] + dW[(int64_t)r * d_in + c];
        out[(int64_t)r * d_in + c] = __builtin_bit_cast(uint16_t, (__bf16)s);
      }
    }
    return;
  }
  // W, dW are [d_in, d_out]: tile rows by.. of W (inputs), columns bx.. (outputs)
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int r = by + ty + k, c = bx + tx;
    if (r < d_in && c < d_out) t[ty + k][tx] = W[(int64_t)r * d_out + c] + dW[(int64_t)r * d_out + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int o = bx + ty + k, i = by + tx;   // out[o][i] = sum[i][o]
    if (o < d_out && i < d_in) out[(int64_t)o * d_in + i] = __builtin_bit_cast(uint16_t, (__bf16)t[tx][ty + k]);
  }
}

// ---- projection ----------------------------------------------------------------------------------
constexpr int kThreads = 256;
constexpr int BT = 128;                       // output tile (rows of A x rows of W_new)
constexpr int BK = 32;                        // k per stage
constexpr int NS = 4;                         // stages in the ring
constexpr int RB = BK * 2;                    // bytes of one tile row in a stage (32 bf16)
constexpr int kPart = BT * RB;                // one operand's share of a stage (8 KB)
constexpr int kStage = 2 * kPart;             // 16 KB
constexpr int kCopies = kStage / 1024 / 4;    // 1 KB copy instructions per wave per stage

static __device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[4];

#define ISPA_PROJ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
#define ISPA_PROJ_LDS_BARRIER()          \
  do {                                   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_waitcnt(0xc07f);  \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  } while (0)

struct ProjArgs {
  const uint16_t *a, *w;
  uint16_t *y;
  int64_t n, lda, ldy;
  int d_in, d_out, tiles_n;
};

// A stage holds each operand as [tile row][32 k], 64 bytes per row, with the four 16-byte chunks of
// row r stored at slot c ^ ((r / 4) mod 4): the 16 rows read by one 16-lane group then fall on 16
// distinct bank groups.
__device__ __forceinline__ int chunk_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ void __launch_bounds__(kThreads, 2) proj_bf16_kernel(ProjArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kStage];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_m = (int)((g.n + BT - 1) / BT);
  const int tile = xcd_remap(blockIdx.x, tiles_m * g.tiles_n);
  const int tm = tile / g.tiles_n, tn = tile % g.tiles_n;
  const int64_t m0 = (int64_t)tm * BT;
  const int n0 = tn * BT;
  const int nst = g.d_in / BK;

  // Copy instruction ii of wave w fills 1 KB block blk = w + 4 ii of a stage: blocks 0-7 hold 16 rows
  // of A each, 8-15 16 rows of W_new. Lane l lands at byte 16 l: row 16 (blk mod 8) + l / 4, slot
  // l mod 4, which holds source chunk (l mod 4) ^ ((row / 4) mod 4), i.e. k = 8 chunk .. +7.
  // Rows past the ends read the zero chunk (A) or are clamped (W_new; their outputs are not stored).
  const uint8_t *src[kCopies];
  int64_t row_stride[kCopies];
#pragma unroll
  for (int ii = 0; ii < kCopies; ++ii) {
    const int blk = w + 4 * ii;
    const int op = blk >> 3;
    const int r = 16 * (blk & 7) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    if (op == 0) {
      const int64_t row = m0 + r;
      src[ii] = row < g.n ? (const uint8_t *)(g.a + row * g.lda + 8 * c) : nullptr;
      row_stride[ii] = 0;
    } else {
      int row = n0 + r;
      row = row < g.d_out ? row : g.d_out - 1;
      src[ii] = (const uint8_t *)(g.w + (int64_t)row * g.d_in + 8 * c);
      row_stride[ii] = 0;
    }
  }
  uint64_t zero = (uint64_t)(uintptr_t)g_zero_chunk;
  asm volatile("" : "+s"(zero));

  auto copy_stage = [&](int s, uint8_t *slot) {
#pragma unroll
    for (int ii = 0; ii < kCopies; ++ii) {
      const uint8_t *p = (src[ii] != nullptr && s < nst) ? src[ii] + (int64_t)s * RB
                                                          : (const uint8_t *)(uintptr_t)zero;
      copy_to_lds<16>(p, slot + 1024 * (w + 4 * ii));
    }
  };
  // MFMA operand of 32 rows starting at rb, 16-k step t: lane (l32, hf) reads row rb + l32, k chunk
  // 2 t + hf
  auto read_op = [&](const uint8_t *part, int rb, int t) -> bf16x8 {
    const int r = rb + l32;
    const int c = 2 * t + hf;
    return *(const bf16x8 *)(part + r * RB + 16 * chunk_slot(r, c));
  };
  struct Ops {
    bf16x8 a[2][2], b[2][2];   // [k step][block]
  };
  auto read_stage = [&](const uint8_t *slot, Ops &o) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) o.a[t][bi] = read_op(slot, wm * 64 + bi * 32, t);
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) o.b[t][bj] = read_op(slot + kPart, wn * 64 + bj * 32, t);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  // acc rows are A rows (MFMA A operand = 32 rows of A), columns are W_new rows (B operand)
  auto stage = [&](int s, uint8_t *cur, const uint8_t *nxt, const Ops &ocur, Ops &onx) {
    ISPA_PROJ_WAIT_VMCNT(kCopies * (NS - 2));   // this wave's copies of stage s+1 have landed
    ISPA_PROJ_LDS_BARRIER();                    // ... everyone's; all reads of stage s are done
    copy_stage(s + NS, cur);
    read_stage(nxt, onx);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = mfma_bf16_32x32x16(ocur.a[t][bi], ocur.b[t][bj], acc[bi][bj]);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, kCopies, 0);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  };

  Ops oa, ob;
  copy_stage(0, ring0);
  copy_stage(1, ring1);
  copy_stage(2, ring2);
  copy_stage(3, ring3);
  ISPA_PROJ_WAIT_VMCNT(kCopies * (NS - 1));
  ISPA_PROJ_LDS_BARRIER();
  read_stage(ring0, oa);
  for (int s = 0; s < nst; s += NS) {
    stage(s, ring0, ring1, oa, ob);
    stage(s + 1, ring1, ring2, ob, oa);
    stage(s + 2, ring2, ring3, oa, ob);
    stage(s + 3, ring3, ring0, ob, oa);
  }
  ISPA_PROJ_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended

  // lane (l32, hf) of block (bi, bj) holds rows 8 q + 4 hf + e of column l32 (MFMA D layout)
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int col = n0 + wn * 64 + bj * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (row < g.n && col < g.d_out)
          g.y[row * g.ldy + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[bi][bj][v]);
      }
    }
}

}  // namespace

hipError_t launch_apply_delta(const float *W, const float *dW, int d_in, int d_out, int linear,
                              uint16_t *out, hipStream_t s) {
  const int gx = ((linear ? d_in : d_out) + 31) / 32, gy = ((linear ? d_out : d_in) + 31) / 32;
  hipLaunchKernelGGL(apply_delta_kernel, dim3(gx, gy), dim3(256), 0, s, W, dW, d_in, d_out, linear, out);
  return hipGetLastError();
}

hipError_t launch_project_bf16(int64_t n, int d_in, int d_out, const uint16_t *a, int64_t lda,
                               const uint16_t *w, uint16_t *y, int64_t ldy, hipStream_t s) {
  if (n == 0) return hipSuccess;
  ProjArgs g;
  g.a = a;
  g.w = w;
  g.y = y;
  g.n = n;
  g.lda = lda;
  g.ldy = ldy;
  g.d_in = d_in;
  g.d_out = d_out;
  g.tiles_n = (d_out + BT - 1) / BT;
  const int64_t tiles = ((n + BT - 1) / BT) * g.tiles_n;
  hipLaunchKernelGGL(proj_bf16_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace ispa
