// Dual-stream attention for gfx950 (ISPA page, section 2 "Framework Core", stage 1 "Dual-Stream
// Warmup" and its Decomposable Attention paragraph).
//
// One workgroup owns one (head, query tile) and walks the layer's cache once: first the local keys
// (sink tokens, then the current chunk), then the history keys. A single online-softmax state runs
// through both. When the local keys are exhausted the normalised output and log-sum-exp of the local
// branch are stored (A_loc, lse_loc); the running state then continues over the history, with the
// history's own exp-sum kept apart so that lse_hist is available too, and the final state gives
// A_full and lse_full. This is the page's local/historical split with the merge done in registers:
// the merged result is exactly the single-pass softmax over all keys, and no key is visited twice.
//
// bf16 kernel: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulate);
// the query index runs along the MFMA column, so each lane holds whole softmax rows' statistics and
// the row max / row sum need only one exchange between the two wave halves. K and V tiles (64 keys)
// are copied global -> LDS with global_load_lds (no staging registers) into row-major tiles whose
// 16-byte chunks are XOR-swizzled per row; K operands are plain 16-byte LDS reads, V^T operands come
// from ds_read_b64_tr_b16, whose 4-consecutive-key reads match the key order that the score MFMA
// leaves in each lane's probability registers. The loop is software-pipelined by one tile: step t
// issues the scores of tile t, then the value product of tile t-1 next to the softmax of tile t.
// The running max is updated lazily: the accumulator is rescaled only when the max grows by more
// than 2^8, so exp2 values stay <= 256.
#include <type_traits>

#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr float kRescaleThreshold = 8.0f;   // log2 units

// Key/value rows of one segment run. The local run is the sink followed by the current chunk (two
// pointers, split at the sink length); the history run is one pointer. All fields are uniform.
struct SegRun {
  const uint16_t *k0, *v0, *k1, *v1;
  int64_t s0, s1, split, n;
};

__device__ __forceinline__ SegRun seg_run(const AttnArgs &a, bool hist) {
  SegRun r;
  const uint16_t *sk = (const uint16_t *)a.sink_k, *sv = (const uint16_t *)a.sink_v;
  const uint16_t *ck = (const uint16_t *)a.cur_k, *cv = (const uint16_t *)a.cur_v;
  const uint16_t *hk = (const uint16_t *)a.hist_k, *hv = (const uint16_t *)a.hist_v;
  r.k0 = hist ? hk : sk;
  r.v0 = hist ? hv : sv;
  r.s0 = hist ? a.hist_stride : a.sink_stride;
  r.k1 = hist ? hk : ck;
  r.v1 = hist ? hv : cv;
  r.s1 = hist ? a.hist_stride : a.cur_stride;
  r.n = hist ? a.hist_n : a.sink_n + a.cur_n;
  r.split = hist ? r.n : a.sink_n;
  return r;
}

// Key/value tiles live in LDS row-major ([key][d], D*2 bytes per row) with the 16-byte chunks of
// row r stored at position chunk ^ swz(r). For D = 128 the swizzle is the bit-rotation
// 4 (r mod 4) + (r/4 mod 4): the 16 rows of a K-operand read (same chunk) land on 16 different
// positions, and so do the 4 rows x 4 chunks of a transposing V read.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int kv_off(int r, int col) {   // byte offset of element (r, col)
  return r * (D * 2) + ((((col >> 3) ^ kv_swz<D>(r))) << 4) + ((col & 7) << 1);
}

// read in place of the bias of a segment that has none
static __device__ __attribute__((aligned(16))) float g_zero_bias[4];

// Bias pointer of key j (< the run's length) of the local run (sink then current) or the history
// run, for head `head`; the zero word when that segment has no bias.
__device__ __forceinline__ const float *bias_ptr(const AttnArgs &a, bool hist, int64_t j, int head) {
  if (hist) return a.hist_b != nullptr ? a.hist_b + head * a.hist_bhs + j : g_zero_bias;
  if (j < a.sink_n) return a.sink_b != nullptr ? a.sink_b + head * a.sink_bhs + j : g_zero_bias;
  return a.cur_b != nullptr ? a.cur_b + head * a.cur_bhs + (j - a.sink_n) : g_zero_bias;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int s32x2 __attribute__((ext_vector_type(2)));

// Tile of BK keys from key j0 of a run, when it lies whole inside one of the run's two pointers: its
// base (`tb`, with the head's column offset) and row stride (`st`, elements). Each lane's 64-bit
// source address is then the tile base plus its row and chunk offset; rows (< BK) and strides
// (< 2^23 elements) both fit in 24 bits, so the offset is one full-rate 24-bit multiply (exact: the
// product is below 2^29). Returns false for a tile that crosses the sink/current boundary or the
// run's end (those copies clamp per lane).
template <int BK, bool VALUE>
__device__ __forceinline__ bool tile_plan(const SegRun &run, int64_t j0, int head_off, const uint16_t *&tb,
                                          uint32_t &st) {
  const int64_t j1 = j0 + BK;
  const bool in_first = j1 <= run.split && j1 <= run.n;
  const bool in_second = j0 >= run.split && j1 <= run.n;
  const uint16_t *base0 = VALUE ? run.v0 : run.k0;
  const uint16_t *base1 = VALUE ? run.v1 : run.k1;
  tb = (in_first ? base0 + j0 * run.s0 : base1 + (j0 - run.split) * run.s1) + head_off;
  st = (uint32_t)(in_first ? run.s0 : run.s1);
  return in_first || in_second;
}

// Stage one K or V tile (BK rows) into LDS with direct global->LDS loads: each wave instruction
// fills 1 KiB (1024 / (2D) rows); lane l writes LDS position base + 16 l, so it fetches the global
// chunk that the swizzle assigns to that position. The per-lane (row, chunk) of each of the wave's
// instructions is fixed (`rr`, `cc8` = 8 * chunk), computed once by the caller.
template <int D, int BK, bool VALUE>
__device__ __forceinline__ void dma_tile(const SegRun &run, int64_t j0, int head_off, uint8_t *lds_tile,
                                         int w, const int (&rr)[BK * D * 2 / 4096],
                                         const int (&cc8)[BK * D * 2 / 4096]) {
  constexpr int NW = BK * D * 2 / 4096;     // instructions per wave per tile
  const uint16_t *tb;
  uint32_t st;
  if (tile_plan<BK, VALUE>(run, j0, head_off, tb, st)) {
#pragma unroll
    for (int ii = 0; ii < NW; ++ii)
      copy_to_lds<16>(tb + (__umul24((uint32_t)rr[ii], st) + (uint32_t)cc8[ii]), lds_tile + 1024 * (w + 4 * ii));
    return;
  }
  const uint16_t *base0 = VALUE ? run.v0 : run.k0;
  const uint16_t *base1 = VALUE ? run.v1 : run.k1;
#pragma unroll
  for (int ii = 0; ii < NW; ++ii) {
    int64_t j = j0 + rr[ii];
    j = j < run.n ? j : run.n - 1;
    const bool second = j >= run.split;
    const int64_t jj = second ? j - run.split : j;
    const uint16_t *src = (second ? base1 : base0) + jj * (second ? run.s1 : run.s0) + head_off + cc8[ii];
    copy_to_lds<16>(src, lds_tile + 1024 * (w + 4 * ii));
  }
}

// e4m3 key tile: row r holds D bytes; its 16-byte chunk c is stored at c ^ ((r / 2) mod 8), so the 16
// rows of one operand read (same chunk) spread over the 16 bank groups. Each wave instruction fills
// 1 KiB (1024 / D rows); `rr`, `cc` = the lane's row and source byte offset, fixed per instruction.
template <int D>
__device__ __forceinline__ int k8_off(int r, int byte) {
  return r * D + ((((byte >> 4) ^ ((r >> 1) & 7))) << 4) + (byte & 15);
}
// The same copy serves e4m3 value tiles (VALUE), with the value tile's own chunk placement (v8_off).
template <int D, int BK, bool VALUE = false>
__device__ __forceinline__ void dma_tile_k8(const AttnArgs &a, bool hist, int64_t j0, int head_off, uint8_t *lds_tile,
                                            int w, const int (&rr)[BK * D / 4096], const int (&cc)[BK * D / 4096]) {
  constexpr int NW = BK * D / 4096;
  const uint8_t *k0 = (const uint8_t *)(VALUE ? (hist ? a.hist_v : a.sink_v) : (hist ? a.hist_k : a.sink_k));
  const uint8_t *k1 = (const uint8_t *)(VALUE ? (hist ? a.hist_v : a.cur_v) : (hist ? a.hist_k : a.cur_k));
  const int64_t s0 = hist ? a.hist_stride : a.sink_stride, s1 = hist ? a.hist_stride : a.cur_stride;
  const int64_t n = hist ? a.hist_n : a.sink_n + a.cur_n, split = hist ? n : a.sink_n;
  const int64_t j1 = j0 + BK;
  const bool in_first = j1 <= split && j1 <= n;
  const bool in_second = j0 >= split && j1 <= n;
  if (in_first || in_second) {
    // whole tile inside one segment: a uniform tile base plus the lane's row and chunk offset, one
    // 24-bit multiply (rows < 64, byte strides < 2^23)
    const uint8_t *tb = (in_first ? k0 + j0 * s0 : k1 + (j0 - split) * s1) + head_off;
    const uint32_t st = (uint32_t)(in_first ? s0 : s1);
#pragma unroll
    for (int ii = 0; ii < NW; ++ii)
      copy_to_lds<16>(tb + (__umul24((uint32_t)rr[ii], st) + (uint32_t)cc[ii]), lds_tile + 1024 * (w + 4 * ii));
    return;
  }
#pragma unroll
  for (int ii = 0; ii < NW; ++ii) {
    int64_t j = j0 + rr[ii];
    j = j < n ? j : n - 1;
    const bool second = j >= split;
    const uint8_t *src = (second ? k1 + (j - split) * s1 : k0 + j * s0) + head_off + cc[ii];
    copy_to_lds<16>(src, lds_tile + 1024 * (w + 4 * ii));
  }
}

// e4m3 value tile (D = 128: 64 keys x 128 B): chunk c of key row r is stored at c ^ v8_swz(r), with
// v8_swz(r) = 4 * bit3(r) + 2 * bit1(r). A V^T operand read (ds_read_b64_tr_b8) of one half-wave takes
// the 8 keys 16m + 8a + 4h + 2b + p, (a, b, p) in {0,1}^3 (h fixed per half-wave, see vread8 in the
// kernel), and two adjacent chunks 2j, 2j+1: the 16 (row, chunk) pairs land in the 16 distinct bank
// groups 8p + (chunk ^ v8_swz) of a 256-byte LDS line.
__device__ __forceinline__ int v8_swz(int r) { return (((r >> 3) & 1) << 2) | (((r >> 1) & 1) << 1); }
template <int D>
__device__ __forceinline__ int v8_off(int r, int byte) {
  static_assert(D == 128, "e4m3 value tiles are laid out for 128-byte rows");
  return r * D + ((((byte >> 4) ^ v8_swz(r))) << 4) + (byte & 15);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define ISPA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)

// Workgroup barrier that orders LDS accesses only: waits for this wave's LDS operations, not for its
// outstanding global->LDS copies (those are waited for explicitly with ISPA_WAIT_VMCNT before the
// barrier that publishes them). The empty asm statements keep the compiler from moving memory
// accesses across it.
#define ISPA_LDS_BARRIER()                 \
  do {                                     \
    asm volatile("" ::: "memory");         \
    __builtin_amdgcn_s_waitcnt(0xc07f);    \
    __builtin_amdgcn_s_barrier();          \
    asm volatile("" ::: "memory");         \
  } while (0)

// Store one normalised 32-query block of the O^T accumulator as bf16 rows of A. Lane (l32, hf)
// holds query l32 and, per 32-wide column block db, columns 8g + 4hf + {0..3}.
template <int D>
__device__ __forceinline__ void write_rows(const f32x16 (&o)[D / 32], float inv, void *out, int qi,
                                           int n_q, int out_stride, int head_off, int hf) {
  if (out == nullptr || qi >= n_q) return;
  uint16_t *dst = (uint16_t *)out + (int64_t)qi * out_stride + head_off + 4 * hf;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      pk[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2 *)(dst + 32 * db + 8 * g) = pk;
    }
}

__device__ __forceinline__ void write_lse(float *out, float val, int head, int qi, int n_q, int hf) {
  if (out != nullptr && hf == 0 && qi < n_q) out[(int64_t)head * n_q + qi] = val;
}

#ifndef ISPA_ATTN_BK
#define ISPA_ATTN_BK 64
#endif
#ifndef ISPA_ATTN_PIPE
#define ISPA_ATTN_PIPE 1
#endif
#ifndef ISPA_ATTN_WGS
#define ISPA_ATTN_WGS 2
#endif
#ifndef ISPA_ATTN_VCOPY_VEC
#define ISPA_ATTN_VCOPY_VEC 1   // ping-pong kernel, bf16 values: value copies in the vector phase
#endif
#ifndef ISPA_ATTN_VCOPY_B
#define ISPA_ATTN_VCOPY_B 1     // ping-pong kernel with value products: group B copies the values
#endif
// Ping-pong kernel: a wave runs its matrix phase at this priority (s_setprio) and drops back to 0 after
// the matrix products (mode 1) or after the phase's copies (mode 2). Where both waves of a SIMD have an
// instruction ready, the one in its matrix phase issues first: the MFMAs and their operand reads are the
// critical path, the other wave's softmax fills the cycles between them. 0 turns it off.
#ifndef ISPA_ATTN_PRIO
#define ISPA_ATTN_PRIO 1
#endif
#ifndef ISPA_ATTN_PRIO_MODE
#define ISPA_ATTN_PRIO_MODE 1
#endif
#ifndef ISPA_ATTN_LANE_OFFS
#define ISPA_ATTN_LANE_OFFS 1   // ping-pong kernel: K and V^T operand reads from per-lane offsets set once
#endif

template <int D, bool BIAS>
__global__ void __launch_bounds__(kThreads, ISPA_ATTN_WGS) attn_dual_bf16_kernel(AttnArgs a, int n_qt) {
  constexpr int BK = ISPA_ATTN_BK;    // keys per tile
  constexpr bool PIPE = ISPA_ATTN_PIPE;
  constexpr int TB = BK * D * 2;      // bytes per K or V tile
  constexpr int NKK = D / 16;         // MFMA k-steps of Q.K
  constexpr int NDB = D / 32;         // 32-wide output column blocks
  constexpr int NB = BK / 32;         // 32-key blocks per tile

  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][TB];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int vid = xcd_remap(blockIdx.x, n_qt * a.n_heads);
  const int head = vid / n_qt, qt = vid % n_qt;
  const int head_off = head * D;
  const int qrow0 = qt * 128 + w * 32;
  const int qi = qrow0 + l32;
  const int n_q = a.n_q;
  const int out_stride = a.n_heads * D;
  const float sl2 = a.scale_log2;

  // Q^T operand, kept in registers for the whole pass: lane holds query l32, d = 16kk + 8hf .. +8.
  bf16x8 qr[NKK];
  {
    const bool ok = qi < n_q;
    const uint16_t *src = (const uint16_t *)a.q + (int64_t)(ok ? qi : 0) * a.q_stride + head_off + hf * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = *(const u32x4 *)(src + kk * 16);
      if (!ok) x = u32x4{0u, 0u, 0u, 0u};
      qr[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t n_loc = a.sink_n + a.cur_n;
  const int nt_loc = (int)((n_loc + BK - 1) / BK);
  const int nt_hist = (int)((a.hist_n + BK - 1) / BK);
  const int nt = nt_loc + nt_hist;

  // per-lane geometry of this wave's DMA instructions (same for K and V tiles)
  constexpr int NW = BK * D * 2 / 4096;
  int drow[NW], dcol8[NW];
#pragma unroll
  for (int ii = 0; ii < NW; ++ii) {
    constexpr int CPR = D / 8;
    const int r = (w + 4 * ii) * (1024 / (2 * D)) + lane / CPR;
    drow[ii] = r;
    dcol8[ii] = 8 * ((lane % CPR) ^ kv_swz<D>(r));
  }
  auto tile_j0 = [&](int t) -> int64_t { return (int64_t)(t >= nt_loc ? t - nt_loc : t) * BK; };
  auto dma_k = [&](int t, int buf) {
    dma_tile<D, BK, false>(seg_run(a, t >= nt_loc), tile_j0(t), head_off, kbuf[buf], w, drow, dcol8);
  };
  auto dma_v = [&](int t, int buf) {
    dma_tile<D, BK, true>(seg_run(a, t >= nt_loc), tile_j0(t), head_off, vbuf[buf], w, drow, dcol8);
  };
  auto n_valid_of = [&](int t) -> int {
    const int64_t nseg = t >= nt_loc ? a.hist_n : n_loc;
    const int64_t rem = nseg - tile_j0(t);
    return (int)(rem < BK ? rem : BK);
  };

  // S^T[key][query] = K Q^T for one tile (K operand: one 16-byte read per MFMA, read one MFMA
  // ahead so that LDS latency hides behind the previous MFMA).
  auto kread = [&](int buf, int i) -> bf16x8 {
    const int kk = i / NB, b = i % NB;
    return *(const bf16x8 *)(kbuf[buf] + kv_off<D>(32 * b + l32, 16 * kk + 8 * hf));
  };
  auto qk = [&](f32x16 (&s)[NB], int buf) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[b][v] = 0.f;
    bf16x8 kcur = kread(buf, 0);
#pragma unroll
    for (int i = 0; i < NKK * NB; ++i) {
      const bf16x8 knext = kread(buf, i + 1 < NKK * NB ? i + 1 : i);
      s[i % NB] = mfma_bf16_32x32x16(kcur, qr[i / NB], s[i % NB]);
      kcur = knext;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = -INFINITY, l = 0.f, l_loc = 0.f;

  // O^T[d][query] += V^T P^T for tile u; V^T operands by transposing reads of the row-major V tile:
  // rows 32b + 16h2 + 4hf + (0..3) and the same + 8, matching the key order of p[b][h2].
  // MFMA i of a tile covers column block db = i / (2 NB), key block b = (i / 2) % NB, half h2 = i % 2.
  constexpr int NPV = NDB * NB * 2;
  const int g = lane >> 4, sl = lane & 15;
  auto vread = [&](int u, int i) -> bf16x8 {
    const uint8_t *vt = vbuf[u & 1];
    const int db = i / (2 * NB), b = (i / 2) % NB, h2 = i % 2;
    const int col = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
    const int row = 32 * b + 16 * h2 + 4 * (g >> 1) + (sl >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(vt + kv_off<D>(row, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(vt + kv_off<D>(row + 8, col)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv = [&](int u, const bf16x8 (&p)[NB][2]) {
    bf16x8 vcur = vread(u, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const bf16x8 vnext = vread(u, i + 1 < NPV ? i + 1 : i);
      const int db = i / (2 * NB), b = (i / 2) % NB, h2 = i % 2;
      o[db] = mfma_bf16_32x32x16(vcur, p[b][h2], o[db]);
      vcur = vnext;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Store A_loc / lse_loc once the local tiles are all in the accumulator; the history then keeps
  // adding to the same state with its exp-sum kept apart.
  auto snapshot_local = [&]() {
    const float tot = halves_sum(l);
    const float inv = 1.0f / tot;
    const float lse = (m + __log2f(tot)) * kLn2;
    write_rows<D>(o, inv, a.a_loc, qi, n_q, out_stride, head_off, hf);
    write_lse(a.lse_loc, lse, head, qi, n_q, hf);
    if (nt_hist == 0) {
      write_rows<D>(o, inv, a.a_full, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_full, lse, head, qi, n_q, hf);
      write_lse(a.lse_hist, -INFINITY, head, qi, n_q, hf);
    }
    l_loc = l;
    l = 0.f;
  };

  // Step t (software-pipelined by one tile): loads for the next step, the scores of tile t, then
  // the value product of tile t-1 (MFMA) interleaved with the softmax of tile t (VALU), which are
  // independent; a rare rescale of the accumulator when the running max grew by more than 2^8.
  auto step = [&](auto has_pv, int t, const bf16x8 (&pp)[NB][2], bf16x8 (&pc)[NB][2]) {
    if constexpr (PIPE) {
      if (t + 1 < nt) dma_k(t + 1, (t + 1) & 1);
      dma_v(t, t & 1);
    } else {
      if (t + 1 < nt) {
        dma_k(t + 1, (t + 1) & 1);
        dma_v(t + 1, (t + 1) & 1);
      }
    }
    f32x16 sc[NB];
    qk(sc, t & 1);
    if constexpr (BIAS) {
      // sc += b / tau, read straight from global memory (key 32b + 8(v/4) + 4hf + v%4 of the tile)
      const bool hist = t >= nt_loc;
      const int64_t nseg = hist ? a.hist_n : n_loc;
      const int64_t j0 = tile_j0(t);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int64_t j = j0 + 32 * b + 8 * (v >> 2) + 4 * hf + (v & 3);
          j = j < nseg ? j : nseg - 1;
          sc[b][v] = __builtin_fmaf(*bias_ptr(a, hist, j, head), a.bias_to_score, sc[b][v]);
        }
    }
    const int n_valid = n_valid_of(t);
    if (n_valid < BK) {
      const int nv = n_valid - 4 * hf;   // key 32b + 8(v/4) + 4hf + v%4 < n_valid
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[b][v] = 32 * b + 8 * (v >> 2) + (v & 3) < nv ? sc[b][v] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[b][v]);
    mx = halves_max(mx);
    const float mnew = mx * sl2;
    const bool need = mnew > m + kRescaleThreshold;
    const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;
    const float mt = need ? mnew : m;
    const float mneg = -mt;
    float sum = 0.f;
    // The 32 probabilities of this tile are produced in NPV slices, one after each MFMA of the
    // previous tile's value product, so the VALU work overlaps the matrix pipe.
    constexpr int EPS = NB * 16 / NPV;       // elements per slice
    static_assert(EPS >= 2 && EPS * NPV == NB * 16, "slices must cover the tile");
    uint32_t pw[NB * 8];
    bf16x8 vcur;
    if constexpr (decltype(has_pv)::value) vcur = vread(t - 1, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      bf16x8 vnext;
      if constexpr (decltype(has_pv)::value) {
        vnext = vread(t - 1, i + 1 < NPV ? i + 1 : i);
        const int db = i / (2 * NB), b = (i / 2) % NB, h2 = i % 2;
        o[db] = mfma_bf16_32x32x16(vcur, pp[b][h2], o[db]);
      }
      const float mneg_i = mneg;
#pragma unroll
      for (int e = 0; e < EPS; e += 2) {
        const int f = i * EPS + e;            // flattened element: block f / 16, index f % 16
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[f / 16][f % 16], sl2, mneg_i));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[f / 16][f % 16 + 1], sl2, mneg_i));
        sum += p0 + p1;
        pw[f / 2] = pack_bf16x2(p0, p1);
      }
      if constexpr (decltype(has_pv)::value) vcur = vnext;
    }
#ifdef ISPA_IGLP
    __builtin_amdgcn_iglp_opt(ISPA_IGLP);
#endif
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 u;
        u[0] = pw[b * 8 + h2 * 4 + 0];
        u[1] = pw[b * 8 + h2 * 4 + 1];
        u[2] = pw[b * 8 + h2 * 4 + 2];
        u[3] = pw[b * 8 + h2 * 4 + 3];
        pc[b][h2] = __builtin_bit_cast(bf16x8, u);
      }
    // the accumulator now holds tiles 0..t-1 at the previous max
    if constexpr (PIPE) {
      if (t - 1 == nt_loc - 1) snapshot_local();
    }
    if (__ballot(need) != 0ull) {
      l *= alpha;
      l_loc *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    m = mt;
    l += sum;
    if constexpr (!PIPE) {
      pv(t, pc);
      if (t == nt_loc - 1) snapshot_local();
    }
    ISPA_WAIT_VMCNT(0);   // this wave's loads of K(t+1) and V(t) have landed
    __syncthreads();      // ... and everyone's; all reads of this step's buffers are done
  };

  using no_pv = std::integral_constant<bool, false>;
  using with_pv = std::integral_constant<bool, true>;
  bf16x8 pa[NB][2], pb[NB][2];
  if constexpr (PIPE) {
    dma_k(0, 0);
    ISPA_WAIT_VMCNT(0);
    __syncthreads();
    step(no_pv{}, 0, pb, pa);
    int t = 1;
    for (; t + 1 < nt; t += 2) {
      step(with_pv{}, t, pa, pb);
      step(with_pv{}, t + 1, pb, pa);
    }
    if (t < nt) {
      step(with_pv{}, t, pa, pb);
      pv(t, pb);
    } else {
      pv(t - 1, pa);
    }
    if (nt - 1 == nt_loc - 1) snapshot_local();
  } else {
    dma_k(0, 0);
    dma_v(0, 0);
    ISPA_WAIT_VMCNT(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) step(no_pv{}, t, pb, pa);
  }

  if (nt_hist > 0) {
    const float th = halves_sum(l);
    const float tl = halves_sum(l_loc);
    const float tot = th + tl;
    write_rows<D>(o, 1.0f / tot, a.a_full, qi, n_q, out_stride, head_off, hf);
    write_lse(a.lse_full, (m + __log2f(tot)) * kLn2, head, qi, n_q, hf);
    write_lse(a.lse_hist, th > 0.f ? (m + __log2f(th)) * kLn2 : -INFINITY, head, qi, n_q, hf);
  }
}

// Balanced schedule (SPLIT form of the ping-pong kernel). XCD x (workgroup id mod 8) keeps the units the
// plain schedule gives it, [us, us + nx), and their lockstep walk over the keys, so that each K/V tile
// is still fetched about once per XCD: main workgroup j (id x + 8 j, j < nx) takes key tiles [0, R) of
// unit us + j, and the XCD's E = S - nx spare workgroups (S per XCD) share the remaining tiles [R, nt)
// of those units, laid end to end, in E equal ranges. Every piece stores its online-softmax state to
// workspace slot 4 u + k (k = 0 the main piece, then the remaining tiles' pieces in key order); the
// workgroup that completes a unit's last piece merges them in that order. Which workgroup runs on which
// XCD decides the speed only: the partition is a function of the workgroup id.
#ifndef ISPA_SPLIT_MARGIN
#define ISPA_SPLIT_MARGIN 6
#endif
constexpr int kSplitSlots = 4;                               // per unit
// pieces of one workgroup: a spare range of nx L / E tiles meets at most ceil(nx / E) + 1 units, each cut at
// most once more at the local end; the host keeps 2 (ceil(nx / E) + 1) within this table
constexpr int kSplitMaxPieces = 72;
constexpr size_t kSplitScal = 16 * 512 * 4;                 // floats of one stored accumulator
constexpr size_t kSplitSlotFloats = kSplitScal + 4 * 512;

struct SplitGeom {
  int us, nx, R, L, E;   // units [us, us + nx); main tiles [0, R); L = nt - R tiles left per unit; E spares
  int64_t len;           // nx L: the XCD's remaining tiles, end to end
};
__device__ __forceinline__ SplitGeom split_geom(int x, int units, int S, int nt) {
  SplitGeom g;
  const int per = units / 8, rem = units % 8;
  g.us = x * per + (x < rem ? x : rem);
  g.nx = per + (x < rem ? 1 : 0);
  // main workgroups take ISPA_SPLIT_MARGIN tiles more than an equal share: the spare ones, which run
  // several pieces, then tend to finish first, and each main workgroup merges its own unit
  const int r = (int)((int64_t)g.nx * nt / S) + ISPA_SPLIT_MARGIN;
  g.R = r < nt - 1 ? r : nt - 1;
  g.L = nt - g.R;
  g.E = S - g.nx;
  g.len = (int64_t)g.nx * g.L;
  return g;
}

// Cuts strictly inside the remaining tiles (R, nt) of the XCD's unit k, in order: the spare-range
// boundary that falls there (ranges are at least L tiles long when nx >= E, so at most one) and the
// local end (a piece never holds keys of both branches unless it starts at tile 0).
struct UnitCuts {
  int n, c0, c1;
};
__device__ __forceinline__ UnitCuts unit_cuts(const SplitGeom &g, int k, int nt, int nt_loc) {
  const int64_t u0 = (int64_t)k * g.L;
  // the first range start floor(e len / E) above u0
  const int64_t e = ((u0 + 1) * g.E + g.len - 1) / g.len;
  int bc = -1;
  if (e < g.E) {
    const int64_t bnd = e * g.len / g.E;
    if (bnd < u0 + g.L) bc = g.R + (int)(bnd - u0);
  }
  const int lc = (g.R < nt_loc && nt_loc < nt) ? nt_loc : -1;
  UnitCuts r;
  if (bc >= 0 && lc >= 0 && bc != lc) {
    r.n = 2;
    r.c0 = bc < lc ? bc : lc;
    r.c1 = bc < lc ? lc : bc;
  } else {
    r.n = (bc >= 0 || lc >= 0) ? 1 : 0;
    r.c0 = r.c1 = bc >= 0 ? bc : lc;
  }
  return r;
}

// Merge of unit us + k's pieces (all 512 threads; bf16 values, head_dim 128) in slot order. Each piece
// holds its accumulator o and running maximum m (log2 units) with the exp-sum l of its keys; the main
// piece, when it completed the local keys (and wrote A_loc itself), holds l of its history keys and
// l_loc of its local keys. A_full and lse_full merge every piece, lse_hist the pieces with history keys,
// and A_loc and lse_loc, when the main piece ends inside the local keys, the pieces inside them.
__device__ __forceinline__ void merge_unit(const AttnArgs &a, const SplitGeom &sg, int k, int nt, int nt_loc,
                                           int nt_hist, int n_qt, int tid) {
  constexpr int D = 128, NDB = 4;
  const int vid = sg.us + k;
  const int lane = tid & 63, hf = lane >> 5;
  const int head = vid / n_qt, qt = vid % n_qt;
  const int qi = qt * 256 + (tid >> 6) * 32 + (lane & 31);
  const int head_off = head * D, out_stride = a.n_heads * D, n_q = a.n_q;
  const UnitCuts cu = unit_cuts(sg, k, nt, nt_loc);
  const int np = 2 + cu.n;
  // last key tile (exclusive) of piece p
  auto hi = [&](int p) { return p == 0 ? sg.R : (p == 1 && cu.n >= 1) ? cu.c0 : (p == 2 && cu.n == 2) ? cu.c1 : nt; };
  const float *base = a.split_ws + (size_t)kSplitSlots * vid * kSplitSlotFloats;
  auto pass = [&](auto local_c) {
    constexpr bool LOCAL = decltype(local_c)::value;
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p) {
      if (LOCAL && hi(p) > nt_loc) continue;
      mx = fmaxf(mx, base[(size_t)p * kSplitSlotFloats + kSplitScal + tid]);
    }
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
    float ls = 0.f, lh = 0.f;
    for (int p = 0; p < np; ++p) {
      if (LOCAL && hi(p) > nt_loc) continue;
      const float *sl = base + (size_t)p * kSplitSlotFloats;
      const float m = sl[kSplitScal + tid], l = sl[kSplitScal + 512 + tid];
      const float c = __builtin_amdgcn_exp2f(m - mx);
      ls += (LOCAL ? l : l + sl[kSplitScal + 1024 + tid]) * c;
      if (!LOCAL && hi(p) > nt_loc) lh += l * c;   // a piece with history keys: l is their sum
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 x = *(const f32x4 *)(sl + 4 * ((db * 4 + g4) * 512 + tid));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * g4 + e] += x[e] * c;
        }
    }
    const float tot = halves_sum(ls);
    if constexpr (LOCAL) {
      write_rows<D>(acc, 1.0f / tot, a.a_loc, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_loc, (mx + __log2f(tot)) * kLn2, head, qi, n_q, hf);
    } else {
      write_rows<D>(acc, 1.0f / tot, a.a_full, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_full, (mx + __log2f(tot)) * kLn2, head, qi, n_q, hf);
      const float th = halves_sum(lh);
      write_lse(a.lse_hist, nt_hist > 0 && th > 0.f ? (mx + __log2f(th)) * kLn2 : -INFINITY, head, qi, n_q, hf);
    }
  };
  pass(std::integral_constant<bool, false>{});
  if (sg.R < nt_loc) pass(std::integral_constant<bool, true>{});
  if (tid == 0) a.split_count[vid] = 0;   // ready for the next call
}

// ------------------------------------------------------------------------------------------------
// Ping-pong kernel: 8 waves (two per SIMD), 256 queries per workgroup. Waves 0-3 (group A) and
// 4-7 (group B) run the same loop, B one barrier behind A; every iteration has a matrix phase
// (scores of tile i, value product of tile i-1) and a vector phase (softmax of tile i), separated by
// workgroup barriers, so on each SIMD one wave's MFMAs run while the other wave's softmax runs.
// Both groups read the same K/V tiles one phase apart; group A issues the global->LDS copies after
// its matrix phase's LDS reads, and (bf16 values) the value copies at the start of its vector phase,
// which has no LDS access: the compiler turns every LDS-read wait into a full wait while a global->LDS
// copy is in flight, so no copy may be pending across a phase with LDS reads. A burst of copies
// stalls the issuing wave for hundreds of cycles; splitting it between the two phases keeps either
// phase from growing past the other group's phase beside it. In the matrix phase no copy is in flight
// and the operand reads run four operands ahead of the MFMAs (scheduling groups below).
// ------------------------------------------------------------------------------------------------
// LSE_ONLY: only the log-sum-exp outputs are wanted (no value copies, no value product, no A rows).
// FP8: q and the keys are e4m3 bytes (per-head scales): the scores run on v_mfma_f32_32x32x64_f8f6f4,
// two k-steps of 64 per 32-key block, and a key tile is half the bytes; values stay bf16.
// FP8V (with FP8): the values are e4m3 bytes too (one scale per head) and the probabilities are rounded
// to e4m3 for the value product, one 32x32x64 MFMA per 32-column block and tile: P^T's 64 keys are the
// 32 probabilities each lane holds after the softmax, in register order, and the V^T operand is read
// with ds_read_b64_tr_b8 in that same key order. The exp-sum keeps the unrounded probabilities; the
// value scale multiplies the normalised rows.
template <int D, bool BIAS, bool LSE_ONLY = false, bool FP8 = false, bool FP8V = false, bool SPLIT = false>
__global__ void __launch_bounds__(512, 1) attn_dual_bf16_pp_kernel(AttnArgs a, int n_qt) {
  static_assert(FP8 || !FP8V, "the FP8 value product comes with FP8 scores");
  static_assert(!(SPLIT && LSE_ONLY), "the LSE-only form has its own key split");
  constexpr int BK = 64;
  constexpr int TB = BK * D * 2;
  constexpr int TBK = FP8 ? BK * D : TB;     // bytes of a key tile
  constexpr int TBV = FP8V ? BK * D : TB;    // bytes of a value tile
  // where group A issues the value copies: beside the softmax where the matrix phase is the longer one
  constexpr bool VCOPY_VEC = !LSE_ONLY && !FP8V && ISPA_ATTN_VCOPY_VEC;
  // bf16 or e4m3 values: group B copies V(i+1) at the start of its vector phase of tile i, beside group A's
  // matrix phase i+1. Issuing a 1 KiB global->LDS copy holds a wave for about 40 cycles, more while
  // other copies are in flight, so the copies go to the phases with slack: B's softmax is shorter than A's
  // matrix phase plus A's key copies, and A's vector phase then carries no copies at all
  constexpr bool VCOPY_B = !LSE_ONLY && ISPA_ATTN_VCOPY_B;
  constexpr int NKK = D / 16;
  constexpr int NK8 = D / 64;                // e4m3 k-steps
  constexpr int NDB = D / 32;
  constexpr int NB = BK / 32;
  constexpr int NPV = NDB * NB * 2;

  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][TBK];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][TBV];
  __shared__ __attribute__((aligned(256))) float bbuf[2][BIAS ? BK : 1];   // bias of tiles, beside K
  __shared__ uint64_t s_merge;   // SPLIT: the units (bit k - k_lo) whose merge falls to this workgroup
  __shared__ int4 s_piece[SPLIT ? kSplitMaxPieces : 1];   // SPLIT: this workgroup's pieces
  __shared__ int s_npiece, s_klo, s_khi;
  __shared__ uint64_t s_two;

  const int tid = threadIdx.x;
  // the wave index as a uniform value (group branches and LDS bases stay scalar)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int grp = w >> 2, wl = w & 3;
  const int n_q = a.n_q;
  const int out_stride = a.n_heads * D;
  const int64_t n_loc = a.sink_n + a.cur_n;
  const int nt_loc = (int)((n_loc + BK - 1) / BK);
  const int nt_hist = (int)((a.hist_n + BK - 1) / BK);
  const int nt = nt_loc + nt_hist;            // key tiles of every (head, query tile) unit
  const int nsplit = LSE_ONLY ? a.lse_splits : 1;   // key ranges per unit in the LSE-only form

  // SPLIT (balanced schedule, see split_geom): a main workgroup runs one piece, [0, R) of its unit; a
  // spare one walks its range of the XCD's remaining tiles piece by piece (a piece ends at a unit's end
  // and at the local end). Thread 0 lists the pieces (unit, first tile, end tile, slot) in LDS before
  // the tile loops, so that the schedule's state is not held in registers across them (it spilled
  // scalar registers inside the tile loop). Otherwise one pass: the workgroup's own unit (and key range).
  int npiece = 1;
  if constexpr (SPLIT) {
    if (tid == 0) {
      const int jw = (int)(blockIdx.x >> 3);
      const SplitGeom sg = split_geom((int)(blockIdx.x & 7), n_qt * a.n_heads, (int)(gridDim.x >> 3), nt);
      int n = 0, k_lo = -1, k_hi = -1;
      uint64_t two = 0;
      if (jw < sg.nx) {
        s_piece[n++] = int4{sg.us + jw, 0, sg.R, kSplitSlots * (sg.us + jw)};
        k_lo = k_hi = jw;
      } else {
        int64_t pos = (int64_t)(jw - sg.nx) * sg.len / sg.E;
        const int64_t end = (int64_t)(jw - sg.nx + 1) * sg.len / sg.E;
        while (pos < end && n < kSplitMaxPieces) {
          const int k = (int)(pos / sg.L);
          const int t0 = sg.R + (int)(pos - (int64_t)k * sg.L);
          const int64_t e = end - (int64_t)k * sg.L;
          int t1 = sg.R + e < nt ? (int)(sg.R + e) : nt;
          if (t0 < nt_loc && nt_loc < t1) t1 = nt_loc;
          const UnitCuts cu = unit_cuts(sg, k, nt, nt_loc);
          const int slot = kSplitSlots * (sg.us + k) + 1 + (cu.n >= 1 && cu.c0 <= t0) + (cu.n == 2 && cu.c1 <= t0);
          s_piece[n++] = int4{sg.us + k, t0, t1, slot};
          pos = (int64_t)k * sg.L + (t1 - sg.R);
          if (k_lo < 0) k_lo = k;
          if (k == k_hi) two |= 1ull << (k - k_lo);
          k_hi = k;
        }
      }
      s_npiece = n;
      s_klo = k_lo;
      s_khi = k_hi;
      s_two = two;
    }
    __syncthreads();
    npiece = s_npiece;
  }
  auto piece_body = [&](int pi) {
  int vid, split = 0, t0, t1, slot = 0;
  if constexpr (SPLIT) {
    const int4 pc = s_piece[pi];
    vid = pc.x;
    t0 = pc.y;
    t1 = pc.z;
    slot = pc.w;
  } else {
    const int lin = xcd_remap(blockIdx.x, n_qt * a.n_heads * nsplit);
    vid = lin / nsplit;
    split = lin % nsplit;
    // tiles of this workgroup: all of them, or one contiguous range per split in the LSE-only form
    t0 = LSE_ONLY ? (int)((int64_t)split * nt / nsplit) : 0;
    t1 = LSE_ONLY ? (int)((int64_t)(split + 1) * nt / nsplit) : nt;
  }
  const int head = vid / n_qt, qt = vid % n_qt;
  const int head_off = head * D;
  const int qi = qt * 256 + w * 32 + l32;
  float sl2 = a.scale_log2;
  if constexpr (FP8) sl2 *= a.q_scale[head] * a.k_scale[head];   // scores of the dequantised values
  const float v_mul = FP8V ? a.v_scale[head] : 1.0f;              // values of the dequantised codes

  bf16x8 qr[FP8 ? 1 : NKK];
  i32x8 qf[FP8 ? NK8 : 1];   // e4m3 q: lane holds dims 64ks + 32hf .. +31
  if constexpr (FP8) {
    const bool ok = qi < n_q;
    const uint8_t *src = (const uint8_t *)a.q + (int64_t)(ok ? qi : 0) * a.q_stride + head_off + hf * 32;
#pragma unroll
    for (int ks = 0; ks < NK8; ++ks) {
      u32x4 x0 = *(const u32x4 *)(src + 64 * ks), x1 = *(const u32x4 *)(src + 64 * ks + 16);
      if (!ok) x0 = x1 = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  } else {
    const bool ok = qi < n_q;
    const uint16_t *src = (const uint16_t *)a.q + (int64_t)(ok ? qi : 0) * a.q_stride + head_off + hf * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = *(const u32x4 *)(src + kk * 16);
      if (!ok) x = u32x4{0u, 0u, 0u, 0u};
      qr[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }


  constexpr int NW = BK * D * 2 / 4096;   // copy instructions per group-A wave per tile
  int drow[NW], dcol8[NW];
#pragma unroll
  for (int ii = 0; ii < NW; ++ii) {
    constexpr int CPR = D / 8;
    const int r = (wl + 4 * ii) * (1024 / (2 * D)) + lane / CPR;
    drow[ii] = r;
    dcol8[ii] = 8 * ((lane % CPR) ^ kv_swz<D>(r));
  }
  constexpr int NW8 = FP8 ? BK * D / 4096 : 1;   // e4m3 key copies per group-A wave per tile
  int k8row[NW8], k8col[NW8];
  if constexpr (FP8) {
#pragma unroll
    for (int ii = 0; ii < NW8; ++ii) {
      const int r = (wl + 4 * ii) * (1024 / D) + lane / (D / 16);
      k8row[ii] = r;
      k8col[ii] = 16 * ((lane % (D / 16)) ^ ((r >> 1) & 7));
    }
  }
  auto tile_j0 = [&](int t) -> int64_t { return (int64_t)(t >= nt_loc ? t - nt_loc : t) * BK; };
  auto dma_k = [&](int t, int buf) {
    if constexpr (FP8)
      dma_tile_k8<D, BK>(a, t >= nt_loc, tile_j0(t), head_off, kbuf[buf], wl, k8row, k8col);
    else
      dma_tile<D, BK, false>(seg_run(a, t >= nt_loc), tile_j0(t), head_off, kbuf[buf], wl, drow, dcol8);
  };
  int v8row[FP8V ? NW8 : 1], v8col[FP8V ? NW8 : 1];
  if constexpr (FP8V) {
#pragma unroll
    for (int ii = 0; ii < NW8; ++ii) {
      const int r = (wl + 4 * ii) * (1024 / D) + lane / (D / 16);
      v8row[ii] = r;
      v8col[ii] = 16 * ((lane % (D / 16)) ^ v8_swz(r));
    }
  }
  auto dma_v = [&](int t, int buf) {
    if constexpr (FP8V)
      dma_tile_k8<D, BK, true>(a, t >= nt_loc, tile_j0(t), head_off, vbuf[buf], wl, v8row, v8col);
    else
      dma_tile<D, BK, true>(seg_run(a, t >= nt_loc), tile_j0(t), head_off, vbuf[buf], wl, drow, dcol8);
  };
  auto n_valid_of = [&](int t) -> int {
    const int64_t nseg = t >= nt_loc ? a.hist_n : n_loc;
    const int64_t rem = nseg - tile_j0(t);
    return (int)(rem < BK ? rem : BK);
  };
  // bias of tile t (one wave, 4 bytes per lane = key j0 + lane; keys past the end repeat the last)
  auto dma_b = [&](int t, int buf) {
    const bool hist = t >= nt_loc;
    const int64_t nseg = hist ? a.hist_n : n_loc;
    int64_t j = tile_j0(t) + lane;
    j = j < nseg ? j : nseg - 1;
    copy_to_lds<4>(bias_ptr(a, hist, j, head), bbuf[buf]);
  };
  const int g = lane >> 4, sl = lane & 15;
  // The swizzle of a tile row depends on the row mod 16 only, so the byte offset of (R0 + r, col) is
  // R0 * 2D + that of (r, col) for R0 a multiple of 16: a lane's K and V^T operand reads differ by their
  // 32-key block b (and the 16-row half h2 of a V^T read) only in an immediate. With LANE_OFFS the
  // lane's offsets of the 32-key block 0 (8 for K, one per 16-column step; 2 per 32-column block for
  // V^T) are formed once, before the tile loop, and kept (the empty asm stops the compiler from forming
  // them again in every tile, which it did: about 56 address instructions per wave and tile).
  constexpr bool LOFFS = ISPA_ATTN_LANE_OFFS && !FP8;        // bf16 keys
  constexpr bool LOFFS_V = ISPA_ATTN_LANE_OFFS && !FP8V && !LSE_ONLY;   // bf16 values
  int koff[LOFFS ? NKK : 1], voff[LOFFS_V ? 2 * NDB : 1];
  if constexpr (LOFFS) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      koff[kk] = kv_off<D>(l32, 16 * kk + 8 * hf);
      asm volatile("" : "+v"(koff[kk]));
    }
  }
  if constexpr (LOFFS_V) {
    const int r = 4 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
      voff[2 * db] = kv_off<D>(r, col);
      voff[2 * db + 1] = kv_off<D>(r + 8, col);
      asm volatile("" : "+v"(voff[2 * db]), "+v"(voff[2 * db + 1]));
    }
  }
  auto kread = [&](int buf, int i) -> bf16x8 {
    const int kk = i / NB, b = i % NB;
    if constexpr (LOFFS) return *(const bf16x8 *)(kbuf[buf] + koff[kk] + 32 * b * (D * 2));
    return *(const bf16x8 *)(kbuf[buf] + kv_off<D>(32 * b + l32, 16 * kk + 8 * hf));
  };
  auto vread = [&](int u, int i) -> bf16x8 {
    const uint8_t *vt = vbuf[u & 1];
    const int db = i / (2 * NB), b = (i / 2) % NB, h2 = i % 2;
    const int col = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
    const int row = 32 * b + 16 * h2 + 4 * (g >> 1) + (sl >> 2);
    const int off_lo = LOFFS_V ? voff[LOFFS_V ? 2 * db : 0] + (32 * b + 16 * h2) * (D * 2) : kv_off<D>(row, col);
    const int off_hi = LOFFS_V ? voff[LOFFS_V ? 2 * db + 1 : 0] + (32 * b + 16 * h2) * (D * 2) : kv_off<D>(row + 8, col);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(vt + off_lo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(vt + off_hi));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // e4m3 V^T operand of 32-column block db for the 64 keys of a tile: byte j of lane (column l32, half
  // hf) must hold the key whose probability sits in byte j of the P^T operand, i.e. key
  // 32 (j/16) + 8 ((j mod 16)/4) + 4 hf + j mod 4. Read m (bytes 8m .. 8m+7) therefore takes keys
  // 16m + 8 (e/4) + 4 hf + e mod 4, e = 0..7: lane s of each 16-lane group addresses key e = s/2 of that
  // list and bytes 32 db + 16 (g mod 2) + 8 (s mod 2) .. +7, and receives column 32 db + l32 of the 8
  // keys. The lane's row and swizzle do not depend on m, so the 16 reads of a tile share 4 addresses.
  int v8addr[FP8V ? NDB : 1];
  if constexpr (FP8V) {
    const int e = sl >> 1, hh = g >> 1;
    const int r0 = 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) v8addr[db] = v8_off<D>(r0, 32 * db + 16 * (g & 1) + 8 * (sl & 1));
  }
  auto vread8 = [&](int u, int db) -> i32x8 {
    const uint8_t *vt = vbuf[u & 1] + v8addr[db];
    s32x2 r[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
      r[mm] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) s32x2 *)(vt + 16 * D * mm));
    return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = -INFINITY, l = 0.f, l_loc = 0.f;
  f32x16 sc[NB];
  bf16x8 pk[FP8V ? 1 : NB][2];
  i32x8 pf = {};   // FP8V: the tile's 32 probabilities of this lane as e4m3, in register order

  // SPLIT workspace slot: the state (o as 16 float4 per thread, thread-minor) at 0 and per-thread
  // scalars at kSplitScal + k * 512 (k: 0 m, 1 l, 2 l_loc)
  float *const slot_ws = SPLIT ? a.split_ws + (size_t)slot * kSplitSlotFloats : nullptr;
  auto store_state = [&](float *dst) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4 *)(dst + 4 * ((db * 4 + g4) * 512 + tid)) =
            f32x4{o[db][4 * g4], o[db][4 * g4 + 1], o[db][4 * g4 + 2], o[db][4 * g4 + 3]};
  };
  auto snapshot_local = [&]() {
    const float tot = halves_sum(l);
    const float inv = 1.0f / tot;
    const float lse = (m + __log2f(tot)) * kLn2;
    if constexpr (!LSE_ONLY) write_rows<D>(o, inv * v_mul, a.a_loc, qi, n_q, out_stride, head_off, hf);
    write_lse(a.lse_loc, lse, head, qi, n_q, hf);
    if (nt_hist == 0) {
      if constexpr (!LSE_ONLY) write_rows<D>(o, inv * v_mul, a.a_full, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_full, lse, head, qi, n_q, hf);
      write_lse(a.lse_hist, -INFINITY, head, qi, n_q, hf);
    }
    l_loc = l;
    l = 0.f;
  };

  // prologue: K(t0) for everyone; group B then falls one barrier behind
  if (grp == 0) {
    if (!LSE_ONLY || t0 < t1) dma_k(t0, t0 & 1);
    if (VCOPY_B && t0 < t1) dma_v(t0, t0 & 1);   // group B copies the later value tiles
    if (BIAS && wl == 0) dma_b(t0, t0 & 1);
    ISPA_WAIT_VMCNT(0);
  }
  ISPA_LDS_BARRIER();
  if (grp == 1) ISPA_LDS_BARRIER();

  // e4m3 key operand of block b, k-step ks: row 32b + l32, bytes 64ks + 32hf .. +31 (two chunks)
  auto kread8 = [&](int buf, int b, int ks) -> i32x8 {
    const uint8_t *kt = kbuf[buf];
    const int r = 32 * b + l32;
    const u32x4 x0 = *(const u32x4 *)(kt + k8_off<D>(r, 64 * ks + 32 * hf));
    const u32x4 x1 = *(const u32x4 *)(kt + k8_off<D>(r, 64 * ks + 32 * hf + 16));
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };

  for (int i = t0; i <= t1; ++i) {
    // ---- matrix phase: scores of tile i, value product of tile i-1 ----
    if constexpr (ISPA_ATTN_PRIO > 0) __builtin_amdgcn_s_setprio(ISPA_ATTN_PRIO);
    if (i < t1) {
      if constexpr (BIAS) {
        // the score accumulators start at b / tau instead of 0, so the softmax below sees
        // tau q.k + b (lane element v of block b is key 32b + 8(v/4) + 4hf + v%4)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 x = *(const f32x4 *)(bbuf[i & 1] + 32 * b + 8 * q4 + 4 * hf);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[b][4 * q4 + e] = x[e] * a.bias_to_score;
          }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[b][v] = 0.f;
      }
      if constexpr (FP8) {
        i32x8 ka[NB * NK8];
#pragma unroll
        for (int j = 0; j < NB * NK8; ++j) ka[j] = kread8(i & 1, j / NK8, j % NK8);
#pragma unroll
        for (int j = 0; j < NB * NK8; ++j) sc[j / NK8] = mfma_e4m3_32x32x64(ka[j], qf[j % NK8], sc[j / NK8]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int g = 0; g < NB * NK8 - 2; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      } else {
        // operands two ahead of the MFMAs
        bf16x8 k0 = kread(i & 1, 0), k1 = kread(i & 1, 1);
#pragma unroll
        for (int j = 0; j < NKK * NB; ++j) {
          const bf16x8 k2 = kread(i & 1, j + 2 < NKK * NB ? j + 2 : NKK * NB - 1);
          sc[j % NB] = mfma_bf16_32x32x16(k0, qr[j / NB], sc[j % NB]);
          k0 = k1;
          k1 = k2;
        }
        // keep four operand reads in flight ahead of the MFMAs (the bias reads, if any, go first)
        if constexpr (BIAS) __builtin_amdgcn_sched_group_barrier(0x100, NB * 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int g = 0; g < NKK * NB / 2 - 2; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
    // the value product of tile i-1 belongs to this range only when i-1 >= t0
    if (FP8V && i > t0) {
      i32x8 vt[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) vt[db] = vread8(i - 1, db);
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = mfma_e4m3_32x32x64(vt[db], pf, o[db]);
      // four transposing reads per operand: two operands ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g2 = 0; g2 < NDB - 2; ++g2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    } else if (!LSE_ONLY && i > t0) {
      bf16x8 v0 = vread(i - 1, 0), v1 = vread(i - 1, 1);
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        const bf16x8 v2 = vread(i - 1, j + 2 < NPV ? j + 2 : NPV - 1);
        const int db = j / (2 * NB), b = (j / 2) % NB, h2 = j % 2;
        o[db] = mfma_bf16_32x32x16(v0, pk[b][h2], o[db]);
        v0 = v1;
        v1 = v2;
      }
      // each V operand is two ds_read_b64_tr_b16: eight reads (four operands) ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < NPV / 2 - 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    if constexpr (ISPA_ATTN_PRIO > 0 && ISPA_ATTN_PRIO_MODE == 1) __builtin_amdgcn_s_setprio(0);
    // copies after this phase's LDS reads: K(i+1) and the bias of tile i+1 here; V(i) here as well when
    // the copies go in the matrix phase (VCOPY_VEC false), else at the start of the vector phase, which
    // has no LDS access (the compiler adds no wait for it) and runs beside group B's matrix phase, which
    // reads only the other buffers (K(i), V(i-1))
    if (grp == 0) {
      if (i + 1 < t1) {
        dma_k(i + 1, (i + 1) & 1);
        if (BIAS && wl == 0) dma_b(i + 1, (i + 1) & 1);
      }
      if (!VCOPY_B && !VCOPY_VEC && !LSE_ONLY && i < t1) dma_v(i, i & 1);
    }
    // VCOPY_B: group B's copies of V(i) (issued in its vector phase of tile i-1) land before group A's
    // matrix phase i+1 reads them
    if (VCOPY_B && grp == 1) ISPA_WAIT_VMCNT(0);
    if constexpr (ISPA_ATTN_PRIO > 0 && ISPA_ATTN_PRIO_MODE == 2) __builtin_amdgcn_s_setprio(0);
    ISPA_LDS_BARRIER();
    if (!VCOPY_B && VCOPY_VEC && grp == 0 && i < t1) dma_v(i, i & 1);
    // V(i+1) goes to the buffer of V(i-1), which both groups finished reading in their matrix phases i
    if (VCOPY_B && grp == 1 && i + 1 < t1) dma_v(i + 1, (i + 1) & 1);
    // ---- vector phase: softmax of tile i ----
    // accumulator holds tiles 0 .. nt_loc-1: the local keys end here (a piece that begins later inside
    // the local keys ends at their end, and its state is merged)
    if (!LSE_ONLY && i == nt_loc && t0 == 0) snapshot_local();
    if (i < t1) {
      const int n_valid = n_valid_of(i);
      if (n_valid < BK) {
        // key 32b + 8(v/4) + 4hf + v%4 < n_valid, with the lane's part moved to the bound so that the
        // key offsets stay immediates
        const int nv = n_valid - 4 * hf;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[b][v] = 32 * b + 8 * (v >> 2) + (v & 3) < nv ? sc[b][v] : -INFINITY;
      }
      // probabilities of the tile against the running maximum m, packed for the value product; returns
      // the lane's sum of its 32 unrounded probabilities
      auto probs = [&](float mneg) -> float {
        float sum = 0.f;
        if constexpr (FP8V) {
          // byte j of pf = probability sc[j / 16][j mod 16] rounded to e4m3 (nearest even; p <= 2^8 < 448)
#pragma unroll
          for (int w4 = 0; w4 < 8; ++w4) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[w4 / 4][4 * (w4 % 4) + e], sl2, mneg));
              sum += p[e];
            }
            // both halves of the word are written: the previous tile's word serves as the untouched input
            const int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf[w4], false);
            pf[w4] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
          }
        } else
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][8 * h2 + e], sl2, mneg));
              sum += p[e];
            }
            u32x4 u;
            u[0] = pack_bf16x2(p[0], p[1]);
            u[1] = pack_bf16x2(p[2], p[3]);
            u[2] = pack_bf16x2(p[4], p[5]);
            u[3] = pack_bf16x2(p[6], p[7]);
            pk[b][h2] = __builtin_bit_cast(bf16x8, u);
          }
        return sum;
      };
      // Lazy maximum: m moves only when the tile's row maximum lies more than 8 (log2 units) above it.
      // A row whose maximum moves has a probability of 2^8 (to within the last bit of exp2) against the
      // current m, so where every lane's sum of its probabilities is at most 255 no row moves and the
      // one pass stands (all probabilities <= 255). Otherwise (the first tile, or scores far above m)
      // the row maxima are formed, m is raised where needed, the accumulator is rescaled and the
      // probabilities are recomputed: the results are those of forming the maximum on every tile.
      float sum = probs(-m);
      if (__ballot(!(sum <= 255.0f)) != 0ull) {
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[b][v]);
        mx = halves_max(mx);
        const float mnew = mx * sl2;
        const bool need = mnew > m + kRescaleThreshold;
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;
        m = need ? mnew : m;
        sum = probs(-m);
        if (__ballot(need) != 0ull) {
          l *= alpha;
          l_loc *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        }
      }
      l += sum;
    }
    // this step's copies of group A (K(i+1), and V(i) unless group B copies the values) have landed;
    // group B waits for its value copies at the end of its next matrix phase instead
    if (!VCOPY_B || grp == 0) ISPA_WAIT_VMCNT(0);
    ISPA_LDS_BARRIER();
  }
  if (grp == 0) ISPA_LDS_BARRIER();     // matches group B's extra prologue barrier

  if constexpr (LSE_ONLY) {
    // partial state of this key range: running max (log2 units) and exp-sum, merged by lse_merge_kernel
    const float tot = halves_sum(l);
    if (hf == 0 && qi < n_q) {
      float *dst = a.lse_part + 2 * (((int64_t)split * a.n_heads + head) * n_q + qi);
      *(f32x2 *)dst = f32x2{m, tot};
    }
  } else if (!SPLIT || (t0 == 0 && t1 == nt)) {
    if (nt_hist > 0) {
      const float th = halves_sum(l);
      const float tl = halves_sum(l_loc);
      const float tot = th + tl;
      write_rows<D>(o, v_mul / tot, a.a_full, qi, n_q, out_stride, head_off, hf);
      write_lse(a.lse_full, (m + __log2f(tot)) * kLn2, head, qi, n_q, hf);
      write_lse(a.lse_hist, th > 0.f ? (m + __log2f(th)) * kLn2 : -INFINITY, head, qi, n_q, hf);
    }
  } else {
    // a cut unit: store this piece's state (counted once the workgroup's last piece is stored)
    store_state(slot_ws);
    slot_ws[kSplitScal + tid] = m;
    slot_ws[kSplitScal + 512 + tid] = l;
    slot_ws[kSplitScal + 2 * 512 + tid] = l_loc;
  }
  };   // pieces
  // One call for a workgroup with a single piece (every workgroup of the plain schedule, the main ones of
  // the balanced schedule), else one per piece. Written this way the plain kernel's tile loop comes out
  // of the compiler about 1 % faster than from the loop over pieces around the body (0.5412-0.5419
  // against 0.5471-0.5475 ms on the 18,720-key chunk, 2.834 against 2.870 ms on workload 5); the
  // balanced schedule gains nothing from its single-piece copy (0.555 against 0.550-0.553 ms).
  if (npiece == 1) piece_body(0);
  else
    for (int pi = 0; pi < npiece; ++pi) piece_body(pi);
  if constexpr (SPLIT) {
    // the XCD's geometry again, from an opaque copy of the workgroup id (the first one is not kept live
    // across the tile loops), and the touched units from LDS
    int xw = (int)blockIdx.x;
    asm volatile("" : "+s"(xw));
    const SplitGeom sg = split_geom(xw & 7, n_qt * a.n_heads, (int)(gridDim.x >> 3), nt);
    const int k_lo = s_klo, k_hi = s_khi;
    const uint64_t two = s_two;
    // Every wave's stores complete in L2; then wave 0 makes them visible at agent scope with one release
    // (a write-back of the XCD's L2; a sequentially consistent fence would also invalidate it, dropping
    // the K/V tiles the XCD's other workgroups are reading) and counts each unit's pieces, one lane per
    // unit. The increment that completes a unit's count gives its merge to this workgroup.
    ISPA_WAIT_VMCNT(0);
    __syncthreads();
    if (w == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int k = k_lo + lane;
      bool last = false;
      if (k_lo >= 0 && k <= k_hi) {
        const int here = 1 + (int)((two >> lane) & 1);
        const int npc = 2 + unit_cuts(sg, k, nt, nt_loc).n;
        last = atomicAdd(a.split_count + sg.us + k, here) + here == npc;
      }
      const uint64_t mine = __ballot(last);
      if (mine != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other pieces' states
      if (lane == 0) s_merge = mine;
    }
    __syncthreads();
    for (uint64_t p = s_merge; p != 0; p &= p - 1)
      merge_unit(a, sg, k_lo + __builtin_ctzll(p), nt, nt_loc, nt_hist, n_qt, tid);
  }
}

// lse = log sum_s l_s 2^(m_s) over the key ranges, in split order
__global__ void __launch_bounds__(256) lse_merge_kernel(const float *part, int splits, int64_t n, float *lse) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part[2 * (s * n + i)]);
  float sum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ms = part[2 * (s * n + i)], ls = part[2 * (s * n + i) + 1];
    if (ls > 0.f) sum += ls * __builtin_amdgcn_exp2f(ms - mx);
  }
  lse[i] = sum > 0.f ? (mx + __log2f(sum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------------------------------------
// fp32 kernel: VALU, one query per thread. Same single pass and the same local/history split.
// ------------------------------------------------------------------------------------------------
template <int D, bool BIAS>
__global__ void __launch_bounds__(128) attn_dual_f32_kernel(AttnArgs a, int n_qt) {
  constexpr int BK = 32;
  constexpr int NT = 128;
  __shared__ float k_lds[BK][D];
  __shared__ float v_lds[BK][D];
  __shared__ float b_lds[BK];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int qi = qt * NT + tid;
  const bool qok = qi < a.n_q;
  const int head_off = head * D;

  float q[D], o[D];
  const float *qsrc = (const float *)a.q + (int64_t)(qok ? qi : 0) * a.q_stride + head_off;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qok ? qsrc[c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f, l_loc = 0.f;
  const int64_t n_loc = a.sink_n + a.cur_n;
  const int nt_loc = (int)((n_loc + BK - 1) / BK);
  const int nt_hist = (int)((a.hist_n + BK - 1) / BK);
  const int nt = nt_loc + nt_hist;

  auto row_ptr = [&](bool hist, int64_t j, bool value) -> const float * {
    if (hist) return (const float *)(value ? a.hist_v : a.hist_k) + j * a.hist_stride + head_off;
    if (j < a.sink_n) return (const float *)(value ? a.sink_v : a.sink_k) + j * a.sink_stride + head_off;
    j -= a.sink_n;
    return (const float *)(value ? a.cur_v : a.cur_k) + j * a.cur_stride + head_off;
  };
  auto store_out = [&](void *out, float inv) {
    if (!qok || out == nullptr) return;
    float *dst = (float *)out + (int64_t)qi * (a.n_heads * D) + head_off;
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = o[c] * inv;
  };
  auto store_lse = [&](float *out, float val) {
    if (qok && out != nullptr) out[(int64_t)head * a.n_q + qi] = val;
  };

  for (int t = 0; t < nt; ++t) {
    const bool hist = t >= nt_loc;
    const int64_t j0 = (int64_t)(hist ? t - nt_loc : t) * BK;
    const int64_t nseg = hist ? a.hist_n : n_loc;
    const int n_valid = (int)((nseg - j0) < BK ? (nseg - j0) : BK);
    __syncthreads();
    for (int idx = tid; idx < BK * D; idx += NT) {
      const int r = idx / D, c = idx % D;
      int64_t j = j0 + r;
      j = j < nseg ? j : nseg - 1;
      k_lds[r][c] = row_ptr(hist, j, false)[c];
      v_lds[r][c] = row_ptr(hist, j, true)[c];
    }
    if (BIAS && tid < BK) {
      int64_t j = j0 + tid;
      j = j < nseg ? j : nseg - 1;
      b_lds[tid] = *bias_ptr(a, hist, j, head) * a.bias_to_score;
    }
    __syncthreads();
    float s[BK];
    float mx = -INFINITY;
    for (int r = 0; r < BK; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], k_lds[r][c], acc);
      if (BIAS) acc += b_lds[r];
      s[r] = r < n_valid ? acc * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    if (mx > m) {
      const float alpha = exp2f(m - mx);
      m = mx;
      l *= alpha;
      l_loc *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
    }
    for (int r = 0; r < BK; ++r) {
      const float p = exp2f(s[r] - m);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, v_lds[r][c], o[c]);
    }
    if (t == nt_loc - 1) {
      const float inv = 1.0f / l;
      const float lse = (m + log2f(l)) * kLn2;
      store_out(a.a_loc, inv);
      store_lse(a.lse_loc, lse);
      if (nt_hist == 0) {
        store_out(a.a_full, inv);
        store_lse(a.lse_full, lse);
        store_lse(a.lse_hist, -INFINITY);
      }
      l_loc = l;
      l = 0.f;
    }
  }
  if (nt_hist > 0) {
    const float tot = l + l_loc;
    store_out(a.a_full, 1.0f / tot);
    store_lse(a.lse_full, (m + log2f(tot)) * kLn2);
    store_lse(a.lse_hist, l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY);
  }
}

#ifndef ISPA_ATTN_PP
#define ISPA_ATTN_PP 1
#endif

template <bool BIAS>
hipError_t launch_attn_bf16_t(const AttnArgs &a, int head_dim, hipStream_t s) {
  if (ISPA_ATTN_PP && head_dim == 128) {
    const int n_qt = (a.n_q + 255) / 256;
    const int grid = n_qt * a.n_heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_dual_bf16_pp_kernel<128, BIAS>), dim3(grid), dim3(512), 0, s, a, n_qt);
    return hipGetLastError();
  }
  const int n_qt = (a.n_q + 127) / 128;
  const int grid = n_qt * a.n_heads;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) {
    // only built when the ping-pong kernel is switched off at compile time
    if constexpr (!ISPA_ATTN_PP)
      hipLaunchKernelGGL((attn_dual_bf16_kernel<128, BIAS>), dim3(grid), dim3(kThreads), 0, s, a, n_qt);
  } else {
    hipLaunchKernelGGL((attn_dual_bf16_kernel<64, BIAS>), dim3(grid), dim3(kThreads), 0, s, a, n_qt);
  }
  return hipGetLastError();
}

template <bool BIAS>
hipError_t launch_attn_f32_t(const AttnArgs &a, int head_dim, hipStream_t s) {
  const int n_qt = (a.n_q + 127) / 128;
  const int grid = n_qt * a.n_heads;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_dual_f32_kernel<128, BIAS>), dim3(grid), dim3(128), 0, s, a, n_qt);
  else
    hipLaunchKernelGGL((attn_dual_f32_kernel<64, BIAS>), dim3(grid), dim3(128), 0, s, a, n_qt);
  return hipGetLastError();
}

bool has_bias(const AttnArgs &a) { return a.sink_b != nullptr || a.cur_b != nullptr || a.hist_b != nullptr; }

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs &a, int head_dim, hipStream_t s) {
  if (head_dim != 128 || has_bias(a) || a.q_scale == nullptr || a.k_scale == nullptr) return hipErrorInvalidValue;
  const int n_qt = (a.n_q + 255) / 256;
  const int grid = n_qt * a.n_heads;
  if (grid == 0) return hipSuccess;
  if (a.v_scale != nullptr)
    hipLaunchKernelGGL((attn_dual_bf16_pp_kernel<128, false, false, true, true>), dim3(grid), dim3(512), 0, s, a,
                       n_qt);
  else
    hipLaunchKernelGGL((attn_dual_bf16_pp_kernel<128, false, false, true>), dim3(grid), dim3(512), 0, s, a, n_qt);
  return hipGetLastError();
}

// Balanced schedule: one workgroup per compute unit over the tile sequence of all units, when the
// units alone would leave a tenth or more of the compute units idle in their last round.
int attn_balanced_grid(int64_t n_q, int n_heads, int64_t n_keys_loc, int64_t n_keys_hist, int cus) {
  const int64_t units = ((n_q + 255) / 256) * (int64_t)n_heads;
  const int64_t nt = (n_keys_loc + 63) / 64 + (n_keys_hist + 63) / 64;
  if (units <= 0 || cus <= 0 || cus % 8 != 0 || nt < 16) return 0;
  const int64_t S = cus / 8, nx_min = units / 8, nx_max = (units + 7) / 8;
  // a tenth or more of the compute units idle under the plain schedule; spare workgroups on every XCD;
  // at least as many main workgroups as spare ones (a unit's remaining tiles then meet at most one
  // spare-range boundary); one bit per unit of an XCD in a 64-bit mask
  if (units * 10 >= (int64_t)cus * 9 || nx_max >= S || 2 * nx_min < S || S > 64) return 0;
  // the pieces of a spare workgroup fit its table
  const int64_t e_min = S - nx_max;
  if (2 * ((nx_max + e_min - 1) / e_min + 1) > kSplitMaxPieces) return 0;
  return cus;
}

size_t attn_balanced_ws_bytes(int64_t n_q, int n_heads, int grid) {
  if (grid <= 0) return 0;
  const int64_t units = ((n_q + 255) / 256) * (int64_t)n_heads;
  const size_t slots = (size_t)kSplitSlots * units * kSplitSlotFloats * sizeof(float);
  return slots + (((size_t)units * sizeof(int) + 255) / 256) * 256;
}

namespace {
__global__ void __launch_bounds__(256) zero_counts_kernel(int *c, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) c[i] = 0;
}
}  // namespace

hipError_t launch_attn_bf16_balanced(const AttnArgs &a, int head_dim, int grid, void *ws, hipStream_t s) {
  if (head_dim != 128 || has_bias(a) || grid <= 0 || ws == nullptr) return hipErrorInvalidValue;
  const int n_qt = (a.n_q + 255) / 256;
  const int64_t units = (int64_t)n_qt * a.n_heads;
  if (units == 0) return hipSuccess;
  AttnArgs b = a;
  b.split_ws = (float *)ws;
  b.split_count = (int *)((char *)ws + (size_t)kSplitSlots * units * kSplitSlotFloats * sizeof(float));
  hipLaunchKernelGGL(zero_counts_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, b.split_count, units);
  hipLaunchKernelGGL((attn_dual_bf16_pp_kernel<128, false, false, false, false, true>), dim3(grid), dim3(512), 0, s,
                     b, n_qt);
  return hipGetLastError();
}

int lse_splits_for(int64_t n_q, int n_heads) {
  // about one workgroup per CU: split the keys when the query tiles alone leave CUs idle
  const int64_t tiles = ((n_q + 255) / 256) * (int64_t)n_heads;
  if (tiles <= 0) return 1;
  const int64_t sp = (256 + tiles / 2) / tiles;
  return (int)(sp < 1 ? 1 : sp > 16 ? 16 : sp);
}

hipError_t launch_attn_lse_bf16(const AttnArgs &a, int head_dim, hipStream_t s) {
  if (has_bias(a) || a.a_loc != nullptr || a.a_full != nullptr) return hipErrorInvalidValue;
  if (ISPA_ATTN_PP && head_dim == 128) {
    const int n_qt = (a.n_q + 255) / 256;
    const int grid = n_qt * a.n_heads;
    if (grid == 0) return hipSuccess;
    if (a.lse_part == nullptr || a.lse_full == nullptr || a.lse_splits != lse_splits_for(a.n_q, a.n_heads))
      return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_dual_bf16_pp_kernel<128, false, true>), dim3(grid * a.lse_splits), dim3(512), 0, s,
                       a, n_qt);
    const int64_t n = (int64_t)a.n_heads * a.n_q;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.lse_part,
                       a.lse_splits, n, a.lse_full);
    return hipGetLastError();
  }
  return launch_attn_bf16_t<false>(a, head_dim, s);   // rows are not stored (NULL outputs)
}

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t s) {
  return has_bias(a) ? launch_attn_bf16_t<true>(a, head_dim, s) : launch_attn_bf16_t<false>(a, head_dim, s);
}

hipError_t launch_attn_f32(const AttnArgs &a, int head_dim, hipStream_t s) {
  return has_bias(a) ? launch_attn_f32_t<true>(a, head_dim, s) : launch_attn_f32_t<false>(a, head_dim, s);
}

}  // namespace ispa
