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
//
// Operand rows reach LDS through a ring of four 32-row stages filled by global_load_lds (no staging
// registers, no LDS store instructions): while stage s is multiplied, stages s+1..s+3 are in flight.
// Rows past the end of the chunk are copied from a 16-byte block of zeros, so the loop always runs
// whole turns of the ring and a partial stage adds exact zeros.
#include <type_traits>

#include "ispa_internal.hpp"
#include "device_common.hpp"

namespace ispa {
namespace {

constexpr int kThreads = 256;                 // 4 waves, each a 64x64 quarter of the tile
constexpr int BT = 128;                       // output tile
constexpr int BR = 32;                        // rows per stage
constexpr int NS = 4;                         // stages in the ring
constexpr int RB = BT * 2;                    // bytes of one tile row (128 bf16)
constexpr int kPart = BR * RB;                // one operand's share of a stage (8 KB)
constexpr int kStage = 2 * kPart;             // 16 KB
constexpr int kCopies = kStage / 1024 / 4;    // 1 KB copy instructions per wave per stage

static __device__ __attribute__((aligned(16))) uint32_t g_zero_row[4];

// s_waitcnt with vmcnt = n and no wait on the other counters
#define ISPA_GRAM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
// Workgroup barrier that waits for this wave's LDS reads but not for its copies in flight (those are
// waited for explicitly, before the barrier that publishes them). The empty asm statements keep the
// compiler from moving memory accesses across it.
#define ISPA_GRAM_LDS_BARRIER()          \
  do {                                   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_waitcnt(0xc07f);  \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  } while (0)

// One launch covers the tiles of up to kMaxGramLayers layers (same n_rows and d): workgroup ids run
// over (layer, tile) pairs, tiles of one layer consecutive, in an XCD-aware order (the 128 x 128 kernel:
// each XCD takes a contiguous range, so the tiles that share a layer's rows share an L2, measured better
// than giving every XCD a share of each layer, which spreads an XCD's concurrent tiles over several
// layers; the 256 x 256 kernel: blocks of 32 consecutive ids in turn over the XCDs, see there).
constexpr int kMaxGramLayers = 48;
struct GramArgs {
  const uint16_t *a_loc[kMaxGramLayers], *a_full[kMaxGramLayers];
  float *G[kMaxGramLayers], *X[kMaxGramLayers], *F[kMaxGramLayers];
  int64_t n_rows;
  int d, T, n_upper, with_f, tiles;   // T: tiles per dimension; tiles: per layer
  // 128 x 128 kernel only: tail_first >= 0 makes it cover the 256 x 256 tiles tail_first, tail_first + 1,
  // ... of a wide launch's tile list (Tw, n_upper_w, tiles_w: that list's geometry), workgroup 4 u + q
  // taking quarter q of tile tail_first + u
  int tail_first, Tw, n_upper_w, tiles_w;
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

// tile idx of a layer's list: the upper tiles of G, the upper tiles of F (if present), all tiles of X
__device__ __forceinline__ void decode_tile(int idx, int T, int n_upper, int with_f, int &mat, int &ti, int &tj) {
  if (idx < n_upper) {
    mat = 0;
    tri_decode(idx, T, ti, tj);
  } else if (with_f && idx < 2 * n_upper) {
    mat = 1;
    tri_decode(idx - n_upper, T, ti, tj);
  } else {
    mat = 2;
    idx -= n_upper * (with_f ? 2 : 1);
    ti = idx / T;
    tj = idx % T;
  }
}

// A stage holds each operand row-major ([row of the chunk][128 columns], 256 bytes per row) with the
// 16-byte chunks of row r stored at position c ^ (4 (r mod 4)). ds_read_b64_tr_b16 then yields MFMA
// operands directly: in each 16-lane group, source lane s addresses row k0 + s/4, columns
// n0 + 4 (s mod 4) .. +3, and result lane i receives column n0 + i of rows k0 .. k0+3. The swizzle
// spreads the 4 rows of one read over distinct banks.
__device__ __forceinline__ int swz_off(int r, int col) {   // byte offset of (r, col) in a stage part
  const int c = col >> 3;
  return r * RB + (((c ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 read_operand(const uint8_t *part, int cb, int kb, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int n0 = cb + 16 * (g & 1);
  const int k0 = kb + 8 * (g >> 1);
  const int col = n0 + 4 * (s & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(part + swz_off(k0 + (s >> 2), col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(part + swz_off(k0 + 4 + (s >> 2), col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct StageOps {
  bf16x8 a[2][2], b[2][2];   // [16-row step][32-column block]
};

__global__ void __launch_bounds__(kThreads, 2) gram_bf16_kernel(GramArgs g) {
  // Four separate arrays (not one indexed ring): the compiler then tracks the copies into each stage
  // on their own and waits only for the ones a read may touch.
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kStage];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  int layer, mat, ti, tj;   // mat: 0 = G, 1 = F, 2 = X
  if (g.tail_first >= 0) {
    // a quarter of a 256 x 256 tile of a wide launch's list; a quarter that lies past d, or below the
    // diagonal of G or F (its elements come from the mirror of the quarter above), has no work. Every
    // element is the same fixed-order sum as in the 256 x 256 kernel.
    const int u = g.tail_first + (int)(blockIdx.x >> 2), q = (int)(blockIdx.x & 3);
    layer = u / g.tiles_w;
    int TI, TJ;
    decode_tile(u % g.tiles_w, g.Tw, g.n_upper_w, g.with_f, mat, TI, TJ);
    ti = 2 * TI + (q >> 1);
    tj = 2 * TJ + (q & 1);
    if (ti >= g.T || tj >= g.T || (mat != 2 && ti > tj)) return;   // uniform: the whole workgroup
  } else {
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    layer = lin / g.tiles;
    decode_tile(lin % g.tiles, g.T, g.n_upper, g.with_f, mat, ti, tj);
  }
  const uint16_t *P = (mat == 1) ? g.a_full[layer] : g.a_loc[layer];   // rows of the left factor
  const uint16_t *Q = (mat == 0) ? g.a_loc[layer] : g.a_full[layer];   // rows of the right factor
  float *out = (mat == 0) ? g.G[layer] : (mat == 1) ? g.F[layer] : g.X[layer];
  const int i0 = ti * BT, j0 = tj * BT;
  const int d = g.d;
  const int64_t n_rows = g.n_rows;
  const int nst = (int)((n_rows + BR - 1) / BR);

  // Copy instruction ii of wave w fills 1 KB block blk = w + 4 ii of a stage: blocks 0-7 are the left
  // operand, 8-15 the right one, 4 rows each. Lane l lands at byte 16 l of the block, i.e. row
  // 4 (blk mod 8) + l / 16, stored chunk l mod 16, which holds source chunk (l mod 16) ^ (4 (l / 16)).
  // Columns past d are clamped (their outputs are not stored).
  const uint8_t *src[kCopies];
  int crow[kCopies];
#pragma unroll
  for (int ii = 0; ii < kCopies; ++ii) {
    const int blk = w + 4 * ii;
    const int op = blk >> 3;
    const int r = 4 * (blk & 7) + (lane >> 4);
    const int c = (lane & 15) ^ (4 * (lane >> 4));
    int col = (op ? j0 : i0) + 8 * c;
    col = col < d ? col : d - 8;
    crow[ii] = r;
    src[ii] = (const uint8_t *)((op ? Q : P) + (int64_t)r * d + col);
  }
  const int64_t stage_bytes = (int64_t)BR * d * 2;
  uint64_t zero_row = (uint64_t)(uintptr_t)g_zero_row;
  asm volatile("" : "+s"(zero_row));   // keep the address in registers, not reloaded per stage

  auto copy_stage = [&](int s, uint8_t *slot) {
#pragma unroll
    for (int ii = 0; ii < kCopies; ++ii) {
      const int64_t n = (int64_t)s * BR + crow[ii];
      const uint8_t *p = src[ii] + (int64_t)s * stage_bytes;
      p = n < n_rows ? p : (const uint8_t *)(uintptr_t)zero_row;
      copy_to_lds<16>(p, slot + 1024 * (w + 4 * ii));
    }
  };
  auto read_stage = [&](const uint8_t *slot, StageOps &o) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) o.a[t][bi] = read_operand(slot, wm * 64 + bi * 32, 16 * t, lane);
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) o.b[t][bj] = read_operand(slot + kPart, wn * 64 + bj * 32, 16 * t, lane);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  // Stage s: its operands are already in registers (`ocur`); stage s+1 is read into `onx` while
  // stage s is multiplied, and the slot of stage s is refilled with stage s+4.
  auto stage = [&](int s, uint8_t *cur, const uint8_t *nxt, const StageOps &ocur, StageOps &onx) {
    ISPA_GRAM_WAIT_VMCNT(kCopies * (NS - 2));   // this wave's copies of stage s+1 have landed
    ISPA_GRAM_LDS_BARRIER();                    // ... everyone's; all reads of stage s are done
    copy_stage(s + NS, cur);
    read_stage(nxt, onx);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = mfma_bf16_32x32x16(ocur.a[t][bi], ocur.b[t][bj], acc[bi][bj]);
    // issue order: one MFMA, the copies, then the LDS reads two at a time between the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, kCopies, 0);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  };

  StageOps oa, ob;
  copy_stage(0, ring0);
  copy_stage(1, ring1);
  copy_stage(2, ring2);
  copy_stage(3, ring3);
  ISPA_GRAM_WAIT_VMCNT(kCopies * (NS - 1));
  ISPA_GRAM_LDS_BARRIER();
  read_stage(ring0, oa);
  for (int s = 0; s < nst; s += NS) {
    stage(s, ring0, ring1, oa, ob);
    stage(s + 1, ring1, ring2, ob, oa);
    stage(s + 2, ring2, ring3, oa, ob);
    stage(s + 3, ring3, ring0, ob, oa);
  }
  ISPA_GRAM_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended

  // Add the tile to the running sums straight from the accumulators: lane (l32, hf) of block
  // (bi, bj) holds rows 8 q + 4 hf + e (q, e < 4) of column l32. Each thread issues its loads before
  // any add, so the round trips overlap.
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int cl = j0 + wn * 64 + bj * 32 + l32;
      const int clc = cl < d ? cl : d - 1;
      float cur[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int rwc = rw < d ? rw : d - 1;
        cur[v] = out[(int64_t)rwc * d + clc];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (rw < d && cl < d) out[(int64_t)rw * d + cl] = cur[v] + acc[bi][bj][v];
      }
    }
  if (mat != 2 && ti != tj) {
    // mirror of an off-diagonal G or F tile: out[c][r] += tile[r][c]; the four rows e of one q are
    // four consecutive columns of the mirror, written as one 16-byte access
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int mr = j0 + wn * 64 + bj * 32 + l32;
        const int mrc = mr < d ? mr : d - 1;
        f32x4 cur[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 64 + bi * 32 + 8 * q + 4 * hf;
          const int mcc = mc < d ? mc : d - 4;
          cur[q] = *(const f32x4 *)&out[(int64_t)mrc * d + mcc];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 64 + bi * 32 + 8 * q + 4 * hf;
          f32x4 add;
#pragma unroll
          for (int e = 0; e < 4; ++e) add[e] = acc[bi][bj][4 * q + e];
          if (mr < d && mc < d) *(f32x4 *)&out[(int64_t)mr * d + mc] = cur[q] + add;
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Wide tiles: one workgroup per 256 x 256 output tile, 4 waves of 128 x 128 (a 4 x 4 grid of 32 x 32
// MFMA blocks each, 256 fp32 accumulators per lane; one workgroup per CU). Per 32-row stage a wave
// reads 16 KB of operands for 32 MFMAs, half the LDS bytes per FLOP of the 128 x 128 form, and the
// workgroup takes in half the rows per FLOP. A stage holds four 8 KB half-panels in the layout of
// the 128 x 128 kernel (32 rows x 128 columns, chunk c of row r at c ^ 4 (r mod 4)): A columns i0..,
// i0+128.., B columns j0.., j0+128..; wave (wm, wn) reads half-panels wm and 2 + wn only.
// ---------------------------------------------------------------------------------------------
#ifndef ISPA_GRAM_WAVES
#define ISPA_GRAM_WAVES 8   // waves of the 256 x 256 tile kernel: 4 (128 x 128 each) or 8 (128 x 64 each)
#endif
constexpr int BTW = 256;                      // output tile
constexpr int kStageW = 4 * kPart;            // 32 KB

template <int BJ>
struct HalfOpsW {
  bf16x8 a[4], b[BJ];   // one 16-row step: [32-column block]
};

// NWV = 4: waves of 128 x 128 (one wave per SIMD); NWV = 8: waves of 128 x 64 (two per SIMD, so that one
// wave's MFMAs run while the other is held issuing its global->LDS copies, which take tens to hundreds of
// cycles each and otherwise leave the matrix core idle)
template <int NWV>
__global__ void __launch_bounds__(64 * NWV, 1) gram_bf16_wide_kernel(GramArgs g) {
  constexpr int BJ = NWV == 8 ? 2 : 4;               // 32-column blocks of a wave
  constexpr int kCW = kStageW / 1024 / NWV;          // copy instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStageW];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStageW];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStageW];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kStageW];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = NWV == 8 ? w >> 2 : w >> 1, wn = NWV == 8 ? w & 3 : w & 1;
  // the wave's B half-panel and its first column in it
  const int bpart = NWV == 8 ? 2 + (wn >> 1) : 2 + wn, bcol = NWV == 8 ? 64 * (wn & 1) : 0;

  // Workgroup b runs on XCD b mod 8 as that XCD's (b / 8)-th workgroup; an XCD runs 32 at a time, one per
  // CU. Each XCD's next 32 are the next unclaimed block of 32 consecutive (layer, tile) ids: the XCD's
  // concurrent tiles share one layer's rows in its L2, and the 8 XCDs together hold about 256 consecutive
  // tiles (a few layers) rather than 8 ranges far apart, so rows that miss an L2 are more often in the
  // memory-side cache. Workgroups past the last whole round of 256 keep their own id.
  int lin;
  {
    const int b = (int)blockIdx.x, full = (int)(gridDim.x / 256) * 256;
    if (b < full) {
      const int x = b & 7, slot = b >> 3;
      lin = (((slot >> 5) << 3) + x) * 32 + (slot & 31);
    } else {
      lin = b;
    }
  }
  const int layer = lin / g.tiles;
  int idx = lin % g.tiles;
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
  const uint16_t *P = (mat == 1) ? g.a_full[layer] : g.a_loc[layer];
  const uint16_t *Q = (mat == 0) ? g.a_loc[layer] : g.a_full[layer];
  float *out = (mat == 0) ? g.G[layer] : (mat == 1) ? g.F[layer] : g.X[layer];
  const int i0 = ti * BTW, j0 = tj * BTW;
  const int d = g.d;
  const int64_t n_rows = g.n_rows;
  const int nst = (int)((n_rows + BR - 1) / BR);

  // Copy instruction ii of wave w fills 1 KB block blk = w + 4 ii of a stage: half-panel blk / 8, rows
  // 4 (blk mod 8) .. +3; lane l lands at row 4 (blk mod 8) + l / 16, stored chunk l mod 16, which holds
  // source chunk (l mod 16) ^ (4 (l / 16)). Columns past d are clamped (their outputs are not stored).
  const uint8_t *src[kCW];
  int crow[kCW];
#pragma unroll
  for (int ii = 0; ii < kCW; ++ii) {
    const int blk = w + NWV * ii;
    const int part = blk >> 3;
    const int r = 4 * (blk & 7) + (lane >> 4);
    const int c = (lane & 15) ^ (4 * (lane >> 4));
    int col = (part < 2 ? i0 + 128 * part : j0 + 128 * (part - 2)) + 8 * c;
    col = col < d ? col : d - 8;
    crow[ii] = r;
    src[ii] = (const uint8_t *)((part < 2 ? P : Q) + (int64_t)r * d + col);
  }
  const int64_t stage_bytes = (int64_t)BR * d * 2;
  uint64_t zero_row = (uint64_t)(uintptr_t)g_zero_row;
  asm volatile("" : "+s"(zero_row));

  // Stages whose rows all exist are copied with one address add per instruction (FULL); a stage that
  // reaches past the last row selects the zero block per lane.
  auto copy_stage = [&](auto full, int s, uint8_t *slot) {
#pragma unroll
    for (int ii = 0; ii < kCW; ++ii) {
      const uint8_t *p = src[ii] + (int64_t)s * stage_bytes;
      if constexpr (!decltype(full)::value) {
        const int64_t n = (int64_t)s * BR + crow[ii];
        p = n < n_rows ? p : (const uint8_t *)(uintptr_t)zero_row;
      }
      copy_to_lds<16>(p, slot + 1024 * (w + NWV * ii));
    }
  };
  auto read_half = [&](const uint8_t *slot, int t, HalfOpsW<BJ> &o) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) o.a[bi] = read_operand(slot + kPart * wm, bi * 32, 16 * t, lane);
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) o.b[bj] = read_operand(slot + kPart * bpart, bcol + bj * 32, 16 * t, lane);
  };

  f32x16 acc[4][BJ];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;
  if constexpr (NWV == 8) {
    // two waves per SIMD share 512 registers: the accumulators are pinned to AGPRs, which leaves the
    // VGPRs to the operands and addresses (left to itself the compiler kept all in VGPRs and spilled)
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) asm volatile("" : "+a"(acc[bi][bj]));
  }
  auto mma = [&](const HalfOpsW<BJ> &o) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) acc[bi][bj] = mfma_bf16_32x32x16(o.a[bi], o.b[bj], acc[bi][bj]);
  };
  constexpr int M = 4 * BJ;          // MFMAs per half-stage
  constexpr int R = 2 * (4 + BJ);    // operand reads per half-stage (two per operand)

  // Stage s, pipelined by half-stage (16 rows): the first half's operands are in registers (h0); the
  // second half is read while the first is multiplied; then, once every wave is done with the slot and
  // this wave's copies of stage s+1 have landed, the slot is refilled with stage s+4 and the first half
  // of stage s+1 is read while the second half of stage s is multiplied.
  HalfOpsW<BJ> h0, h1;
  auto stage = [&](auto full, int s, uint8_t *cur, const uint8_t *nxt) {
    read_half(cur, 1, h1);
    mma(h0);
    // one MFMA first (the wait for h0's reads then precedes h1's reads), h1's reads two per MFMA, and
    // the remaining MFMAs to cover their latency before the barrier's wait
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M - 1 - R / 2, 0);
    ISPA_GRAM_WAIT_VMCNT(kCW * (NS - 2));   // this wave's copies of stage s+1 have landed
    ISPA_GRAM_LDS_BARRIER();                // ... everyone's; all reads of stage s are done
    copy_stage(full, s + NS, cur);
    read_half(nxt, 0, h0);
    mma(h1);
    // per MFMA: one copy while copies remain, two operand reads while reads remain
#pragma unroll
    for (int i = 0; i < M; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kCW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i < R / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  using full_t = std::integral_constant<bool, true>;
  using part_t = std::integral_constant<bool, false>;
  copy_stage(part_t{}, 0, ring0);
  copy_stage(part_t{}, 1, ring1);
  copy_stage(part_t{}, 2, ring2);
  copy_stage(part_t{}, 3, ring3);
  ISPA_GRAM_WAIT_VMCNT(kCW * (NS - 1));
  ISPA_GRAM_LDS_BARRIER();
  read_half(ring0, 0, h0);
  // turns of the ring whose refills (stages s + 4 .. s + 7) hold only existing rows, then the rest
  const int n_full = (int)(n_rows / BR);
  int s = 0;
  for (; s + 2 * NS <= n_full; s += NS) {
    stage(full_t{}, s, ring0, ring1);
    stage(full_t{}, s + 1, ring1, ring2);
    stage(full_t{}, s + 2, ring2, ring3);
    stage(full_t{}, s + 3, ring3, ring0);
  }
  for (; s < nst; s += NS) {
    stage(part_t{}, s, ring0, ring1);
    stage(part_t{}, s + 1, ring1, ring2);
    stage(part_t{}, s + 2, ring2, ring3);
    stage(part_t{}, s + 3, ring3, ring0);
  }
  ISPA_GRAM_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended

  // Add the tile to the running sums (lane (l32, hf) of block (bi, bj) holds rows 8 q + 4 hf + e of
  // column l32), and mirror off-diagonal G and F tiles with 16-byte accesses.
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) {
      const int cl = j0 + 128 * (bpart - 2) + bcol + bj * 32 + l32;
      const int clc = cl < d ? cl : d - 1;
      float cur[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 128 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int rwc = rw < d ? rw : d - 1;
        cur[v] = out[(int64_t)rwc * d + clc];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 128 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (rw < d && cl < d) out[(int64_t)rw * d + cl] = cur[v] + acc[bi][bj][v];
      }
    }
  if (mat != 2 && ti != tj) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) {
        const int mr = j0 + 128 * (bpart - 2) + bcol + bj * 32 + l32;
        const int mrc = mr < d ? mr : d - 1;
        f32x4 cur[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 128 + bi * 32 + 8 * q + 4 * hf;
          const int mcc = mc < d ? mc : d - 4;
          cur[q] = *(const f32x4 *)&out[(int64_t)mrc * d + mcc];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 128 + bi * 32 + 8 * q + 4 * hf;
          f32x4 add;
#pragma unroll
          for (int e = 0; e < 4; ++e) add[e] = acc[bi][bj][4 * q + e];
          if (mr < d && mc < d) *(f32x4 *)&out[(int64_t)mr * d + mc] = cur[q] + add;
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------
// e4m3 rows (OCP FP8 E4M3 with one scale per head): the same 128x128 tiles and ring, 64 rows per stage
// (one v_mfma_f32_32x32x64_f8f6f4 k-step), 128-byte stage rows whose 16-byte chunk c is stored at
// c ^ ((r / 2) mod 8). ds_read_b64_tr_b8 builds the operands: in each 16-lane group, lane s addresses
// row k0 + s/2, bytes n0 + 8 (s mod 2) .. +7, and result lane i receives column n0 + i of rows k0 ..
// k0+7; four reads give a lane its 32 rows. The per-head scales multiply each tile in the epilogue.
// ---------------------------------------------------------------------------------------------
constexpr int BR8 = 64;                       // rows per stage
constexpr int RB8 = BT;                       // bytes of one stage row (128 e4m3 columns)
constexpr int kPart8 = BR8 * RB8;             // 8 KB
constexpr int kStage8 = 2 * kPart8;           // 16 KB
constexpr int kCopies8 = kStage8 / 1024 / 4;  // 4

struct GramArgs8 {
  const uint8_t *a_loc, *a_full;
  const float *s_loc, *s_full;                // per-head scales
  float *G, *X, *F;
  int64_t n_rows;
  int d, T, n_upper, with_f, head_dim;
};

__device__ __forceinline__ int swz8_off(int r, int col) {   // byte offset of (r, col) in a stage part
  return r * RB8 + ((((col >> 4) ^ ((r >> 1) & 7))) << 4) + (col & 15);
}

typedef int s32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ i32x8 read_operand8(const uint8_t *part, int cb, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int n0 = cb + 16 * (g & 1) + 8 * (s & 1);
  const int k0 = 32 * (g >> 1) + (s >> 1);
  s32x2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) s32x2 *)(part + swz8_off(k0 + 8 * j, n0)));
  return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

struct StageOps8 {
  i32x8 a[2], b[2];   // [32-column block]
};

__global__ void __launch_bounds__(kThreads, 2) gram_fp8_kernel(GramArgs8 g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStage8];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStage8];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStage8];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kStage8];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  const int n_tiles = g.n_upper * (g.with_f ? 2 : 1) + g.T * g.T;
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
  const uint8_t *P = (mat == 1) ? g.a_full : g.a_loc;
  const uint8_t *Q = (mat == 0) ? g.a_loc : g.a_full;
  const float *sP = (mat == 1) ? g.s_full : g.s_loc;
  const float *sQ = (mat == 0) ? g.s_loc : g.s_full;
  float *out = (mat == 0) ? g.G : (mat == 1) ? g.F : g.X;
  const int i0 = ti * BT, j0 = tj * BT;
  const int d = g.d;
  const int64_t n_rows = g.n_rows;
  const int nst = (int)((n_rows + BR8 - 1) / BR8);

  // copy instruction ii of wave w fills 1 KB block blk = w + 4 ii: blocks 0-7 the left operand, 8-15
  // the right one, 8 rows each; lane l lands at row 8 (blk mod 8) + l / 8, stored chunk l mod 8, which
  // holds source chunk (l mod 8) ^ ((row / 2) mod 8). Columns past d are clamped (not stored).
  const uint8_t *src[kCopies8];
  int crow[kCopies8];
#pragma unroll
  for (int ii = 0; ii < kCopies8; ++ii) {
    const int blk = w + 4 * ii;
    const int op = blk >> 3;
    const int r = 8 * (blk & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int col = (op ? j0 : i0) + 16 * c;
    col = col < d ? col : d - 16;
    crow[ii] = r;
    src[ii] = (op ? Q : P) + (int64_t)r * d + col;
  }
  const int64_t stage_bytes = (int64_t)BR8 * d;
  uint64_t zero_row = (uint64_t)(uintptr_t)g_zero_row;
  asm volatile("" : "+s"(zero_row));

  auto copy_stage = [&](int s, uint8_t *slot) {
#pragma unroll
    for (int ii = 0; ii < kCopies8; ++ii) {
      const int64_t n = (int64_t)s * BR8 + crow[ii];
      const uint8_t *p = src[ii] + (int64_t)s * stage_bytes;
      p = n < n_rows ? p : (const uint8_t *)(uintptr_t)zero_row;
      copy_to_lds<16>(p, slot + 1024 * (w + 4 * ii));
    }
  };
  auto read_stage = [&](const uint8_t *slot, StageOps8 &o) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) o.a[bi] = read_operand8(slot, wm * 64 + bi * 32, lane);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) o.b[bj] = read_operand8(slot + kPart8, wn * 64 + bj * 32, lane);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  auto stage = [&](int s, uint8_t *cur, const uint8_t *nxt, const StageOps8 &ocur, StageOps8 &onx) {
    ISPA_GRAM_WAIT_VMCNT(kCopies8 * (NS - 2));
    ISPA_GRAM_LDS_BARRIER();
    copy_stage(s + NS, cur);
    read_stage(nxt, onx);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma_e4m3_32x32x64(ocur.a[bi], ocur.b[bj], acc[bi][bj]);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, kCopies8, 0);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  };

  StageOps8 oa, ob;
  copy_stage(0, ring0);
  copy_stage(1, ring1);
  copy_stage(2, ring2);
  copy_stage(3, ring3);
  ISPA_GRAM_WAIT_VMCNT(kCopies8 * (NS - 1));
  ISPA_GRAM_LDS_BARRIER();
  read_stage(ring0, oa);
  for (int s = 0; s < nst; s += NS) {
    stage(s, ring0, ring1, oa, ob);
    stage(s + 1, ring1, ring2, ob, oa);
    stage(s + 2, ring2, ring3, oa, ob);
    stage(s + 3, ring3, ring0, ob, oa);
  }
  ISPA_GRAM_WAIT_VMCNT(0);   // no copy may land in LDS after the workgroup has ended

  // per-head scales: element (row i, column j) of the tile times sP[i / head_dim] * sQ[j / head_dim]
  const int hd = g.head_dim;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      int cl = j0 + wn * 64 + bj * 32 + l32;
      cl = cl < d ? cl : d - 1;
      const float sq = sQ[cl / hd];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int rw = i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        rw = rw < d ? rw : d - 1;
        acc[bi][bj][v] *= sP[rw / hd] * sq;
      }
    }
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int cl = j0 + wn * 64 + bj * 32 + l32;
      const int clc = cl < d ? cl : d - 1;
      float cur[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        const int rwc = rw < d ? rw : d - 1;
        cur[v] = out[(int64_t)rwc * d + clc];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rw = i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (rw < d && cl < d) out[(int64_t)rw * d + cl] = cur[v] + acc[bi][bj][v];
      }
    }
  if (mat != 2 && ti != tj) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int mr = j0 + wn * 64 + bj * 32 + l32;
        const int mrc = mr < d ? mr : d - 1;
        f32x4 cur[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 64 + bi * 32 + 8 * q + 4 * hf;
          const int mcc = mc < d ? mc : d - 4;
          cur[q] = *(const f32x4 *)&out[(int64_t)mrc * d + mcc];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = i0 + wm * 64 + bi * 32 + 8 * q + 4 * hf;
          f32x4 add;
#pragma unroll
          for (int e = 0; e < 4; ++e) add[e] = acc[bi][bj][4 * q + e];
          if (mr < d && mc < d) *(f32x4 *)&out[(int64_t)mr * d + mc] = cur[q] + add;
        }
      }
  }
}

}  // namespace

hipError_t launch_gram_fp8(int64_t n_rows, int d, int head_dim, const uint8_t *a_loc, const float *s_loc,
                           const uint8_t *a_full, const float *s_full, float *G, float *X, float *F, hipStream_t s) {
  GramArgs8 g;
  g.a_loc = a_loc;
  g.a_full = a_full;
  g.s_loc = s_loc;
  g.s_full = s_full;
  g.G = G;
  g.X = X;
  g.F = F;
  g.n_rows = n_rows;
  g.d = d;
  g.T = (d + BT - 1) / BT;
  g.n_upper = g.T * (g.T + 1) / 2;
  g.with_f = F != nullptr;
  g.head_dim = head_dim;
  const int n_tiles = g.n_upper * (g.with_f ? 2 : 1) + g.T * g.T;
  if (n_rows == 0 || n_tiles == 0 || d < 16) return hipSuccess;
  hipLaunchKernelGGL(gram_fp8_kernel, dim3(n_tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

int gram_tiles(int d, int bt, bool with_f) {
  const int T = (d + bt - 1) / bt;
  return T * (T + 1) / 2 * (with_f ? 2 : 1) + T * T;
}

#ifndef ISPA_GRAM_TAIL_SPLIT
#define ISPA_GRAM_TAIL_SPLIT 1   // tiles of a wide launch's last partial round of 256 go to the 128 x 128 kernel
#endif
#ifndef ISPA_GRAM_WIDE_MIN
#define ISPA_GRAM_WIDE_MIN 512   // wide-tile workgroups a launch needs before the wide kernel is used
#endif

hipError_t launch_gram_bf16_batch(int64_t n_rows, int d, int batch, const uint16_t *const *a_loc,
                                  const uint16_t *const *a_full, float *const *G, float *const *X,
                                  float *const *F, hipStream_t s) {
  if (n_rows == 0 || batch <= 0 || d < 8) return hipSuccess;
  const bool with_f = F != nullptr;
  for (int p0 = 0; p0 < batch; p0 += kMaxGramLayers) {
    const int cnt = batch - p0 < kMaxGramLayers ? batch - p0 : kMaxGramLayers;
    const bool wide = (int64_t)gram_tiles(d, BTW, with_f) * cnt >= ISPA_GRAM_WIDE_MIN;
    const int bt = wide ? BTW : BT;
    GramArgs g;
    for (int i = 0; i < cnt; ++i) {
      g.a_loc[i] = a_loc[p0 + i];
      g.a_full[i] = a_full[p0 + i];
      g.G[i] = G[p0 + i];
      g.X[i] = X[p0 + i];
      g.F[i] = with_f ? F[p0 + i] : nullptr;
    }
    g.n_rows = n_rows;
    g.d = d;
    g.T = (d + bt - 1) / bt;
    g.n_upper = g.T * (g.T + 1) / 2;
    g.with_f = with_f;
    g.tiles = gram_tiles(d, bt, with_f);
    g.tail_first = -1;
    g.Tw = g.n_upper_w = g.tiles_w = 0;
    const int n_wg = g.tiles * cnt;
    if (wide) {
      // The 256 x 256 kernel runs whole rounds of 256 workgroups (one per CU); the tiles of a last,
      // partial round would hold a few CUs for a whole tile while the rest idle, so they go to the
      // 128 x 128 kernel as quarters (four times the workgroups, two per CU), launched after it.
      const int full = ISPA_GRAM_TAIL_SPLIT ? n_wg / 256 * 256 : n_wg;
      const int tail = full > 0 ? n_wg - full : 0;
      const int main_wg = n_wg - tail;
      if (ISPA_GRAM_WAVES == 8)
        hipLaunchKernelGGL(gram_bf16_wide_kernel<8>, dim3((unsigned)main_wg), dim3(512), 0, s, g);
      else
        hipLaunchKernelGGL(gram_bf16_wide_kernel<4>, dim3((unsigned)main_wg), dim3(256), 0, s, g);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (tail > 0) {
        GramArgs gt = g;
        gt.Tw = g.T;
        gt.n_upper_w = g.n_upper;
        gt.tiles_w = g.tiles;
        gt.tail_first = main_wg;
        gt.T = (d + BT - 1) / BT;
        gt.n_upper = gt.T * (gt.T + 1) / 2;
        gt.tiles = gram_tiles(d, BT, with_f);
        hipLaunchKernelGGL(gram_bf16_kernel, dim3((unsigned)(4 * tail)), dim3(kThreads), 0, s, gt);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    } else {
      hipLaunchKernelGGL(gram_bf16_kernel, dim3((unsigned)n_wg), dim3(kThreads), 0, s, g);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gram_bf16(int64_t n_rows, int d, const uint16_t *a_loc, const uint16_t *a_full,
                            float *G, float *X, float *F, hipStream_t s) {
  return launch_gram_bf16_batch(n_rows, d, 1, &a_loc, &a_full, &G, &X, F != nullptr ? &F : nullptr, s);
}

}  // namespace ispa
