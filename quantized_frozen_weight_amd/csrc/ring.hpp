// Shared pieces of the MFMA products: the direct-to-LDS stage ring and the
// low-rank epilogue.
//
// Stage ring. Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (16 bytes per lane; lane l of one instruction lands
// at LDS base + 16 l), so no registers hold tiles in flight and no wave spends
// instructions copying them. S stages rotate through the ring: the block waits
// for stage kt with an explicit partial vector-memory count (the loads of the
// later stages stay in flight), crosses one barrier, refills the slot freed by
// stage kt - 1 and computes on stage kt. Rows of 128 bytes hold eight
// 16-byte chunks stored at chunk ^ ((row >> 1) & 7): the 16 rows one MFMA
// operand read touches then cover all 64 banks once.
#pragma once

#include "common.hpp"

namespace qlora {

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters unconstrained
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

// s_waitcnt immediate that waits for every LDS operation of this wave
// (lgkmcnt 0) and leaves the other counters unconstrained.
constexpr int lgkmcnt0_imm() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }

// Index of the calling wave in its block, as a wave-uniform (scalar) value.
// Plain threadIdx.x / 64 is not known to be uniform to the compiler, which
// then guards code that depends on it with an exec mask; MFMA instructions
// ignore the exec mask, so such a guard would not hold.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
}

// Wait until at most min(n, MAXI) stages of LPS loads each are outstanding.
template <int LPS, int I, int MAXI>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (I >= MAXI) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(MAXI * LPS));
  } else {
    if (n <= I) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(I * LPS));
      return;
    }
    wait_stages<LPS, I + 1, MAXI>(n);
  }
}

// Tile (row mt, column kt) of block b in a grid of tm x tx tiles. The
// dispatcher deals blocks to the eight XCDs in turn, each XCD with its own
// L2; numbering logical blocks L = (b % 8) (blocks / 8) + b / 8 and laying
// them out in bands of gw tile columns, row-major inside a band, gives each
// XCD a compact rectangle of tiles, so that its L2 fetches a few row and
// column panels instead of a slice of all of them. Grids that do not divide
// evenly keep the row-major order.
__device__ __forceinline__ void xcd_tile(int b, int tm, int tx, int& mt, int& kt) {
  const int nb = tm * tx;
  const int gw = tx % 8 == 0 ? 8 : tx % 4 == 0 ? 4 : 0;
  if ((nb & 7) == 0 && gw != 0) {
    const int L = (b & 7) * (nb >> 3) + (b >> 3);
    const int band = L / (tm * gw), r = L - band * (tm * gw);
    mt = r / gw;
    kt = band * gw + r % gw;
  } else {
    mt = b / tx;
    kt = b % tx;
  }
}

// Zero bytes: the source of direct-to-LDS lanes whose 16-byte chunk lies past
// the end of the contraction axis (every shape keeps that axis a multiple of
// 16, so a chunk is wholly inside or wholly outside).
static __device__ __attribute__((aligned(256))) int8_t g_zero_chunks[256] = {};

__device__ __forceinline__ const int8_t* zero_chunk(int lane) {
  return g_zero_chunks + 16 * (lane & 15);
}

// Copy one 16-byte chunk per lane from global memory into LDS; lane l writes
// dst + 16 l.
__device__ __forceinline__ void lds_dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Byte offset of logical 16-byte chunk c of row `row` in a 128-byte-row tile.
__device__ __forceinline__ int swz128(int row, int c) {
  return row * 128 + ((c ^ ((row >> 1) & 7)) << 4);
}

// ---------------------------------------------------------------------------
// Low-rank epilogue: out[m, n] = fma(s, sum_j P[m, j] Q(j, n), base[m, n])
// with base = float(acc) * (rs[m] * cs[n]) or the float accumulator itself,
// or (affine weights, AFF) base = rs[m] * (acc + ra[m]) with acc already the
// float c * (integer product) + correction of the affine grid, and a per-row
// term ra[m] = b * as[m] (b the grid's value of code 0, as[m] a row sum of
// the activation codes).
// The rank-R product runs on v_mfma_f32_16x16x4_f32 (float32 operands and
// accumulation), R / 4 instructions per 16 x 16 block, and lands in the same
// lane layout as the main accumulator. The block's operands are fetched into
// registers when the kernel starts (loads from clamped addresses, masked
// afterwards, so no branch waits on them) and written to LDS once the main
// loop has released the ring:
//   ts [BM][R]   P rows of the tile, ranks past r zero
//   qs [R][BN]   Q of the tile's columns, ranks past r zero
//   rsv [BM], csv [BN]             (SCALED)
//   rav [BM]                       (AFF)
// ---------------------------------------------------------------------------
template <int BM, int BN, int R, bool SCALED, bool AFF = false> struct EpiOps {
  static constexpr int kFloats = (BM + BN) * R + BM + BN + (AFF ? BM : 0);
  static constexpr int NT = (BM * R + 255) / 256;
  static constexpr int NQ = (BN * R + 255) / 256;
  float t[NT], q[NQ], rs, cs, ra;

  // P float32 [M, r]; Q(j, n) = Q[head_index(j, n, r, hd)] ([r][N], or
  // [heads][r][hd]); rsrc [M] / csrc [N]
  // read when SCALED (csrc NULL: column scale 1). Nothing here consumes the
  // loaded values: a use would make the wave wait for these loads before the
  // main loop starts. The masks are applied by store().
  __device__ __forceinline__ void load(int M, int N, int m0, int n0, int r,
                                       const float* __restrict__ P,
                                       const float* __restrict__ Q, int hd,
                                       const float* __restrict__ rsrc,
                                       const float* __restrict__ csrc) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = tid + 256 * i;
      const int row = e / R, j = e % R, gm = m0 + row;
      t[i] = P[(long)(gm < M ? gm : M - 1) * r + (j < r ? j : r - 1)];
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 256 * i;
      const int j = e / BN, col = e % BN, gn = n0 + col;
      q[i] = Q[head_index(j < r ? j : r - 1, gn < N ? gn : N - 1, r, hd)];
    }
    if constexpr (SCALED) {
      const int im = m0 + (tid < BM ? tid : BM - 1), in = n0 + (tid < BN ? tid : BN - 1);
      rs = rsrc[im < M ? im : M - 1];
      cs = csrc != nullptr ? csrc[in < N ? in : N - 1] : 1.f;   // no column scale: 1
    }
  }

  // AFF: the row sums as[M] of the activation codes (the grid's bias times
  // them is the per-row term); read like the scales above.
  __device__ __forceinline__ void load_rows(int M, int m0, const float* __restrict__ asrc) {
    const int tid = threadIdx.x;
    const int im = m0 + (tid < BM ? tid : BM - 1);
    ra = asrc[im < M ? im : M - 1];
  }

  __device__ __forceinline__ void store(float* E, int M, int N, int m0, int n0, int r) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = tid + 256 * i;
      const int row = e / R, j = e % R;
      if (e < BM * R) E[e] = (j < r && m0 + row < M) ? t[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 256 * i;
      const int j = e / BN, col = e % BN;
      if (e < BN * R) E[BM * R + e] = (j < r && n0 + col < N) ? q[i] : 0.f;
    }
    if constexpr (SCALED) {
      if (tid < BM) E[(BM + BN) * R + tid] = m0 + tid < M ? rs : 0.f;
      if (tid < BN) E[(BM + BN) * R + BM + tid] = n0 + tid < N ? cs : 0.f;
    }
  }

  // AFF: rav[m] = bias * as[m]
  __device__ __forceinline__ void store_rows(float* E, int M, int m0, float bias) const {
    const int tid = threadIdx.x;
    if (tid < BM) E[(BM + BN) * R + BM + BN + tid] = m0 + tid < M ? bias * ra : 0.f;
  }
};


// LDS bytes of one wave's output staging strip in epilogue_lowrank: 16 rows
// of FN * 16 outputs, each row padded by 16 bytes (so that the four row
// groups of one write instruction fall in different banks).
template <typename OutT, int FN>
constexpr int epi_strip_bytes() {
  return 16 * (FN * 16 * (int)sizeof(OutT) + 16);
}

// Apply the epilogue to a wave's FM x FN grid of 16 x 16 accumulator blocks
// whose top-left output is (wr0, wc0) inside the tile (the lane holds rows
// 4 (lane / 16) + ii of column lane % 16 of each block). The results leave
// through `strip` (epi_strip_bytes<OutT, FN>() of LDS owned by this wave):
// one 16-row strip at a time is written there in the accumulator layout and
// read back as 16-byte pieces of rows, so each global store instruction
// writes whole 16-byte runs of a row instead of one element per lane.
template <int BM, int BN, int R, bool SCALED, bool AFF = false, typename OutT, typename AccT,
          int FM, int FN>
__device__ __forceinline__ void epilogue_lowrank(const AccT (&acc)[FM][FN], const float* E,
                                                 int M, int N, int m0, int n0, int wr0,
                                                 int wc0, float s, OutT* __restrict__ out,
                                                 int8_t* strip) {
  static_assert(!AFF || SCALED, "the affine form uses the row scales");
  const int lane = threadIdx.x & 63;
  const float* ts = E;
  const float* qs = E + BM * R;
  const float* rsv = E + (BM + BN) * R;
  const float* csv = rsv + BM;
  const float* rav = csv + BN;
  f32x4 low[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) low[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A operand lane l: P[row l % 16][rank 4 kc + l / 16]; B operand lane l:
  // Q(rank 4 kc + l / 16, column l % 16).
#pragma unroll
  for (int kc = 0; kc < R / 4; ++kc) {
    const int j = kc * 4 + (lane >> 4);
    float ta[FM], qb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ta[i] = ts[(wr0 + i * 16 + (lane & 15)) * R + j];
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) qb[jn] = qs[j * BN + wc0 + jn * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        low[i][jn] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[i], qb[jn], low[i][jn], 0, 0, 0);
  }
  constexpr int ROWB = FN * 16 * (int)sizeof(OutT);   // bytes of one strip row
  constexpr int PITCH = ROWB + 16;
  constexpr int CPR = ROWB / 16;                      // 16-byte pieces per row
  constexpr int EPC = 16 / (int)sizeof(OutT);         // outputs per piece
  static_assert(CPR * 16 % 64 == 0, "whole pieces per lane");
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const int nl = wc0 + jn * 16 + (lane & 15);
      const float csn = SCALED ? csv[nl] : 1.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rl = (lane >> 4) * 4 + ii;             // row inside the strip
        const int ml = wr0 + i * 16 + rl;
        float base;
        if constexpr (AFF)
          base = rsv[ml] * ((float)acc[i][jn][ii] + rav[ml]);
        else
          base = SCALED ? (float)acc[i][jn][ii] * (rsv[ml] * csn) : (float)acc[i][jn][ii];
        store_out(reinterpret_cast<OutT*>(strip + rl * PITCH) + jn * 16 + (lane & 15),
                  __builtin_fmaf(s, low[i][jn][ii], base));
      }
    }
    // (no wait between the strip's writes and its read-back, nor before the
    // next strip's writes: the LDS executes one wave's instructions in issue
    // order, and the strip belongs to this wave alone; measured 1-2 % on the
    // products)
#pragma unroll
    for (int p = 0; p < CPR * 16 / 64; ++p) {
      const int q = lane + 64 * p, rl = q / CPR, cq = q % CPR;
      const int m = m0 + wr0 + i * 16 + rl, n = n0 + wc0 + cq * EPC;
      const u32x4 v = *reinterpret_cast<const u32x4*>(strip + rl * PITCH + cq * 16);
      if (m < M && n < N) *reinterpret_cast<u32x4*>(out + (long)m * N + n) = v;
    }
  }
}

}  // namespace qlora
