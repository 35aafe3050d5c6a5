// Integer forward of the 4-bit layer with int8 activations, on
// v_mfma_i32_16x16x64_i8:
//
//   acc_g[m, n] = sum_{k in group g} xq[m, k] q[n, k]        (exact int32)
//   y[m, n]     = fma(s, sum_j t[m, j] B[j, n], sx[m] sum_g sc[n, g] acc_g[m, n])
//
// ("Simplified Int4Variable quantization": two 4-bit codes per byte; "How to
// fine-tune the 4-bit model?": narrow frozen weights under a float adapter
// raise the arithmetic intensity; "Introduce QLoRA-like technique",
// "Highlights": the int8 x int8 integer product of the int8 path, here with
// 4-bit weight codes.) The alternative to the dequantized bf16 product of
// gemm_w4.hip: the activation codes and scales come from the same per-row
// quantizer as the int8 weights use.
//
// A stage covers one 128-wide group of k. Two tiles per stage move global ->
// LDS without registers (ring.hpp): the activation codes [BM rows][128 bytes]
// and the packed weight codes [BN n][64 bytes], both chunk-swizzled; the
// block's fp16 group scales [BN][K / 128] come in once before the loop. Each
// wave widens the nibbles of its own operand rows in registers: 8 bytes of a
// row give the 16 consecutive k of one MFMA operand, each nibble
// sign-extended into a byte (x | (x & 8) * 30 sets the upper nibble when bit
// 3 is set) and the even-k and odd-k bytes interleaved with v_perm_b32. After
// the group's two 64-wide steps the int32 sums are weighted by the group's
// scale and added into float32 accumulators; the epilogue multiplies by
// sx[m] and adds the adapter term (ring.hpp).
#include "launch.hpp"
#include "ring.hpp"

namespace qlora {

namespace {

constexpr int kCUs = 256;

struct A8W4Args {
  int M, N, K;
  const int8_t* xq;         // [M, K]
  const float* sx;          // [M]
  const uint8_t* packed;    // [N, K / 2], low nibble = even k
  const _Float16* scales;   // [N, K / 128]
  const float* t;           // [M, r]
  const float* B;           // [r, N], or [heads, r, hd]
  int hd;                   // head width (N: one head)
  int r;
  float s;
  uint16_t* y;              // [M, N] bf16
  int tiles_x;
};

// Sixteen consecutive 4-bit codes (8 bytes, the even k in each low nibble)
// as sixteen int8 values in k order.
__device__ __forceinline__ i32x4 widen_nibbles(u32x2 w) {
  i32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t lo = w[h] & 0x0F0F0F0Fu;             // k = 0, 2, 4, 6 of this dword
    uint32_t hi = (w[h] >> 4) & 0x0F0F0F0Fu;      // k = 1, 3, 5, 7
    lo |= (lo & 0x08080808u) * 30u;               // sign-extend each nibble
    hi |= (hi & 0x08080808u) * 30u;
    out[2 * h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);      // k 0..3
    out[2 * h + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u);  // k 4..7
  }
  return out;
}

// G: the largest number of 128-wide k groups the block's scale slab holds.
template <int BM, int BN, int S, int R, int G>
__global__ __launch_bounds__(256) void fwd_a8w4_kernel(A8W4Args a) {
  constexpr int BK = 128;                          // k per stage = one scale group
  constexpr int ASZ = BM * 128, BSZ = BN * 64, STG = ASZ + BSZ;
  constexpr int AI = BM / 32, BI = BN / 64, LPS = AI + BI;   // DMA per wave per stage
  constexpr int FM = BM / 32, FN = BN / 32;
  static_assert(BN == 128, "code rows of 64 bytes: 16 rows per DMA instruction");
  static_assert(BN * G * 2 % 1024 == 0, "the scale slab takes whole 1 KB DMA instructions");
  // after the loop the ring holds the epilogue operands, then one output
  // staging strip per wave
  constexpr int EPB = (EpiOps<BM, BN, R, true>::kFloats * 4 + 15) / 16 * 16;
  static_assert(EPB + 4 * epi_strip_bytes<uint16_t, FN>() <= S * STG, "epilogue fits in the ring");
  __shared__ __attribute__((aligned(1024))) int8_t lds[S * STG + BN * G * 2];
  int8_t* ring = lds;
  const _Float16* SC = reinterpret_cast<const _Float16*>(lds + S * STG);   // [BN][ngrp]

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int wm = wid >> 1, wn = wid & 1;
  int mt, nt;
  xcd_tile((int)blockIdx.x, (a.M + BM - 1) / BM, a.tiles_x, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int ngrp = K / BK;

  // epilogue operands: t, B, and the row scales sx (no column scale)
  EpiOps<BM, BN, R, true> ep;
  ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, a.sx, nullptr);

  // the block's scale slab: rows n0 .. n0 + BN of [N][ngrp], contiguous
  {
    const int bytes = BN * ngrp * 2;                // a multiple of 16
    const int8_t* src0 = reinterpret_cast<const int8_t*>(a.scales) + (long)n0 * ngrp * 2;
    const long valid = ((long)N - n0) * ngrp * 2;    // bytes that exist past src0
    for (int o = wid * 1024; o < bytes; o += 4096) {
      const int e = o + lane * 16;
      const int8_t* src = (e < bytes && e < valid) ? src0 + e : zero_chunk(lane);
      lds_dma16(src, lds + S * STG + o);
    }
  }
  // Loads from a wave-wide base (the stage's first k) plus a fixed 32-bit
  // lane offset. Rows past M repeat row M - 1 and weight rows past N repeat
  // row N - 1: their products land only in outputs that are never stored.
  uint32_t voA[AI], voB[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int rb = wid * (BM / 4) + i * 8, row = rb + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    voA[i] = (uint32_t)((long)(gm < M ? gm : M - 1) * K + c * 16);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int rb = (wid * BI + i) * 16, row = rb + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3), gn = n0 + row;
    voB[i] = (uint32_t)((long)(gn < N ? gn : N - 1) * (K / 2) + c * 16);
  }
  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
    const int8_t* xb = a.xq + kt * BK;
    const int8_t* pb = reinterpret_cast<const int8_t*>(a.packed) + kt * 64;
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(xb + voA[i], base + (wid * (BM / 4) + i * 8) * 128);
#pragma unroll
    for (int i = 0; i < BI; ++i) lds_dma16(pb + voB[i], base + ASZ + (wid * BI + i) * 16 * 64);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < ngrp) issue(st, st);
  // The scale slab went out before stage 0: loads complete in issue order,
  // so every wave's share has landed once its stage 0 has, and the first
  // barrier covers all waves.

  int slot = 0;
  for (int kt = 0; kt < ngrp; ++kt) {
    wait_stages<LPS, 0, S - 2>(ngrp - 1 - kt);
    __builtin_amdgcn_s_barrier();                    // stage kt landed; slot kt - 1 free
    if (kt + S - 1 < ngrp) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;

    i32x4 part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) part[i][j] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < BK / 64; ++kk) {
      const int c = kk * 4 + (lane >> 4);            // 16-byte chunk of the A rows
      // the B operand: 16 k = 8 bytes of a packed row, at byte 8 c
      const int cb = c >> 1, half = c & 1;
      i32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(As + swz128(wm * (BM / 2) + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * (BN / 2) + j * 16 + (lane & 15);
        const u32x2 w = *reinterpret_cast<const u32x2*>(Bs + n * 64 + ((cb ^ ((n >> 2) & 3)) << 4) + half * 8);
        bf[j] = widen_nibbles(w);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          part[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], part[i][j], 0, 0, 0);
    }
    // weight the group's exact sums by its scale (the lane's column of each
    // 16 x 16 block is lane % 16)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = wn * (BN / 2) + j * 16 + (lane & 15);
      const float sc = (float)SC[nl * ngrp + kt];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          acc[i][j][ii] = __builtin_fmaf((float)part[i][j][ii], sc, acc[i][j][ii]);
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  float* E = reinterpret_cast<float*>(ring);
  __syncthreads();                                    // every wave is done with the ring
  ep.store(E, M, N, m0, n0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, BN, R, true>(acc, E, M, N, m0, n0, wm * (BM / 2), wn * (BN / 2), a.s, a.y,
                                    ring + EPB + wid * epi_strip_bytes<uint16_t, FN>());
}

template <int BM, int S, int G>
void launch_tiles(A8W4Args a, hipStream_t st) {
  constexpr int BN = 128;
  a.tiles_x = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM)));
  if (a.r <= 4) fwd_a8w4_kernel<BM, BN, S, 4, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_a8w4_kernel<BM, BN, S, 8, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_a8w4_kernel<BM, BN, S, 16, G><<<grid, 256, 0, st>>>(a);
  else fwd_a8w4_kernel<BM, BN, S, 32, G><<<grid, 256, 0, st>>>(a);
}

template <int BM, int S>
void launch_groups(const A8W4Args& a, hipStream_t st) {
  const int ngrp = a.K / 128;                      // validated: <= kW4MaxGroups
  if (ngrp <= 8) launch_tiles<BM, S, 8>(a, st);
  else if (ngrp <= 32) launch_tiles<BM, S, 32>(a, st);
  else launch_tiles<BM, S, kW4MaxGroups>(a, st);
}

}  // namespace

void launch_gemm_fwd_a8w4(int M, int N, int K, const int8_t* xq, const float* sx,
                          const uint8_t* packed, const _Float16* scales,
                          const float* t, const float* B, int hd, int r, float s,
                          uint16_t* y, hipStream_t st) {
  A8W4Args a{};
  a.M = M; a.N = N; a.K = K; a.xq = xq; a.sx = sx; a.packed = packed; a.scales = scales;
  a.t = t; a.B = B; a.hd = hd; a.r = r; a.s = s; a.y = y;
  const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= kCUs) launch_groups<128, 2>(a, st);
  else launch_groups<64, 3>(a, st);
}

}  // namespace qlora
