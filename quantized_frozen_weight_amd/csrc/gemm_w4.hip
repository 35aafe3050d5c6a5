// Forward product of the frozen 4-bit layer on v_mfma_f32_16x16x32_bf16:
//
//   y[m, n] = fma(s, sum_j t[m, j] B[j, n], sum_k x[m, k] deq4[k, n])
//   deq4[k, n] = q[n, k] sc[n, k / 128]
//
// ("How to fine-tune the 4-bit model?": the frozen weight is dequantized
// and multiplied in float; "Simplified Int4Variable quantization": two 4-bit
// values per byte. "Parameter-efficient fine-tuning of GPT-2 with LoRA",
// "LoRA equation" and "Create LoRA layer": the adapter term, scaled by
// alpha / rank.)
//
// A stage covers half of one 128-wide group of k, so one fp16 scale per
// output column applies to the whole stage. Two tiles move global -> LDS
// without registers (ring.hpp): the x rows (bf16, 128-byte rows swizzled by
// 16-byte chunk) and the packed codes [BN n][32 bytes]; once before the loop
// the block's scales [BN][K / 128] (a contiguous slab of the scale array)
// follow the same path. Each wave widens the codes of its own columns from
// LDS straight into MFMA operand registers (below). The adapter term runs in
// the epilogue on v_mfma_f32_16x16x4_f32 (ring.hpp).
//
// Few 128-row tiles over a long k axis split it (up to 8 ways): each block
// multiplies one range of k and leaves its float32 accumulators in the
// workspace, and a second launch adds them in split order and applies the
// epilogue.
#include "launch.hpp"
#include "ring.hpp"

namespace qlora {

namespace {

constexpr int kCUs = 256;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct W4Args {
  int M, N, K;
  const uint16_t* x;        // [M, K] bf16
  const uint8_t* packed;    // [N, K / 2], low nibble = even k
  const _Float16* scales;   // [N, K / 128]
  const float* t;           // [M, r]
  const float* B;           // [r, N], or [heads, r, hd]
  int hd;                   // head width (N: one head)
  int r;
  float s;
  uint16_t* y;              // [M, N] bf16
  int tiles_x;
  // split contraction (128-row tiles): float32 partial sums in the
  // accumulator layout, the split count and stages of 64 k per split
  float* pacc;              // [splits, tiles, 4 waves, 16 fragments, 64 lanes] float4
  int splits, nks;
};

constexpr int kMaxW4Splits = 8;

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The eight nibbles of a packed word (nibble e = the code of k offset e,
// two's complement) times sc, as four bf16 pairs: w ^ 0x88888888 turns each
// code q into q + 8 in [0, 15], two masks spread the nibbles over bytes
// (v_cvt_f32_ubyte takes a byte in one instruction), and
// fma(q + 8, sc, -8 sc) rounds q sc exactly once, as q * sc would.
__device__ __forceinline__ u32x4 nibbles_bf16(uint32_t w, float sc) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0f0f0f0fu, hi = (u >> 4) & 0x0f0f0f0fu;   // even, odd e
  const float nsc = -8.f * sc;
  float v[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = __builtin_fmaf((float)((lo >> (8 * b)) & 0xffu), sc, nsc);
    v[2 * b + 1] = __builtin_fmaf((float)((hi >> (8 * b)) & 0xffu), sc, nsc);
  }
  return u32x4{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]), pk_bf16(v[4], v[5]), pk_bf16(v[6], v[7])};
}

// G: the largest number of 128-wide k groups the block's scale slab holds.
//
// A block owns BM rows x 128 columns of y. Wave w owns columns
// [32 w, 32 w + 32) and every row of the block, so the codes it multiplies
// are its own: each lane reads the packed word holding the 8 codes of its
// operand slot (column n, 8 consecutive k -- exactly one 32-bit word of the
// [n][k / 2] layout) and widens it straight into the MFMA operand register,
// with no converted copy in LDS and no second barrier per stage. The
// widening of one operand then overlaps the matrix work of the previous one
// inside the wave.
template <int BM, int S, int R, int G, bool SPLIT = false>
__global__ __launch_bounds__(256, 2) void fwd_w4_kernel(W4Args a) {
  static_assert(!SPLIT || BM == 128, "split contraction: 128-row tiles");
  constexpr int BN = 128, BK = 64;                 // k per stage: half a scale group
  constexpr int ASZ = BM * 128, BSZ = BN * 32, STG = ASZ + BSZ;
  constexpr int AI = BM / 32, LPS = AI + 1;        // DMA per wave per stage: x rows, code rows
  constexpr int FM = BM / 16, FN = 2;              // the wave's 16 x 16 blocks: all rows, 32 columns
  // after the loop the ring holds the epilogue operands, then one output
  // staging strip per wave
  constexpr int EPB = (EpiOps<BM, BN, R, false>::kFloats * 4 + 15) / 16 * 16;
  static_assert(EPB + 4 * epi_strip_bytes<uint16_t, FN>() <= S * STG, "epilogue fits");
  const int K = a.K, M = a.M, N = a.N;
  const int ngrp = K / 128;
  static_assert(BN * G * 2 % 1024 == 0, "the scale slab takes whole 1 KB DMA instructions");
  // scales of the block's columns: [BN][ngrp] fp16, ngrp <= G
  __shared__ __attribute__((aligned(1024))) int8_t lds[S * STG + BN * G * 2];
  int8_t* ring = lds;
  const _Float16* SC = reinterpret_cast<const _Float16*>(lds + S * STG);

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  // SPLIT: blocks (split, tile), split-major, renumbered so that the blocks
  // the dispatcher deals to one XCD (every eighth) share one split's k range
  int bid = (int)blockIdx.x, split = 0;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  int mt, nt;
  if constexpr (SPLIT) {
    const int nb = (int)gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    split = bid / tiles;
    bid -= split * tiles;
    mt = bid / a.tiles_x;
    nt = bid % a.tiles_x;
  } else {
    xcd_tile(bid, (M + BM - 1) / BM, a.tiles_x, mt, nt);
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk = 2 * ngrp;
  // stages [kt0, kt1) of the contraction
  const int kt0 = SPLIT ? split * a.nks : 0;
  const int kt1 = SPLIT ? (kt0 + a.nks < nk ? kt0 + a.nks : nk) : nk;

  EpiOps<BM, BN, R, false> ep;
  if constexpr (!SPLIT) ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, nullptr, nullptr);

  // the block's scale slab: rows n0 .. n0 + BN of [N][ngrp], contiguous
  {
    const int bytes = BN * ngrp * 2;                // multiple of 16 (ngrp >= 1, BN = 128)
    const int8_t* src0 = reinterpret_cast<const int8_t*>(a.scales) + (long)n0 * ngrp * 2;
    const long valid = ((long)N - n0) * ngrp * 2;    // bytes that exist past src0
    for (int o = wid * 1024; o < bytes; o += 4096) {
      const int e = o + lane * 16;
      const int8_t* src = (e < bytes && e < valid) ? src0 + e : zero_chunk(lane);
      lds_dma16(src, lds + S * STG + o);
    }
  }
  // Loads from a wave-wide base (the stage's first k) plus a fixed 32-bit
  // lane offset: x as 128-byte rows swizzled by 16-byte chunk, 8 rows per
  // instruction; the codes as 32-byte rows, 32 per instruction (lanes 2 i
  // and 2 i + 1 take the two halves of row i), wave w loading the rows of
  // its own columns. Rows past M repeat row M - 1 and weight rows past N
  // repeat row N - 1: their products land only in outputs that are never
  // stored.
  uint32_t voA[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = wid * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    voA[i] = (uint32_t)(((long)(gm < M ? gm : M - 1) * K + c * 8) * 2);
  }
  const int brow = wid * 32 + (lane >> 1), gn = n0 + brow;
  const uint32_t voB = (uint32_t)((long)(gn < N ? gn : N - 1) * (K / 2) + (lane & 1) * 16);
  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
    const int8_t* xb = reinterpret_cast<const int8_t*>(a.x) + 2L * kt * BK;
    const int8_t* pb = reinterpret_cast<const int8_t*>(a.packed) + kt * (BK / 2);
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(xb + voA[i], base + (wid * (BM / 4) + i * 8) * 128);
    lds_dma16(pb + voB, base + ASZ + wid * 32 * 32);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (kt0 + st < kt1) issue(kt0 + st, st);
  // The scale slab went out before the first stage (its per-wave
  // instruction count may differ): loads complete in issue order, so every
  // wave's share has landed once its first stage has, and the first barrier
  // covers all waves.

  // the lane's operand slots: column 32 wid + 16 jf + lane % 16 (code row
  // in the tile), k 8 (lane / 16) .. + 8 of each 32-wide step
  const int nl = 32 * wid + (lane & 15);
  int slot = 0;
  for (int kt = kt0; kt < kt1; ++kt) {
    wait_stages<LPS, 0, S - 2>(kt1 - 1 - kt);
    __builtin_amdgcn_s_barrier();                    // stage kt landed; slot of kt - 1 free
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;
    uint32_t raw[FN][BK / 32];
    float sc[FN];
#pragma unroll
    for (int jf = 0; jf < FN; ++jf) {
      sc[jf] = (float)SC[(nl + 16 * jf) * ngrp + (kt >> 1)];
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk)
        raw[jf][kk] = *reinterpret_cast<const uint32_t*>(Bs + (nl + 16 * jf) * 32 + kk * 16 + (lane >> 4) * 4);
    }
    // the next stage's loads, into the slot stage kt - 1 left, once this
    // stage's codes are read
    if (kt + S - 1 < kt1) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 bf[FN];
#pragma unroll
      for (int jf = 0; jf < FN; ++jf) bf[jf] = __builtin_bit_cast(bf16x8, nibbles_bf16(raw[jf][kk], sc[jf]));
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(As + swz128(i * 16 + (lane & 15), c));
#pragma unroll
        for (int jf = 0; jf < FN; ++jf)
          acc[i][jf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[jf], acc[i][jf], 0, 0, 0);
      }
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  if constexpr (SPLIT) {
    // float4 unit (((split tiles + tile) 4 + wave) F + f) 64 + lane for
    // fragment f = i FN + jf of F = FM FN: each store writes 1 KB of
    // consecutive bytes
    f32x4* P = reinterpret_cast<f32x4*>(a.pacc) +
               ((long)(split * tiles + bid) * 4 + wid) * (FM * FN * 64) + lane;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jf = 0; jf < FN; ++jf) P[(i * FN + jf) * 64] = acc[i][jf];
    return;
  }

  float* E = reinterpret_cast<float*>(ring);
  __syncthreads();
  ep.store(E, M, N, m0, n0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, BN, R, false>(acc, E, M, N, m0, n0, 0, 32 * wid, a.s, a.y,
                                     ring + EPB + wid * epi_strip_bytes<uint16_t, FN>());
}

// Second launch of the split contraction, one 512-thread block per 32-column
// strip of a 128 x 128 tile (the strip one wave of the product kernel owns):
// the partial sums added in split order, then the epilogue. Wave v takes the
// strip's 16-row block v.
template <int R, int NSPL>
__global__ __launch_bounds__(512) void fwd_w4_fixup_kernel(W4Args a) {
  constexpr int BM = 128, HN = 32, FM = 8, FN = 2;
  using Ep = EpiOps<BM, HN, R, false>;
  constexpr int EPB = (Ep::kFloats * 4 + 15) / 16 * 16;
  constexpr int STRIP = epi_strip_bytes<uint16_t, FN>();
  __shared__ __attribute__((aligned(1024))) int8_t lds[EPB + 8 * STRIP];
  float* E = reinterpret_cast<float*>(lds);

  const int tid = threadIdx.x, lane = tid & 63, v = wave_id();
  const int M = a.M, N = a.N, nsp = a.splits;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  const int tile = (int)blockIdx.x >> 2, q = (int)blockIdx.x & 3;
  const int m0 = (tile / a.tiles_x) * BM, n0 = (tile % a.tiles_x) * 128 + q * HN;

  const f32x4* P = reinterpret_cast<const f32x4*>(a.pacc) + ((long)tile * 4 + q) * (FM * FN * 64) +
                   v * FN * 64 + lane;
  const long pstride = (long)tiles * 4 * FM * FN * 64;  // float4 units per split
  f32x4 pv[NSPL][FN];
#pragma unroll
  for (int sp = 0; sp < NSPL; ++sp)
#pragma unroll
    for (int j = 0; j < FN; ++j) pv[sp][j] = P[(sp < nsp ? sp : 0) * pstride + j * 64];

  Ep ep;
  if (tid < 256) ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, nullptr, nullptr);
  f32x4 acc[1][FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    acc[0][j] = pv[0][j];
#pragma unroll
    for (int sp = 1; sp < NSPL; ++sp)
      if (sp < nsp) acc[0][j] += pv[sp][j];
  }
  if (tid < 256) ep.store(E, M, N, m0, n0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, HN, R, false>(acc, E, M, N, m0, n0, 16 * v, 0, a.s, a.y,
                                     lds + EPB + v * STRIP);
}

template <int BM, int S, int G>
void launch_tiles(W4Args a, hipStream_t st) {
  constexpr int BN = 128;
  a.tiles_x = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM)));
  if (a.r <= 4) fwd_w4_kernel<BM, S, 4, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_w4_kernel<BM, S, 8, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_w4_kernel<BM, S, 16, G><<<grid, 256, 0, st>>>(a);
  else fwd_w4_kernel<BM, S, 32, G><<<grid, 256, 0, st>>>(a);
}

template <int S, int G>
void launch_split_tiles(W4Args a, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  a.tiles_x = (a.N + BN - 1) / BN;
  const int tiles = a.tiles_x * ((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles * a.splits)), fgrid((unsigned)(4 * tiles));
  if (a.r <= 4) fwd_w4_kernel<BM, S, 4, G, true><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_w4_kernel<BM, S, 8, G, true><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_w4_kernel<BM, S, 16, G, true><<<grid, 256, 0, st>>>(a);
  else fwd_w4_kernel<BM, S, 32, G, true><<<grid, 256, 0, st>>>(a);
  if (a.splits <= 4) {
    if (a.r <= 4) fwd_w4_fixup_kernel<4, 4><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 8) fwd_w4_fixup_kernel<8, 4><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 16) fwd_w4_fixup_kernel<16, 4><<<fgrid, 512, 0, st>>>(a);
    else fwd_w4_fixup_kernel<32, 4><<<fgrid, 512, 0, st>>>(a);
  } else {
    if (a.r <= 4) fwd_w4_fixup_kernel<4, kMaxW4Splits><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 8) fwd_w4_fixup_kernel<8, kMaxW4Splits><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 16) fwd_w4_fixup_kernel<16, kMaxW4Splits><<<fgrid, 512, 0, st>>>(a);
    else fwd_w4_fixup_kernel<32, kMaxW4Splits><<<fgrid, 512, 0, st>>>(a);
  }
}

// Split count and stages of 64 k per split: only for at most 128 tiles of
// 128 x 128, doubling (up to 8) while the grid stays within two blocks per
// compute unit and each split keeps at least 8 stages.
void w4_split_plan(int M, int N, int K, int* splits, int* nks) {
  const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  const int nk = K / 64;
  int sp = 1;
  if (tiles <= 128)
    while (sp < kMaxW4Splits && tiles * sp * 2 <= 2 * kCUs && nk / (sp * 2) >= 8) sp *= 2;
  *nks = (nk + sp - 1) / sp;
  *splits = (nk + *nks - 1) / *nks;
}

// Three ring slots where they fit beside the scale slab at two blocks per
// compute unit (80 KB each), else two.
template <int BM>
void launch_groups(const W4Args& a, hipStream_t st) {
  const int ngrp = a.K / 128;                      // validated: <= kW4MaxGroups
  if (a.splits > 1) {
    if (ngrp <= 8) launch_split_tiles<3, 8>(a, st);
    else if (ngrp <= 32) launch_split_tiles<3, 32>(a, st);
    else launch_split_tiles<2, kW4MaxGroups>(a, st);
    return;
  }
  if (ngrp <= 8) launch_tiles<BM, 3, 8>(a, st);
  else if (ngrp <= 32) launch_tiles<BM, 3, 32>(a, st);
  else launch_tiles<BM, BM == 128 ? 2 : 3, kW4MaxGroups>(a, st);
}

}  // namespace

size_t fwd_w4_split_floats(int M, int N, int K) {
  int sp, nks;
  w4_split_plan(M, N, K, &sp, &nks);
  if (sp == 1) return 0;
  const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((N + 127) / 128);
  return (size_t)sp * tiles * 128 * 128;
}

void launch_gemm_fwd_w4(int M, int N, int K, const uint16_t* x,
                        const uint8_t* packed, const _Float16* scales,
                        const float* t, const float* B, int hd, int r, float s,
                        uint16_t* y, float* pacc, hipStream_t st) {
  W4Args a{};
  a.M = M; a.N = N; a.K = K; a.x = x; a.packed = packed; a.scales = scales;
  a.t = t; a.B = B; a.hd = hd; a.r = r; a.s = s; a.y = y;
  a.splits = 1;
  if (pacc != nullptr) {
    w4_split_plan(M, N, K, &a.splits, &a.nks);
    a.pacc = pacc;
  }
  const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= kCUs || a.splits > 1) launch_groups<128>(a, st);
  else launch_groups<64>(a, st);
}

}  // namespace qlora
