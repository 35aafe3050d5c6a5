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
// output column applies to the whole stage, and a 128 x 128 block needs
// 64 KB of LDS (two per compute unit). Three tiles move global -> LDS
// without registers (ring.hpp): the x rows (bf16, 128-byte rows swizzled by
// 16-byte chunk), the packed codes [BN n][32 bytes], and, once before the
// loop, the block's scales [BN][K / 128] (a contiguous slab of the scale
// array). Once a stage has landed the block converts its codes in one
// cooperative pass, every nibble once: CB [BN n][64 k] = bf16(q sc), stored
// like the x rows. The MFMA loop then reads both operands with plain 16-byte
// LDS reads. The adapter term runs in the epilogue on v_mfma_f32_16x16x4_f32
// (ring.hpp).
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
};

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
template <int BM, int BN, int S, int R, int G>
__global__ __launch_bounds__(256) void fwd_w4_kernel(W4Args a) {
  constexpr int BK = 64;                           // k per stage: half a scale group
  constexpr int ASZ = BM * 128, BSZ = BN * 32, STG = ASZ + BSZ;
  constexpr int AI = BM / 32, BI = BN / 128, LPS = AI + BI;   // DMA per wave per stage
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int CBSZ = BN * 128;
  static_assert(BN == 128, "code rows of 32 bytes: 32 rows per DMA instruction, one per wave");
  // after the loop the ring and the converted-code buffer hold the epilogue
  // operands, then one output staging strip per wave
  constexpr int EPB = (EpiOps<BM, BN, R, false>::kFloats * 4 + 15) / 16 * 16;
  static_assert(EPB + 4 * epi_strip_bytes<uint16_t, FN>() <= S * STG + CBSZ, "epilogue fits");
  const int K = a.K, M = a.M, N = a.N;
  const int ngrp = K / 128;
  static_assert(BN * G * 2 % 1024 == 0, "the scale slab takes whole 1 KB DMA instructions");
  // scales of the block's columns: [BN][ngrp] fp16, ngrp <= G
  __shared__ __attribute__((aligned(1024))) int8_t lds[S * STG + CBSZ + BN * G * 2];
  int8_t* ring = lds;
  int8_t* CB = lds + S * STG;
  const _Float16* SC = reinterpret_cast<const _Float16*>(lds + S * STG + CBSZ);

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int wm = wid >> 1, wn = wid & 1;
  int mt, nt;
  xcd_tile((int)blockIdx.x, (a.M + BM - 1) / BM, a.tiles_x, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk = 2 * ngrp;

  EpiOps<BM, BN, R, false> ep;
  ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, nullptr, nullptr);

  // the block's scale slab: rows n0 .. n0 + BN of [N][ngrp], contiguous
  {
    const int bytes = BN * ngrp * 2;                // multiple of 16 (ngrp >= 1, BN = 128)
    const int8_t* src0 = reinterpret_cast<const int8_t*>(a.scales) + (long)n0 * ngrp * 2;
    const long valid = ((long)N - n0) * ngrp * 2;    // bytes that exist past src0
    for (int o = wid * 1024; o < bytes; o += 4096) {
      const int e = o + lane * 16;
      const int8_t* src = (e < bytes && e < valid) ? src0 + e : zero_chunk(lane);
      lds_dma16(src, lds + S * STG + CBSZ + o);
    }
  }
  // Loads from a wave-wide base (the stage's first k) plus a fixed 32-bit
  // lane offset: x as 128-byte rows swizzled by 16-byte chunk, 8 rows per
  // instruction; the codes as 32-byte rows, 32 per instruction (lanes 2 i and
  // 2 i + 1 take the two halves of row i, read back in that order). Rows past
  // M repeat row M - 1 and weight rows past N repeat row N - 1: their products
  // land only in outputs that are never stored.
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
    if (st < nk) issue(st, st);
  // The scale slab went out before stage 0 (its per-wave instruction count
  // may differ): loads complete in issue order, so every wave's share has
  // landed once its stage 0 has, and the first barrier covers all waves.

  const int crow = tid >> 1, chalf = tid & 1;        // conversion: row n, 32 k half
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_stages<LPS, 0, S - 2>(nk - 1 - kt);
    __builtin_amdgcn_s_barrier();                    // stage kt landed; CB free
    if (kt + S - 1 < nk) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;

    // CB[n][k] = bf16(q[n][k] sc[n][kt / 2]) for row crow, k in [32 chalf, 32 chalf + 32)
    {
      const float sc = (float)SC[crow * ngrp + (kt >> 1)];
      const u32x4 w = *reinterpret_cast<const u32x4*>(Bs + crow * 32 + chalf * 16);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        *reinterpret_cast<u32x4*>(CB + swz128(crow, 4 * chalf + d)) = nibbles_bf16(w[d], sc);
    }
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    __builtin_amdgcn_s_barrier();                    // CB visible

#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + swz128(wm * (BM / 2) + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(CB + swz128(wn * (BN / 2) + j * 16 + (lane & 15), c));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  float* E = reinterpret_cast<float*>(ring);
  __syncthreads();
  ep.store(E, M, N, m0, n0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, BN, R, false>(acc, E, M, N, m0, n0, wm * (BM / 2), wn * (BN / 2), a.s, a.y,
                                     ring + EPB + wid * epi_strip_bytes<uint16_t, FN>());
}

template <int BM, int S, int G>
void launch_tiles(W4Args a, hipStream_t st) {
  constexpr int BN = 128;
  a.tiles_x = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM)));
  if (a.r <= 4) fwd_w4_kernel<BM, BN, S, 4, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_w4_kernel<BM, BN, S, 8, G><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_w4_kernel<BM, BN, S, 16, G><<<grid, 256, 0, st>>>(a);
  else fwd_w4_kernel<BM, BN, S, 32, G><<<grid, 256, 0, st>>>(a);
}

template <int BM, int S>
void launch_groups(const W4Args& a, hipStream_t st) {
  const int ngrp = a.K / 128;                      // validated: <= kW4MaxGroups
  if (ngrp <= 8) launch_tiles<BM, S, 8>(a, st);
  else if (ngrp <= 32) launch_tiles<BM, S, 32>(a, st);
  else launch_tiles<BM, S, kW4MaxGroups>(a, st);
}

}  // namespace

void launch_gemm_fwd_w4(int M, int N, int K, const uint16_t* x,
                        const uint8_t* packed, const _Float16* scales,
                        const float* t, const float* B, int hd, int r, float s,
                        uint16_t* y, hipStream_t st) {
  W4Args a{};
  a.M = M; a.N = N; a.K = K; a.x = x; a.packed = packed; a.scales = scales;
  a.t = t; a.B = B; a.hd = hd; a.r = r; a.s = s; a.y = y;
  const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= kCUs) launch_groups<128, 2>(a, st);
  else launch_groups<64, 2>(a, st);
}

}  // namespace qlora
