// Backward of the frozen-weight layer (int8, or 4-bit with fp16 group
// scales) with its adapter, in one launch (plus the fixed-order combine of
// the adapter-gradient partial sums):
//
//   u  = dy B^T                                  [M, r]
//   dx = dy deq(W)^T + s u A^T,  deq(W)[k, n] = q[n, k] sw[n]
//                                 (4-bit: q[n, k] sc[n, k / 128])
//   dB = s t^T dy                                [r, N]
//   dA = s x^T u                                 [K, r]
//
// ("Parameter-efficient fine-tuning of GPT-2 with LoRA", "LoRA equation" and
// "Why does LoRA reduce memory footprint?": gradients only for the adapter;
// the quantizer of x is passed straight through; "How to fine-tune the 4-bit
// model?": the transposed quantized product.)
//
// A block owns BM rows x BN columns of dx and walks the whole contraction
// over n in stages of 64, so on the way it sees every dy value of its rows.
// The stage ring (ring.hpp) carries three tiles per stage, all moved
// global -> LDS without registers: the dy rows (swizzled 128-byte rows), the
// codes [64 n][BN k] in their stored layout (chunk-swizzled), and an aux tile
// with the stage's weight scales and the adapter's B columns for those n.
// Once a stage has landed it is converted in one cooperative pass (every code
// read and widened once, not once per wave that uses it):
//   * CB [BN k][64 n] = bf16(deq(W)[k, n]), the transposed dequantized
//     weight, as swizzled 128-byte rows (4-bit: the nibbles unpacked and
//     scaled by their group's fp16 scale, one 128-wide group per block);
//   * BU [3 R j][64 n]: B[j, n] as three bf16 parts, hi | mid | lo
//     (pk_bf16_split3 below), so that the rank-r products keep float32
//     accuracy.
// Then per 32 n, on v_mfma_f32_16x16x32_bf16:
//   * dx += dy CB^T;
//   * u  += dy BU^T, one MFMA per row block and column block of BU (the two
//     column waves of a row split the row blocks);
//   * dB: the block whose column index equals the stage index modulo the
//     column-tile count adds t^T dy over its rows for the stage's 64 n
//     (dy^T through transposing LDS reads, t as three bf16 parts), giving
//     one partial per row block.
// After the loop u goes to LDS and the dA partial x^T u over the block's
// rows is taken from an x tile loaded into LDS: on the 64-row tiles a
// float32 vector-ALU sum in row order (beside the consumers' epilogue), on
// the 128-row tiles bf16 MFMAs with u split into hi, mid and lo parts like
// B and t; the dx epilogue adds s u A^T on v_mfma_f32_16x16x4_f32. The
// partials of dA and dB are added in row-block order by a small second
// launch. No atomics: results are bitwise reproducible.
//
// Outlier-compensated int8 weights (keras-llm-light README, "Simplified
// Int8Variable quantization"; format in outlier.hpp) take the 64-row tiles:
// the producers widen each code v - 128 to bf16(c (v - 128) + b') with the
// weight's one grid step c and code-0 value b', and then write every outlier
// of the stage over its place in the converted tile as bf16(value) -- the
// weight the pages reconstruct before the layer runs, built in LDS one stage
// at a time. Producer wave w converts k in [k0 + 16 w, k0 + 16 w + 16), which
// is one backward cell of the outlier lists (64 n x 16 k); it reads its
// cell's outliers one stage ahead, one per lane, and each lane writes its
// outlier after the wave's own conversion stores (in program order, so the
// outlier wins).
//
// Two block shapes share this scheme:
//   * 64-row tiles, 512 threads in two roles (producer waves load and
//     convert stage kt + 1 while consumer waves multiply stage kt), for
//     shapes with at most two such tiles per compute unit;
//   * 128 x 128 (or, for int8 grids of fewer 128 x 128 tiles than compute
//     units, 128 x 64) tiles, 256 threads that all do every step, for larger
//     shapes, where sharing each loaded tile among more outputs matters more
//     than overlapping the steps.
// Few 128 x 128 tiles over a long contraction split it: up to 8 blocks per
// tile each take a range of n and leave their float32 accumulators and
// partial u in the workspace, and a second launch adds them in split order
// and does what the one-pass kernel does after its loop (u, the dA partial,
// the epilogue).
#include "launch.hpp"
#include "outlier.hpp"
#include "ring.hpp"

namespace qlora {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWideSplits = 8;   // contraction splits of the 128 x 128 backward

struct BwdArgs {
  int M, K, N;
  const uint16_t* dy;      // [M, N] bf16
  const int8_t* codes;     // int8 [N, K], or packed 4-bit [N, K / 2]
  const float* sw;         // int8: channel scales [N]
  const uint16_t* sc4;     // 4-bit: fp16 group scales [N, K / 128] (bit patterns)
  const float* B;          // [r, N], or [heads, r, hd]
  int hd;                  // head width of B (N: one head)
  const float* A;          // [K, r]
  const float* t;          // [M, r]
  const uint16_t* x;       // [M, K] bf16
  int r;
  float s;
  uint16_t* dx;            // [M, K] bf16
  float* partA;            // [row blocks, r, K]
  float* partB;            // [row blocks, r, N]
  // outlier-compensated weights
  const W8OHeader* w8o;    // grid step and code-0 value
  const int* bptr;         // backward cells, outlier.hpp
  const u32x2* bent;
  int kg;                  // 16-row k groups
  int tiles_x;
  // split contraction (128 x 128 tiles): the partial products in the
  // accumulator layout, the partial u, the split count and stages per split
  float* pdx;              // [splits, tiles, 4 waves, 16 fragments, 64 lanes] float4
  float* pu;               // [splits, M, r]
  int splits, nks;
};

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two float32 values each as a sum of three bf16 values, v = hi + mid + lo:
// hi is the bf16 nearest to v, mid the bf16 nearest to the remainder
// v - hi, lo the bf16 nearest to v - hi - mid (both remainders exact in
// float32). Products with a bf16 operand on the matrix cores then carry v to
// float32 precision (relative error at most 2^-24) instead of 8 significant
// bits, which keeps the float32 adapter's gradients float32-accurate: B (for
// u = dy B^T) and t (for dB = s t^T dy) enter their products as hi, mid and
// lo columns of one operand. A non-finite hi (v infinite or NaN, or past the
// bf16 range) takes mid = lo = 0, so hi alone carries the infinity or NaN.
// Returns the packed hi pair; the mid and lo pairs go to mid2 and lo2.
__device__ __forceinline__ uint32_t pk_bf16_split3(float a, float b, uint32_t& mid2, uint32_t& lo2) {
  const uint32_t h = pk_bf16(a, b);
  const bool fa = (h & 0x7f80u) != 0x7f80u, fb = (h & 0x7f800000u) != 0x7f800000u;
  const float ra = fa ? a - __uint_as_float(h << 16) : 0.f;
  const float rb = fb ? b - __uint_as_float(h & 0xffff0000u) : 0.f;
  mid2 = pk_bf16(ra, rb);
  lo2 = pk_bf16(ra - __uint_as_float(mid2 << 16), rb - __uint_as_float(mid2 & 0xffff0000u));
  return h;
}

// The rank-r products u = dy B^T and dB^T = dy^T t run with 3R operand
// columns: j in [0, R) the hi parts, [R, 2R) the mid parts, [2R, 3R) the lo
// parts. The sum for rank j (j = cb * 16 + lane % 16 < R) of its columns j,
// j + R, j + 2R of the accumulators (column c at block c / 16, lane c % 16 of
// the 16-lane group): R = 4 and 8 put some of them in other lanes of the
// group, read through a lane permute that every lane executes; for R >= 16
// all three are the same lane of blocks cb, cb + R / 16, cb + R / 8.
template <int R, int UCB>
__device__ __forceinline__ float split3_sum(const f32x4 (&v)[UCB], int cb, int ii, int lane) {
  if constexpr (R == 4) {
    static_assert(UCB == 1, "12 columns in one block");
    const int g = lane & ~15;
    return v[0][ii] + __shfl(v[0][ii], g | ((lane + 4) & 15)) + __shfl(v[0][ii], g | ((lane + 8) & 15));
  } else if constexpr (R == 8) {
    static_assert(UCB == 2, "24 columns in two blocks");
    return v[0][ii] + __shfl(v[0][ii], (lane & ~15) | ((lane + 8) & 15)) + v[1][ii];
  } else {
    static_assert(R % 16 == 0 && UCB == 3 * R / 16, "whole blocks per part");
    return v[cb][ii] + v[cb + R / 16][ii] + v[cb + R / 8][ii];
  }
}

// NR transposing LDS reads (ds_read_b64_tr_b16) issued together and completed
// in the same asm block. Written as asm because the builtin form makes the
// compiler wait for every direct-to-LDS load in flight (the ring's later
// stages included) before each read.
template <int NR>
__device__ __forceinline__ void tr16_reads(const uint32_t (&addr)[NR], uint64_t (&out)[NR]) {
  static_assert(NR == 4 || NR == 8, "4 or 8 reads");
  if constexpr (NR == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]),
          "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]),
          "v"(addr[4]), "v"(addr[5]), "v"(addr[6]), "v"(addr[7])
        : "memory");
  }
}

// The eight codes of a packed 4-bit word (nibble e = k offset e, two's
// complement) times sc: w ^ 0x88888888 turns each code q into q + 8 in
// [0, 15], two masks spread the nibbles over bytes (v_cvt_f32_ubyte takes a
// byte in one instruction), and fma(q + 8, sc, -8 sc) rounds q sc exactly
// once, as q * sc would.
__device__ __forceinline__ void nibble_vals(uint32_t w, float sc, float (&v)[8]) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0f0f0f0fu, hi = (u >> 4) & 0x0f0f0f0fu;   // even, odd e
  const float nsc = -8.f * sc;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = __builtin_fmaf((float)((lo >> (8 * b)) & 0xffu), sc, nsc);
    v[2 * b + 1] = __builtin_fmaf((float)((hi >> (8 * b)) & 0xffu), sc, nsc);
  }
}

// a0 or a1 by a wave-uniform flag, as selects rather than a branch (the u
// products take the odd or even row blocks of A by the wave's column half)
__device__ __forceinline__ bf16x8 pick_frag(const bf16x8& a0, const bf16x8& a1, bool second) {
  const u32x4 x = __builtin_bit_cast(u32x4, a0), y = __builtin_bit_cast(u32x4, a1);
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = second ? y[e] : x[e];
  return __builtin_bit_cast(bf16x8, r);
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Chunk swizzle of a code tile with RB-byte rows (RB = 64 or 128).
template <int RB>
__device__ __forceinline__ int code_swz(int row) {
  return (row >> (RB == 64 ? 2 : 1)) & (RB / 16 - 1);
}

// dA partial over a block's rows, in row order:
//   da[jj] = sum over m < rows of x[m][kl] U[m][jb + TPK jj]
// with x the block's bf16 tile [BM][BN] (swizzled 128-byte row halves, as
// the x tile loads lay it out) and U = E [BM][R]. The wave's 64 lanes hold
// 64 consecutive columns of one row half (lane = kl % 64). The tile is read
// four rows at a time through transposing reads: in each 16-lane group,
// lane 4 i + p fetches the 4 columns at 16 g + 4 p of row i, and lane q
// receives column 16 g + q of the four rows.
template <int BM, int BN, int R, int TPK, int JPT>
__device__ __forceinline__ void da_partial(const int8_t* Xs, const float* E, int kl, int jb,
                                           int rows, float (&da)[JPT]) {
  constexpr int RH = BN / 64;
  const int lane = threadIdx.x & 63, g = lane >> 4, q = lane & 15, h = kl / 64;
  auto batch = [&](int b0, bool check) {            // rows [b0, b0 + 16)
    uint32_t ad[4];
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int hrow = (b0 + 4 * u + (q >> 2)) * RH + h;
      ad[u] = lds_addr(Xs + swz128(hrow, 2 * g + ((q & 3) >> 1)) + 8 * (q & 1));
    }
    tr16_reads<4>(ad, v);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = b0 + 4 * u + i;
        if (check && m >= rows) continue;            // uniform
        const float xv = __uint_as_float((uint32_t)(v[u] >> (16 * i)) << 16);
#pragma unroll
        for (int jj = 0; jj < JPT; ++jj) da[jj] = __builtin_fmaf(xv, E[m * R + jb + TPK * jj], da[jj]);
      }
  };
  int b0 = 0;
  for (; b0 + 16 <= rows; b0 += 16) batch(b0, false);
  if (b0 < rows) batch(b0, true);
}

// W4: 4-bit weights (two codes per byte, fp16 scale per 128 k); else int8.
// S: ring slots (at least 3: stage kt is multiplied while stage kt + 1 is
// converted and the later stages are in flight).
//
// 512 threads in two roles. Waves 0-3 (consumers) own the accumulators and
// run the products; waves 4-7 (producers) issue every direct-to-LDS load and
// convert the codes. In iteration kt the consumers multiply stage kt while
// the producers refill the ring with stage kt + S - 1 and convert stage
// kt + 1 into the other buffer, so a compute unit overlaps the matrix work
// of one wave with the vector work of the other on each SIMD. One barrier
// per stage hands the buffers over.
// BRES (int8 weights of one head, N <= kBresN): the channel scales sw [N]
// and B [R][N] stay in LDS for the whole kernel, loaded once before the
// loop, so that a stage's loads are only its dy and code rows.
constexpr int kBresN = 1024;

template <bool W4, int BM, int BN, int S, int R, bool AFF = false, bool BRES = false>
__global__ __launch_bounds__(512) void bwd_pc_kernel(BwdArgs a) {
  constexpr int KC = 64;                              // n per stage
  constexpr int RB = W4 ? BN / 2 : BN;                // code bytes per row of n
  static_assert(!AFF || (!W4 && BN == 64 && KC == kW8OBwdCellN), "affine: int8, 64 x 64 cells");
  static_assert(!BRES || (!W4 && !AFF), "resident scales and B: plain int8 weights");
  // aux tile: a header with the stage's weight scales (int8: sw[n], 64
  // floats; 4-bit: for each n the 16-byte chunk of the scale array that holds
  // sc[n][k0 / 128]; affine weights: none), then the B columns [R][64] float
  // (none with BRES)
  constexpr int HDR = AFF ? 0 : W4 ? 1024 : 256;
  constexpr int AUXI = BRES ? 0 : (HDR + R * 256 + 4095) / 4096;  // aux DMA instructions per producer wave
  constexpr int BRSZ = BRES ? (1 + R) * kBresN * 4 : 0;           // resident sw [kBresN] | B [R][kBresN]
  constexpr int ASZ = BM * 128, BSZ = KC * RB, XSZ = 4 * AUXI * 1024;
  constexpr int STG = ASZ + BSZ + XSZ;
  // per producer wave and stage: dy rows, code rows, aux
  constexpr int AI = BM / 32, BI = RB / 64, LPS = AI + BI + AUXI;
  constexpr int FM = BM / 32, FN = BN / 32;
  static_assert(FM % 2 == 0, "the u products pair the 16-row blocks by column half");
  constexpr int RPI = 1024 / RB, CPR = RB / 16;
  static_assert(RB == 64 || RB == 128, "code rows of 64 or 128 bytes");
  static_assert(S >= 3, "stage kt + 1 is resident while stage kt is used");
  static_assert(!W4 || BN == 128, "4-bit: one 128-wide k group per block");
  constexpr int UCB = (3 * R + 15) / 16;              // operand column blocks of 16: B (t) hi | mid | lo
  constexpr int RCB = (R + 15) / 16;                  // column blocks of the ranks
  constexpr bool XPRE = BM * BN * 2 <= 8192;          // x tile kept outside the ring
  constexpr int CBSZ = BN * 128;                      // converted codes [BN][64] bf16
  constexpr int BUSZ = UCB * 16 * 128;                // converted B [16 UCB][64] bf16: hi | mid | lo
  constexpr int TSZ = BM * R * 4;                     // t tile (pitch r)
  constexpr int XTSZ = BM * BN * 2;
  constexpr int AQSZ = BN * R * 4;                    // the block's rows of A [BN][r]
  constexpr int EFL = (BM + BN) * R;                  // epilogue floats: U [BM][R], A^T [R][BN]
  static_assert(EFL * 4 + (XPRE ? 0 : XTSZ) <= S * STG, "epilogue and x tile fit in the ring");
  // One LDS array for everything: with a second __shared__ object the
  // compiler can no longer tell that the ring's reads do not wait on the
  // direct-to-LDS loads still in flight, and waits for all of them.
  // Converted codes and B are double-buffered: buffer kt % 2 feeds the
  // products of stage kt while stage kt + 1 is converted into the other.
  // the dB operand, t as bf16 hi, mid and lo columns in the MFMA operand
  // layout [UCB][BM / 32][64 lanes][16 B], built once by the consumers
  constexpr int TFSZ = UCB * (BM / 32) * 1024;
  __shared__ __attribute__((aligned(1024))) int8_t ring[S * STG + 2 * CBSZ + 2 * BUSZ + TSZ + AQSZ + TFSZ + (XPRE ? XTSZ : 0) + BRSZ];
  int8_t* CB0 = ring + S * STG;
  int8_t* BU0 = CB0 + 2 * CBSZ;
  float* Ts = reinterpret_cast<float*>(BU0 + 2 * BUSZ);                        // [BM][r]
  const float* Aq = reinterpret_cast<const float*>(BU0 + 2 * BUSZ + TSZ);    // [BN][r]
  int8_t* TF = BU0 + 2 * BUSZ + TSZ + AQSZ;                                    // t operand
  int8_t* Xs = XPRE ? TF + TFSZ : ring + EFL * 4;                              // [BM][BN] bf16
  float* BRs = reinterpret_cast<float*>(TF + TFSZ + (XPRE ? XTSZ : 0));        // BRES: sw | B

  const int lane = threadIdx.x & 63, wid = wave_id();
  const bool producer = wid >= 4;
  const int pw = wid - 4;                             // producer wave 0..3
  const int ptid = (int)threadIdx.x - 256;            // producer thread 0..255
  const int ctid = threadIdx.x;                       // consumer thread 0..255
  const int wm = (wid >> 1) & 1, wn = wid & 1;        // consumer wave position
  int mt, kt_blk;
  xcd_tile((int)blockIdx.x, (a.M + BM - 1) / BM, a.tiles_x, mt, kt_blk);
  const int m0 = mt * BM, k0 = kt_blk * BN;
  const int M = a.M, K = a.K, N = a.N, r = a.r;
  const int nk = (N + KC - 1) / KC;
  const int G = K / 128;                              // 4-bit: scale groups per row

  // consumers: t rows of the block (for dB), then A^T of the block's columns
  // (for the epilogue); masks are applied when stored
  constexpr int NT = (BM * R + 255) / 256;
  float tv[NT];
  if (!producer) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = ctid + 256 * i, row = e / R, j = e % R, gm = m0 + row;
      tv[i] = a.t[(long)(gm < M ? gm : M - 1) * r + (j < r ? j : r - 1)];
    }
  }

  // producers: x tile [BM][BN] bf16 as swizzled 128-byte rows (64 columns
  // per row half)
  auto issue_x = [&]() {
    constexpr int RH = BN / 64;                        // 128-byte halves per row
#pragma unroll
    for (int i = 0; i < BM * RH / 32; ++i) {
      const int rb = (pw * (BM * RH / 32) + i) * 8, hrow = rb + (lane >> 3);
      const int row = hrow / RH, half = hrow % RH;
      const int c = (lane & 7) ^ ((hrow >> 1) & 7);
      const int gm = m0 + row, gk = k0 + half * 64 + c * 8;
      const void* src = gk < K ? (const void*)(a.x + (long)(gm < M ? gm : M - 1) * K + gk)
                               : (const void*)zero_chunk(lane);
      lds_dma16(src, Xs + rb * 128);
    }
  };

  // Producers' per-lane sources of the stage loads at stage 0; stage kt
  // moves each by kt * 64 n. Lanes whose chunk is outside the operand point
  // at the zero page and do not move. Only a ragged last stage needs the n
  // bound checked.
  const int8_t* srcA[AI];
  int nA[AI];                                          // first n of the lane's chunk
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = pw * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    nA[i] = c * 8;
    srcA[i] = reinterpret_cast<const int8_t*>(a.dy + (long)(gm < M ? gm : M - 1) * N + c * 8);
  }
  const long crs = W4 ? K / 2 : K;                    // code bytes per row in memory
  const int8_t* srcB[BI];
  int nB[BI];
  bool okB[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (pw * BI + i) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ code_swz<RB>(row), gk = (W4 ? k0 / 2 : k0) + c * 16;
    nB[i] = row;
    okB[i] = gk < crs;
    srcB[i] = okB[i] ? a.codes + (long)row * crs + gk : zero_chunk(lane);
  }
  // the dy and code loads as 32-bit offsets from a base shared by the wave
  // (the stage's first n), for every stage but a ragged last one; a code
  // chunk past the row's K bytes reads the row's last chunk instead of
  // zeros, which only reaches output columns past K (never stored)
  uint32_t voA[AI], voB[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = pw * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    voA[i] = (uint32_t)(((long)(gm < M ? gm : M - 1) * N + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (pw * BI + i) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ code_swz<RB>(row), gk = (W4 ? k0 / 2 : k0) + c * 16;
    voB[i] = (uint32_t)((long)row * crs + (gk < crs ? gk : crs - 16));
  }
  // aux chunk ci of the tile: header chunks first, then B [j][64 n] in
  // 4-float chunks; a header source moves by adv bytes per n of the stage, a
  // B source (adv 0) by the stage's offset in B (a stage of 64 n lies inside
  // one head: the head width is a multiple of 64)
  constexpr int AUXA = AUXI > 0 ? AUXI : 1;         // (array extent: none used when AUXI = 0)
  const int8_t* srcX[AUXA];
  int nX[AUXA], advX[AUXA];
  bool okX[AUXA];
#pragma unroll
  for (int i = 0; i < AUXI; ++i) {
    const int ci = (pw * AUXI + i) * 64 + lane;
    if (ci < HDR / 16) {
      if constexpr (W4) {
        // n = ci: the aligned 16 bytes around sc[n][k0 / 128]
        const long byte = 2L * ((long)ci * G + k0 / 128);
        nX[i] = ci;
        advX[i] = 2 * G;
        okX[i] = true;
        srcX[i] = reinterpret_cast<const int8_t*>(a.sc4) + (byte & ~15L);
      } else {
        nX[i] = 4 * ci;
        advX[i] = 4;
        okX[i] = true;
        srcX[i] = reinterpret_cast<const int8_t*>(a.sw + 4 * ci);
      }
    } else {
      const int e = (ci - HDR / 16) * 4, j = e / 64, nn = e % 64;
      nX[i] = nn;
      advX[i] = 0;
      okX[i] = j < r;
      srcX[i] = j < r ? reinterpret_cast<const int8_t*>(a.B + (long)j * a.hd + nn) : zero_chunk(lane);
    }
  }
  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
    const int nb = kt * KC;
    const bool tail = nb + KC > N;
    // (affine weights keep one branch-free form: their loop waits for loads
    // by count, and a branch here makes the compiler wait for all of them)
    if (!AFF && !tail) {
      const int8_t* dyb = reinterpret_cast<const int8_t*>(a.dy) + 2L * nb;
      const int8_t* cdb = a.codes + (long)nb * crs;
#pragma unroll
      for (int i = 0; i < AI; ++i) lds_dma16(dyb + voA[i], base + (pw * (BM / 4) + i * 8) * 128);
#pragma unroll
      for (int i = 0; i < BI; ++i) lds_dma16(cdb + voB[i], base + ASZ + (pw * BI + i) * RPI * RB);
    } else {
#pragma unroll
      for (int i = 0; i < AI; ++i) {
        const int8_t* src = srcA[i] + 2L * nb;
        if (tail && nb + nA[i] >= N) src = zero_chunk(lane);
        lds_dma16(src, base + (pw * (BM / 4) + i * 8) * 128);
      }
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int8_t* src = okB[i] ? srcB[i] + (long)nb * crs : srcB[i];
        if (tail && nb + nB[i] >= N) src = zero_chunk(lane);
        lds_dma16(src, base + ASZ + (pw * BI + i) * RPI * RB);
      }
    }
    const long boff = 4 * head_index(0, nb, r, a.hd);   // bytes: B column nb, rank 0
#pragma unroll
    for (int i = 0; i < AUXI; ++i) {
      const int8_t* src = okX[i] ? srcX[i] + (advX[i] ? (long)advX[i] * nb : boff) : srcX[i];
      if (tail && nb + nX[i] >= N) src = zero_chunk(lane);
      lds_dma16(src, base + ASZ + BSZ + (pw * AUXI + i) * 1024);
    }
  };

  // producers' cooperative conversion: thread -> n quad nq, k quads kq0 + 16 h
  const int nq = ptid & 15, kq0 = (ptid >> 4) & 15;
  // 4-bit: byte offset of sc[n][k0 / 128] inside the header chunk of n, for
  // the thread's 4 n
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) soff[i] = 16 * (4 * nq + i) + ((2 * ((4 * nq + i) * G + k0 / 128)) & 15);

  // Conversion of the stage in ring slot `slot` into buffer `buf`:
  //   CB[k][n] = bf16(q[n][k] sw[n]) for the 4 n of nq and 4 k per quad
  //   (4-bit: bf16(q[n][k] sc[n][k0 / 128]) for the 4 n of nq and 8 k);
  //   BU[j][n] = bf16(B[j][n]), 2 n per entry.
  constexpr int NBU = (R * 32 + 255) / 256;
  float cstep = 0.f, cbias = 0.f;
  if constexpr (AFF) {
    cstep = a.w8o->scale;
    cbias = a.w8o->bias_q;
  }
  // affine weights: outliers (k, n, value) of this producer wave's cell in a
  // stage, one per lane from the cell's first entry, and the cell's range
  // (past K the range is empty, lo == hi)
  struct Outl {
    u32x2 e;
    int lo, hi;
  };
  const int kgw = k0 / kW8OBwdCellK + (pw & 3);       // the wave's 16-row k group
  const int kgl = kgw < a.kg ? kgw : a.kg, kgh = kgw + 1 < a.kg ? kgw + 1 : a.kg;
  CellRanges cr;
  auto outl_range = [&](int st, Outl& o) { cr.get(st, o.lo, o.hi); };
  auto outl_load = [&](Outl& o) { o.e = a.bent[o.lo + lane]; };
  // write the lane's outlier over the converted tile
  auto outl_put = [&](int8_t* CB, uint32_t kn, uint32_t vbits) {
    const int kl = (int)(kn >> 6) - k0, nl = (int)(kn & 63), nqo = nl >> 2;
    if ((unsigned)kl < (unsigned)BN)
      *reinterpret_cast<uint16_t*>(CB + swz128(kl, nqo >> 1) + (nqo & 1) * 8 + 2 * (nl & 3)) =
          (uint16_t)f32_to_bf16(__uint_as_float(vbits));
  };
  auto convert = [&](int slot, int buf, const Outl& ol, int nb, auto&& hook) {
    const int8_t* Bs = ring + slot * STG + ASZ;
    const int8_t* Xb = Bs + BSZ;
    // the stage's sw [64] and B [R] columns: the aux tile, or (BRES) the
    // resident copies at the stage's first n
    const float* Xa = BRES ? BRs + nb : reinterpret_cast<const float*>(Xb);
    constexpr int BP = BRES ? kBresN : 64;           // pitch of B's rows
    constexpr int BO = BRES ? kBresN : HDR / 4;      // offset of B's first row
    int8_t* CB = CB0 + buf * CBSZ;
    int8_t* BU = BU0 + buf * BUSZ;
    hook();
    f32x2 bq[NBU];
#pragma unroll
    for (int q = 0; q < NBU; ++q) {
      const int e = ptid + 256 * q;
      const int j = e >> 5, p = e & 31;
      if (e < R * 32) bq[q] = *reinterpret_cast<const f32x2*>(Xa + BO + BP * j + 2 * p);
    }
    if constexpr (W4) {
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = (float)*reinterpret_cast<const _Float16*>(Xb + soff[i]);
      const int kq8 = kq0;                           // k in [8 kq8, 8 kq8 + 8)
      uint32_t raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * nq + i;
        raw[i] = *reinterpret_cast<const uint32_t*>(Bs + n * RB + (((kq8 >> 2) ^ code_swz<RB>(n)) << 4) + (kq8 & 3) * 4);
      }
      float v[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) nibble_vals(raw[i], sc[i], v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x2*>(CB + swz128(8 * kq8 + e, nq >> 1) + (nq & 1) * 8) =
            u32x2{pk_bf16(v[0][e], v[1][e]), pk_bf16(v[2][e], v[3][e])};
    } else {
      f32x4 swv = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!AFF) swv = *reinterpret_cast<const f32x4*>(Xa + 4 * nq);
#pragma unroll
      for (int h = 0; h < BN / 64; ++h) {
        const int kcol = 4 * (kq0 + 16 * h);
        int raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 4 * nq + i;
          raw[i] = *reinterpret_cast<const int*>(Bs + n * RB + ((((kcol >> 4) ^ code_swz<RB>(n))) << 4) + (kcol & 15));
        }
#pragma unroll
        for (int kk2 = 0; kk2 < 4; ++kk2) {
          float v0, v1, v2, v3;
          if constexpr (AFF) {
            v0 = __builtin_fmaf((float)(int8_t)(raw[0] >> (8 * kk2)), cstep, cbias);
            v1 = __builtin_fmaf((float)(int8_t)(raw[1] >> (8 * kk2)), cstep, cbias);
            v2 = __builtin_fmaf((float)(int8_t)(raw[2] >> (8 * kk2)), cstep, cbias);
            v3 = __builtin_fmaf((float)(int8_t)(raw[3] >> (8 * kk2)), cstep, cbias);
          } else {
            v0 = (float)(int8_t)(raw[0] >> (8 * kk2)) * swv.x;
            v1 = (float)(int8_t)(raw[1] >> (8 * kk2)) * swv.y;
            v2 = (float)(int8_t)(raw[2] >> (8 * kk2)) * swv.z;
            v3 = (float)(int8_t)(raw[3] >> (8 * kk2)) * swv.w;
          }
          *reinterpret_cast<u32x2*>(CB + swz128(kcol + kk2, nq >> 1) + (nq & 1) * 8) =
              u32x2{pk_bf16(v0, v1), pk_bf16(v2, v3)};
        }
      }
      if constexpr (AFF) {
        const int cnt = ol.hi - ol.lo;
        if (lane < cnt) outl_put(CB, ol.e.x, ol.e.y);
        for (int b0 = 64; b0 < cnt; b0 += 64) {      // more than 64 in one cell
          const u32x2 ev = a.bent[ol.lo + b0 + lane];
          if (lane < cnt - b0) outl_put(CB, ev.x, ev.y);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NBU; ++q) {
      const int e = ptid + 256 * q;
      const int j = e >> 5, p = e & 31;
      if (e < R * 32) {
        uint32_t mid2, lo2;
        const uint32_t hi2 = pk_bf16_split3(bq[q].x, bq[q].y, mid2, lo2);
        *reinterpret_cast<uint32_t*>(BU + swz128(j, p >> 2) + (p & 3) * 4) = hi2;
        *reinterpret_cast<uint32_t*>(BU + swz128(R + j, p >> 2) + (p & 3) * 4) = mid2;
        *reinterpret_cast<uint32_t*>(BU + swz128(2 * R + j, p >> 2) + (p & 3) * 4) = lo2;
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 uacc[(FM + 1) / 2][UCB];
#pragma unroll
  for (int i = 0; i < (FM + 1) / 2; ++i)
#pragma unroll
    for (int j = 0; j < UCB; ++j) uacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // affine weights (producers): outliers of the stage converted next (ocur)
  // and the range of the stage after it (onext)
  Outl ocur{};
  if (producer) {
    if constexpr (AFF) cr.init(a.bptr, a.kg, kgl, kgh, nk);
    // the block's rows of A, contiguous in memory: (K - k0 or BN) * r floats
    {
      const int rows = K - k0 < BN ? K - k0 : BN;
      const int bytes = rows * r * 4;                // a multiple of 16
      const int8_t* src0 = reinterpret_cast<const int8_t*>(a.A + (long)k0 * r);
      for (int o = pw * 1024; o < AQSZ; o += 4096) {
        const int e = o + lane * 16;
        lds_dma16(e < bytes ? src0 + e : zero_chunk(lane), const_cast<float*>(Aq) + o / 4);
      }
    }
    if constexpr (XPRE) issue_x();
    if constexpr (BRES) {
      // sw [N] and B [r][N] (rows up to R, columns up to kBresN; zeros past
      // them), 16 bytes per lane, ahead of the stage loads (loads complete in
      // issue order, so they have landed once stage 0 has)
      for (int o = pw * 1024; o < BRSZ; o += 4096) {
        const int e = (o + lane * 16) / 4;             // float index in sw | B
        const int row = e / kBresN, n = e % kBresN;    // row 0: sw; row 1 + j: B[j]
        const float* src = row == 0 ? a.sw + n : a.B + (long)(row - 1) * N + n;
        const bool ok = n < N && (row == 0 || row - 1 < r);
        lds_dma16(ok ? (const void*)src : (const void*)zero_chunk(lane), BRs + o / 4);
      }
    }
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nk) issue(st, st);
    // BU rows past the rank stay zero for good
    for (int e = 3 * R * 32 + ptid; e < UCB * 16 * 32; e += 256) {   // 4-byte pairs
      const int off = swz128(e / 32, (e % 32) >> 2) + (e & 3) * 4;
      *reinterpret_cast<uint32_t*>(BU0 + off) = 0u;
      *reinterpret_cast<uint32_t*>(BU0 + BUSZ + off) = 0u;
    }
    // stage 0 landed (later prologue stages may still be in flight)
    wait_stages<LPS, 0, S - 2>(nk - 1);
  } else {
    // t tile into LDS (pitch r)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = ctid + 256 * i, row = e / R, j = e % R;
      if (e < BM * R && j < r) Ts[row * r + j] = m0 + row < M ? tv[i] : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
  __builtin_amdgcn_s_barrier();
  if (!producer) {
    // the dB operand from the t tile, while the producers convert stage 0:
    // consumer wave w builds fragments f = w, w + 4, ... of the UCB * BM / 32
    // (fragment (cb, c): lane -> column cb * 16 + lane % 16, i.e. part
    // j / R of rank j % R, rows 32 c + 8 (lane / 16) + e)
    for (int f = wid; f < UCB * (BM / 32); f += 4) {
      const int cb = f / (BM / 32), c = f % (BM / 32);
      const int j = cb * 16 + (lane & 15), part = j / R, jr = j - part * R;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 32 * c + 8 * (lane >> 4) + e;
        v[e] = (jr < r && part < 3) ? Ts[m * r + (jr < r ? jr : 0)] : 0.f;
      }
      u32x4 hi, mid, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t me, le;
        hi[e] = pk_bf16_split3(v[2 * e], v[2 * e + 1], me, le);
        mid[e] = me;
        lo[e] = le;
      }
      *reinterpret_cast<u32x4*>(TF + (f * 64 + lane) * 16) = part == 0 ? hi : part == 1 ? mid : lo;
    }
  }
  if (producer) {
    if constexpr (AFF) {
      outl_range(0, ocur);
      outl_load(ocur);
    }
    convert(0, 0, ocur, 0, [] {});
    if constexpr (AFF) {
      // stage 1's outliers are read before the loop queues more loads
      outl_range(nk > 1 ? 1 : 0, ocur);
      outl_load(ocur);
    }
  }

  const int rows_here = M - m0 < BM ? M - m0 : BM;
  // dB operand: t split into bf16 hi, mid and lo columns, lane -> column
  // (lane % 16), rows 32 c + 8 (lane / 16) + e; rebuilt from the t tile in
  // LDS at each of the block's dB stages rather than held in registers

  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // producers: stage kt + 1 landed and buffer kt % 2 written; then every
    // wave is done with stage kt - 1 (its slot and buffer (kt + 1) % 2)
    if (producer) wait_stages<LPS, 0, S - 3>(nk - 2 - kt);
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    __builtin_amdgcn_s_barrier();
    const int pslot = slot == 0 ? S - 1 : slot - 1;  // slot of stage kt - 1 = kt + S - 1
    const int nslot = slot == S - 1 ? 0 : slot + 1;  // slot of stage kt + 1
    if (producer) {
      // affine weights: read stage kt + 2's outliers ahead of this
      // iteration's loads
      Outl o2{};
      if constexpr (AFF) {
        outl_range(kt + 2 < nk ? kt + 2 : nk - 1, o2);
        outl_load(o2);
        __builtin_amdgcn_sched_barrier(0);         // ahead of the stage loads
      }
      // (affine weights: past the last stage the loads read the zero page into
      // the free slot, so that every iteration queues the same loads and the
      // read-ahead registers can be waited for by count)
      if constexpr (AFF) {
        issue(kt + S - 1, pslot);
        if (kt + 1 < nk) convert(nslot, (kt + 1) & 1, ocur, (kt + 1) * KC, [] {});
      } else if (kt + 1 < nk) {
        // the stage loads are queued from inside the conversion, ahead of
        // its first LDS read (measured: about 5% faster on 1024-wide layers
        // than queueing them before the call, the form the affine weights
        // keep)
        const bool more = kt + S - 1 < nk;
        convert(nslot, (kt + 1) & 1, ocur, (kt + 1) * KC, [&] {
          if (more) issue(kt + S - 1, pslot);
        });
      }
      if constexpr (AFF) {
        // the read-ahead outliers were queued before this iteration's stage
        // loads: all but those loads are done
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
        ocur = o2;
      }
    } else {
      const int8_t* As = ring + slot * STG;
      const int8_t* CB = CB0 + (kt & 1) * CBSZ;
      const int8_t* BU = BU0 + (kt & 1) * BUSZ;
      constexpr int KS = KC / 32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int c = kk * 4 + (lane >> 4);
        bf16x8 af[FM], bf[FN], bu[UCB];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(As + swz128(wm * (BM / 2) + i * 16 + (lane & 15), c));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = *reinterpret_cast<const bf16x8*>(CB + swz128(wn * (BN / 2) + j * 16 + (lane & 15), c));
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb)
          bu[cb] = *reinterpret_cast<const bf16x8*>(BU + swz128(cb * 16 + (lane & 15), c));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb)
#pragma unroll
          for (int h = 0; h < FM / 2; ++h)
            uacc[h][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pick_frag(af[2 * h], af[2 * h + 1], wn != 0),
                                                                 bu[cb], uacc[h][cb], 0, 0, 0);
      }
      // dB partial for this stage's 64 n over the block's rows (one block
      // per row block and stage), on the matrix cores: consumer wave w takes
      // n in [16 w, 16 w + 16); dB^T[n][j] = sum_m dy[m][n] t[m][j]. The dy^T
      // operand comes from the dy tile through transposing reads: in each
      // 16-lane group, lanes 4 i + p fetch the 4 n at 16 w + 4 p of row i,
      // and lane q receives n = 16 w + q of rows 0..3.
      if (kt % a.tiles_x == kt_blk) {
        bf16x8 tfr[UCB][BM / 32];
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb)
#pragma unroll
          for (int c = 0; c < BM / 32; ++c)
            tfr[cb][c] = *reinterpret_cast<const bf16x8*>(TF + ((cb * (BM / 32) + c) * 64 + lane) * 16);
        constexpr int NRD = 2 * (BM / 32);
        uint32_t tra[NRD];
        uint64_t trv[NRD];
        const int q = lane & 15, i4 = q >> 2, p4 = q & 3;
#pragma unroll
        for (int c = 0; c < BM / 32; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = 32 * c + 8 * (lane >> 4) + 4 * h + i4;
            const int n = 16 * wid + 4 * p4;
            tra[2 * c + h] = lds_addr(As + swz128(m, n >> 3) + (n & 7) * 2);
          }
        tr16_reads<NRD>(tra, trv);
        f32x4 dbacc[UCB];
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb) dbacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < BM / 32; ++c) {
          const bf16x8 dyT = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)trv[2 * c], (uint32_t)(trv[2 * c] >> 32),
                                                              (uint32_t)trv[2 * c + 1], (uint32_t)(trv[2 * c + 1] >> 32)});
#pragma unroll
          for (int cb = 0; cb < UCB; ++cb)
            dbacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dyT, tfr[cb][c], dbacc[cb], 0, 0, 0);
        }
#pragma unroll
        for (int cb = 0; cb < RCB; ++cb) {
          const int j = cb * 16 + (lane & 15);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float dbv = split3_sum<R, UCB>(dbacc, cb, ii, lane);
            const int gn = kt * KC + 16 * wid + 4 * (lane >> 4) + ii;
            if (j < r && gn < N) a.partB[((long)mt * r + j) * N + gn] = dbv;
          }
        }
      }
    }
    slot = nslot;
  }

  // ---- after the contraction: u to LDS, x tile, then the dA partial
  // (producers) beside the dx epilogue (consumers) ----
  float* E = reinterpret_cast<float*>(ring);             // U [BM][R] | A^T [R][BN]
  __syncthreads();                                        // ring released
  if (producer) {
    if constexpr (!XPRE) issue_x();
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if ((i & 1) != wn) continue;
#pragma unroll
      for (int cb = 0; cb < RCB; ++cb) {
        const int j = cb * 16 + (lane & 15);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float uv = split3_sum<R, UCB>(uacc[i >> 1], cb, ii, lane);
          const int ml = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
          if (j < R) E[ml * R + j] = j < r ? uv : 0.f;
        }
      }
    }
  }
  // A^T of the block's columns into the epilogue layout (from LDS)
  for (int e = threadIdx.x; e < BN * R; e += 512) {
    const int j = e / BN, col = e % BN;
    E[BM * R + e] = (j < r && k0 + col < K) ? Aq[col * r + (j < r ? j : 0)] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  if (producer) {
    // dA partial: thread -> column k = ptid % BN, ranks jb + (256 / BN) jj
    constexpr int TPK = 256 / BN, JPT = R / TPK;
    const int kl = ptid % BN, jb = ptid / BN;
    float da[JPT];
#pragma unroll
    for (int jj = 0; jj < JPT; ++jj) da[jj] = 0.f;
    da_partial<BM, BN, R, TPK, JPT>(Xs, E, kl, jb, rows_here, da);
    if (k0 + kl < K) {
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) {
        const int j = jb + TPK * jj;
        if (j < r) a.partA[((long)mt * r + j) * K + k0 + kl] = da[jj];
      }
    }
  } else {
    // output staging strips in the converted-code buffers, free after the loop
    static_assert(4 * epi_strip_bytes<uint16_t, FN>() <= 2 * CBSZ, "staging strips fit");
    epilogue_lowrank<BM, BN, R, false>(acc, E, M, K, m0, k0, wm * (BM / 2), wn * (BN / 2), a.s, a.dx,
                                       CB0 + wid * epi_strip_bytes<uint16_t, FN>());
  }
}



// Wide tiles (128 x 128, 256 threads): every wave issues its share of the
// stage loads, converts its share of the codes and multiplies, with two
// barriers per stage. At this tile size the dy and code tiles are each shared
// by twice the outputs of a 64-row tile, which halves the load traffic per
// product, and the whole block's registers serve one role.
// W4: 4-bit weights (two codes per byte, fp16 scale per 128 k, carried one
// stage ahead in a register); else int8.
template <bool W4, int BM, int BN, int S, int R, bool AFF = false, bool SPLIT = false>
__global__ __launch_bounds__(256, 2) void bwd_wide_kernel(BwdArgs a) {
  constexpr int KC = 64;                              // n per stage
  constexpr int RB = W4 ? BN / 2 : BN;                // code bytes per row of n
  constexpr int AUXI = ((1 + R) * 256 + 4095) / 4096;  // aux DMA instructions per wave
  constexpr int ASZ = BM * 128, BSZ = KC * RB, XSZ = 4 * AUXI * 1024;
  constexpr int STG = ASZ + BSZ + XSZ;
  // per wave and stage: dy rows, code rows, aux, and (4-bit) one scale load
  constexpr int AI = BM / 32, BI = RB / 64, LPS = AI + BI + AUXI + (W4 ? 1 : 0);
  constexpr int FM = BM / 32, FN = BN / 32;
  static_assert(FM % 2 == 0, "the u products pair the 16-row blocks by column half");
  constexpr int RPI = 1024 / RB, CPR = RB / 16;
  static_assert(RB == 64 || RB == 128, "code rows of 64 or 128 bytes");
  static_assert(!W4 || (BN == 128 && S == 2),
                "4-bit: one 128-wide k group per block; the scales ride one stage ahead in a register");
  static_assert(!AFF || (!W4 && BN == 128 && S == 2 && KC == kW8OBwdCellN),
                "affine: int8, the outliers of stage kt read during stage kt - 1");
  constexpr int UCB = (3 * R + 15) / 16;              // operand column blocks of 16: B (t) hi | mid | lo
  constexpr int RCB = (R + 15) / 16;                  // column blocks of the ranks
  constexpr bool XPRE = BM * BN * 2 <= 8192;          // x tile kept outside the ring
  constexpr int CBSZ = BN * 128;                      // converted codes [BN][64] bf16
  constexpr int BUSZ = UCB * 16 * 128;                // converted B [16 UCB][64] bf16: hi | mid | lo
  // The dB operand, t split into bf16 hi, mid and lo columns in the MFMA
  // operand layout [UCB][BM / 32][64 lanes][16 B], built once per block in
  // LDS where it fits beside two blocks per compute unit and the float32 t
  // tile fits in the converted-code buffer it passes through (TFL); else
  // each dB stage rebuilds it from the t tile.
  constexpr bool TFL = R != 8 && BM * R * 4 <= CBSZ;
  constexpr int TSZ = TFL ? UCB * (BM / 32) * 1024 : BM * R * 4;   // t operand, or t tile (pitch r)
  constexpr int XTSZ = BM * BN * 2;
  constexpr int EFL = (BM + BN) * R;                  // epilogue floats: U [BM][R], A^T [R][BN]
  static_assert(EFL * 4 + (XPRE ? 0 : XTSZ) <= S * STG, "epilogue and x tile fit in the ring");
  // One LDS array for everything: with a second __shared__ object the
  // compiler can no longer tell that the ring's reads do not wait on the
  // direct-to-LDS loads still in flight, and waits for all of them.
  constexpr int SCSZ = W4 ? KC * 4 : 0;               // 4-bit: the stage's scales, float
  __shared__ __attribute__((aligned(1024))) int8_t ring[S * STG + CBSZ + BUSZ + TSZ + SCSZ + (XPRE ? XTSZ : 0)];
  int8_t* CB = ring + S * STG;
  int8_t* BU = CB + CBSZ;
  // t tile [BM][r] float32: its own region, or (TFL) the converted-code
  // buffer until the t operand is built from it
  float* Ts = reinterpret_cast<float*>(TFL ? CB : BU + BUSZ);
  int8_t* TF = BU + BUSZ;                                                      // t operand (TFL)
  float* SCs = reinterpret_cast<float*>(BU + BUSZ + TSZ);                      // [64] (4-bit)
  int8_t* Xs = XPRE ? BU + BUSZ + TSZ + SCSZ : ring + EFL * 4;                 // [BM][BN] bf16

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int wm = wid >> 1, wn = wid & 1;
  const int M = a.M, K = a.K, N = a.N, r = a.r;
  const int nk = (N + KC - 1) / KC;
  // SPLIT: blocks (split, tile), split-major; the dispatcher deals blocks to
  // the eight XCDs in turn, so block b runs as logical block
  // (b % 8) * (blocks / 8) + b / 8 and the blocks of one XCD share one
  // split's n range (its dy columns and code rows stay in that XCD's L2)
  int bid = (int)blockIdx.x, split = 0;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  if constexpr (SPLIT) {
    const int nb = (int)gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    split = bid / tiles;
    bid -= split * tiles;
  }
  int mt, kt_blk;
  if constexpr (SPLIT) {
    mt = bid / a.tiles_x;
    kt_blk = bid % a.tiles_x;
  } else {
    xcd_tile(bid, (M + BM - 1) / BM, a.tiles_x, mt, kt_blk);
  }
  const int m0 = mt * BM, k0 = kt_blk * BN;
  // stages [kt0, kt1) of the contraction; nend bounds the n loaded
  const int kt0 = SPLIT ? split * a.nks : 0;
  const int kt1 = SPLIT ? (kt0 + a.nks < nk ? kt0 + a.nks : nk) : nk;
  const int nend = kt1 * KC < N ? kt1 * KC : N;

  // t rows of the block (for dB), then A^T of the block's columns (for the
  // epilogue); masks are applied when stored
  constexpr int NT = (BM * R + 255) / 256, NQ = (BN * R + 255) / 256;
  float tv[NT], qv[NQ];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = tid + 256 * i, row = e / R, j = e % R, gm = m0 + row;
    tv[i] = a.t[(long)(gm < M ? gm : M - 1) * r + (j < r ? j : r - 1)];
  }
  if constexpr (!SPLIT) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 256 * i, j = e / BN, col = e % BN, gk = k0 + col;
      qv[i] = a.A[(long)(gk < K ? gk : K - 1) * r + (j < r ? j : r - 1)];
    }
  }

  // x tile [BM][BN] bf16 as swizzled 128-byte rows (64 columns per row
  // half), zeros past M and K
  auto issue_x = [&]() {
    constexpr int RH = BN / 64;                        // 128-byte halves per row
#pragma unroll
    for (int i = 0; i < BM * RH / 32; ++i) {
      const int rb = (wid * (BM * RH / 32) + i) * 8, hrow = rb + (lane >> 3);
      const int row = hrow / RH, half = hrow % RH;
      const int c = (lane & 7) ^ ((hrow >> 1) & 7);
      const int gm = m0 + row, gk = k0 + half * 64 + c * 8;
      const void* src = gk < K && gm < M ? (const void*)(a.x + (long)gm * K + gk)
                                         : (const void*)zero_chunk(lane);
      lds_dma16(src, Xs + rb * 128);
    }
  };
  if constexpr (XPRE) issue_x();

  // Per-lane sources of the stage loads at stage 0; stage kt adds kt * 64 n.
  // Lanes whose chunk is outside the operand point at the zero page and do
  // not move. Only a ragged last stage needs the n bound checked.
  const int8_t* srcA[AI];
  int nA[AI];                                          // first n of the lane's chunk
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = wid * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    nA[i] = c * 8;
    srcA[i] = reinterpret_cast<const int8_t*>(a.dy + (long)(gm < M ? gm : M - 1) * N + c * 8);
  }
  const long crs = W4 ? K / 2 : K;                    // code bytes per row in memory
  const int8_t* srcB[BI];
  int nB[BI];
  bool okB[BI];
  // the same loads as 32-bit offsets from a base shared by the wave (dy and
  // the codes at the stage's first n), for every stage but a ragged last
  // one; a code chunk past the row's K bytes reads the row's last chunk
  // instead of zeros, which only reaches output columns past K (never
  // stored)
  uint32_t voA[AI], voB[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = wid * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    voA[i] = (uint32_t)(((long)(gm < M ? gm : M - 1) * N + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (wid * BI + i) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ code_swz<RB>(row), gk = (W4 ? k0 / 2 : k0) + c * 16;
    nB[i] = row;
    okB[i] = gk < crs;
    srcB[i] = okB[i] ? a.codes + (long)row * crs + gk : zero_chunk(lane);
    voB[i] = (uint32_t)((long)row * crs + (okB[i] ? gk : crs - 16));
  }
  // aux chunks: sw (row -1), then B [j][64 n]; sw moves by 4 bytes per n of
  // the stage, B by the stage's offset in B (a stage of 64 n lies inside one
  // head: the head width is a multiple of 64)
  const int8_t* srcX[AUXI];
  int nX[AUXI];
  bool okX[AUXI], isB[AUXI];
#pragma unroll
  for (int i = 0; i < AUXI; ++i) {
    const int e = ((wid * AUXI + i) * 64 + lane) * 4;   // aux float index
    const int j = e / 64 - 1, nn = e % 64;
    nX[i] = nn;
    isB[i] = j >= 0;
    okX[i] = j < r;
    okX[i] = okX[i] && !((W4 || AFF) && j < 0);        // 4-bit, affine: no channel scales
    srcX[i] = j < 0 ? ((W4 || AFF) ? zero_chunk(lane) : reinterpret_cast<const int8_t*>(a.sw + nn))
                    : (j < r ? reinterpret_cast<const int8_t*>(a.B + (long)j * a.hd + nn) : zero_chunk(lane));
  }
  // 4-bit: lane l of wave w loads the scale of n = 16 w + l % 16 of the
  // stage (k group k0 / 128); kept as raw bits until the stage has landed
  uint16_t scr = 0;
  const int scn = 16 * wid + (lane & 15);
  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
    const int nb = kt * KC;
    const bool tail = nb + KC > nend;
    // (affine weights keep one branch-free form: their loop waits for loads
    // by count, and a branch here makes the compiler wait for all of them)
    if (!AFF && !tail) {
      const int8_t* dyb = reinterpret_cast<const int8_t*>(a.dy) + 2L * nb;
      const int8_t* cdb = a.codes + (long)nb * crs;
#pragma unroll
      for (int i = 0; i < AI; ++i) lds_dma16(dyb + voA[i], base + (wid * (BM / 4) + i * 8) * 128);
#pragma unroll
      for (int i = 0; i < BI; ++i) lds_dma16(cdb + voB[i], base + ASZ + (wid * BI + i) * RPI * RB);
    } else {
#pragma unroll
      for (int i = 0; i < AI; ++i) {
        const int8_t* src = srcA[i] + 2L * nb;
        if (tail && nb + nA[i] >= nend) src = zero_chunk(lane);
        lds_dma16(src, base + (wid * (BM / 4) + i * 8) * 128);
      }
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int8_t* src = okB[i] ? srcB[i] + (long)nb * crs : srcB[i];
        if (tail && nb + nB[i] >= nend) src = zero_chunk(lane);
        lds_dma16(src, base + ASZ + (wid * BI + i) * RPI * RB);
      }
    }
    const long boff = 4 * head_index(0, nb, r, a.hd);   // bytes: B column nb, rank 0
#pragma unroll
    for (int i = 0; i < AUXI; ++i) {
      const int8_t* src = okX[i] ? srcX[i] + (isB[i] ? boff : 4L * nb) : srcX[i];
      if (tail && nb + nX[i] >= nend) src = zero_chunk(lane);
      lds_dma16(src, base + ASZ + BSZ + (wid * AUXI + i) * 1024);
    }
    if constexpr (W4) {
      const int n = nb + scn;
      scr = a.sc4[(long)(n < N ? n : N - 1) * (K / 128) + k0 / 128];
    }
  };

  // affine weights: wave w converts k in [k0 + 16 w, +16) and
  // [k0 + 64 + 16 w, +16), two backward cells of the outlier lists; their
  // outliers in a stage, one per lane from each cell's first entry, and the
  // cells' entry ranges
  float cstep = 0.f, cbias = 0.f;
  if constexpr (AFF) {
    cstep = a.w8o->scale;
    cbias = a.w8o->bias_q;
  }
  struct Outl2 {
    u32x2 e[2];
    int lo[2], hi[2];
  };
  const int kgw0 = k0 / kW8OBwdCellK + wid;
  CellRanges cr2[2];
  auto outl_range = [&](int st, Outl2& o) {
#pragma unroll
    for (int h = 0; h < 2; ++h) cr2[h].get(st, o.lo[h], o.hi[h]);
  };
  auto outl_load = [&](Outl2& o) {
#pragma unroll
    for (int h = 0; h < 2; ++h) o.e[h] = a.bent[o.lo[h] + lane];
  };
  auto outl_put = [&](uint32_t kn, uint32_t vbits) {
    const int kl = (int)(kn >> 6) - k0, nl = (int)(kn & 63), nqo = nl >> 2;
    if ((unsigned)kl < (unsigned)BN)
      *reinterpret_cast<uint16_t*>(CB + swz128(kl, nqo >> 1) + (nqo & 1) * 8 + 2 * (nl & 3)) =
          (uint16_t)f32_to_bf16(__uint_as_float(vbits));
  };
  // the first two stages' ranges are read before the stage loads, so that
  // reading the first entries waits for them alone
  Outl2 ocur{};
  if constexpr (AFF) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kg = kgw0 + 4 * h;
      cr2[h].init(a.bptr, a.kg, kg < a.kg ? kg : a.kg, kg + 1 < a.kg ? kg + 1 : a.kg, nk, kt0);
    }
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 uacc[(FM + 1) / 2][UCB];
#pragma unroll
  for (int i = 0; i < (FM + 1) / 2; ++i)
#pragma unroll
    for (int j = 0; j < UCB; ++j) uacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (kt0 + st < kt1) issue(kt0 + st, st);
  if constexpr (AFF) {
    outl_range(kt0, ocur);
    outl_load(ocur);
  }

  // t tile into LDS (pitch r); BU rows past the rank stay zero for good
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = tid + 256 * i, row = e / R, j = e % R;
    if (e < BM * R && j < r) Ts[row * r + j] = m0 + row < M ? tv[i] : 0.f;
  }
  for (int e = 3 * R * 32 + tid; e < UCB * 16 * 32; e += 256)      // 4-byte pairs
    *reinterpret_cast<uint32_t*>(BU + swz128(e / 32, (e % 32) >> 2) + (e & 3) * 4) = 0u;
  __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());    // stores land before the first barrier
  if constexpr (TFL) {
    // the t operand from the t tile (which sits in the converted-code
    // buffer: the loop's first barrier comes before the first conversion);
    // wave w builds fragments f = w, w + 4, ... of the UCB * BM / 32
    __syncthreads();
    for (int f = wid; f < UCB * (BM / 32); f += 4) {
      const int cb = f / (BM / 32), c = f % (BM / 32);
      const int j = cb * 16 + (lane & 15), part = j / R, jr = j - part * R;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 32 * c + 8 * (lane >> 4) + e;
        v[e] = (jr < r && part < 3) ? Ts[m * r + (jr < r ? jr : 0)] : 0.f;
      }
      u32x4 hi, mid, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t me, le;
        hi[e] = pk_bf16_split3(v[2 * e], v[2 * e + 1], me, le);
        mid[e] = me;
        lo[e] = le;
      }
      *reinterpret_cast<u32x4*>(TF + (f * 64 + lane) * 16) = part == 0 ? hi : part == 1 ? mid : lo;
    }
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
  }

  const int rows_here = M - m0 < BM ? M - m0 : BM;
  // dB operand: t split into bf16 hi, mid and lo columns, lane -> column
  // (lane % 16), rows 32 c + 8 (lane / 16) + e; rebuilt from the t tile in
  // LDS at each of the block's dB stages rather than held in registers
  // cooperative conversion: thread -> n quad nq, k quads kq0 + 16 h
  const int nq = tid & 15, kq0 = tid >> 4;

  int slot = 0;
  for (int kt = kt0; kt < kt1; ++kt) {
    wait_stages<LPS, 0, S - 2>(kt1 - 1 - kt);
    if constexpr (W4) {                              // the stage's scales, as float
      if (lane < 16) SCs[scn] = (float)__builtin_bit_cast(_Float16, scr);
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    }
    __builtin_amdgcn_s_barrier();                    // stage kt landed; CB, BU free
    // affine weights: read stage kt + 1's outliers ahead of this
    // iteration's loads
    Outl2 o1{};
    if constexpr (AFF) {
      outl_range(kt + 1 < kt1 ? kt + 1 : kt, o1);
      outl_load(o1);
      __builtin_amdgcn_sched_barrier(0);           // ahead of the stage loads
    }
    // (affine weights: every iteration queues the same loads; see the 64-row
    // kernel)
    // The loads of stage kt + S - 1 (into the slot that stage kt - 1 left)
    // are queued where the wave stalls least on the memory pipeline taking
    // them (measured): 4-bit weights once this stage's codes have been read,
    // int8 weights after the second barrier, beside the products; the
    // affine weights' outlier read-ahead counts on them being queued here.
    auto issue_next = [&] {
      if (AFF || kt + S - 1 < kt1) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
    };
    if constexpr (AFF) issue_next();
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;
    const float* Xa = reinterpret_cast<const float*>(Bs + BSZ);

    // CB[k][n] = bf16(q[n][k] sw[n]) for the 4 n of nq and 4 k per quad
    // (4-bit: bf16(q[n][k] sc[n][k0 / 128]) for the 4 n of nq and 8 k)
    if constexpr (W4) {
      const f32x4 scv = *reinterpret_cast<const f32x4*>(SCs + 4 * nq);
      const int kq8 = kq0;                           // k in [8 kq8, 8 kq8 + 8)
      uint32_t raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * nq + i;
        raw[i] = *reinterpret_cast<const uint32_t*>(Bs + n * RB + (((kq8 >> 2) ^ code_swz<RB>(n)) << 4) + (kq8 & 3) * 4);
      }
      issue_next();
      float v[4][8];
      nibble_vals(raw[0], scv.x, v[0]);
      nibble_vals(raw[1], scv.y, v[1]);
      nibble_vals(raw[2], scv.z, v[2]);
      nibble_vals(raw[3], scv.w, v[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x2*>(CB + swz128(8 * kq8 + e, nq >> 1) + (nq & 1) * 8) =
            u32x2{pk_bf16(v[0][e], v[1][e]), pk_bf16(v[2][e], v[3][e])};
    } else {
      f32x4 swv = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!AFF) swv = *reinterpret_cast<const f32x4*>(Xa + 4 * nq);
#pragma unroll
      for (int h = 0; h < BN / 64; ++h) {
        const int kcol = 4 * (kq0 + 16 * h);
        int raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 4 * nq + i;
          raw[i] = *reinterpret_cast<const int*>(Bs + n * RB + ((((kcol >> 4) ^ code_swz<RB>(n))) << 4) + (kcol & 15));
        }
#pragma unroll
        for (int kk2 = 0; kk2 < 4; ++kk2) {
          float v0, v1, v2, v3;
          if constexpr (AFF) {
            v0 = __builtin_fmaf((float)(int8_t)(raw[0] >> (8 * kk2)), cstep, cbias);
            v1 = __builtin_fmaf((float)(int8_t)(raw[1] >> (8 * kk2)), cstep, cbias);
            v2 = __builtin_fmaf((float)(int8_t)(raw[2] >> (8 * kk2)), cstep, cbias);
            v3 = __builtin_fmaf((float)(int8_t)(raw[3] >> (8 * kk2)), cstep, cbias);
          } else {
            v0 = (float)(int8_t)(raw[0] >> (8 * kk2)) * swv.x;
            v1 = (float)(int8_t)(raw[1] >> (8 * kk2)) * swv.y;
            v2 = (float)(int8_t)(raw[2] >> (8 * kk2)) * swv.z;
            v3 = (float)(int8_t)(raw[3] >> (8 * kk2)) * swv.w;
          }
          *reinterpret_cast<u32x2*>(CB + swz128(kcol + kk2, nq >> 1) + (nq & 1) * 8) =
              u32x2{pk_bf16(v0, v1), pk_bf16(v2, v3)};
        }
      }
      if constexpr (AFF) {
        // the wave's outliers over its own conversion stores
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int cnt = ocur.hi[h] - ocur.lo[h];
          if (lane < cnt) outl_put(ocur.e[h].x, ocur.e[h].y);
          for (int b0 = 64; b0 < cnt; b0 += 64) {    // more than 64 in one cell
            const u32x2 ev = a.bent[ocur.lo[h] + b0 + lane];
            if (lane < cnt - b0) outl_put(ev.x, ev.y);
          }
        }
        // the read-ahead outliers were queued before this iteration's stage
        // loads: all but those loads are done
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
        ocur = o1;
      }
    }
    // BU[j][n], BU[R + j][n], BU[2 R + j][n] = the bf16 hi, mid and lo parts of
    // B[j][n], 2 n per entry
#pragma unroll
    for (int e = tid; e < R * 32; e += 256) {
      const int j = e >> 5, p = e & 31;
      const f32x2 b = *reinterpret_cast<const f32x2*>(Xa + 64 * (1 + j) + 2 * p);
      uint32_t mid2, lo2;
      const uint32_t hi2 = pk_bf16_split3(b.x, b.y, mid2, lo2);
      *reinterpret_cast<uint32_t*>(BU + swz128(j, p >> 2) + (p & 3) * 4) = hi2;
      *reinterpret_cast<uint32_t*>(BU + swz128(R + j, p >> 2) + (p & 3) * 4) = mid2;
      *reinterpret_cast<uint32_t*>(BU + swz128(2 * R + j, p >> 2) + (p & 3) * 4) = lo2;
    }
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    __builtin_amdgcn_s_barrier();                    // CB, BU visible
    if constexpr (!W4 && !AFF) issue_next();

#pragma unroll
    for (int kk = 0; kk < KC / 32; ++kk) {
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
#pragma unroll
      for (int cb = 0; cb < UCB; ++cb) {
        const bf16x8 bu = *reinterpret_cast<const bf16x8*>(BU + swz128(cb * 16 + (lane & 15), c));
#pragma unroll
        for (int h = 0; h < FM / 2; ++h)
          uacc[h][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pick_frag(af[2 * h], af[2 * h + 1], wn != 0),
                                                               bu, uacc[h][cb], 0, 0, 0);
      }
    }
    // dB partial for this stage's 64 n over the block's rows (one block per
    // row block and stage), on the matrix cores: wave w takes n in
    // [16 w, 16 w + 16); dB^T[n][j] = sum_m dy[m][n] t[m][j]. The dy^T operand
    // comes from the dy tile through transposing reads: in each 16-lane group,
    // lanes 4 i + p fetch the 4 n at 16 w + 4 p of row i, and lane q receives
    // n = 16 w + q of rows 0..3.
    if (kt % a.tiles_x == kt_blk) {
      constexpr int NRD = 2 * (BM / 32);
      uint32_t tra[NRD];
      uint64_t trv[NRD];
      const int q = lane & 15, i4 = q >> 2, p4 = q & 3;
#pragma unroll
      for (int c = 0; c < BM / 32; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int m = 32 * c + 8 * (lane >> 4) + 4 * h + i4;
          const int n = 16 * wid + 4 * p4;
          tra[2 * c + h] = lds_addr(As + swz128(m, n >> 3) + (n & 7) * 2);
        }
      tr16_reads<NRD>(tra, trv);
      f32x4 dbacc[UCB];
#pragma unroll
      for (int cb = 0; cb < UCB; ++cb) dbacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < BM / 32; ++c) {
        const bf16x8 dyT = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)trv[2 * c], (uint32_t)(trv[2 * c] >> 32),
                                                            (uint32_t)trv[2 * c + 1], (uint32_t)(trv[2 * c + 1] >> 32)});
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb) {
          // the t operand's fragment (cb, c): from LDS, or (rank 8) rebuilt
          // from the t tile here, one fragment at a time (fewer registers
          // live): column j is part j / R (hi, mid, lo) of t[., j % R]
          bf16x8 tf;
          if constexpr (TFL) {
            tf = *reinterpret_cast<const bf16x8*>(TF + ((cb * (BM / 32) + c) * 64 + lane) * 16);
          } else {
            const int j = cb * 16 + (lane & 15), part = j / R, jr = j - part * R;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int m = 32 * c + 8 * (lane >> 4) + e;
              v[e] = (jr < r && part < 3) ? Ts[m * r + (jr < r ? jr : 0)] : 0.f;
            }
            u32x4 hi, mid, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              uint32_t me, le;
              hi[e] = pk_bf16_split3(v[2 * e], v[2 * e + 1], me, le);
              mid[e] = me;
              lo[e] = le;
            }
            tf = __builtin_bit_cast(bf16x8, part == 0 ? hi : part == 1 ? mid : lo);
          }
          dbacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dyT, tf, dbacc[cb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int cb = 0; cb < RCB; ++cb) {
        const int j = cb * 16 + (lane & 15);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float dbv = split3_sum<R, UCB>(dbacc, cb, ii, lane);
          const int gn = kt * KC + 16 * wid + 4 * (lane >> 4) + ii;
          if (j < r && gn < N) a.partB[((long)mt * r + j) * N + gn] = dbv;
        }
      }
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  if constexpr (SPLIT) {
    // partial products, float4 unit ((split tiles + tile) 4 + wave) F + f)
    // 64 + lane for fragment f = i FN + j of F = FM FN: each store writes
    // 1 KB of consecutive bytes. The column-tile-0 block of each row block
    // writes its split's partial u.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));        // ring loads done before the block ends
    f32x4* P = reinterpret_cast<f32x4*>(a.pdx) +
               ((long)(split * tiles + bid) * 4 + wid) * (FM * FN * 64) + lane;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) P[(i * FN + j) * 64] = acc[i][j];
    if (kt_blk == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if ((i & 1) != wn) continue;
#pragma unroll
        for (int cb = 0; cb < RCB; ++cb) {
          const int j = cb * 16 + (lane & 15);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float uv = split3_sum<R, UCB>(uacc[i >> 1], cb, ii, lane);
            const int gm = m0 + wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
            if (j < r && gm < M) a.pu[((long)split * M + gm) * r + j] = uv;
          }
        }
      }
    }
    return;
  }

  // ---- after the contraction: u to LDS, x tile, dA partial, dx epilogue ----
  float* E = reinterpret_cast<float*>(ring);             // U [BM][R] | A^T [R][BN]
  __syncthreads();                                        // ring released
  if constexpr (!XPRE) issue_x();
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if ((i & 1) != wn) continue;
#pragma unroll
    for (int cb = 0; cb < RCB; ++cb) {
      const int j = cb * 16 + (lane & 15);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float uv = split3_sum<R, UCB>(uacc[i >> 1], cb, ii, lane);
        const int ml = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
        if (j < R) E[ml * R + j] = j < r ? uv : 0.f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = tid + 256 * i, j = e / BN, col = e % BN;
    if (e < BN * R) E[BM * R + e] = (j < r && k0 + col < K) ? qv[i] : 0.f;
  }
  __syncthreads();

  // dA partial on the matrix cores: dA^T[k][j] = sum_m x[m][k] u[m][j] over
  // the block's rows, with u split like B and t into bf16 hi, mid and lo
  // columns (the u operand, [UCB][BM / 32][64 lanes][16 B] in the B and t
  // buffers the loop has released; wave w builds fragments w, w + 4, ...;
  // rows past M are zero there and in the x tile) and x^T read from the x
  // tile through transposing reads (in each 16-lane group lane 4 i + p
  // fetches the 4 columns at c0 + 4 p of row i, and lane q receives column
  // c0 + q of rows 0..3). Wave w takes the columns [BN / 4 w, BN / 4 (w + 1)).
  int8_t* UF = BU;
  static_assert(UCB * (BM / 32) * 1024 <= BUSZ + TSZ, "u operand fits in the B and t buffers");
  for (int f = wid; f < UCB * (BM / 32); f += 4) {
    const int cb = f / (BM / 32), c = f % (BM / 32);
    const int j = cb * 16 + (lane & 15), part = j / R, jr = j - part * R;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 32 * c + 8 * (lane >> 4) + e;
      v[e] = (jr < r && part < 3 && m < rows_here) ? E[m * R + (jr < r ? jr : 0)] : 0.f;
    }
    u32x4 hi, mid, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t me, le;
      hi[e] = pk_bf16_split3(v[2 * e], v[2 * e + 1], me, le);
      mid[e] = me;
      lo[e] = le;
    }
    *reinterpret_cast<u32x4*>(UF + (f * 64 + lane) * 16) = part == 0 ? hi : part == 1 ? mid : lo;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));              // the x tile
  __syncthreads();
  {
    constexpr int KB = BN / 64, RH = BN / 64;          // 16-column blocks per wave
    f32x4 dacc[KB][UCB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cb = 0; cb < UCB; ++cb) dacc[kb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int q = lane & 15, i4 = q >> 2, p4 = q & 3;
#pragma unroll
    for (int c0 = 0; c0 < BM / 32; c0 += 2) {
      uint32_t tra[4 * KB];
      uint64_t trv[4 * KB];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = 32 * (c0 + cc) + 8 * (lane >> 4) + 4 * h + i4;
            const int col = (BN / 4) * wid + 16 * kb + 4 * p4;
            tra[(cc * KB + kb) * 2 + h] = lds_addr(Xs + swz128(m * RH + col / 64, (col % 64) >> 3) + (col & 7) * 2);
          }
      tr16_reads<4 * KB>(tra, trv);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = c0 + cc;
        bf16x8 uf[UCB];
#pragma unroll
        for (int cb = 0; cb < UCB; ++cb)
          uf[cb] = *reinterpret_cast<const bf16x8*>(UF + ((cb * (BM / 32) + c) * 64 + lane) * 16);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int t0 = (cc * KB + kb) * 2;
          const bf16x8 xT = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)trv[t0], (uint32_t)(trv[t0] >> 32),
                                                             (uint32_t)trv[t0 + 1], (uint32_t)(trv[t0 + 1] >> 32)});
#pragma unroll
          for (int cb = 0; cb < UCB; ++cb)
            dacc[kb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xT, uf[cb], dacc[kb][cb], 0, 0, 0);
        }
      }
    }
    float dav[KB][RCB][4];
    bool nan = false;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cb = 0; cb < RCB; ++cb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          dav[kb][cb][ii] = split3_sum<R, UCB>(dacc[kb], cb, ii, lane);
          nan |= dav[kb][cb][ii] != dav[kb][cb][ii];
        }
    if (__builtin_amdgcn_ballot_w64(nan) == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int cb = 0; cb < RCB; ++cb) {
          const int j = cb * 16 + (lane & 15);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int kl = (BN / 4) * wid + 16 * kb + 4 * (lane >> 4) + ii;
            if (j < r && k0 + kl < K) a.partA[((long)mt * r + j) * K + k0 + kl] = dav[kb][cb][ii];
          }
        }
    } else {
      // A NaN in the wave's columns: an infinite x times the three parts of
      // u can give inf - inf where the plain product is infinite, so the
      // wave takes its columns again as float32 sums in row order (lane ->
      // column (BN / 4) w + lane % (BN / 4), ranks jb + TPK jj).
      constexpr int CPW = BN / 4, TPK = 64 / CPW, JPT = (R + TPK - 1) / TPK;
      const int kl = CPW * wid + lane % CPW, jb = lane / CPW;
      float da[JPT];
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) da[jj] = 0.f;
      for (int m = 0; m < rows_here; ++m) {
        const int e = kl % 64;
        const uint16_t xb = *reinterpret_cast<const uint16_t*>(Xs + swz128(m * RH + kl / 64, e >> 3) + 2 * (e & 7));
        const float xv = __uint_as_float((uint32_t)xb << 16);
#pragma unroll
        for (int jj = 0; jj < JPT; ++jj)
          if (jb + TPK * jj < R) da[jj] = __builtin_fmaf(xv, E[m * R + jb + TPK * jj], da[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) {
        const int j = jb + TPK * jj;
        if (j < r && k0 + kl < K) a.partA[((long)mt * r + j) * K + k0 + kl] = da[jj];
      }
    }
  }

  // output staging strips in the converted-code buffer, free after the loop
  static_assert(4 * epi_strip_bytes<uint16_t, FN>() <= CBSZ, "staging strips fit");
  epilogue_lowrank<BM, BN, R, false>(acc, E, M, K, m0, k0, wm * (BM / 2), wn * (BN / 2), a.s, a.dx,
                                     CB + wid * epi_strip_bytes<uint16_t, FN>());
}


// Second launch of the split contraction, one block per 128-row x 32-column
// quarter of a 128 x 128 tile (so that twice as many compute units read the
// partial sums as with halves): the partial products added in split order,
// u added in split order from its partials, the dA partial of the 128-row
// block over these 32 columns, and dx = bf16(sum + s u A^T) through the
// common epilogue. Wave v takes rows [16 v, 16 v + 16): fragment row v % 4,
// fragment columns 2 (q % 2) + {0, 1} of the wide kernel's wave
// 2 (v / 4) + q / 2 for quarter q. Every split's loads are issued before
// the first add (NSPL: the split count's bound; splits past the count read
// split 0 and are dropped by a select).
template <int R, int NSPL>
__global__ __launch_bounds__(512) void bwd_fixup_kernel(BwdArgs a) {
  constexpr int BM = 128, HN = 32, FN = 2;
  constexpr int EFL = (BM + HN) * R;                    // U [BM][R] | A^T [R][HN]
  constexpr int XSZ = BM * HN * 2;                      // x [BM][HN] bf16, 64-byte rows
  constexpr int STRIP = epi_strip_bytes<uint16_t, FN>();
  __shared__ __attribute__((aligned(1024))) int8_t lds[XSZ + EFL * 4 + 8 * STRIP];
  int8_t* Xs = lds;
  float* E = reinterpret_cast<float*>(lds + XSZ);
  int8_t* strips = lds + XSZ + EFL * 4;

  const int tid = threadIdx.x, lane = tid & 63, v = wave_id();
  const int M = a.M, K = a.K, r = a.r, nsp = a.splits;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  const int tile = (int)blockIdx.x >> 2, q = (int)blockIdx.x & 3;
  const int mt = tile / a.tiles_x;
  const int m0 = mt * BM, k0 = (tile % a.tiles_x) * 128 + q * HN;

  // partial products of this wave's two fragments, all splits in flight
  const int w = 2 * (v >> 2) + (q >> 1), fi = v & 3;
  const f32x4* P = reinterpret_cast<const f32x4*>(a.pdx) + ((long)tile * 4 + w) * (16 * 64) +
                   (fi * 4 + 2 * (q & 1)) * 64 + lane;
  const long pstride = (long)tiles * 4 * 16 * 64;       // float4 units per split
  f32x4 pv[NSPL][FN];
#pragma unroll
  for (int sp = 0; sp < NSPL; ++sp)
#pragma unroll
    for (int j = 0; j < FN; ++j) pv[sp][j] = P[(sp < nsp ? sp : 0) * pstride + j * 64];

  // x tile by DMA: [128 rows][32 columns] as 64-byte rows, 16 per
  // instruction; wave v moves rows 16 v .. + 16 (chunk c of row r lands at
  // 64 r + 16 (c ^ ((r >> 2) & 3)))
  {
    const int row = 16 * v + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3), gm = m0 + row, gk = k0 + c * 8;
    const void* src = gk < K ? (const void*)(a.x + (long)(gm < M ? gm : M - 1) * K + gk)
                             : (const void*)zero_chunk(lane);
    lds_dma16(src, Xs + 16 * v * 64);
  }

  // U[m][j] = sum over splits of the partial u (rows past M and ranks past r: 0)
  for (int e = tid; e < BM * R; e += 512) {
    const int m = e / R, j = e % R, gm = m0 + m;
    const bool ok = j < r && gm < M;
    const float* pu = a.pu + ((long)(gm < M ? gm : M - 1)) * r + (j < r ? j : 0);
    float uv[NSPL];
#pragma unroll
    for (int sp = 0; sp < NSPL; ++sp) uv[sp] = pu[(long)(sp < nsp ? sp : 0) * M * r];
    float u = 0.f;
#pragma unroll
    for (int sp = 0; sp < NSPL; ++sp) u += sp < nsp ? uv[sp] : 0.f;
    E[e] = ok ? u : 0.f;
  }
  for (int e = tid; e < R * HN; e += 512) {
    const int j = e / HN, col = e % HN, gk = k0 + col;
    E[BM * R + e] = (j < r && gk < K) ? a.A[(long)gk * r + j] : 0.f;
  }

  f32x4 acc[1][FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    acc[0][j] = pv[0][j];
#pragma unroll
    for (int sp = 1; sp < NSPL; ++sp)
      if (sp < nsp) acc[0][j] += pv[sp][j];
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // dA partial over the block's rows: thread -> column tid % 32, ranks
  // tid / 32 + 16 jj
  {
    constexpr int JPT = (R + 15) / 16;
    const int kl = tid % HN, jb = tid / HN;
    const int rows_here = M - m0 < BM ? M - m0 : BM;
    float da[JPT];
#pragma unroll
    for (int jj = 0; jj < JPT; ++jj) da[jj] = 0.f;
    if (jb < R) {
#pragma unroll 8
      for (int m = 0; m < rows_here; ++m) {
        const uint16_t xb = *reinterpret_cast<const uint16_t*>(
            Xs + m * 64 + (((kl >> 3) ^ ((m >> 2) & 3)) << 4) + 2 * (kl & 7));
        const float xv = __uint_as_float((uint32_t)xb << 16);
#pragma unroll
        for (int jj = 0; jj < JPT; ++jj)
          if (jb + 16 * jj < R) da[jj] = __builtin_fmaf(xv, E[m * R + jb + 16 * jj], da[jj]);
      }
    }
    if (k0 + kl < K) {
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) {
        const int j = jb + 16 * jj;
        if (j < r) a.partA[((long)mt * r + j) * K + k0 + kl] = da[jj];
      }
    }
  }

  epilogue_lowrank<BM, HN, R, false>(acc, E, M, K, m0, k0, 16 * v, 0, a.s, a.dx,
                                     strips + v * STRIP);
}

template <bool W4, int BN, int S, bool AFF = false>
void launch_pc(BwdArgs a, hipStream_t st) {
  constexpr int BM = 64;
  a.tiles_x = (a.K + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM)));
  if constexpr (!W4 && !AFF) {
    // plain int8 of one head and at most kBresN outputs, rank 5 to 8, at
    // least 512 rows: scales and B resident in LDS (measured: 1-1.5 % faster
    // on 1024-row layers; on short grids loading them up front costs more
    // than it saves). The block takes 112 KB, one per compute unit as
    // without them; at rank 4 they would cost the second block.
    if (a.N <= kBresN && a.hd == a.N && a.r > 4 && a.r <= 8 && a.M >= 512) {
      bwd_pc_kernel<false, BM, BN, S, 8, false, true><<<grid, 512, 0, st>>>(a);
      return;
    }
  }
  if (a.r <= 4) bwd_pc_kernel<W4, BM, BN, S, 4, AFF><<<grid, 512, 0, st>>>(a);
  else if (a.r <= 8) bwd_pc_kernel<W4, BM, BN, S, 8, AFF><<<grid, 512, 0, st>>>(a);
  else if (a.r <= 16) bwd_pc_kernel<W4, BM, BN, S, 16, AFF><<<grid, 512, 0, st>>>(a);
  else if constexpr (!W4) bwd_pc_kernel<W4, BM, BN, S, 32, AFF><<<grid, 512, 0, st>>>(a);
  // (4-bit layers of rank above 16 take the 128 x 128 tiles: bwd_row_block)
}

template <bool W4, bool AFF = false, bool SPLIT = false, int BN = 128>
void launch_wide(BwdArgs a, hipStream_t st) {
  static_assert(BN == 128 || (!W4 && !AFF && !SPLIT), "64-wide tiles: plain int8, one pass");
  constexpr int BM = 128, S = 2;
  a.tiles_x = (a.K + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM) * (SPLIT ? a.splits : 1)));
  if (a.r <= 4) bwd_wide_kernel<W4, BM, BN, S, 4, AFF, SPLIT><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) bwd_wide_kernel<W4, BM, BN, S, 8, AFF, SPLIT><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) bwd_wide_kernel<W4, BM, BN, S, 16, AFF, SPLIT><<<grid, 256, 0, st>>>(a);
  else bwd_wide_kernel<W4, BM, BN, S, 32, AFF, SPLIT><<<grid, 256, 0, st>>>(a);
  if constexpr (SPLIT) {
    const dim3 fgrid((unsigned)(4 * a.tiles_x * ((a.M + BM - 1) / BM)));
    if (a.splits <= 4) {
      if (a.r <= 4) bwd_fixup_kernel<4, 4><<<fgrid, 512, 0, st>>>(a);
      else if (a.r <= 8) bwd_fixup_kernel<8, 4><<<fgrid, 512, 0, st>>>(a);
      else if (a.r <= 16) bwd_fixup_kernel<16, 4><<<fgrid, 512, 0, st>>>(a);
      else bwd_fixup_kernel<32, 4><<<fgrid, 512, 0, st>>>(a);
    } else {
      if (a.r <= 4) bwd_fixup_kernel<4, kMaxWideSplits><<<fgrid, 512, 0, st>>>(a);
      else if (a.r <= 8) bwd_fixup_kernel<8, kMaxWideSplits><<<fgrid, 512, 0, st>>>(a);
      else if (a.r <= 16) bwd_fixup_kernel<16, kMaxWideSplits><<<fgrid, 512, 0, st>>>(a);
      else bwd_fixup_kernel<32, kMaxWideSplits><<<fgrid, 512, 0, st>>>(a);
    }
  }
}

// Stages per split of the 128 x 128 contraction, and the split count: split
// only while the tiles would leave most compute units idle (at most 128
// tiles) and the contraction is long (two splits of at least 16 stages),
// then keep doubling (up to 8) while the grid stays within two blocks per
// compute unit and each split keeps at least 8 stages (measured: 8 stages
// per split beat 16 by 5-25 % on layers of 128-1024 rows; the shapes that
// would split only at fewer than 16 stages are faster on 64-row tiles).
void wide_split_plan(int M, int K, int N, int* splits, int* nks) {
  const long tiles = (long)((M + 127) / 128) * ((K + 127) / 128);
  const int nk = (N + 63) / 64;
  int sp = 1;
  if (tiles <= 128)
    while (sp < kMaxWideSplits && tiles * sp * 2 <= 512 && nk / (sp * 2) >= (sp == 1 ? 16 : 8)) sp *= 2;
  *nks = (nk + sp - 1) / sp;
  *splits = (nk + *nks - 1) / *nks;
}

}  // namespace

void bwd_split_sizes(int M, int K, int N, int r, size_t* pdx_floats, size_t* pu_floats) {
  int sp, nks;
  wide_split_plan(M, K, N, &sp, &nks);
  if (sp == 1) {
    *pdx_floats = 0;
    *pu_floats = 0;
    return;
  }
  const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((K + 127) / 128);
  *pdx_floats = (size_t)sp * tiles * 128 * 128;
  *pu_floats = (size_t)sp * (size_t)M * (size_t)r;
}

int bwd_row_block(int fmt, int M, int K, int N, int r) {
  int sp, nks;
  wide_split_plan(M, K, N, &sp, &nks);
  if (sp > 1) return 128;                         // split 128 x 128 tiles
  if (fmt == 1 && r > 16) return 128;             // the 64-row 4-bit tile at rank 32 exceeds the LDS
  const int bn = fmt == 1 ? 128 : 64;             // k per 64-row tile
  const long t64 = (long)((M + 63) / 64) * ((K + bn - 1) / bn);
  return t64 <= 512 ? 64 : 128;
}

namespace {
// The fused backward's block shape for a layer: split 128 x 128 tiles for
// few tiles over a long contraction; else 64-row tiles (producer/consumer)
// while they make at most two blocks per compute unit; else 128 x 64 tiles
// (plain int8) while 128 x 128 ones would be fewer than the compute units;
// else 128 x 128 tiles.
enum class BwdKind { kSplit, kPC, kWide64, kWide128 };
BwdKind bwd_kind(int fmt, int M, int K, int N, int r) {
  int sp, nks;
  wide_split_plan(M, K, N, &sp, &nks);
  if (sp > 1) return BwdKind::kSplit;
  if (bwd_row_block(fmt, M, K, N, r) == 64) return BwdKind::kPC;
  const long t128 = (long)((M + 127) / 128) * ((K + 127) / 128);
  if (fmt == 0 && t128 < 256) return BwdKind::kWide64;
  return BwdKind::kWide128;
}
}  // namespace

const char* bwd_fused_kernel_name(int fmt, int M, int K, int N, int r) {
  switch (bwd_kind(fmt, M, K, N, r)) {
    case BwdKind::kSplit: return "bwd_wide_kernel<SPLIT> + bwd_fixup_kernel";
    case BwdKind::kPC: return "bwd_pc_kernel";
    case BwdKind::kWide64: return "bwd_wide_kernel (128 x 64 tiles)";
    default: return "bwd_wide_kernel";
  }
}

void launch_bwd_fused(int fmt, int M, int K, int N, const uint16_t* dy,
                      const void* codes, const void* scales, const float* B, int hd,
                      const float* A, const float* t, const uint16_t* x, int r,
                      float s, uint16_t* dx, float* partA, float* partB,
                      float* pdx, float* pu, hipStream_t st) {
  BwdArgs a{};
  a.M = M; a.K = K; a.N = N; a.dy = dy; a.codes = static_cast<const int8_t*>(codes);
  a.B = B; a.hd = hd; a.A = A; a.t = t; a.x = x; a.r = r; a.s = s; a.dx = dx; a.partA = partA;
  a.partB = partB;
  a.pdx = pdx; a.pu = pu;
  wide_split_plan(M, K, N, &a.splits, &a.nks);
  const BwdKind kind = bwd_kind(fmt, M, K, N, r);
  if (fmt == 2) {
    const W8OLayout L = w8o_layout(K, N);
    const char* sb = static_cast<const char*>(scales);
    a.w8o = reinterpret_cast<const W8OHeader*>(sb);
    a.bptr = reinterpret_cast<const int*>(sb + L.bptr);
    a.bent = reinterpret_cast<const u32x2*>(sb + L.bent);
    a.kg = L.kg;
    if (kind == BwdKind::kSplit) launch_wide<false, true, true>(a, st);
    else if (kind == BwdKind::kPC) launch_pc<false, 64, 3, true>(a, st);
    else launch_wide<false, true>(a, st);
  } else if (fmt == 0) {
    a.sw = static_cast<const float*>(scales);
    if (kind == BwdKind::kSplit) launch_wide<false, false, true>(a, st);
    else if (kind == BwdKind::kPC) launch_pc<false, 64, 3>(a, st);
    else if (kind == BwdKind::kWide64) launch_wide<false, false, false, 64>(a, st);
    else launch_wide<false>(a, st);
  } else {
    a.sc4 = static_cast<const uint16_t*>(scales);
    if (kind == BwdKind::kSplit) launch_wide<true, false, true>(a, st);
    else if (kind == BwdKind::kPC) launch_pc<true, 128, 3>(a, st);
    else launch_wide<true>(a, st);
  }
}

}  // namespace qlora
