// Input gradient of the frozen int8 layer on v_mfma_f32_16x16x32_bf16.
//
//   dx[m, k] = sum_n g[m, n] q[n, k] + s sum_j u[m, j] A[k, j]
//
// with g = bf16(dy * sw) (the channel scale folded into the gradient rows by
// the row pass) and q the raw codes, exact in bfloat16. The quantizer of x is
// taken as the identity (straight-through estimator), so this is the frozen
// layer's transposed product plus the adapter's input gradient
// ("Parameter-efficient fine-tuning of GPT-2 with LoRA", "LoRA equation";
// "How to fine-tune the 4-bit model?": adapter training needs the transposed
// quantized product).
//
// The codes are stored [N, K] (K contiguous) while this product contracts over
// n. Both operands still go straight into the LDS stage ring (ring.hpp) in
// their stored layout: g rows as swizzled 128-byte rows (64 n per stage) and
// the codes as [64 n][BN k] byte rows. The transpose happens in the LDS read:
// ds_read_b64_tr_b8 gives each lane the 8 bytes of one k column at 8
// consecutive n, which is the MFMA B operand after widening to bfloat16 in
// registers (one sign-extending convert per byte, one permute per pair).
// Code rows are swizzled by 16-byte chunk so that the transposing reads of 16
// rows cover all 64 banks.
//
// Extra blocks past the output tiles run stage 1 of the adapter-gradient
// reductions (skinny.hpp), which only needs the row pass's outputs.
#include "launch.hpp"
#include "ring.hpp"
#include "skinny.hpp"

namespace qlora {

namespace {

constexpr int kCUs = 256;

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

struct Dx8Args {
  int M, K, N;                 // rows, output columns, contraction length
  const uint16_t* g;           // [M, N] bfloat16
  const int8_t* codes;         // [N, K]
  const float* u;              // [M, r]
  const float* A;              // [K, r]
  int r;
  float s;
  uint16_t* dx;                // [M, K] bfloat16
  int tiles_x, tiles;
};

// Chunk swizzle of a code tile with RB-byte rows (RB = 64 or 128): rows that
// share banks (256 / RB of them per 256 bytes) get distinct chunk masks.
template <int RB>
__device__ __forceinline__ int code_swz(int row) {
  return (row >> (RB == 64 ? 2 : 1)) & (RB / 16 - 1);
}

// Widen 8 signed bytes to 8 bfloat16 (exact: |q| <= 127).
__device__ __forceinline__ bf16x8 widen_i8(i32x2 w) {
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int x = w[d];
    const float f0 = (float)(int8_t)x, f1 = (float)(int8_t)(x >> 8);
    const float f2 = (float)(int8_t)(x >> 16), f3 = (float)(x >> 24);
    o[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    o[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, o);
}

template <int BM, int BN, int S, int R>
__global__ __launch_bounds__(256) void dx8_kernel(Dx8Args a, SkinnyJobs sk) {
  constexpr int KC = 64;                          // contraction per stage (n)
  constexpr int ASZ = BM * 2 * KC, BSZ = KC * BN, STG = ASZ + BSZ;
  constexpr int AI = BM / 32;                     // A: 8 rows of 128 B per instruction
  constexpr int BI = BN / 64;                     // B: 1024 / BN rows per instruction
  constexpr int LPS = AI + BI;
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int RPI = 1024 / BN, CPR = BN / 16;   // code rows per instruction, chunks per row
  static_assert(EpiOps<BM, BN, R, false>::kFloats * 4 <= S * STG, "epilogue fits in the ring");
  static_assert(4 * (R < 4 ? R : 4) * kSkCols * 4 <= S * STG, "stage 1 fits in the ring");
  __shared__ __attribute__((aligned(1024))) int8_t ring[S * STG];

  if ((int)blockIdx.x >= a.tiles) {
    skinny_partial_block<BF16, R>(sk, blockIdx.x - a.tiles, reinterpret_cast<float*>(ring));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = ((int)blockIdx.x / a.tiles_x) * BM, k0 = ((int)blockIdx.x % a.tiles_x) * BN;
  const int M = a.M, K = a.K, N = a.N;
  const int nk = (N + KC - 1) / KC;

  EpiOps<BM, BN, R, false> ep;
  ep.load(M, K, m0, k0, a.r, a.u, a.A, 1, a.r, nullptr, nullptr);

  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int rb = wid * (BM / 4) + i * 8, row = rb + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      const int gn = kt * KC + c * 8, gm = m0 + row;
      const void* src = gn < N ? (const void*)(a.g + (long)(gm < M ? gm : M - 1) * N + gn)
                               : (const void*)zero_chunk(lane);
      lds_dma16(src, base + rb * 128);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int rb = (wid * BI + i) * RPI, row = rb + lane / CPR;
      const int c = (lane % CPR) ^ code_swz<BN>(row);
      const int gn = kt * KC + row, gk = k0 + c * 16;
      const int8_t* src = (gn < N && gk < K) ? a.codes + (long)gn * K + gk : zero_chunk(lane);
      lds_dma16(src, base + ASZ + rb * BN);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transposing-read address of lane l for 16 columns: lanes 2i, 2i+1 of each
  // 16-lane group fetch the two 8-byte halves of code row 8 (l / 16) + i
  const int tr_row = 8 * (lane >> 4) + ((lane & 15) >> 1), tr_half = lane & 1;

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nk) issue(st, st);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_stages<LPS, 0, S - 2>(nk - 1 - kt);
    __builtin_amdgcn_s_barrier();
    if (kt + S - 1 < nk) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;
#pragma unroll
    for (int kk = 0; kk < KC / 32; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + swz128(wm * (BM / 2) + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = kk * 32 + tr_row;
        const int col = wn * (BN / 2) + j * 16;                 // multiple of 16
        const int off = row * BN + (((col >> 4) ^ code_swz<BN>(row)) << 4) + 8 * tr_half;
        bf[j] = widen_i8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Bs + off)));
      }
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
  ep.store(E, M, K, m0, k0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, BN, R, false>(acc, E, M, K, m0, k0, wm * (BM / 2), wn * (BN / 2), a.s, a.dx);
}

template <int BM, int BN, int S>
void launch_tiles(Dx8Args a, const SkinnyJobs& sk, hipStream_t st) {
  a.tiles_x = (a.K + BN - 1) / BN;
  a.tiles = a.tiles_x * ((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(a.tiles + (sk.njobs > 0 ? sk.blocks() : 0)));
  if (a.r <= 4) dx8_kernel<BM, BN, S, 4><<<grid, 256, 0, st>>>(a, sk);
  else if (a.r <= 8) dx8_kernel<BM, BN, S, 8><<<grid, 256, 0, st>>>(a, sk);
  else if (a.r <= 16) dx8_kernel<BM, BN, S, 16><<<grid, 256, 0, st>>>(a, sk);
  else dx8_kernel<BM, BN, S, 32><<<grid, 256, 0, st>>>(a, sk);
}

}  // namespace

void launch_gemm_dx_w8(int M, int K, int N, const uint16_t* dys,
                       const int8_t* codes, const float* u, const float* A,
                       int r, float s, uint16_t* dx, const SkinnyJobs* sk,
                       hipStream_t st) {
  Dx8Args a{};
  a.M = M; a.K = K; a.N = N; a.g = dys; a.codes = codes; a.u = u; a.A = A;
  a.r = r; a.s = s; a.dx = dx;
  SkinnyJobs none{};
  const SkinnyJobs& j = sk != nullptr ? *sk : none;
  const long t64 = (long)((M + 63) / 64) * ((K + 63) / 64);
  if (t64 <= 2 * kCUs) launch_tiles<64, 64, 4>(a, j, st);
  else launch_tiles<128, 128, 3>(a, j, st);
}

}  // namespace qlora
