// Forward products on MFMA.
//
// int8 path: acc[m, n] = sum_k xq[m, k] * q[n, k]  (v_mfma_i32_16x16x64_i8,
// exact int32), then the fused epilogue
//     y[m, n] = fma(s, sum_j t[m, j] B[j, n], float(acc) * (sx[m] * sw[n]))
// rounded once to the output dtype ("Parameter-efficient fine-tuning of GPT-2
// with LoRA", "LoRA equation": the adapter branch is added to the frozen
// layer's output; "Create LoRA layer": scaled by alpha / rank).
//
// 4-bit path: y = x deq4(W) + s t B with bf16 MFMA (v_mfma_f32_16x16x32_bf16);
// the packed nibbles are unpacked, scaled by their fp16 group scale and
// rounded to bf16 while being staged into LDS ("How to fine-tune the 4-bit
// model?": dequantize at operand load, feeding the matrix unit).
//
// Both operands are staged K-contiguous in LDS ([row][k], rows padded by 16
// bytes so that the 16 rows one MFMA operand reads fall in distinct banks);
// global -> register prefetch of the next K-slice overlaps the MFMAs on the
// current one (double-buffered LDS, one barrier per K-slice).
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int BM = 128, BN = 128;   // block tile (rows of x, output channels)
constexpr int BK8 = 128;            // int8: K bytes per LDS slice
constexpr int P8 = BK8 + 16;        // int8 LDS row pitch in bytes

template <typename OutT, bool ACC_OUT>
__global__ __launch_bounds__(256, 1) void gemm_fwd_w8_kernel(
    int M, int N, int K, const int8_t* __restrict__ xq,
    const int8_t* __restrict__ codes, const float* __restrict__ sx,
    const float* __restrict__ sw, const float* __restrict__ t,
    const float* __restrict__ B, int r, float s, OutT* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * P8];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * P8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  // chunk c = tid + 256 i of a 128 x 128-byte slice: row c / 8, 16 bytes
  const int lrow = tid >> 3, lcol = (tid & 7) * 16;

  u32x4 ra[4], rb[4];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
    const int gk = k0 + lcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      const int gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M && gk < K)
                  ? *reinterpret_cast<const u32x4*>(xq + (long)gm * K + gk) : zero;
      rb[i] = (gn < N && gk < K)
                  ? *reinterpret_cast<const u32x4*>(codes + (long)gn * K + gk) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<u32x4*>(&As[buf][row * P8 + lcol]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][row * P8 + lcol]) = rb[i];
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  const int nk = (K + BK8 - 1) / BK8;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK8);
#pragma unroll
    for (int kk = 0; kk < BK8 / 64; ++kk) {
      i32x4 af[4], bf[4];
      const int koff = kk * 64 + (lane >> 4) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(
            &As[cur][(wm * 64 + i * 16 + (lane & 15)) * P8 + koff]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(
            &Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * P8 + koff]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j],
                                                            acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  if (ACC_OUT) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + ii;
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          if (m < M && n < N) acc_out[(long)m * N + n] = acc[i][j][ii];
        }
    return;
  }
  tile_epilogue<BM, BN, OutT>(acc, M, N, m0, n0, wm, wn, lane, sx, sw, t, B,
                              N, 1, r, s, reinterpret_cast<float*>(&As[0][0]),
                              reinterpret_cast<float*>(&Bs[0][0]), y);
}

// ---------------------------------------------------------------------------
// 4-bit forward: bf16 x [M, K] times deq4 [K, N] (packed [N, K/2] + fp16
// scales [N, K/128]); K slice of 64 per stage.
// ---------------------------------------------------------------------------
constexpr int BK16 = 64;             // bf16 elements of K per LDS slice
constexpr int P16 = BK16 + 8;        // LDS row pitch in bf16 elements

__global__ __launch_bounds__(256, 1) void gemm_fwd_w4_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ packed, const _Float16* __restrict__ scales,
    const float* __restrict__ t, const float* __restrict__ B, int r, float s,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * P16];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * P16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  // x slice: 128 rows x 64 bf16 = 1024 chunks of 8: row c / 8, col 8 (c % 8)
  const int arow = tid >> 3, acol = (tid & 7) * 8;
  // packed slice: 128 rows x 32 bytes: row tid / 2, 16 bytes = 32 codes
  const int brow = tid >> 1, bhalf = tid & 1;
  const int KB = K / 2, G = K / 128;

  u32x4 ra[4], rb;
  float bscale;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gm = m0 + arow + 32 * i;
      ra[i] = (gm < M) ? *reinterpret_cast<const u32x4*>(x + (long)gm * K + k0 + acol)
                       : zero;
    }
    const int gn = n0 + brow;
    const int kb = k0 / 2 + bhalf * 16;
    if (gn < N) {
      rb = *reinterpret_cast<const u32x4*>(packed + (long)gn * KB + kb);
      bscale = (float)scales[(long)gn * G + (k0 + 32 * bhalf) / 128];
    } else {
      rb = zero;
      bscale = 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][(arow + 32 * i) * P16 + acol]) = ra[i];
    // 32 nibbles -> 32 bf16 (q * scale, rounded to nearest even)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t w = rb[d];
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        int q0 = ((int)(w << (28 - 8 * p))) >> 28;      // nibble 2p
        int q1 = ((int)(w << (24 - 8 * p))) >> 28;      // nibble 2p + 1
        o[p] = pack_bf16x2((float)q0 * bscale, (float)q1 * bscale);
      }
      u32x4 ov = {o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4*>(&Bs[buf][brow * P16 + bhalf * 32 + d * 8]) = ov;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK16;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK16);
#pragma unroll
    for (int kk = 0; kk < BK16 / 32; ++kk) {
      bf16x8 af[4], bf[4];
      const int koff = kk * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &As[cur][(wm * 64 + i * 16 + (lane & 15)) * P16 + koff]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * P16 + koff]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
  tile_epilogue<BM, BN, uint16_t>(acc, M, N, m0, n0, wm, wn, lane, nullptr,
                                  nullptr, t, B, N, 1, r, s,
                                  reinterpret_cast<float*>(&As[0][0]),
                                  reinterpret_cast<float*>(&Bs[0][0]), y);
}

}  // namespace

void launch_gemm_fwd_w8(int dtype, int M, int N, int K, const int8_t* xq,
                        const int8_t* codes, const float* sx, const float* sw,
                        const float* t, const float* B, int r, float s,
                        void* y, int32_t* acc_out, hipStream_t st) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (acc_out != nullptr)
    gemm_fwd_w8_kernel<float, true><<<grid, 256, 0, st>>>(
        M, N, K, xq, codes, sx, sw, t, B, r, s, nullptr, acc_out);
  else if (dtype == 0)
    gemm_fwd_w8_kernel<float, false><<<grid, 256, 0, st>>>(
        M, N, K, xq, codes, sx, sw, t, B, r, s, reinterpret_cast<float*>(y),
        nullptr);
  else
    gemm_fwd_w8_kernel<uint16_t, false><<<grid, 256, 0, st>>>(
        M, N, K, xq, codes, sx, sw, t, B, r, s, reinterpret_cast<uint16_t*>(y),
        nullptr);
}

void launch_gemm_fwd_w4(int M, int N, int K, const uint16_t* x,
                        const uint8_t* packed, const _Float16* scales,
                        const float* t, const float* B, int r, float s,
                        uint16_t* y, hipStream_t st) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  gemm_fwd_w4_kernel<<<grid, 256, 0, st>>>(M, N, K, x, packed, scales, t, B, r,
                                           s, y);
}

}  // namespace qlora
