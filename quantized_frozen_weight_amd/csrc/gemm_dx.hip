// Input gradient through the frozen weight (straight-through past the
// activation quantizer):
//     dx[m, k] = sum_n dy[m, n] deq(W)[k, n] + s sum_j u[m, j] A[k, j]
// This is the product with the transposed quantized matrix that "How to
// fine-tune the 4-bit model?" names as the missing piece for adapter
// training; the frozen weight itself receives no gradient ("Parameter-
// efficient fine-tuning of GPT-2 with LoRA", "Create LoRA layer").
//
// bf16 path (int8 codes): the per-channel scale sw[n] is folded into the
// gradient rows (dys = bf16(dy * sw), produced by the backward row pass), so
// the weight operand is the raw codes, which are exact in bf16. The codes are
// stored [N, K] (K contiguous) but the contraction runs over n, so each block
// transposes its [64 n x 128 k] code slice while widening it to bf16 on the
// way into LDS ([k][n], n contiguous). MFMA v_mfma_f32_16x16x32_bf16.
//
// 4-bit path: same structure, nibbles unpacked and multiplied by their fp16
// group scale (which depends on k and n, so it cannot be folded into dy),
// rounded to bf16 in LDS.
//
// float32 path: plain LDS-tiled FMA kernel (no bf16 rounding anywhere).
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int BM = 128, BN = 128;   // rows of dy, columns of dx (k)
constexpr int BKN = 64;             // contraction slice (n) per stage
constexpr int P16 = BKN + 8;        // LDS row pitch in bf16 elements

template <bool W4>
__global__ __launch_bounds__(256, 1) void gemm_dx_kernel(
    int M, int K, int N, const uint16_t* __restrict__ g,   // dys or dy [M, N]
    const void* __restrict__ wcodes, const _Float16* __restrict__ scales,
    const float* __restrict__ u, const float* __restrict__ A, int r, float s,
    uint16_t* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * P16];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * P16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * BM, k0 = blockIdx.x * BN;
  // gradient slice: 128 rows x 64 n: row c / 8, 8 elements at 8 (c % 8)
  const int arow = tid >> 3, acol = (tid & 7) * 8;

  u32x4 ra[4];
  uint32_t rb[8];
  float bsc[8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // int8: thread -> k quad kq = tid % 32 (k = 4 kq .. 4 kq + 3), n octet
  // no = tid / 32 (n = 8 no .. 8 no + 7): eight dword loads, one per n row.
  // 4-bit: thread -> k octet ko = tid % 16 (k = 8 ko .. +7, one dword of
  // nibbles), n quad nq = tid / 16 (n = 4 nq .. +3): four dword loads.
  auto gload = [&](int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gm = m0 + arow + 32 * i, gn = n0 + acol;
      ra[i] = (gm < M && gn < N)
                  ? *reinterpret_cast<const u32x4*>(g + (long)gm * N + gn) : zero;
    }
    if (!W4) {
      const int8_t* codes = reinterpret_cast<const int8_t*>(wcodes);
      const int kq = tid & 31, no = tid >> 5;
      const int gk = k0 + 4 * kq;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gn = n0 + 8 * no + i;
        rb[i] = (gn < N && gk < K)
                    ? *reinterpret_cast<const uint32_t*>(codes + (long)gn * K + gk) : 0u;
      }
    } else {
      const uint8_t* packed = reinterpret_cast<const uint8_t*>(wcodes);
      const int ko = tid & 15, nq = tid >> 4;
      const int gk = k0 + 8 * ko;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gn = n0 + 4 * nq + i;
        const bool ok = gn < N && gk < K;
        rb[i] = ok ? *reinterpret_cast<const uint32_t*>(packed + (long)gn * (K / 2) + gk / 2)
                   : 0u;
        bsc[i] = ok ? (float)scales[(long)gn * (K / 128) + gk / 128] : 0.f;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][(arow + 32 * i) * P16 + acol]) = ra[i];
    if (!W4) {
      const int kq = tid & 31, no = tid >> 5;
#pragma unroll
      for (int jk = 0; jk < 4; ++jk) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          int q0 = ((int)(rb[2 * p] << (24 - 8 * jk))) >> 24;
          int q1 = ((int)(rb[2 * p + 1] << (24 - 8 * jk))) >> 24;
          o[p] = pack_int_bf16x2(q0, q1);
        }
        u32x4 ov = {o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4*>(&Bs[buf][(4 * kq + jk) * P16 + 8 * no]) = ov;
      }
    } else {
      const int ko = tid & 15, nq = tid >> 4;
#pragma unroll
      for (int jk = 0; jk < 8; ++jk) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int q = ((int)(rb[i] << (28 - 4 * jk))) >> 28;
          v[i] = (float)q * bsc[i];
        }
        u32x2 ov = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(&Bs[buf][(8 * ko + jk) * P16 + 4 * nq]) = ov;
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (N + BKN - 1) / BKN;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BKN);
#pragma unroll
    for (int kk = 0; kk < BKN / 32; ++kk) {
      bf16x8 af[4], bf[4];
      const int off = kk * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &As[cur][(wm * 64 + i * 16 + (lane & 15)) * P16 + off]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * P16 + off]);
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
  // dx[m, k] = acc + s sum_j u[m, j] A[k, j]   (A [K, r] read transposed)
  tile_epilogue<BM, BN, uint16_t>(acc, M, K, m0, k0, wm, wn, lane, nullptr,
                                  nullptr, u, A, 1, r, r, s,
                                  reinterpret_cast<float*>(&As[0][0]),
                                  reinterpret_cast<float*>(&Bs[0][0]), dx);
}

// ---------------------------------------------------------------------------
// float32 input gradient: 64 x 64 output tile, 16-wide contraction slices,
// each thread a 4 x 4 register tile. dy * sw is formed once per element (one
// float32 rounding), then multiplied by the exact integer code.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_dx_f32_kernel(
    int M, int K, int N, const float* __restrict__ dy,
    const int8_t* __restrict__ codes, const float* __restrict__ sw,
    const float* __restrict__ u, const float* __restrict__ A, int r, float s,
    float* __restrict__ dx) {
  __shared__ float Ds[16][64 + 4];   // [n][m]
  __shared__ float Ws[16][64 + 4];   // [n][k]
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const int tm = tid >> 4, tk = tid & 15;
  float acc[4][4] = {};
  for (int n0 = 0; n0 < N; n0 += 16) {
    {
      const int ml = tid >> 2, nq = (tid & 3) * 4;
      const int gm = m0 + ml;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gn = n0 + nq + i;
        Ds[nq + i][ml] = (gm < M && gn < N) ? dy[(long)gm * N + gn] * sw[gn] : 0.f;
      }
      const int nl = tid >> 4, kq = (tid & 15) * 4;
      const int gn = n0 + nl, gk = k0 + kq;
      uint32_t w = (gn < N && gk < K)
                       ? *reinterpret_cast<const uint32_t*>(codes + (long)gn * K + gk) : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Ws[nl][kq + i] = (float)(((int)(w << (24 - 8 * i))) >> 24);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = Ds[n][4 * tm + i]; b[i] = Ws[n][4 * tk + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + 4 * tk + j;
      if (k >= K) continue;
      float low = 0.f;
      for (int jj = 0; jj < r; ++jj)
        low = __builtin_fmaf(u[(long)m * r + jj], A[(long)k * r + jj], low);
      dx[(long)m * K + k] = __builtin_fmaf(s, low, acc[i][j]);
    }
  }
}

}  // namespace

void launch_gemm_dx_w8(int M, int K, int N, const uint16_t* dys,
                       const int8_t* codes, const float* u, const float* A,
                       int r, float s, uint16_t* dx, hipStream_t st) {
  dim3 grid((K + BN - 1) / BN, (M + BM - 1) / BM);
  gemm_dx_kernel<false><<<grid, 256, 0, st>>>(M, K, N, dys, codes, nullptr, u,
                                              A, r, s, dx);
}

void launch_gemm_dx_w4(int M, int K, int N, const uint16_t* dy,
                       const uint8_t* packed, const _Float16* scales,
                       const float* u, const float* A, int r, float s,
                       uint16_t* dx, hipStream_t st) {
  dim3 grid((K + BN - 1) / BN, (M + BM - 1) / BM);
  gemm_dx_kernel<true><<<grid, 256, 0, st>>>(M, K, N, dy, packed, scales, u, A,
                                             r, s, dx);
}

void launch_gemm_dx_f32(int M, int K, int N, const float* dy,
                        const int8_t* codes, const float* sw, const float* u,
                        const float* A, int r, float s, float* dx,
                        hipStream_t st) {
  dim3 grid((K + 63) / 64, (M + 63) / 64);
  gemm_dx_f32_kernel<<<grid, 256, 0, st>>>(M, K, N, dy, codes, sw, u, A, r, s,
                                           dx);
}

}  // namespace qlora
