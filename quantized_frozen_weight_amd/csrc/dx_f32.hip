// float32 input gradient through the frozen int8 weight (straight-through
// past the activation quantizer, "How to fine-tune the 4-bit model?": the
// gradient needs the product with the transposed quantized matrix):
//     dx[m, k] = sum_n (dy[m, n] * sw[n]) q[n, k] + s sum_j u[m, j] A[k, j]
// Plain LDS-tiled FMA kernel, no reduced-precision rounding anywhere; used
// for the float32 compute dtype.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

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

void launch_gemm_dx_f32(int M, int K, int N, const float* dy,
                        const int8_t* codes, const float* sw, const float* u,
                        const float* A, int r, float s, float* dx,
                        hipStream_t st) {
  dim3 grid((K + 63) / 64, (M + 63) / 64);
  gemm_dx_f32_kernel<<<grid, 256, 0, st>>>(M, K, N, dy, codes, sw, u, A, r, s,
                                           dx);
}

}  // namespace qlora
