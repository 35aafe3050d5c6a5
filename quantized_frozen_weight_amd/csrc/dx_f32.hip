// float32 input gradient through the frozen int8 weight (straight-through
// past the activation quantizer, "How to fine-tune the 4-bit model?": the
// gradient needs the product with the transposed quantized matrix):
//     dx[m, k] = sum_n (dy[m, n] * sw[n]) q[n, k] + s sum_j u[m, j] A[k, j]
// Plain LDS-tiled FMA kernel, no reduced-precision rounding anywhere; used
// for the float32 compute dtype (small layers).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

// ---------------------------------------------------------------------------
// 32 x 32 output tile per block (small layers still spread over many compute
// units), contraction in slices of 128 n (small layers are latency-bound:
// each slice is one round trip to memory), each thread a 2 x 2 register
// tile. The next slice is fetched into registers (16-byte loads from
// clamped addresses, masked when used) while the current one is used, and
// nothing consumes the fetched values before the slice's products are done.
// dy * sw is formed once per element (one float32 rounding) as it goes to
// LDS, then multiplied by the exact integer code.
// ---------------------------------------------------------------------------
constexpr int kT = 32, kS = 128;

__global__ __launch_bounds__(256) void gemm_dx_f32_kernel(
    int M, int K, int N, const float* __restrict__ dy,
    const int8_t* __restrict__ codes, const float* __restrict__ sw,
    const float* __restrict__ u, const float* __restrict__ A, int r, float s,
    float* __restrict__ dx) {
  __shared__ float Ds[kS][kT + 1];   // [n][m]
  __shared__ float Ws[kS][kT + 1];   // [n][k]
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kT, k0 = blockIdx.x * kT;
  const int tm = tid >> 4, tk = tid & 15;      // outputs rows 2 tm + i, cols 2 tk + j
  // loader roles per slice: dy rows tid / 32 + 8 p, 4 n from 4 (tid % 32);
  // code rows (n) tid / 8 + 32 p, 4 k from 4 (tid % 8); p = 0..3
  const int lm = tid >> 5, ln = (tid & 31) * 4;
  const int wn = tid >> 3, wk = (tid & 7) * 4;
  // N and K are multiples of 16, so a thread's 4 consecutive n (or k) are
  // all inside or all outside
  f32x4 dv[4], swv;
  uint32_t wv[4];
  bool okn = false, okw[4];
  auto fetch = [&](int n0) {
    const int gn = n0 + ln;
    okn = gn < N;
    const int gnc = okn ? gn : 0;
    swv = *reinterpret_cast<const f32x4*>(sw + gnc);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int gm = m0 + lm + 8 * p;
      dv[p] = *reinterpret_cast<const f32x4*>(dy + (long)(gm < M ? gm : M - 1) * N + gnc);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int gw = n0 + wn + 32 * p, gk = k0 + wk;
      okw[p] = gw < N && gk < K;
      wv[p] = *reinterpret_cast<const uint32_t*>(codes + (long)(gw < N ? gw : 0) * K + (gk < K ? gk : 0));
    }
  };
  float acc[2][2] = {};
  fetch(0);
  for (int n0 = 0; n0 < N; n0 += kS) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool ok = okn && m0 + lm + 8 * p < M;
#pragma unroll
      for (int i = 0; i < 4; ++i) Ds[ln + i][lm + 8 * p] = ok ? dv[p][i] * swv[i] : 0.f;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Ws[wn + 32 * p][wk + i] = okw[p] ? (float)(((int)(wv[p] << (24 - 8 * i))) >> 24) : 0.f;
    __syncthreads();
    if (n0 + kS < N) fetch(n0 + kS);
#pragma unroll 8
    for (int n = 0; n < kS; ++n) {
      const float a0 = Ds[n][2 * tm], a1 = Ds[n][2 * tm + 1];
      const float b0 = Ws[n][2 * tk], b1 = Ws[n][2 * tk + 1];
      acc[0][0] = __builtin_fmaf(a0, b0, acc[0][0]);
      acc[0][1] = __builtin_fmaf(a0, b1, acc[0][1]);
      acc[1][0] = __builtin_fmaf(a1, b0, acc[1][0]);
      acc[1][1] = __builtin_fmaf(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 2 * tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + 2 * tk + j;
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
  dim3 grid((K + kT - 1) / kT, (M + kT - 1) / kT);
  gemm_dx_f32_kernel<<<grid, 256, 0, st>>>(M, K, N, dy, codes, sw, u, A, r, s,
                                           dx);
}

}  // namespace qlora
