// Shared epilogue of the 128 x 128 MFMA tiles: low-rank term added to the
// product, one rounding to the output dtype.
//
//   out[m, n] = fma(s, sum_j P[m, j] Q(j, n), base(acc[m, n]))
//   base      = float(acc) * (rs[m] * cs[n])   when rs != nullptr
//             = acc                             otherwise
//
// P is float32 [M, r] (row-major); Q(j, n) = Q[j * ldj + n * ldn] so the same
// code serves B [r, N] (forward: ldj = N, ldn = 1) and A [K, r] read as its
// transpose (input gradient: ldj = 1, ldn = r).
#pragma once
#include "common.hpp"

namespace qlora {

// 16x16 MFMA accumulator layout (wave64): lane l holds rows 4 (l / 16) + ii,
// ii = 0..3, of column l % 16.
template <int TM, int TN, typename OutT, typename AccT>
__device__ __forceinline__ void tile_epilogue(
    const AccT (&acc)[4][4], int M, int N, int m0, int n0, int wm, int wn,
    int lane, const float* __restrict__ rs, const float* __restrict__ cs,
    const float* __restrict__ P, const float* __restrict__ Q, long ldj,
    long ldn, int r, float s, float* ts, float* qs, OutT* __restrict__ out) {
  for (int e = threadIdx.x; e < TM * r; e += blockDim.x) {
    int gm = m0 + e / r;
    ts[e] = gm < M ? P[(long)gm * r + e % r] : 0.f;
  }
  for (int e = threadIdx.x; e < r * TN; e += blockDim.x) {
    int gn = n0 + e % TN;
    qs[e] = gn < N ? Q[(long)(e / TN) * ldj + (long)gn * ldn] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = wn * 64 + j * 16 + (lane & 15);
    const int n = n0 + nl;
    if (n >= N) continue;
    const float csn = cs != nullptr ? cs[n] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int ml = wm * 64 + i * 16 + (lane >> 4) * 4 + ii;
        const int m = m0 + ml;
        if (m >= M) continue;
        float low = 0.f;
        for (int jj = 0; jj < r; ++jj)
          low = __builtin_fmaf(ts[ml * r + jj], qs[jj * TN + nl], low);
        float base;
        if (rs != nullptr) base = (float)acc[i][j][ii] * (rs[m] * csn);
        else base = (float)acc[i][j][ii];
        store_out(out + (long)m * N + n, __builtin_fmaf(s, low, base));
      }
    }
  }
}

}  // namespace qlora
