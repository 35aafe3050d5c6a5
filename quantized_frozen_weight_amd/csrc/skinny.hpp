// Adapter gradients, the reductions over the M rows ("Parameter-efficient
// fine-tuning of GPT-2 with LoRA", "Why does LoRA reduce memory footprint?":
// gradients exist only for the small trainable A and B):
//
//   dB[j, n] = s sum_m t[m, j] dy[m, n]        (P = t, Q = dy, C = N)
//   dA[k, j] = s sum_m x[m, k] u[m, j]         (P = u, Q = x,  C = K, stored [K, r])
//
// Stage 1 (a block type that runs inside another launch): a block owns 256
// columns of one product and one split of the rows; its four waves take a
// quarter of the split each (4 columns per lane; the P row is wave-uniform),
// every load of a group of rows is issued before the first one is used, and
// the waves are added in a fixed order through LDS into the split's partial
// sum. Stage 2 (its own small launch) adds the splits in split order and
// scales by s. No atomics and no cross-block waiting: results are bitwise
// reproducible.
#pragma once
#include "common.hpp"

namespace qlora {

constexpr int kSkCols = 256;       // columns per stage-1 block (64 lanes x 4)
constexpr int kSkMaxSplit = 32;
constexpr int kFinishBatch = 32;   // layers per launch of the batched stage 2
constexpr int kSkGroup = 8;        // rows whose loads are in flight together

struct SkinnyJobs {
  const float* P[2];   // [M, r]
  const void* Q[2];    // [M, C] in the compute dtype
  float* partial[2];   // [nsplit, r, C]
  float* out[2];       // dB [r, C] or dA [C, r]
  int C[2];
  int ncb[2];          // column blocks per job
  int transpose[2];
  int hd0;             // job 0's output (dB): head width ([heads, r, hd]; C[0]: [r, C])
  int njobs, M, r, nsplit, rows_per_split;
  float s;
  int blocks() const { return (ncb[0] + (njobs > 1 ? ncb[1] : 0)) * nsplit; }
};

inline int skinny_nsplit_host(int M) {
  int n = (M + 63) / 64;
  return n < 1 ? 1 : (n > kSkMaxSplit ? kSkMaxSplit : n);
}

__device__ __forceinline__ void sk_load4(const float* p, float q[4]) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
}
__device__ __forceinline__ void sk_load4(const uint16_t* p, float q[4]) {
  u32x2 v = *reinterpret_cast<const u32x2*>(p);
  q[0] = __uint_as_float(v.x << 16); q[1] = __uint_as_float(v.x & 0xffff0000u);
  q[2] = __uint_as_float(v.y << 16); q[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Stage 1 for block b of the skinny grid. Needs 4 * min(R, 4) * 256 floats of
// LDS at red (and two barriers of the whole block).
template <typename T, int R>
__device__ __forceinline__ void skinny_partial_block(const SkinnyJobs& p, int b,
                                                     float* red) {
  constexpr int JC = R < 4 ? R : 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int job = b < p.ncb[0] * p.nsplit ? 0 : 1;
  if (job) b -= p.ncb[0] * p.nsplit;
  const int ncb = p.ncb[job], C = p.C[job], r = p.r;
  const int cb = b % ncb, sp = b / ncb;
  const float* __restrict__ P = p.P[job];
  const auto* __restrict__ Q = reinterpret_cast<const typename Elem<T>::type*>(p.Q[job]);
  const int c0 = cb * kSkCols + 4 * lane;
  const bool col_ok = c0 < C;                // C % 16 == 0: 4 columns all in or out

  float acc[4][R];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[i][j] = 0.f;

  const int q4 = p.rows_per_split / 4;
  const int m0 = sp * p.rows_per_split + w * q4;
  const int m1 = min(p.M, m0 + q4);
  // loads are unconditional from clamped addresses (masked afterwards) so a
  // whole group of rows is in flight at once
  const int cc0 = col_ok ? c0 : 0;
  for (int g0 = m0; g0 < m1; g0 += kSkGroup) {
    float q[kSkGroup][4], pv[kSkGroup][R];
#pragma unroll
    for (int g = 0; g < kSkGroup; ++g) {
      const int m = g0 + g;
      const int mc = m < m1 ? m : m0;
      sk_load4(Q + (long)mc * C + cc0, q[g]);
#pragma unroll
      for (int j = 0; j < R; ++j) pv[g][j] = P[(long)mc * r + (j < r ? j : 0)];
    }
#pragma unroll
    for (int g = 0; g < kSkGroup; ++g) {
      const bool ok = col_ok && g0 + g < m1;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float pj = (ok && j < r) ? pv[g][j] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_fmaf(pj, q[g][i], acc[i][j]);
      }
    }
  }

  // combine the four waves (wave order fixed), JC values of j per round
  float* __restrict__ part = p.partial[job] + (long)sp * r * C;
  const int c = cb * kSkCols + tid;
#pragma unroll
  for (int jb = 0; jb < R; jb += JC) {
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < JC; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(w * JC + jj) * kSkCols + 4 * lane + i] = acc[i][jb + jj];
    __syncthreads();
    if (c < C) {
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        const int j = jb + jj;
        if (j < r) {
          const float v = ((red[(0 * JC + jj) * kSkCols + tid] + red[(1 * JC + jj) * kSkCols + tid]) +
                           red[(2 * JC + jj) * kSkCols + tid]) + red[(3 * JC + jj) * kSkCols + tid];
          part[(long)j * C + c] = v;
        }
      }
    }
  }
}

}  // namespace qlora
