// Rank-r pieces of the backward ("Parameter-efficient fine-tuning of GPT-2
// with LoRA", "Why does LoRA reduce memory footprint?": gradients exist only
// for the small trainable A and B):
//
//   u  = dy B^T                 one wave per row, reduction along N
//   dB = s t^T dy,  dA = s x^T u    reductions over the M rows
//
// The M reductions are split into fixed 64-row chunks whose partial sums are
// added in chunk order by a second kernel, so results are bitwise
// reproducible (no float atomics).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int kSplitRows = 64;

// u[m, j] = sum_n dy[m, n] B[j, n]; optionally dys[m, n] = bf16(dy * sw[n])
// (the per-channel weight scale folded into the gradient for the input-
// gradient product).
template <typename T, int RMAX, bool DYS>
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const typename Elem<T>::type* __restrict__ dy, int M, int N,
    const float* __restrict__ B, int r, const float* __restrict__ sw,
    uint16_t* __restrict__ dys, float* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const auto* g = dy + (long)row * N;
  float acc[RMAX];
#pragma unroll
  for (int j = 0; j < RMAX; ++j) acc[j] = 0.f;
  for (int c = lane; c < N / 8; c += 64) {
    float v[8];
    load8(g + 8 * c, v);
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      if (j < r) {
        float b[8];
        load8(B + (long)j * N + 8 * c, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j] = __builtin_fmaf(v[i], b[i], acc[j]);
      }
    }
    if (DYS) {
      float w[8];
      load8(sw + 8 * c, w);
      u32x4 o = {pack_bf16x2(v[0] * w[0], v[1] * w[1]),
                 pack_bf16x2(v[2] * w[2], v[3] * w[3]),
                 pack_bf16x2(v[4] * w[4], v[5] * w[5]),
                 pack_bf16x2(v[6] * w[6], v[7] * w[7])};
      *reinterpret_cast<u32x4*>(dys + (long)row * N + 8 * c) = o;
    }
  }
#pragma unroll
  for (int j = 0; j < RMAX; ++j) {
    if (j < r) {
      float sum = wave_sum(acc[j]);
      if (lane == 0) u[(long)row * r + j] = sum;
    }
  }
}

template <typename T, bool DYS>
void bwd_rows_dispatch(const void* dy, int M, int N, const float* B, int r,
                       const float* sw, uint16_t* dys, float* u, hipStream_t st) {
  dim3 grid((M + 3) / 4);
  const auto* g = reinterpret_cast<const typename Elem<T>::type*>(dy);
  if (r <= 4) bwd_rows_kernel<T, 4, DYS><<<grid, 256, 0, st>>>(g, M, N, B, r, sw, dys, u);
  else if (r <= 8) bwd_rows_kernel<T, 8, DYS><<<grid, 256, 0, st>>>(g, M, N, B, r, sw, dys, u);
  else if (r <= 16) bwd_rows_kernel<T, 16, DYS><<<grid, 256, 0, st>>>(g, M, N, B, r, sw, dys, u);
  else bwd_rows_kernel<T, 32, DYS><<<grid, 256, 0, st>>>(g, M, N, B, r, sw, dys, u);
}

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }

// partial[split][j][c] = sum over the split's rows of P[m, j] Q[m, c]
template <typename T, int RMAX>
__global__ __launch_bounds__(256) void skinny_partial_kernel(
    int M, int r, int C, const float* __restrict__ P,
    const typename Elem<T>::type* __restrict__ Q, float* __restrict__ partial) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int split = blockIdx.y;
  if (c >= C) return;
  const int m0 = split * kSplitRows, m1 = min(M, m0 + kSplitRows);
  float acc[RMAX];
#pragma unroll
  for (int j = 0; j < RMAX; ++j) acc[j] = 0.f;
  for (int m = m0; m < m1; ++m) {
    const float q = load1(Q + (long)m * C + c);
#pragma unroll
    for (int j = 0; j < RMAX; ++j)
      if (j < r) acc[j] = __builtin_fmaf(P[(long)m * r + j], q, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < RMAX; ++j)
    if (j < r) partial[((long)split * r + j) * C + c] = acc[j];
}

// out = s * (sum of the splits in order)
__global__ __launch_bounds__(256) void skinny_reduce_kernel(
    int nsplit, int r, int C, const float* __restrict__ partial, float s,
    float* __restrict__ out, int transpose_out) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)r * C) return;
  const int j = (int)(e / C), c = (int)(e % C);
  float sum = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) sum += partial[((long)sp * r + j) * C + c];
  const float v = s * sum;
  if (transpose_out) out[(long)c * r + j] = v;
  else out[(long)j * C + c] = v;
}

template <typename T>
void skinny_dispatch(int M, int r, int C, const float* P, const void* Q,
                     float* partial, hipStream_t st) {
  const int nsplit = (M + kSplitRows - 1) / kSplitRows;
  dim3 grid((C + 255) / 256, nsplit);
  const auto* q = reinterpret_cast<const typename Elem<T>::type*>(Q);
  if (r <= 4) skinny_partial_kernel<T, 4><<<grid, 256, 0, st>>>(M, r, C, P, q, partial);
  else if (r <= 8) skinny_partial_kernel<T, 8><<<grid, 256, 0, st>>>(M, r, C, P, q, partial);
  else if (r <= 16) skinny_partial_kernel<T, 16><<<grid, 256, 0, st>>>(M, r, C, P, q, partial);
  else skinny_partial_kernel<T, 32><<<grid, 256, 0, st>>>(M, r, C, P, q, partial);
}

}  // namespace

void launch_bwd_rows(int dtype, const void* dy, int M, int N, const float* B,
                     int r, const float* sw, uint16_t* dys, float* u,
                     hipStream_t st) {
  if (dtype == 0) bwd_rows_dispatch<F32, false>(dy, M, N, B, r, sw, dys, u, st);
  else if (dys != nullptr) bwd_rows_dispatch<BF16, true>(dy, M, N, B, r, sw, dys, u, st);
  else bwd_rows_dispatch<BF16, false>(dy, M, N, B, r, sw, dys, u, st);
}

size_t skinny_partial_floats(int M, int r, int C) {
  const size_t nsplit = (size_t)((M + kSplitRows - 1) / kSplitRows);
  return nsplit * (size_t)r * (size_t)C;
}

void launch_skinny(int dtype, int M, int r, int C, const float* P,
                   const void* Q, float s, float* out, bool transpose_out,
                   float* partial, hipStream_t st) {
  if (dtype == 0) skinny_dispatch<F32>(M, r, C, P, Q, partial, st);
  else skinny_dispatch<BF16>(M, r, C, P, Q, partial, st);
  const int nsplit = (M + kSplitRows - 1) / kSplitRows;
  const long total = (long)r * C;
  skinny_reduce_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, st>>>(
      nsplit, r, C, partial, s, out, transpose_out ? 1 : 0);
}

}  // namespace qlora
