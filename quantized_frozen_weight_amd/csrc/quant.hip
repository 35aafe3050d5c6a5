// Weight quantizers: one-time preparation of the frozen weight.
//
// Formats ("Introduce QLoRA-like technique", "Highlights": int8 frozen
// kernels; keras-llm-light README, "Simplified Int4Variable quantization":
// two 4-bit values per byte). The abs-max rules are the readings stated in
// include/qlora.h.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, long n) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  long stride = (long)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// ---------------------------------------------------------------------------
// int8 weights, per output channel n (a column of W [K, N]; element (k, n)
// at head_index(k, n, K, hd) when W is stored per head [heads, K, hd]).
// Pass 1: column abs-max as ordered bits, combined across K-slices with an
// integer atomic max (order-independent, hence deterministic). A thread
// covers 4 adjacent columns (N % 16 == 0) of an 8-row slice, all 8 row loads
// in flight at once.
// ---------------------------------------------------------------------------
constexpr int kColmaxRows = 8;

__global__ __launch_bounds__(256) void w8_colmax_kernel(
    const float* __restrict__ W, int K, int N, int hd, uint32_t* __restrict__ amax) {
  const int n = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (n >= N) return;
  const int k0 = blockIdx.y * kColmaxRows;
  f32x4 v[kColmaxRows];
#pragma unroll
  for (int i = 0; i < kColmaxRows; ++i) {
    const int k = k0 + i < K ? k0 + i : K - 1;     // repeats of a real row do not change a max
    v[i] = *reinterpret_cast<const f32x4*>(W + head_index(k, n, K, hd));   // 4 n in one head
  }
  uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kColmaxRows; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t b = abs_bits(v[i][c]);
      m[c] = b > m[c] ? b : m[c];
    }
#pragma unroll
  for (int c = 0; c < 4; ++c) atomicMax(amax + n + c, m[c]);
}

// Pass 2: codes for a 64(k) x 64(n) tile, transposed through LDS so that the
// [N, K] code rows are written 16 bytes at a time.
__global__ __launch_bounds__(256) void w8_codes_kernel(
    const float* __restrict__ W, int K, int N, int hd,
    const uint32_t* __restrict__ amax, int8_t* __restrict__ codes) {
  __shared__ int8_t tile[64][64 + 16];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int tn = threadIdx.x & 63, tk = threadIdx.x >> 6;
  const int n = n0 + tn;
  QuantParams p{0.f, 0.f, false};
  if (n < N) p = absmax_params(amax[n], 127.f);
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    int kl = tk + 4 * i, k = k0 + kl;
    int q = 0;
    if (n < N && k < K && p.live) q = quant_code(W[head_index(k, n, K, hd)], p.inv, 127.f);
    tile[tn][kl] = (int8_t)q;
  }
  __syncthreads();
  const int row = threadIdx.x >> 2, c = threadIdx.x & 3;
  const int nr = n0 + row, kc = k0 + 16 * c;
  if (nr < N && kc < K) {
    *reinterpret_cast<u32x4*>(codes + (long)nr * K + kc) =
        *reinterpret_cast<const u32x4*>(&tile[row][16 * c]);
  }
}

// Pass 3: replace the abs-max bits by the stored scale absmax / 127.
__global__ void w8_scales_kernel(uint32_t* __restrict__ amax_then_scale, int N) {
  int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  QuantParams p = absmax_params(amax_then_scale[n], 127.f);
  amax_then_scale[n] = __float_as_uint(p.scale);
}

// ---------------------------------------------------------------------------
// Merging the adapter into the int8 weight ("Parameter-efficient fine-tuning
// of GPT-2 with LoRA", "Merge weights and generate text!": the merged kernel
// is the frozen one plus the adapter product; "Introduce QLoRA-like
// technique", results-table footnote: merging into int8 is lossy):
//
//   W'[k, n] = fl32( q[n, k] sw[n] + s sum_j A[k, j] B[j, n] )
//
// evaluated in float64 with a fixed sequence: q sw and every A B product are
// exact; the r products are added in index order; one multiply by s, one
// add, one rounding to float32 (explicitly rounded operations, no fused
// multiply-add). W' is then quantized with the int8 rule above. A 64 n x 64 k
// tile per block; a thread owns 16 consecutive k of one row n (one 16-byte
// code load and, in pass 2, one 16-byte code store). W' is recomputed in
// pass 2 rather than stored.
// ---------------------------------------------------------------------------
struct MergeSrc {
  const int8_t* codes;   // [N, K]
  const float* sw;       // [N]
  const float* A;        // [K, r]
  const float* B;        // [r, N], or [heads, r, hd]
  int hd;                // head width of B (N: one head)
  int K, N, r;
  double s;
};

constexpr int kMergeMaxR = 32;

// W' for the thread's 16 k of row n: A [64 k][r] and B [r][64 n] of the tile
// are in LDS.
__device__ __forceinline__ void merged_row16(const MergeSrc& p, const float (*As)[kMergeMaxR + 1],
                                             const float (*Bs)[64], int nl, int kl0, u32x4 qraw,
                                             float swn, float w[16]) {
  const int8_t* q = reinterpret_cast<const int8_t*>(&qraw);
  const double sw64 = (double)swn;
  for (int i = 0; i < 16; ++i) {
    double acc = 0.0;
    for (int j = 0; j < p.r; ++j)
      acc = __dadd_rn(acc, __dmul_rn((double)As[kl0 + i][j], (double)Bs[j][nl]));
    const double d = __dmul_rn((double)q[i], sw64);            // exact
    w[i] = __double2float_rn(__dadd_rn(d, __dmul_rn(p.s, acc)));
  }
}

template <bool CODES>
__global__ __launch_bounds__(256) void merge_kernel(MergeSrc p, uint32_t* __restrict__ amax,
                                                    int8_t* __restrict__ codes_out) {
  __shared__ float As[64][kMergeMaxR + 1];
  __shared__ float Bs[kMergeMaxR][64];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int tid = threadIdx.x, K = p.K, N = p.N, r = p.r;
  for (int e = tid; e < 64 * r; e += 256) {
    const int kl = e / r, j = e % r, k = k0 + kl;
    As[kl][j] = k < K ? p.A[(long)k * r + j] : 0.f;
  }
  for (int e = tid; e < 64 * r; e += 256) {
    const int j = e / 64, nl = e % 64, n = n0 + nl;
    Bs[j][nl] = n < N ? p.B[head_index(j, n, r, p.hd)] : 0.f;
  }
  __syncthreads();
  const int nl = tid >> 2, kl0 = (tid & 3) * 16;
  const int n = n0 + nl, k = k0 + kl0;
  const bool live = n < N && k < K;                 // K % 16 == 0: 16 k all in or out
  u32x4 qraw = {0u, 0u, 0u, 0u};
  float swn = 0.f;
  if (live) {
    qraw = *reinterpret_cast<const u32x4*>(p.codes + (long)n * K + k);
    swn = p.sw[n];
  }
  float w[16];
  merged_row16(p, As, Bs, nl, kl0, qraw, swn, w);
  if constexpr (!CODES) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = abs_bits(w[i]);
      m = b > m ? b : m;
    }
    // the 4 threads of a row are adjacent lanes
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
    if (live && (tid & 3) == 0) atomicMax(amax + n, m);
  } else {
    if (!live) return;
    const QuantParams qp = absmax_params(amax[n], 127.f);
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c = qp.live ? quant_code(w[4 * d + b], qp.inv, 127.f) : 0;
        v |= (uint32_t)(uint8_t)(int8_t)c << (8 * b);
      }
      o[d] = v;
    }
    *reinterpret_cast<u32x4*>(codes_out + (long)n * K + k) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

void launch_merge_w8(const int8_t* codes, const float* sw, const float* A,
                     const float* B, int hd, int K, int N, int r, float s,
                     int8_t* codes_out, float* scales_out, hipStream_t st) {
  MergeSrc p{codes, sw, A, B, hd, K, N, r, (double)s};
  uint32_t* amax = reinterpret_cast<uint32_t*>(scales_out);
  fill_u32_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, 0u, N);
  const dim3 grid((N + 63) / 64, (K + 63) / 64);
  merge_kernel<false><<<grid, 256, 0, st>>>(p, amax, nullptr);
  merge_kernel<true><<<grid, 256, 0, st>>>(p, amax, codes_out);
  w8_scales_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, N);
}

void launch_quantize_w8(const float* W, int K, int N, int hd, int8_t* codes,
                        float* scales, hipStream_t st) {
  uint32_t* amax = reinterpret_cast<uint32_t*>(scales);
  fill_u32_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, 0u, N);
  w8_colmax_kernel<<<dim3((N + 1023) / 1024, (K + kColmaxRows - 1) / kColmaxRows),
                     256, 0, st>>>(W, K, N, hd, amax);
  w8_codes_kernel<<<dim3((N + 63) / 64, (K + 63) / 64), 256, 0, st>>>(
      W, K, N, hd, amax, codes);
  w8_scales_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, N);
}

// ---------------------------------------------------------------------------
// 4-bit weights: one block per (64 output channels, one 128-input group).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4_quant_kernel(
    const float* __restrict__ W, int K, int N, int hd, uint8_t* __restrict__ packed,
    _Float16* __restrict__ scales) {
  __shared__ int8_t tile[64][128 + 16];
  __shared__ uint32_t part[4][64];
  const int n0 = blockIdx.x * 64, g = blockIdx.y, k0 = g * 128;
  const int tn = threadIdx.x & 63, tk = threadIdx.x >> 6;
  const int n = n0 + tn;
  float v[32];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int k = k0 + tk + 4 * i;
    v[i] = (n < N) ? W[head_index(k, n, K, hd)] : 0.f;
    uint32_t b = abs_bits(v[i]);
    m = b > m ? b : m;
  }
  part[tk][tn] = m;
  __syncthreads();
  uint32_t a_bits = part[0][tn];
#pragma unroll
  for (int j = 1; j < 4; ++j) a_bits = part[j][tn] > a_bits ? part[j][tn] : a_bits;
  const float a = __uint_as_float(a_bits);
  // fp16 scale of fl32(a / 7), round to nearest even (overflow -> inf)
  _Float16 s16 = (_Float16)(a / 7.0f);
  float sc = (float)s16;
  bool bad = a_bits >= 0x7f800000u || !(__builtin_fabsf(sc) <= 65504.f);
  bool live = !bad && sc != 0.f;
  float inv = live ? 1.0f / sc : 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    tile[tn][tk + 4 * i] = (int8_t)(live ? quant_code(v[i], inv, 7.f) : 0);
  if (tk == 0 && n < N)
    scales[(long)n * (K / 128) + g] =
        bad ? (_Float16)__uint_as_float(0x7fc00000u) : s16;
  __syncthreads();
  // pack: thread -> (row, 32 codes) -> 16 bytes, even k in the low nibble
  const int row = threadIdx.x >> 2, c = threadIdx.x & 3;
  if (n0 + row < N) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t acc = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        uint32_t nib = (uint32_t)tile[row][32 * c + 8 * d + b] & 0xfu;
        acc |= nib << (4 * b);
      }
      w[d] = acc;
    }
    u32x4 out = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(packed + (long)(n0 + row) * (K / 2) + g * 64 + 16 * c) = out;
  }
}

void launch_quantize_w4(const float* W, int K, int N, int hd, uint8_t* packed,
                        _Float16* scales, hipStream_t st) {
  w4_quant_kernel<<<dim3((N + 63) / 64, K / 128), 256, 0, st>>>(W, K, N, hd, packed,
                                                               scales);
}

}  // namespace qlora
