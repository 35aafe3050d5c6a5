// Weight quantizers (one-time preparation of the frozen weight) and the
// forward prologue: per-row activation quantization fused with the LoRA down
// projection t = x A.
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
// int8 weights, per output channel n (a column of W [K, N]).
// Pass 1: column abs-max as ordered bits, combined across K-slices with an
// integer atomic max (order-independent, hence deterministic).
// ---------------------------------------------------------------------------
constexpr int kColmaxRows = 256;

__global__ __launch_bounds__(256) void w8_colmax_kernel(
    const float* __restrict__ W, int K, int N, uint32_t* __restrict__ amax) {
  int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  int k0 = blockIdx.y * kColmaxRows;
  int k1 = min(K, k0 + kColmaxRows);
  uint32_t m = 0;
  for (int k = k0; k < k1; ++k) {
    uint32_t b = abs_bits(W[(long)k * N + n]);
    m = b > m ? b : m;
  }
  atomicMax(amax + n, m);
}

// Pass 2: codes for a 64(k) x 64(n) tile, transposed through LDS so that the
// [N, K] code rows are written 16 bytes at a time.
__global__ __launch_bounds__(256) void w8_codes_kernel(
    const float* __restrict__ W, int K, int N,
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
    if (n < N && k < K && p.live) q = quant_code(W[(long)k * N + n], p.inv, 127.f);
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

void launch_quantize_w8(const float* W, int K, int N, int8_t* codes,
                        float* scales, hipStream_t st) {
  uint32_t* amax = reinterpret_cast<uint32_t*>(scales);
  fill_u32_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, 0u, N);
  w8_colmax_kernel<<<dim3((N + 255) / 256, (K + kColmaxRows - 1) / kColmaxRows),
                     256, 0, st>>>(W, K, N, amax);
  w8_codes_kernel<<<dim3((N + 63) / 64, (K + 63) / 64), 256, 0, st>>>(
      W, K, N, amax, codes);
  w8_scales_kernel<<<dim3((N + 255) / 256), 256, 0, st>>>(amax, N);
}

// ---------------------------------------------------------------------------
// 4-bit weights: one block per (64 output channels, one 128-input group).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4_quant_kernel(
    const float* __restrict__ W, int K, int N, uint8_t* __restrict__ packed,
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
    v[i] = (n < N) ? W[(long)k * N + n] : 0.f;
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

void launch_quantize_w4(const float* W, int K, int N, uint8_t* packed,
                        _Float16* scales, hipStream_t st) {
  w4_quant_kernel<<<dim3((N + 63) / 64, K / 128), 256, 0, st>>>(W, K, N, packed,
                                                               scales);
}

// ---------------------------------------------------------------------------
// Forward prologue, one wave per row:
//   pass 1: row abs-max (integer max of |x| bits, NaN-propagating)
//   pass 2: codes xq = rint(x * 127/absmax), scale sx = absmax/127, and the
//           adapter down projection t[m, :] = x[m, :] A in float32.
// With QUANT = false only t is produced (4-bit forward; backward recompute).
// ---------------------------------------------------------------------------
template <typename T, int RMAX, bool QUANT>
__global__ __launch_bounds__(256) void rowquant_kernel(
    const typename Elem<T>::type* __restrict__ x, int M, int K,
    const float* __restrict__ A, int r, int8_t* __restrict__ xq,
    float* __restrict__ sx, float* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const auto* xr = x + (long)row * K;
  const int nchunk = K / 8;
  QuantParams p{0.f, 0.f, false};
  if (QUANT) {
    uint32_t m = 0;
    for (int c = lane; c < nchunk; c += 64) {
      float v[8];
      load8(xr + 8 * c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t b = abs_bits(v[i]);
        m = b > m ? b : m;
      }
    }
    m = wave_max_u32(m);
    p = absmax_params(m, 127.f);
  }
  float acc[RMAX];
#pragma unroll
  for (int j = 0; j < RMAX; ++j) acc[j] = 0.f;
  for (int c = lane; c < nchunk; c += 64) {
    float v[8];
    load8(xr + 8 * c, v);
    if (QUANT) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t q0 = p.live ? (uint32_t)(quant_code(v[i], p.inv, 127.f) & 0xff) : 0u;
        uint32_t q1 = p.live ? (uint32_t)(quant_code(v[i + 4], p.inv, 127.f) & 0xff) : 0u;
        lo |= q0 << (8 * i);
        hi |= q1 << (8 * i);
      }
      u32x2 pk = {lo, hi};
      *reinterpret_cast<u32x2*>(xq + (long)row * K + 8 * c) = pk;
    }
    if (t != nullptr) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* a = A + (long)(8 * c + i) * r;
#pragma unroll
        for (int j = 0; j < RMAX; ++j)
          if (j < r) acc[j] = __builtin_fmaf(v[i], a[j], acc[j]);
      }
    }
  }
  if (t != nullptr) {
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      if (j < r) {
        float s = wave_sum(acc[j]);
        if (lane == 0) t[(long)row * r + j] = s;
      }
    }
  }
  if (QUANT && lane == 0) sx[row] = p.scale;
}

template <typename T, bool QUANT>
static void rowquant_dispatch(const void* x, int M, int K, const float* A, int r,
                              int8_t* xq, float* sx, float* t, hipStream_t st) {
  dim3 grid((M + 3) / 4);
  const auto* xp = reinterpret_cast<const typename Elem<T>::type*>(x);
  if (t == nullptr || r <= 4)
    rowquant_kernel<T, 4, QUANT><<<grid, 256, 0, st>>>(xp, M, K, A, r, xq, sx, t);
  else if (r <= 8)
    rowquant_kernel<T, 8, QUANT><<<grid, 256, 0, st>>>(xp, M, K, A, r, xq, sx, t);
  else if (r <= 16)
    rowquant_kernel<T, 16, QUANT><<<grid, 256, 0, st>>>(xp, M, K, A, r, xq, sx, t);
  else
    rowquant_kernel<T, 32, QUANT><<<grid, 256, 0, st>>>(xp, M, K, A, r, xq, sx, t);
}

void launch_rowquant(int dtype, const void* x, int M, int K, const float* A,
                     int r, int8_t* xq, float* sx, float* t, hipStream_t st) {
  if (dtype == 0) rowquant_dispatch<F32, true>(x, M, K, A, r, xq, sx, t, st);
  else rowquant_dispatch<BF16, true>(x, M, K, A, r, xq, sx, t, st);
}

void launch_lora_down(int dtype, const void* x, int M, int K, const float* A,
                      int r, float* t, hipStream_t st) {
  if (dtype == 0) rowquant_dispatch<F32, false>(x, M, K, A, r, nullptr, nullptr, t, st);
  else rowquant_dispatch<BF16, false>(x, M, K, A, r, nullptr, nullptr, t, st);
}

}  // namespace qlora
