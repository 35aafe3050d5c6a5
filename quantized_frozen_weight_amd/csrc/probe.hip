// Measurement probes (include/qlora_probe.h): kernels whose work is known
// exactly, for re-measuring on the machine itself the peaks that the
// roofline of the layer's kernels is taken against, and the launch floor.
// None of them is part of the layer's computation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "qlora_probe.h"

namespace qlora {

namespace {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Each wave keeps 8 independent accumulators and issues `iters` rounds of 8
// MFMAs, so the matrix pipe always has independent work queued. The
// operands are derived from the block index (never constant-folded), and
// every accumulator is folded into one value per lane that is stored, so no
// product can be dropped.
__global__ __launch_bounds__(256) void mfma_bf16_probe(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  const float seed = (float)(blockIdx.x & 7) * 0.125f + (float)lane * 0.001f;
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{seed, seed + 0.5f}, b2));
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w, w ^ 0x00010000u, w, w});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{w ^ 1u, w, w, w ^ 0x00010001u});
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_i8_probe(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  const int v = (int)(blockIdx.x * 131u + (unsigned)lane * 7u) & 0x3f3f3f3f;
  const i32x4_t a = i32x4_t{v, v ^ 0x01010101, v, v};
  const i32x4_t b = i32x4_t{v ^ 0x02020202, v, v, v};
  i32x4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = i32x4_t{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[i], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

// Streaming copy: 16-byte loads and stores, each thread 4 chunks per round
// of the grid-stride loop (n16 = bytes / 16, a multiple of 4 * threads).
__global__ __launch_bounds__(256) void copy_probe(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, long n16) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * stride < n16 ? src[i + u * stride] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n16) dst[i + u * stride] = v[u];
  }
}

// Read-only stream: 16-byte loads folded with xor, one 16-byte store per
// thread at the end.
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ src, long n16,
                                                  u32x4* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * stride < n16 ? src[i + u * stride] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  out[(long)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void empty_probe(int never, int* sink) {
  if (never == 0x5eed1e55 && threadIdx.x == 0) sink[0] = 1;
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : 5; }

}  // namespace
}  // namespace qlora

extern "C" {

int qlora_probe_mfma(int kind, int blocks, int iters, void* out, void* stream,
                     double* ops) {
  if (blocks < 1 || iters < 1 || out == nullptr || ops == nullptr) return 1;
  if (kind != QLORA_PROBE_BF16 && kind != QLORA_PROBE_I8) return 1;
  if (hipPeekAtLastError() != hipSuccess) return 5;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // 16 x 16 x 32 (bf16) or 16 x 16 x 64 (int8) multiply-adds per MFMA, two
  // operations each; 4 waves x 8 MFMAs per round
  const double per = kind == QLORA_PROBE_BF16 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 64;
  *ops = per * 8.0 * 4.0 * (double)blocks * (double)iters;
  if (kind == QLORA_PROBE_BF16)
    qlora::mfma_bf16_probe<<<blocks, 256, 0, s>>>(iters, static_cast<float*>(out));
  else
    qlora::mfma_i8_probe<<<blocks, 256, 0, s>>>(iters, static_cast<float*>(out));
  return qlora::status_of(hipGetLastError());
}

int qlora_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16384 || blocks < 1) return 1;
  if (hipPeekAtLastError() != hipSuccess) return 5;
  qlora::copy_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (long)(bytes / 16));
  return qlora::status_of(hipGetLastError());
}

int qlora_probe_read(const void* src, size_t bytes, int blocks, void* out, void* stream) {
  if (!src || !out || bytes == 0 || bytes % 16384 || blocks < 1) return 1;
  if (hipPeekAtLastError() != hipSuccess) return 5;
  qlora::read_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), (long)(bytes / 16), static_cast<u32x4*>(out));
  return qlora::status_of(hipGetLastError());
}

int qlora_probe_empty(int blocks, int threads, void* stream) {
  if (blocks < 1 || threads < 1 || threads > 1024) return 1;
  if (hipPeekAtLastError() != hipSuccess) return 5;
  qlora::empty_probe<<<blocks, threads, 0, static_cast<hipStream_t>(stream)>>>(0, nullptr);
  return qlora::status_of(hipGetLastError());
}

}  // extern "C"
