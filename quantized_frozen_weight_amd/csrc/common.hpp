// Shared device helpers for libqlora (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace qlora {

constexpr int kWave = 64;

// ---- dtype tags -----------------------------------------------------------
struct F32 {};   // float32 activations / gradients
struct BF16 {};  // bfloat16 activations / gradients (stored as uint16_t)

template <typename T> struct Elem;
template <> struct Elem<F32> { typedef float type; static constexpr int bytes = 4; };
template <> struct Elem<BF16> { typedef uint16_t type; static constexpr int bytes = 2; };

// ---- bfloat16 ---------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Small integers (|v| < 256) are exact in bfloat16: take the upper half of
// the float32 pattern, no rounding needed.
__device__ __forceinline__ uint32_t pack_int_bf16x2(int lo, int hi) {
  return (__float_as_uint((float)lo) >> 16) |
         (__float_as_uint((float)hi) & 0xffff0000u);
}

// ---- 8-element loads/stores of a row in either dtype -----------------------
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16(v);
}

// ---- multi-head layouts ---------------------------------------------------
// Element (row, n) of an array stored [heads][rows][hd] with heads = N / hd,
// n = head * hd + d ("Parameter-efficient fine-tuning of GPT-2 with LoRA",
// "Create LoRA layer": the adapter's B keeps the attention projection's
// per-head output shape). With hd = N it is the plain row-major [rows][N].
__device__ __forceinline__ long head_index(int row, int n, int rows, int hd) {
  const int h = n / hd;
  return ((long)h * rows + row) * hd + (n - h * hd);
}

// ---- wave reductions ---------------------------------------------------------
// Sums of R per-lane values over the 64 lanes in one butterfly: the first
// log2 R levels pair lanes across bit 5, 4, 3, ... and each lane keeps half of
// its values (those of its side of the pair) plus the partner's matching
// half; the remaining levels are plain sums. Lane l ends with the total of
// value rank_of_lane<R>(l). The cross-lane steps are v_permlane32_swap and
// v_permlane16_swap (bits 5 and 4), then DPP within rows of 16: row_mirror
// (bit 3), row_half_mirror (bit 2), quad_perm [3,2,1,0] (bit 1) and
// [1,0,3,2] (bit 0) -- each pairs lanes that differ in that bit. Fixed order:
// the same inputs give the same bits.
template <int R>
__device__ __forceinline__ int rank_of_lane(int lane) {
  int j = 0;
#pragma unroll
  for (int b = 0, h = R / 2; h >= 1; ++b, h >>= 1) j += ((lane >> (5 - b)) & 1) ? h : 0;
  return j;
}

__device__ __forceinline__ float dpp_pair(float v, int ctrl_id) {
  // ctrl_id: 0 row_mirror, 1 row_half_mirror, 2 quad_perm [3,2,1,0], 3 quad_perm [1,0,3,2]
  const int iv = __builtin_bit_cast(int, v);
  int r;
  if (ctrl_id == 0) r = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xf, 0xf, false);
  else if (ctrl_id == 1) r = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xf, 0xf, false);
  else if (ctrl_id == 2) r = __builtin_amdgcn_update_dpp(0, iv, 0x1b, 0xf, 0xf, false);
  else r = __builtin_amdgcn_update_dpp(0, iv, 0xb1, 0xf, 0xf, false);
  return __builtin_bit_cast(float, r);
}

template <int R>
__device__ __forceinline__ float wave_sum_ranks(const float (&in)[R]) {
  static_assert(R >= 1 && R <= 32 && (R & (R - 1)) == 0, "R a power of two up to 32");
  const int lane = threadIdx.x & 63;
  float v[R];
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = in[i];
  int n = R;
  // level 0: lanes l and l ^ 32
  {
    const int h = n > 1 ? n / 2 : 1;
#pragma unroll
    for (int i = 0; i < (R > 1 ? R / 2 : 1); ++i) {
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[n > 1 ? i + h : i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(a, b, false, false);
      v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    n = n > 1 ? n / 2 : 1;
  }
  // level 1: lanes l and l ^ 16
  {
    const int h = n > 1 ? n / 2 : 1;
#pragma unroll
    for (int i = 0; i < (R > 2 ? R / 4 : 1); ++i) {
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[n > 1 ? i + h : i]);
      const auto sw = __builtin_amdgcn_permlane16_swap(a, b, false, false);
      v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    n = n > 1 ? n / 2 : 1;
  }
  // levels 2..5 inside rows of 16: bit 3, 2, 1, 0
#pragma unroll
  for (int lvl = 0; lvl < 4; ++lvl) {
    const bool upper = (lane >> (3 - lvl)) & 1;
    if (n > 1) {
      const int h = n / 2;
#pragma unroll
      for (int i = 0; i < R / 8 + 1; ++i) {
        if (i < h) {
          const float keep = upper ? v[i + h] : v[i];
          const float send = upper ? v[i] : v[i + h];
          v[i] = keep + dpp_pair(send, lvl);
        }
      }
      n = h;
    } else {
      v[0] = v[0] + dpp_pair(v[0], lvl);
    }
  }
  return v[0];
}

// All-lane max and sum over the 64 lanes by the same butterfly (every lane
// ends with the result). The sum is used only on integer-valued floats below
// 2^24, which add exactly in any order.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = s32[0] > s32[1] ? s32[0] : s32[1];
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = s16[0] > s16[1] ? s16[0] : s16[1];
#pragma unroll
  for (int lvl = 0; lvl < 4; ++lvl) {
    const uint32_t w = __float_as_uint(dpp_pair(__uint_as_float(v), lvl));
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  const uint32_t b = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const uint32_t c = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(c, c, false, false);
  v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
#pragma unroll
  for (int lvl = 0; lvl < 4; ++lvl) v += dpp_pair(v, lvl);
  return v;
}

// ---- abs-max quantizer shared by weights and activations ----------------------
// |v| as an ordered integer: for non-negative floats the bit patterns sort like
// the values, and every NaN pattern sorts above +inf, so an integer max over
// |v| yields NaN when any element is NaN.
__device__ __forceinline__ uint32_t abs_bits(float v) {
  return __float_as_uint(v) & 0x7fffffffu;
}

struct QuantParams {
  float inv;    // 127 / absmax (meaningful only when live)
  float scale;  // stored scale: absmax / 127, 0, or NaN
  bool live;    // false -> every code is 0
};

// One float32 divide each for the inverse and the scale; see the header for
// the zero / overflow / non-finite rules.
__device__ __forceinline__ QuantParams absmax_params(uint32_t amax_bits,
                                                     float qmax) {
  QuantParams p;
  float a = __uint_as_float(amax_bits);
  if (amax_bits >= 0x7f800000u) {  // inf or NaN
    p.inv = 0.f; p.scale = __uint_as_float(0x7fc00000u); p.live = false;
    return p;
  }
  float inv = qmax / a;
  if (amax_bits == 0u || __float_as_uint(inv) >= 0x7f800000u) {
    p.inv = 0.f; p.scale = 0.f; p.live = false;
    return p;
  }
  p.inv = inv; p.scale = a / qmax; p.live = true;
  return p;
}

__device__ __forceinline__ int quant_code(float v, float inv, float qmax) {
  float q = __builtin_rintf(v * inv);   // v_rndne_f32: ties to even
  q = fminf(fmaxf(q, -qmax), qmax);
  return (int)q;
}

}  // namespace qlora
