// Row passes (one wave per row, four rows per block), shared by the forward
// prologue and the first backward pass:
//
//   forward:  t[m, :] = x[m, :] A            (adapter down projection, float32)
//             xq, sx  = abs-max int8 codes and scale of row m (int8 weights)
//             as[m]   = sum_k xq[m, k] (optional: the affine weights' bias
//                       term, outlier.hpp)
//   backward: u[m, :] = dy[m, :] B^T         (gradient reaching the adapter)
//             dys     = bf16(dy[m, n] * sw[n])   (int8 weights, bf16 compute:
//                       the channel scale folded into the gradient rows that
//                       the input-gradient product consumes)
//
// Sources: "Parameter-efficient fine-tuning of GPT-2 with LoRA", "LoRA
// equation" / "Create LoRA layer" (the adapter branch B(A x) scaled by
// alpha/r); "Introduce QLoRA-like technique", "Highlights" (int8 frozen
// kernels); the row quantizer and the straight-through backward are the
// readings stated in include/qlora.h.
//
// Latency, not bandwidth, decides these small passes, so every global load a
// block needs is issued before anything waits: the row itself (rows of up
// to 4096 entries stay in registers between the abs-max and the quantize
// pass; forward rows of up to 16384 too, two per block with each wave on a
// quarter of them, or -- with t wanted and scratch given -- split over k in
// two launches; longer rows are streamed twice) and the slice of the
// rank-r matrix that the block's rows share, copied to LDS with 16-byte
// loads (for many short rows each wave takes two or four of them, so one
// LDS read of the adapter serves several rows). In LDS
// a lane that holds 8 consecutive row entries k finds the 8 x R adapter
// values it needs contiguous: A keeps its [k][j] order in groups of 8 rows
// padded by 4 floats (so the 16 lanes of one LDS read land in distinct
// banks); B is kept as [j][k].
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kLdsFloats = 17408;          // 68 KB adapter slice budget
constexpr int kHoldChunks = 8;             // 8 chunks x 8 entries x 64 lanes

enum RowMode { kFwdQuant = 0, kFwdT = 1, kBwd = 2 };

// Slice length (row entries per LDS fill): a multiple of 512 whose grouped
// layout (8 R + 4 floats per 8 entries) fits the budget.
template <int R> struct Slice {
  static constexpr int len = (kLdsFloats / (8 * R + 4)) * 8 / 512 * 512;
  static_assert(len >= 512, "slice too short");
};

template <typename T> struct Raw;
template <> struct Raw<BF16> { u32x4 v; };
template <> struct Raw<F32> { f32x4 a, b; };

__device__ __forceinline__ void raw_load(const uint16_t* p, Raw<BF16>& r) {
  r.v = *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void raw_load(const float* p, Raw<F32>& r) {
  r.a = *reinterpret_cast<const f32x4*>(p);
  r.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void raw_zero(Raw<BF16>& r) { r.v = u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void raw_zero(Raw<F32>& r) {
  r.a = f32x4{0.f, 0.f, 0.f, 0.f};
  r.b = r.a;
}
__device__ __forceinline__ void raw_unpack(const Raw<BF16>& r, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r.v[i] << 16);
    v[2 * i + 1] = __uint_as_float(r.v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_unpack(const Raw<F32>& r, float v[8]) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}

// LDS position of adapter entry (k, j) of the current slice.
template <int R, int MODE>
__device__ __forceinline__ int ws_index(int k, int j, int sld) {
  if constexpr (MODE == kBwd) return j * sld + k;
  else return (k >> 3) * (8 * R + 4) + (k & 7) * R + j;
}

// Copy the slice [s0, s0 + len) of the adapter matrix into LDS.
// MODE < kBwd: A [L, r] row-major; kBwd: B [r, L] row-major, or per head
// [heads, r, hd] (4-float units never straddle a head: hd % 4 == 0).
template <int R, int MODE, int SL = Slice<R>::len>
__device__ __forceinline__ void stage_slice(float* Ws, const float* __restrict__ W,
                                            int L, int r, int s0, int len, int sld, int hd) {
  constexpr int PER = (R * SL / 4 + 255) / 256;     // 16-byte units per thread
  if constexpr (MODE == kBwd) {
    // r rows of len floats
    const int upr = len / 4;                         // units per row
    const int n = r * upr;
    f32x4 v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int u = threadIdx.x + 256 * q;
      const int uc = u < n ? u : n - 1;
      v[q] = *reinterpret_cast<const f32x4*>(W + head_index(uc / upr, s0 + 4 * (uc % upr), r, hd));
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int u = threadIdx.x + 256 * q;
      if (u < n) *reinterpret_cast<f32x4*>(&Ws[(u / upr) * sld + 4 * (u % upr)]) = v[q];
    }
  } else {
    if (R >= 4 && r == R) {
      // the slice of A is contiguous: len * R floats
      const int n = len * R / 4;
      const float* src = W + (long)s0 * R;
      f32x4 v[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int u = threadIdx.x + 256 * q;
        v[q] = *reinterpret_cast<const f32x4*>(src + 4 * (u < n ? u : n - 1));
      }
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int u = threadIdx.x + 256 * q;
        if (u < n) {
          const int k = (4 * u) / R, j = (4 * u) % R;
          *reinterpret_cast<f32x4*>(&Ws[ws_index<R, MODE>(k, j, sld)]) = v[q];
        }
      }
    } else {
      // rank below the padded width (or tiny ranks): element by element
      for (int e = threadIdx.x; e < len * R; e += 256) {
        const int k = e / R, j = e % R;
        Ws[ws_index<R, MODE>(k, j, sld)] = j < r ? W[(long)(s0 + k) * r + j] : 0.f;
      }
    }
  }
}

template <typename T, int R, int MODE, bool HOLD>
__global__ __launch_bounds__(256) void row_kernel(
    const typename Elem<T>::type* __restrict__ rows, int M, int L,
    const float* __restrict__ W, int hd, int r, float* __restrict__ out_r,
    int8_t* __restrict__ xq, float* __restrict__ sx, float* __restrict__ asum,
    const float* __restrict__ sw, uint16_t* __restrict__ dys) {
  constexpr int SL = Slice<R>::len;
  extern __shared__ __attribute__((aligned(16))) float Ws[];
  const int sld = min(SL, (L + 511) / 512 * 512);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const bool live = row < M;
  const auto* xr = rows + (long)row * L;
  const int nchunk = L / 8;
  const bool lowrank = out_r != nullptr;

  // Loads are issued unconditionally from clamped addresses and masked
  // afterwards: predicated loads become branches that make the compiler wait
  // for every outstanding load at each join.
  Raw<T> hold[HOLD ? kHoldChunks : 1];
  if constexpr (HOLD) {
    const auto* xr0 = rows + (long)(live ? row : M - 1) * L;
#pragma unroll
    for (int i = 0; i < kHoldChunks; ++i) {
      const int c = lane + 64 * i;
      raw_load(xr0 + 8 * (c < nchunk ? c : nchunk - 1), hold[i]);
    }
#pragma unroll
    for (int i = 0; i < kHoldChunks; ++i) {
      const int c = lane + 64 * i;
      if (!(live && c < nchunk)) raw_zero(hold[i]);
    }
  }

  QuantParams qp{0.f, 0.f, false};
  int csum = 0;                      // sum of this lane's codes (asum)
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;

  for (int s0 = 0; s0 < L; s0 += SL) {
    const int len = min(SL, L - s0);
    if (s0 > 0) __syncthreads();
    if (lowrank) stage_slice<R, MODE>(Ws, W, L, r, s0, len, sld, hd);
    if (MODE == kFwdQuant && s0 == 0 && live) {
      uint32_t m = 0;
      if constexpr (HOLD) {
#pragma unroll
        for (int i = 0; i < kHoldChunks; ++i) {
          float v[8];
          raw_unpack(hold[i], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) { uint32_t b = abs_bits(v[e]); m = b > m ? b : m; }
        }
      } else {
        for (int c = lane; c < nchunk; c += 64) {
          float v[8];
          load8(xr + 8 * c, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) { uint32_t b = abs_bits(v[e]); m = b > m ? b : m; }
        }
      }
      qp = absmax_params(wave_max_u32(m), 127.f);
    }
    __syncthreads();
    if (!live) continue;
    // one 8-entry chunk: quantize / scale-fold, then accumulate against the
    // LDS slice (cl = chunk index within the slice, c = within the row)
    auto chunk = [&](const float (&v)[8], int c, int cl) {
      if (MODE == kFwdQuant) {
        uint32_t lo = 0, hi = 0;
        if (qp.live) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q0 = quant_code(v[e], qp.inv, 127.f), q1 = quant_code(v[e + 4], qp.inv, 127.f);
            lo |= (uint32_t)(q0 & 0xff) << (8 * e);
            hi |= (uint32_t)(q1 & 0xff) << (8 * e);
            csum += q0 + q1;
          }
        }
        *reinterpret_cast<u32x2*>(xq + (long)row * L + 8 * c) = u32x2{lo, hi};
      }
      if (MODE == kBwd && dys != nullptr) {
        float w[8];
        load8(sw + 8 * c, w);
        u32x4 o = {pack_bf16x2(v[0] * w[0], v[1] * w[1]),
                   pack_bf16x2(v[2] * w[2], v[3] * w[3]),
                   pack_bf16x2(v[4] * w[4], v[5] * w[5]),
                   pack_bf16x2(v[6] * w[6], v[7] * w[7])};
        *reinterpret_cast<u32x4*>(dys + (long)row * L + 8 * c) = o;
      }
      if (!lowrank) return;
      if constexpr (MODE == kBwd) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          if (j >= r) break;
          const f32x4 a = *reinterpret_cast<const f32x4*>(&Ws[j * sld + 8 * cl]);
          const f32x4 b = *reinterpret_cast<const f32x4*>(&Ws[j * sld + 8 * cl + 4]);
          float s = acc[j];
          s = __builtin_fmaf(v[0], a.x, s); s = __builtin_fmaf(v[1], a.y, s);
          s = __builtin_fmaf(v[2], a.z, s); s = __builtin_fmaf(v[3], a.w, s);
          s = __builtin_fmaf(v[4], b.x, s); s = __builtin_fmaf(v[5], b.y, s);
          s = __builtin_fmaf(v[6], b.z, s); s = __builtin_fmaf(v[7], b.w, s);
          acc[j] = s;
        }
      } else {
        const float* g = &Ws[cl * (8 * R + 4)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
          for (int j = 0; j < R; ++j) acc[j] = __builtin_fmaf(v[i], g[i * R + j], acc[j]);
        }
      }
    };
    if constexpr (HOLD) {
      // chunk row i covers entries [512 i, 512 i + 512); SL is a multiple of 512
#pragma unroll
      for (int i = 0; i < kHoldChunks; ++i) {
        const int c = lane + 64 * i;
        if (512 * i < s0 || 512 * i >= s0 + SL || c >= nchunk) continue;
        float v[8];
        raw_unpack(hold[i], v);
        chunk(v, c, c - s0 / 8);
      }
    } else {
      for (int cl = lane; 8 * cl < len; cl += 64) {
        const int c = s0 / 8 + cl;
        float v[8];
        load8(xr + 8 * c, v);
        chunk(v, c, cl);
      }
    }
  }
  if (!live) return;
  if (lowrank) {
    // one butterfly for all R sums; lane l holds rank rank_of_lane(l), and
    // the first lane of each group of 64 / R writes it
    const float tot = wave_sum_ranks<R>(acc);
    const int j = rank_of_lane<R>(lane);
    if ((lane & (64 / R - 1)) == 0 && j < r) out_r[(long)row * r + j] = tot;
  }
  if (MODE == kFwdQuant && lane == 0) sx[row] = qp.scale;
  if (MODE == kFwdQuant && asum != nullptr) {
    // |sum| <= 127 K < 2^24 for the shapes the library takes: exact in float
    const float tot = wave_sum((float)csum);
    if (lane == 0) asum[row] = tot;
  }
}

// ---- long rows (4096 < L <= 16384), forward modes, rank up to 8 ------------
// (with t wanted and scratch given, the split pass below takes these rows)
// Two rows per block. Wave w owns the 512-entry groups g = 4 i + w of both
// rows (entries [512 g, 512 g + 512), one 8-entry chunk per lane), so every
// adapter value read from LDS serves two rows, and the rows stay in
// registers between the abs-max and the quantize pass (read once). The
// adapter comes in slices of 2048 entries: slice i holds group i of every
// wave. The row's abs-max, its code sum and its r sums of x A are combined
// across the four waves through LDS in wave order.
constexpr int kLongRows = 2;
constexpr int kLongHold = 8;               // groups per wave: L <= 4 * 8 * 512
constexpr int kLongMax = 4 * kLongHold * 512;
constexpr int kLongSlice = 2048;
constexpr int kLongMaxRank = 8;

// |v| bits of the largest of a chunk's eight values, as float32 bits
__device__ __forceinline__ uint32_t raw_absmax(const Raw<BF16>& r) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = r.v[i] & 0x7fffu, hi = (r.v[i] >> 16) & 0x7fffu;
    m = lo > m ? lo : m;
    m = hi > m ? hi : m;
  }
  return m << 16;
}
__device__ __forceinline__ uint32_t raw_absmax(const Raw<F32>& r) {
  const float v[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) { const uint32_t b = abs_bits(v[e]); m = b > m ? b : m; }
  return m;
}

template <typename T, int R, int MODE>
__global__ __launch_bounds__(256) void row_long_kernel(
    const typename Elem<T>::type* __restrict__ rows, int M, int L,
    const float* __restrict__ W, int r, float* __restrict__ out_r,
    int8_t* __restrict__ xq, float* __restrict__ sx, float* __restrict__ asum) {
  static_assert(MODE == kFwdQuant || MODE == kFwdT, "forward modes");
  static_assert(R <= kLongMaxRank, "a 2048-entry slice fits the LDS budget");
  constexpr int SL = kLongSlice, RB = kLongRows, NH = kLongHold;
  extern __shared__ __attribute__((aligned(16))) float Ws[];
  __shared__ uint32_t red_max[RB][4];
  __shared__ float red_t[RB][4][R];
  __shared__ float red_c[RB][4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int row0 = blockIdx.x * RB;
  const int nchunk = L / 8;
  const bool lowrank = out_r != nullptr;

  // both rows' chunks, from clamped addresses: a chunk past the row repeats
  // the row's last chunk and a row past M repeats row M - 1, which leaves
  // the abs-max unchanged; neither is stored or summed
  Raw<T> hold[RB][NH];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const int row = row0 + rr;
    const auto* xr = rows + (long)(row < M ? row : M - 1) * L;
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int c = 64 * (4 * i + w) + lane;
      raw_load(xr + 8 * (c < nchunk ? c : nchunk - 1), hold[rr][i]);
    }
  }
  if (lowrank) stage_slice<R, MODE, SL>(Ws, W, L, r, 0, SL, SL, 0);

  QuantParams qp[RB];
  if constexpr (MODE == kFwdQuant) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const uint32_t b = raw_absmax(hold[rr][i]);
        m = b > m ? b : m;
      }
      m = wave_max_u32(m);
      if (lane == 0) red_max[rr][w] = m;
    }
  }
  __syncthreads();                                  // slice 0 and the wave maxima
  if constexpr (MODE == kFwdQuant) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      uint32_t m = red_max[rr][0];
#pragma unroll
      for (int q = 1; q < 4; ++q) m = red_max[rr][q] > m ? red_max[rr][q] : m;
      qp[rr] = absmax_params(m, 127.f);
    }
  }

  int csum[RB];
  float acc[RB][R];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    csum[rr] = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) acc[rr][j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    if (SL * i >= L) break;
    if (i > 0) {
      __syncthreads();                              // slice i - 1 is used
      if (lowrank) stage_slice<R, MODE, SL>(Ws, W, L, r, SL * i, min(SL, L - SL * i), SL, 0);
      __syncthreads();
    }
    const int c = 64 * (4 * i + w) + lane;
    if (c < nchunk) {
      float v[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) raw_unpack(hold[rr][i], v[rr]);
      if constexpr (MODE == kFwdQuant) {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const int row = row0 + rr;
          uint32_t lo = 0, hi = 0;
          if (qp[rr].live) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q0 = quant_code(v[rr][e], qp[rr].inv, 127.f);
              const int q1 = quant_code(v[rr][e + 4], qp[rr].inv, 127.f);
              lo |= (uint32_t)(q0 & 0xff) << (8 * e);
              hi |= (uint32_t)(q1 & 0xff) << (8 * e);
              csum[rr] += q0 + q1;
            }
          }
          if (row < M) *reinterpret_cast<u32x2*>(xq + (long)row * L + 8 * c) = u32x2{lo, hi};
        }
      }
      if (lowrank) {
        const float* gA = &Ws[(c - SL / 8 * i) * (8 * R + 4)];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
          for (int j = 0; j < R; ++j) {
            const float a = gA[e * R + j];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) acc[rr][j] = __builtin_fmaf(v[rr][e], a, acc[rr][j]);
          }
        }
      }
    }
  }

  // per-wave totals, then the four waves added in wave order
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    if (lowrank) {
      const float tot = wave_sum_ranks<R>(acc[rr]);
      const int j = rank_of_lane<R>(lane);
      if ((lane & (64 / R - 1)) == 0) red_t[rr][w][j] = tot;
    }
    if (MODE == kFwdQuant && asum != nullptr) {
      // |sum| <= 127 L < 2^24: exact in float
      const float cs = wave_sum((float)csum[rr]);
      if (lane == 0) red_c[rr][w] = cs;
    }
  }
  __syncthreads();
  if (lowrank && tid < RB * R) {
    const int rr = tid / R, j = tid % R, row = row0 + rr;
    if (row < M && j < r)
      out_r[(long)row * r + j] = ((red_t[rr][0][j] + red_t[rr][1][j]) + red_t[rr][2][j]) + red_t[rr][3][j];
  }
  if constexpr (MODE == kFwdQuant) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int row = row0 + rr;
      if (tid == rr && row < M) {
        sx[row] = qp[rr].scale;
        if (asum != nullptr) asum[row] = ((red_c[rr][0] + red_c[rr][1]) + red_c[rr][2]) + red_c[rr][3];
      }
    }
  }
}

// ---- long rows with the adapter product, split over k ---------------------
// row_long_kernel stages the whole adapter through LDS in every block (512
// KiB for 16384 x 8), one global round trip per 2048-entry slice, so its
// blocks wait on those loads. With t wanted this path splits instead:
//   part: block (g, s) takes rows [RB g, RB g + RB) and the 2048-entry slice
//         s; thread i owns chunk 256 s + i (8 entries) of every row and holds
//         that chunk's 8 x R adapter values in registers for all RB rows.
//         It leaves per (row, slice) the abs-max bits and the r sums of the
//         slice (the four waves' totals added in wave order);
//   fin:  one block per row: the abs-max over the slices, the codes (the row
//         read again), the code sum, and t as the slice sums added in slice
//         order (the t-only mode: a small kernel that adds the slice sums).
// Scratch: abs-max bits [M][S] then slice sums [M][S][R], S = ceil(L / 2048).
constexpr int kSplitSlice = 2048;

template <typename T> constexpr int split_rows() { return std::is_same<T, F32>::value ? 8 : 16; }

template <typename T, int R, int MODE>
__global__ __launch_bounds__(256) void row_split_part_kernel(
    const typename Elem<T>::type* __restrict__ rows, int M, int L,
    const float* __restrict__ W, int r, uint32_t* __restrict__ pmax, float* __restrict__ pt) {
  constexpr int RB = split_rows<T>();
  __shared__ uint32_t red_max[RB][4];
  __shared__ float red_t[RB][4][R];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row0 = blockIdx.x * RB, s = blockIdx.y, S = gridDim.y;
  const int nchunk = L / 8;
  const int c = s * (kSplitSlice / 8) + tid;
  const int cc = c < nchunk ? c : nchunk - 1;

  // every row's chunk from clamped addresses; a chunk past the row is zeroed
  // (no abs-max, no sum), a row past M is computed and not stored
  Raw<T> hold[RB];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const int row = row0 + rr;
    raw_load(rows + (long)(row < M ? row : M - 1) * L + 8 * cc, hold[rr]);
  }
  // the adapter rows k = 8 cc .. 8 cc + 7, ranks past r as zeros
  float a[8][R];
  if (r == R) {
    const f32x4* src = reinterpret_cast<const f32x4*>(W + (long)8 * cc * R);
    f32x4 av[2 * R];
#pragma unroll
    for (int q = 0; q < 2 * R; ++q) av[q] = src[q];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < R; ++j) a[e][j] = av[(e * R + j) / 4][(e * R + j) % 4];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < R; ++j) a[e][j] = j < r ? W[(long)(8 * cc + e) * r + j] : 0.f;
  }
  if (c >= nchunk) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) raw_zero(hold[rr]);
  }

#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    if constexpr (MODE == kFwdQuant) {
      const uint32_t m = wave_max_u32(raw_absmax(hold[rr]));
      if (lane == 0) red_max[rr][w] = m;
    }
    float v[8], acc[R];
    raw_unpack(hold[rr], v);
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j] = __builtin_fmaf(v[e], a[e][j], acc[j]);
    const float tot = wave_sum_ranks<R>(acc);
    if ((lane & (64 / R - 1)) == 0) red_t[rr][w][rank_of_lane<R>(lane)] = tot;
  }
  __syncthreads();
  if (tid < RB * R) {
    const int rr = tid / R, j = tid % R, row = row0 + rr;
    if (row < M)
      pt[((long)row * S + s) * R + j] =
          ((red_t[rr][0][j] + red_t[rr][1][j]) + red_t[rr][2][j]) + red_t[rr][3][j];
  }
  if (MODE == kFwdQuant && tid < RB) {
    const int row = row0 + tid;
    uint32_t m = red_max[tid][0];
#pragma unroll
    for (int q = 1; q < 4; ++q) m = red_max[tid][q] > m ? red_max[tid][q] : m;
    if (row < M) pmax[(long)row * S + s] = m;
  }
}

template <typename T, int R>
__global__ __launch_bounds__(256) void row_split_fin_kernel(
    const typename Elem<T>::type* __restrict__ rows, int M, int L, int r, int S,
    const uint32_t* __restrict__ pmax, const float* __restrict__ pt, float* __restrict__ out_r,
    int8_t* __restrict__ xq, float* __restrict__ sx, float* __restrict__ asum) {
  constexpr int NH = kLongMax / 8 / 256;             // chunks per thread
  __shared__ float red_c[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x;
  const int nchunk = L / 8;
  const auto* xr = rows + (long)row * L;
  Raw<T> hold[NH];
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int c = tid + 256 * i;
    raw_load(xr + 8 * (c < nchunk ? c : nchunk - 1), hold[i]);
  }
  // the row's abs-max from its slices' (each wave reads them all)
  const uint32_t m = wave_max_u32(lane < S ? pmax[(long)row * S + lane] : 0u);
  const QuantParams qp = absmax_params(m, 127.f);
  int csum = 0;
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int c = tid + 256 * i;
    if (c < nchunk) {
      float v[8];
      raw_unpack(hold[i], v);
      uint32_t lo = 0, hi = 0;
      if (qp.live) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q0 = quant_code(v[e], qp.inv, 127.f);
          const int q1 = quant_code(v[e + 4], qp.inv, 127.f);
          lo |= (uint32_t)(q0 & 0xff) << (8 * e);
          hi |= (uint32_t)(q1 & 0xff) << (8 * e);
          csum += q0 + q1;
        }
      }
      *reinterpret_cast<u32x2*>(xq + (long)row * L + 8 * c) = u32x2{lo, hi};
    }
  }
  if (tid < r) {
    const float* p = pt + (long)row * S * R + tid;
    float acc = p[0];
    for (int s = 1; s < S; ++s) acc += p[s * R];
    out_r[(long)row * r + tid] = acc;
  }
  if (tid == 0) sx[row] = qp.scale;
  if (asum != nullptr) {
    // |sum| <= 127 L < 2^24: exact in float
    const float cs = wave_sum((float)csum);
    if (lane == 0) red_c[w] = cs;
    __syncthreads();
    if (tid == 0) asum[row] = ((red_c[0] + red_c[1]) + red_c[2]) + red_c[3];
  }
}

template <int R>
__global__ __launch_bounds__(256) void row_split_tsum_kernel(int M, int r, int S,
                                                              const float* __restrict__ pt,
                                                              float* __restrict__ out_r) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(e / R), j = (int)(e % R);
  if (row >= M || j >= r) return;
  const float* p = pt + (long)row * S * R + j;
  float acc = p[0];
  for (int s = 1; s < S; ++s) acc += p[s * R];
  out_r[(long)row * r + j] = acc;
}

// ---- many short rows, forward modes: RW rows per wave ---------------------
// For grids of more than two blocks per compute unit (the multiple is kept
// at 512 blocks or more: 768-wide rows of 4096 ran faster as 512 blocks of
// two rows per wave than as 256 of four), each wave takes RW
// rows (L <= 512 NHC, held in registers) instead of one, so every adapter
// value read from LDS serves RW rows and a block stages the adapter once for
// 4 RW rows. Same chunk mapping, slices, abs-max and sums as row_kernel, per
// row.
template <typename T, int R, int MODE, int RW, int NHC>
__global__ __launch_bounds__(256) void row_multi_kernel(
    const typename Elem<T>::type* __restrict__ rows, int M, int L,
    const float* __restrict__ W, int r, float* __restrict__ out_r,
    int8_t* __restrict__ xq, float* __restrict__ sx, float* __restrict__ asum) {
  static_assert(MODE == kFwdQuant || MODE == kFwdT, "forward modes");
  constexpr int SL = Slice<R>::len;
  extern __shared__ __attribute__((aligned(16))) float Ws[];
  const int sld = min(SL, (L + 511) / 512 * 512);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int row0 = (blockIdx.x * kRowsPerBlock + w) * RW;
  const int nchunk = L / 8;
  const bool lowrank = out_r != nullptr;

  // chunks from clamped addresses (a chunk past the row repeats its last
  // chunk, a row past M repeats row M - 1: neither changes an abs-max, and
  // neither is stored)
  Raw<T> hold[RW][NHC];
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int row = row0 + q;
    const auto* xr = rows + (long)(row < M ? row : M - 1) * L;
#pragma unroll
    for (int i = 0; i < NHC; ++i) {
      const int c = lane + 64 * i;
      raw_load(xr + 8 * (c < nchunk ? c : nchunk - 1), hold[q][i]);
    }
  }

  QuantParams qp[RW];
  int csum[RW];
  float acc[RW][R];
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    csum[q] = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) acc[q][j] = 0.f;
  }
  for (int s0 = 0; s0 < L; s0 += SL) {
    const int len = min(SL, L - s0);
    if (s0 > 0) __syncthreads();
    if (lowrank) stage_slice<R, MODE>(Ws, W, L, r, s0, len, sld, 0);
    if (MODE == kFwdQuant && s0 == 0) {
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < NHC; ++i) {
          const uint32_t b = raw_absmax(hold[q][i]);
          m = b > m ? b : m;
        }
        qp[q] = absmax_params(wave_max_u32(m), 127.f);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NHC; ++i) {
      const int c = lane + 64 * i;
      if (512 * i < s0 || 512 * i >= s0 + SL || c >= nchunk) continue;
      float v[RW][8];
#pragma unroll
      for (int q = 0; q < RW; ++q) raw_unpack(hold[q][i], v[q]);
      if constexpr (MODE == kFwdQuant) {
#pragma unroll
        for (int q = 0; q < RW; ++q) {
          uint32_t lo = 0, hi = 0;
          if (qp[q].live) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q0 = quant_code(v[q][e], qp[q].inv, 127.f);
              const int q1 = quant_code(v[q][e + 4], qp[q].inv, 127.f);
              lo |= (uint32_t)(q0 & 0xff) << (8 * e);
              hi |= (uint32_t)(q1 & 0xff) << (8 * e);
              csum[q] += q0 + q1;
            }
          }
          if (row0 + q < M) *reinterpret_cast<u32x2*>(xq + (long)(row0 + q) * L + 8 * c) = u32x2{lo, hi};
        }
      }
      if (lowrank) {
        const float* g = &Ws[(c - s0 / 8) * (8 * R + 4)];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
          for (int j = 0; j < R; ++j) {
            const float a = g[e * R + j];
#pragma unroll
            for (int q = 0; q < RW; ++q) acc[q][j] = __builtin_fmaf(v[q][e], a, acc[q][j]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int row = row0 + q;
    if (lowrank) {
      const float tot = wave_sum_ranks<R>(acc[q]);
      const int j = rank_of_lane<R>(lane);
      if ((lane & (64 / R - 1)) == 0 && j < r && row < M) out_r[(long)row * r + j] = tot;
    }
    if constexpr (MODE == kFwdQuant) {
      if (lane == 0 && row < M) sx[row] = qp[q].scale;
      if (asum != nullptr) {
        // |sum| <= 127 L < 2^24: exact in float
        const float cs = wave_sum((float)csum[q]);
        if (lane == 0 && row < M) asum[row] = cs;
      }
    }
  }
}

// Rows per wave of the forward row pass for L <= 4096: doubled while the
// grid keeps at least one block per compute unit, up to 4 (2 at rank 16 or
// for float32 rows, 1 at rank 32), and to at most 16 held chunks per lane
// (NHC chunks per row), so that the held rows and the sums fit in registers.
template <typename T, int R>
constexpr int row_multi_max() {
  constexpr int byr = R <= 8 ? 4 : R <= 16 ? 2 : 1;
  return std::is_same<T, F32>::value ? (byr > 1 ? byr / 2 : 1) : byr;
}

template <typename T, int R, int MODE, int RW>
void row_multi_launch(int nhc, dim3 grid, size_t lds, const typename Elem<T>::type* p, int M,
                      int L, const float* W, int r, float* out_r, int8_t* xq, float* sx,
                      float* asum, hipStream_t st) {
  if (nhc <= 2)
    row_multi_kernel<T, R, MODE, RW, 2><<<grid, 256, lds, st>>>(p, M, L, W, r, out_r, xq, sx, asum);
  else if (nhc <= 4)
    row_multi_kernel<T, R, MODE, RW, 4><<<grid, 256, lds, st>>>(p, M, L, W, r, out_r, xq, sx, asum);
  else if constexpr (RW <= 2)
    row_multi_kernel<T, R, MODE, RW, 8><<<grid, 256, lds, st>>>(p, M, L, W, r, out_r, xq, sx, asum);
}

template <typename T, int R, int MODE>
void row_launch(const void* rows, int M, int L, const float* W, int hd, int r,
                float* out_r, int8_t* xq, float* sx, float* asum, const float* sw,
                uint16_t* dys, float* scratch, hipStream_t st) {
  dim3 grid((M + kRowsPerBlock - 1) / kRowsPerBlock);
  const auto* p = reinterpret_cast<const typename Elem<T>::type*>(rows);
  constexpr int SL = Slice<R>::len;
  const int sld = SL < (L + 511) / 512 * 512 ? SL : (L + 511) / 512 * 512;
  size_t lds = 0;
  if (out_r != nullptr)
    lds = (MODE == kBwd ? (size_t)R * sld : (size_t)(sld / 8) * (8 * R + 4)) * sizeof(float);
  if constexpr (MODE != kBwd && R <= kLongMaxRank) {
    if (L > kHoldChunks * 512 && L <= kLongMax && out_r != nullptr && scratch != nullptr) {
      const int S = (L + kSplitSlice - 1) / kSplitSlice;
      uint32_t* pmax = reinterpret_cast<uint32_t*>(scratch);
      float* pt = scratch + (size_t)M * S;
      constexpr int RB = split_rows<T>();
      row_split_part_kernel<T, R, MODE><<<dim3((M + RB - 1) / RB, S), 256, 0, st>>>(p, M, L, W, r, pmax, pt);
      if constexpr (MODE == kFwdQuant)
        row_split_fin_kernel<T, R><<<M, 256, 0, st>>>(p, M, L, r, S, pmax, pt, out_r, xq, sx, asum);
      else
        row_split_tsum_kernel<R><<<(unsigned)(((long)M * R + 255) / 256), 256, 0, st>>>(M, r, S, pt, out_r);
      return;
    }
    if (L > kHoldChunks * 512 && L <= kLongMax) {
      const size_t ldsl = out_r != nullptr ? (size_t)(kLongSlice / 8) * (8 * R + 4) * sizeof(float) : 0;
      const dim3 lgrid((M + kLongRows - 1) / kLongRows);
      row_long_kernel<T, R, MODE><<<lgrid, 256, ldsl, st>>>(p, M, L, W, r, out_r, xq, sx, asum);
      return;
    }
  }
  if constexpr (MODE != kBwd) {
    if (L <= kHoldChunks * 512) {
      constexpr int RWM = row_multi_max<T, R>();
      const int nhc = L <= 1024 ? 2 : L <= 2048 ? 4 : 8;   // held chunks per row
      int rw = 1;
      while (rw < RWM && rw * 2 * nhc <= 16 && (M + 8 * rw - 1) / (8 * rw) >= 512) rw *= 2;
      if (rw > 1) {
        const dim3 mgrid((M + kRowsPerBlock * rw - 1) / (kRowsPerBlock * rw));
        if constexpr (RWM >= 2)
          if (rw == 2)
            row_multi_launch<T, R, MODE, 2>(nhc, mgrid, lds, p, M, L, W, r, out_r, xq, sx, asum, st);
        if constexpr (RWM >= 4)
          if (rw == 4)
            row_multi_launch<T, R, MODE, 4>(nhc, mgrid, lds, p, M, L, W, r, out_r, xq, sx, asum, st);
        return;
      }
      // one row per wave, rows of at most 2048 entries: the same pass with
      // the held chunks sized to the row (row_kernel holds 8 per lane and
      // loads them all)
      if (nhc < kHoldChunks) {
        row_multi_launch<T, R, MODE, 1>(nhc, grid, lds, p, M, L, W, r, out_r, xq, sx, asum, st);
        return;
      }
    }
  }
  if (L <= kHoldChunks * 512)
    row_kernel<T, R, MODE, true><<<grid, 256, lds, st>>>(p, M, L, W, hd, r, out_r, xq, sx,
                                                         asum, sw, dys);
  else
    row_kernel<T, R, MODE, false><<<grid, 256, lds, st>>>(p, M, L, W, hd, r, out_r, xq, sx,
                                                          asum, sw, dys);
}

template <typename T, int MODE>
void row_dispatch_r(int r, const void* rows, int M, int L, const float* W, int hd,
                    float* out_r, int8_t* xq, float* sx, float* asum, const float* sw,
                    uint16_t* dys, hipStream_t st, float* scratch = nullptr) {
  if (r <= 1) row_launch<T, 1, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
  else if (r <= 2) row_launch<T, 2, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
  else if (r <= 4) row_launch<T, 4, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
  else if (r <= 8) row_launch<T, 8, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
  else if (r <= 16) row_launch<T, 16, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
  else row_launch<T, 32, MODE>(rows, M, L, W, hd, r, out_r, xq, sx, asum, sw, dys, scratch, st);
}

}  // namespace

size_t row_split_floats(int M, int K, int r) {
  if (K <= kHoldChunks * 512 || K > kLongMax || r > kLongMaxRank) return 0;
  const int R = r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : 8;   // row_dispatch_r's rank
  const size_t S = (K + kSplitSlice - 1) / kSplitSlice;
  return (size_t)M * S * (1 + R);
}

void launch_rowquant(int dtype, const void* x, int M, int K, const float* A,
                     int r, int8_t* xq, float* sx, float* t, hipStream_t st,
                     float* asum, float* scratch) {
  const int rr = t == nullptr ? 1 : r;
  if (dtype == 0)
    row_dispatch_r<F32, kFwdQuant>(rr, x, M, K, A, K, t, xq, sx, asum, nullptr, nullptr, st, scratch);
  else
    row_dispatch_r<BF16, kFwdQuant>(rr, x, M, K, A, K, t, xq, sx, asum, nullptr, nullptr, st, scratch);
}

void launch_lora_down(int dtype, const void* x, int M, int K, const float* A,
                      int r, float* t, hipStream_t st, float* scratch) {
  if (dtype == 0)
    row_dispatch_r<F32, kFwdT>(r, x, M, K, A, K, t, nullptr, nullptr, nullptr, nullptr, nullptr, st, scratch);
  else
    row_dispatch_r<BF16, kFwdT>(r, x, M, K, A, K, t, nullptr, nullptr, nullptr, nullptr, nullptr, st, scratch);
}

void launch_bwd_rows(int dtype, const void* dy, int M, int N, const float* B, int hd,
                     int r, const float* sw, uint16_t* dys, float* u,
                     hipStream_t st) {
  if (dtype == 0)
    row_dispatch_r<F32, kBwd>(r, dy, M, N, B, hd, u, nullptr, nullptr, nullptr, sw, nullptr, st);
  else
    row_dispatch_r<BF16, kBwd>(r, dy, M, N, B, hd, u, nullptr, nullptr, nullptr, sw, dys, st);
}

}  // namespace qlora
