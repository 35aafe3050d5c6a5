// Quantization into the outlier-compensated int8 format (outlier.hpp;
// keras-llm-light README, "Simplified Int8Variable quantization": cut at the
// 0.1th and 99.9th percentiles, affine 8-bit codes for the clipped weight,
// fp16 values kept for the elements outside the cut).
//
// 1. Exact selection of the two cut values (the elements of nearest rank
//    ceil(n / 1000) and ceil(999 n / 1000) among n = K N) by a three-pass
//    radix select over order-preserving float keys: each pass builds a
//    histogram of the next 11 (11, 10) key bits among the elements that share
//    the prefix found so far (block-private LDS histograms, integer atomics),
//    and one small block picks the bin holding the wanted rank. The last pick
//    also fixes the grid: scale = fl32(d / 255), inverse fl32(255 / d) with
//    d = fl32(hi - lo).
// 2. One wave per 64 x 64 tile of W [K, N] counts the outliers of every row
//    (ballot over the tile's 64 columns), of every 16-row group and of every
//    16-column quarter.
// 3. Prefix sums: per row over the column tiles, then three exclusive scans
//    (rows, backward cells, forward cells), one block each.
// 4. The same tiles again: each lane writes its column's 64 codes as four
//    16-byte stores into codes [N, K] (the transposed layout), and every
//    outlier is written at its precomputed place in the three lists.
// Every count is an integer sum and every list position is fixed by (k, n),
// so the result does not depend on the launch configuration.
#include "common.hpp"
#include "launch.hpp"
#include "outlier.hpp"

namespace qlora {

namespace {

// Unsigned order of the keys is the order of the values: negative values
// have all bits inverted, non-negative ones get the sign bit set.
__device__ __forceinline__ uint32_t order_key(float w) {
  const uint32_t u = __float_as_uint(w);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int PASS> struct SelPass;
template <> struct SelPass<0> { static constexpr int shift = 21, width = 11; };
template <> struct SelPass<1> { static constexpr int shift = 10, width = 11; };
template <> struct SelPass<2> { static constexpr int shift = 0, width = 10; };

__global__ __launch_bounds__(256) void sel_init(W8OHeader* h, uint32_t* hist, long long n,
                                                int cap) {
  for (int i = threadIdx.x; i < 2 * kSelBins; i += 256) hist[i] = 0u;
  if (threadIdx.x == 0) {
    const long long r_lo = (n + 999) / 1000, r_hi = (999 * n + 999) / 1000;   // 1-based
    h->rem[0] = (int)((r_lo > 1 ? r_lo : 1) - 1);
    h->rem[1] = (int)((r_hi > 1 ? r_hi : 1) - 1);
    h->key[0] = 0u;
    h->key[1] = 0u;
    h->cap = cap;
    h->nnz = 0;
  }
}

// Histogram of key bits [shift, shift + width) over the elements whose
// higher bits equal the prefix of target t (pass 0: one histogram, no
// prefix).
template <int PASS>
__global__ __launch_bounds__(256) void sel_hist(const float* __restrict__ W, long long n4,
                                                const W8OHeader* __restrict__ h,
                                                uint32_t* __restrict__ hist) {
  constexpr int SH = SelPass<PASS>::shift, WD = SelPass<PASS>::width, NB = 1 << WD;
  constexpr int NT = PASS == 0 ? 1 : 2;
  __shared__ uint32_t hs[NT * NB];
  for (int i = threadIdx.x; i < NT * NB; i += 256) hs[i] = 0u;
  uint32_t pfx0 = 0u, pfx1 = 0u;
  if constexpr (PASS > 0) {
    pfx0 = h->key[0] >> (SH + WD);
    pfx1 = h->key[1] >> (SH + WD);
  }
  __syncthreads();
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const f32x4 v = reinterpret_cast<const f32x4*>(W)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = order_key(v[e]);
      const uint32_t bin = (key >> SH) & (NB - 1);
      if constexpr (PASS == 0) {
        atomicAdd(&hs[bin], 1u);
      } else {
        const uint32_t top = key >> (SH + WD);
        if (top == pfx0) atomicAdd(&hs[bin], 1u);
        if (top == pfx1) atomicAdd(&hs[NB + bin], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NT * NB; i += 256) {
    const uint32_t c = hs[i];
    if (c) atomicAdd(&hist[(i / NB) * kSelBins + (i % NB)], c);
  }
}

// Find, for each target, the bin that holds its remaining rank; extend the
// key prefix and reduce the rank. Clears the histograms for the next pass.
// After the last pass: the cut values and the grid.
template <int PASS>
__global__ __launch_bounds__(256) void sel_pick(W8OHeader* h, uint32_t* hist) {
  constexpr int SH = SelPass<PASS>::shift, WD = SelPass<PASS>::width, NB = 1 << WD;
  constexpr int PER = NB / 256;
  __shared__ uint32_t part[256];
  __shared__ uint32_t fkey[2];
  __shared__ int frem[2];
  const int tid = threadIdx.x;
  if (tid < 2) {
    fkey[tid] = 0u;
    frem[tid] = 0;
  }
  for (int t = 0; t < 2; ++t) {
    const uint32_t* H = hist + (PASS == 0 ? 0 : t * kSelBins);
    uint32_t loc[PER], s = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      loc[j] = H[tid * PER + j];
      s += loc[j];
    }
    part[tid] = s;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const uint32_t v = tid >= o ? part[tid - o] : 0u;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const uint32_t incl = part[tid], excl = incl - s;
    const uint32_t rem = (uint32_t)h->rem[t];
    if (rem >= excl && rem < incl) {
      uint32_t c = excl;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (rem < c + loc[j]) {
          fkey[t] = (uint32_t)(tid * PER + j) << SH;
          frem[t] = (int)(rem - c);
          break;
        }
        c += loc[j];
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < 2 * kSelBins; i += 256) hist[i] = 0u;
  if (tid == 0) {
    h->key[0] |= fkey[0];
    h->key[1] |= fkey[1];
    h->rem[0] = frem[0];
    h->rem[1] = frem[1];
    if constexpr (PASS == 2) {
      const float lo = key_float(h->key[0]), hi = key_float(h->key[1]);
      const float d = hi - lo;
      float inv = 255.f / d, scale = d / 255.f;
      if (!(d > 0.f) || !__builtin_isfinite(d) || !__builtin_isfinite(inv)) {
        inv = 0.f;
        scale = 0.f;
      }
      h->lo = lo;
      h->hi = hi;
      h->scale = scale;
      h->inv = inv;
      h->bias_q = lo + 128.f * scale;
    }
  }
}

// W [K, N] rows of one 64 x 64 tile into registers: lane = column n, entry kk
// = row k0 + kk (rows past K and columns past N read a valid neighbour; the
// caller masks them).
__device__ __forceinline__ void load_tile(const float* __restrict__ W, int K, int N, int k0,
                                          int n, float (&wv)[64]) {
  const int nc = n < N ? n : N - 1;
#pragma unroll
  for (int kk = 0; kk < 64; ++kk) {
    const int k = k0 + kk < K ? k0 + kk : K - 1;
    wv[kk] = W[(long)k * N + nc];
  }
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Pass 2: outlier counts of one tile per wave.
//   cnt_r[nt][k]   outliers of row k among the tile column's 64 n
//   bcell[nt][kg]  the same summed over 16 rows
//   fcnt[kt][g]    outliers of the tile's 16-column quarter g over its 64 rows
__global__ __launch_bounds__(256) void outlier_count(const float* __restrict__ W,
                                                     const W8OHeader* __restrict__ h,
                                                     W8OLayout L, char* __restrict__ side) {
  const int lane = threadIdx.x & 63;
  const int id = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (id >= L.nkt * L.nnb) return;
  const int K = L.K, N = L.N;
  const int kt = id / L.nnb, nt = id % L.nnb;
  const int k0 = kt * 64, n = nt * 64 + lane, rows = K - k0 < 64 ? K - k0 : 64;
  const bool vn = n < N;
  float wv[64];
  load_tile(W, K, N, k0, n, wv);
  const float lo = h->lo, hi = h->hi;
  int* cnt_r = reinterpret_cast<int*>(side + L.cnt_r);
  int* bcell = reinterpret_cast<int*>(side + L.bcell);
  int* fcnt = reinterpret_cast<int*>(side + L.fcnt);
  int mine = 0, grp = 0, gq[4] = {0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < 64; ++kk) {
    if (kk < rows) {
      const float w = wv[kk];
      const bool o = vn && (w < lo || w > hi);
      const uint64_t mask = __ballot(o);
      const int c = __popcll(mask);
      if (lane == kk) mine = c;
      grp += c;
#pragma unroll
      for (int q = 0; q < 4; ++q) gq[q] += __popc((uint32_t)(mask >> (16 * q)) & 0xffffu);
      if ((kk & 15) == 15) {
        if (lane == 0) bcell[nt * L.kg + kt * 4 + (kk >> 4)] = grp;
        grp = 0;
      }
    }
  }
  if (lane < rows) cnt_r[(long)nt * K + k0 + lane] = mine;
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * nt + q < L.ng) fcnt[kt * L.ng + 4 * nt + q] = gq[q];
  }
}

// Pass 3a: per row k, the exclusive prefix of cnt_r over the column tiles
// (in place) and the row total; per forward cell (kb, g), the sum of its two
// 64-row tiles.
__global__ __launch_bounds__(256) void outlier_prep(W8OLayout L, char* __restrict__ side) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  int* cnt_r = reinterpret_cast<int*>(side + L.cnt_r);
  int* rowtot = reinterpret_cast<int*>(side + L.rowtot);
  const int* fcnt = reinterpret_cast<const int*>(side + L.fcnt);
  int* fcell = reinterpret_cast<int*>(side + L.fcell);
  if (i < L.K) {
    int run = 0;
    for (int nt = 0; nt < L.nnb; ++nt) {
      const long at = (long)nt * L.K + i;
      const int v = cnt_r[at];
      cnt_r[at] = run;
      run += v;
    }
    rowtot[i] = run;
  }
  if (i < L.nkb * L.ng) {
    const int kb = i / L.ng, g = i % L.ng;
    fcell[i] = fcnt[(2 * kb) * L.ng + g] + (2 * kb + 1 < L.nkt ? fcnt[(2 * kb + 1) * L.ng + g] : 0);
  }
}

struct ScanJobs {
  const int* in[3];
  int* out[3];
  int len[3];
  W8OHeader* h;
};

// Pass 3b: out[i] = sum of in[0 .. i) for i <= len (out[len] = total), one
// block per job; job 0 (the rows) also records the outlier count.
__global__ __launch_bounds__(1024) void outlier_scan(ScanJobs j) {
  const int* in = j.in[blockIdx.x];
  int* out = j.out[blockIdx.x];
  const int L = j.len[blockIdx.x];
  const int tid = threadIdx.x;
  const int per = (L + 1023) / 1024, b = tid * per, e = b + per < L ? b + per : L;
  __shared__ int part[1024];
  int s = 0;
  for (int i = b; i < e; ++i) s += in[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int i = b; i < e; ++i) {
    const int v = in[i];
    out[i] = run;
    run += v;
  }
  if (tid == 1023) {
    out[L] = part[1023];
    if (blockIdx.x == 0) j.h->nnz = part[1023];
  }
}

// Pass 4: codes and the three outlier lists, one tile per wave.
__global__ __launch_bounds__(256) void outlier_fill(const float* __restrict__ W,
                                                    const W8OHeader* __restrict__ h,
                                                    W8OLayout L, char* __restrict__ side,
                                                    int8_t* __restrict__ codes) {
  const int lane = threadIdx.x & 63;
  const int id = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (id >= L.nkt * L.nnb) return;
  const int K = L.K, N = L.N, cap = L.cap;
  const int kt = id / L.nnb, nt = id % L.nnb;
  const int k0 = kt * 64, n = nt * 64 + lane, rows = K - k0 < 64 ? K - k0 : 64;
  const bool vn = n < N;
  float wv[64];
  load_tile(W, K, N, k0, n, wv);
  const float lo = h->lo, hi = h->hi, inv = h->inv, scale = h->scale, bias_q = h->bias_q;

  const int* rowptr = reinterpret_cast<const int*>(side + L.rowptr);
  const int* rpre = reinterpret_cast<const int*>(side + L.cnt_r);
  const int* bptr = reinterpret_cast<const int*>(side + L.bptr);
  const int* fptr = reinterpret_cast<const int*>(side + L.fptr);
  const int* fcnt = reinterpret_cast<const int*>(side + L.fcnt);
  int* col = reinterpret_cast<int*>(side + L.col);
  uint16_t* val = reinterpret_cast<uint16_t*>(side + L.val);
  u32x2* fent = reinterpret_cast<u32x2*>(side + L.fent);
  u32x2* bent = reinterpret_cast<u32x2*>(side + L.bent);

  // list bases: lane j holds row j's CSR start; lanes 0..3 the backward
  // cells of the tile's 16-row groups, and the forward cells of its
  // 16-column quarters (plus the first 64-row tile of a 128-row cell)
  const int rbase = lane < rows ? rowptr[k0 + lane] + rpre[(long)nt * K + k0 + lane] : 0;
  const int bbase = (lane < 4 && 16 * lane < rows) ? bptr[nt * L.kg + kt * 4 + lane] : 0;
  int fbase = 0;
  if (lane < 4 && 4 * nt + lane < L.ng) {
    const int g = 4 * nt + lane;
    fbase = fptr[(kt >> 1) * L.ng + g] + ((kt & 1) ? fcnt[(kt - 1) * L.ng + g] : 0);
  }
  const int quarter = lane >> 4;

  uint32_t cw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cw[i] = 0u;
  int runB = 0, runF[4] = {0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < 64; ++kk) {
    if (kk < rows) {
      const float w = wv[kk];
      const bool o = vn && (w < lo || w > hi);
      const float c = fminf(fmaxf(w, lo), hi);
      float v = __builtin_rintf((c - lo) * inv);
      v = fminf(fmaxf(v, 0.f), 255.f);
      const int q = (int)v - 128;
      cw[kk >> 2] |= (uint32_t)(q & 0xff) << (8 * (kk & 3));
      const uint64_t mask = __ballot(o);
      if (mask != 0) {
        const int below = lanes_below(mask);
        // outliers of the lanes of lower quarters
        const int lower = __popcll(mask & ((1ull << (16 * quarter)) - 1ull));
        if (o) {
          const int k = k0 + kk;
          const _Float16 v16 = (_Float16)w;
          const float vf = (float)v16;
          const int pos = __builtin_amdgcn_readlane(rbase, kk) + below;
          if (pos < cap) {
            col[pos] = n;
            val[pos] = __builtin_bit_cast(uint16_t, v16);
          }
          const int posb = __builtin_amdgcn_readlane(bbase, kk >> 4) + runB + below;
          if (posb < cap) bent[posb] = u32x2{((uint32_t)k << 6) | (uint32_t)(n & 63), __float_as_uint(vf)};
          int fb = __builtin_amdgcn_readlane(fbase, 0), rf = runF[0];
#pragma unroll
          for (int q = 1; q < 4; ++q)
            if (quarter == q) {
              fb = __builtin_amdgcn_readlane(fbase, q);
              rf = runF[q];
            }
          const int posf = fb + rf + (below - lower);
          const float d = vf - (bias_q + scale * (float)q);
          if (posf < cap) fent[posf] = u32x2{((uint32_t)n << 7) | (uint32_t)(k & 127), __float_as_uint(d)};
        }
        runB += __popcll(mask);
#pragma unroll
        for (int q = 0; q < 4; ++q) runF[q] += __popc((uint32_t)(mask >> (16 * q)) & 0xffffu);
      }
      if ((kk & 15) == 15) runB = 0;
    }
  }
  if (vn) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (16 * p < rows)
        *reinterpret_cast<u32x4*>(codes + (long)n * K + k0 + 16 * p) =
            u32x4{cw[4 * p], cw[4 * p + 1], cw[4 * p + 2], cw[4 * p + 3]};
  }
}

}  // namespace

void launch_quantize_w8o(const float* W, int K, int N, int8_t* codes, void* side_v,
                         hipStream_t st) {
  const W8OLayout L = w8o_layout(K, N);
  char* side = static_cast<char*>(side_v);
  W8OHeader* h = reinterpret_cast<W8OHeader*>(side);
  uint32_t* hist = reinterpret_cast<uint32_t*>(side + L.hist);
  const long long n = (long long)K * N, n4 = n / 4;
  long long nb = (n4 + 256 * 16 - 1) / (256 * 16);
  const unsigned hb = (unsigned)(nb < 1024 ? nb : 1024);
  sel_init<<<1, 256, 0, st>>>(h, hist, n, L.cap);
  sel_hist<0><<<hb, 256, 0, st>>>(W, n4, h, hist);
  sel_pick<0><<<1, 256, 0, st>>>(h, hist);
  sel_hist<1><<<hb, 256, 0, st>>>(W, n4, h, hist);
  sel_pick<1><<<1, 256, 0, st>>>(h, hist);
  sel_hist<2><<<hb, 256, 0, st>>>(W, n4, h, hist);
  sel_pick<2><<<1, 256, 0, st>>>(h, hist);
  const unsigned tb = (unsigned)((L.nkt * L.nnb + 3) / 4);
  outlier_count<<<tb, 256, 0, st>>>(W, h, L, side);
  const int np = L.K > L.nkb * L.ng ? L.K : L.nkb * L.ng;
  outlier_prep<<<(unsigned)((np + 255) / 256), 256, 0, st>>>(L, side);
  ScanJobs j{};
  j.in[0] = reinterpret_cast<const int*>(side + L.rowtot);
  j.out[0] = reinterpret_cast<int*>(side + L.rowptr);
  j.len[0] = L.K;
  j.in[1] = reinterpret_cast<const int*>(side + L.bcell);
  j.out[1] = reinterpret_cast<int*>(side + L.bptr);
  j.len[1] = L.nnb * L.kg;
  j.in[2] = reinterpret_cast<const int*>(side + L.fcell);
  j.out[2] = reinterpret_cast<int*>(side + L.fptr);
  j.len[2] = L.nkb * L.ng;
  j.h = h;
  outlier_scan<<<3, 1024, 0, st>>>(j);
  outlier_fill<<<tb, 256, 0, st>>>(W, h, L, side, codes);
}

}  // namespace qlora
