// Side buffer of the outlier-compensated int8 weight (keras-llm-light README,
// "Simplified Int8Variable quantization": the weight is cut at its 0.1th and
// 99.9th percentiles, stored as 8-bit codes of an affine grid, and the
// elements outside the cut are kept as fp16 values at their positions).
//
// The codes live in the layer's `codes` array, int8 [N, K] = grid index - 128.
// Everything else lives in one side buffer (the layer's `scales` pointer),
// sections 256-byte aligned:
//
//   header      W8OHeader (the public part first)
//   rowptr      int32 [K + 1]     outliers of weight row k (input k):
//   col         int32 [cap]         [rowptr[k], rowptr[k + 1]) in n order
//   val         fp16  [cap]
//   fptr, fent  the same outliers for the forward product, grouped by cell
//               (k / 128, n / 16) in cell order, (k, n) order inside a cell:
//               fptr int32 [NKB * NG + 1], fent {(n << 7) | k % 128,
//               correction} [cap + 64]; correction = value - the grid's
//               reconstruction at that position
//   bptr, bent  grouped by cell (n / 64, k / 16), (k, n) order inside:
//               bptr int32 [NNB * KG + 1], bent {(k << 6) | n % 64, value}
//               [cap + 64]
//   scratch     used while quantizing only: per-(64-column tile, k) row
//               counts, per-(64-row tile, 16-column group) counts, the
//               16-row group counts, the select histograms
//
// cap bounds the outlier count: with nearest-rank cuts at ranks
// ceil(n / 1000) and ceil(999 n / 1000) of n = K N elements, at most
// floor(n / 1000) elements lie on each side. The entry arrays have 64 spare
// entries so that a wave may read 64 entries from any start inside the list.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qlora {

struct W8OHeader {
  // public (qlora_outlier_header in include/qlora.h)
  float lo, hi, scale;       // cut and grid step; bias = lo
  int32_t nnz;               // outliers stored
  // library-internal
  float inv;                 // 255 / (hi - lo), or 0
  float bias_q;              // lo + 128 scale: the reconstruction of code 0
  int32_t cap;
  uint32_t key[2];           // order keys found by the selection
  int32_t rem[2];            // ranks still to resolve inside the key prefix
};

constexpr int kW8OFwdCellK = 128;   // k per forward cell (the forward's stage)
constexpr int kW8OFwdCellN = 16;    // n per forward cell (a wave's columns)
constexpr int kW8OBwdCellN = 64;    // n per backward cell (the backward's stage)
constexpr int kW8OBwdCellK = 16;    // k per backward cell
constexpr int kW8OPad = 64;         // spare entries after each entry list
constexpr int kSelBins = 2048;      // histogram bins of one selection pass

struct W8OLayout {
  int K, N, cap, nkb, ng, nnb, kg, nkt;
  size_t rowptr, col, val, fptr, fent, bptr, bent;   // byte offsets
  size_t cnt_r, fcnt, bcell, rowtot, fcell, hist;     // scratch
  size_t total;
};

inline size_t w8o_align(size_t v) { return (v + 255) / 256 * 256; }

inline W8OLayout w8o_layout(int K, int N) {
  W8OLayout L{};
  L.K = K; L.N = N;
  const long long n = (long long)K * N;
  L.cap = (int)(2 * (n / 1000) + 2);
  L.nkb = (K + kW8OFwdCellK - 1) / kW8OFwdCellK;
  L.ng = (N + kW8OFwdCellN - 1) / kW8OFwdCellN;
  L.nnb = (N + kW8OBwdCellN - 1) / kW8OBwdCellN;
  L.kg = K / kW8OBwdCellK;
  L.nkt = (K + 63) / 64;
  size_t off = w8o_align(sizeof(W8OHeader));
  L.rowptr = off; off = w8o_align(off + 4 * ((size_t)K + 1));
  L.col = off;    off = w8o_align(off + 4 * (size_t)L.cap);
  L.val = off;    off = w8o_align(off + 2 * (size_t)L.cap);
  L.fptr = off;   off = w8o_align(off + 4 * ((size_t)L.nkb * L.ng + 1));
  L.fent = off;   off = w8o_align(off + 8 * ((size_t)L.cap + kW8OPad));
  L.bptr = off;   off = w8o_align(off + 4 * ((size_t)L.nnb * L.kg + 1));
  L.bent = off;   off = w8o_align(off + 8 * ((size_t)L.cap + kW8OPad));
  L.cnt_r = off;  off = w8o_align(off + 4 * (size_t)L.nnb * K);
  L.fcnt = off;   off = w8o_align(off + 4 * (size_t)L.nkt * L.ng);
  L.bcell = off;  off = w8o_align(off + 4 * (size_t)L.nnb * L.kg);
  L.rowtot = off; off = w8o_align(off + 4 * (size_t)K);
  L.fcell = off;  off = w8o_align(off + 4 * (size_t)L.nkb * L.ng);
  L.hist = off;   off = w8o_align(off + 4 * 2 * (size_t)kSelBins);
  L.total = off;
  return L;
}

}  // namespace qlora

#ifdef __HIPCC__
namespace qlora {

// Entry ranges of one outlier cell for every stage of a product, read 64
// stages at a time into registers: lane i of (lo, hi) holds stage 64 c + i of
// chunk c, and the next chunk is read while this one is used. A stage's range
// is then a readlane with a uniform index -- no load inside the stage loop
// whose result the loop would have to wait for. p[st * stride + olo] and
// p[st * stride + ohi] are the stage's first and one-past-last entries.
struct CellRanges {
  int lo, hi, nlo, nhi, chunk;
  const int* p;
  int stride, olo, ohi, nst;

  __device__ __forceinline__ void read(int c, int& l, int& h) const {
    int st = c * 64 + (int)(threadIdx.x & 63);
    st = st < nst ? st : nst - 1;
    l = p[(long)st * stride + olo];
    h = p[(long)st * stride + ohi];
  }
  // st0: the first stage that get() will be asked for
  __device__ __forceinline__ void init(const int* p_, int stride_, int olo_, int ohi_, int nst_,
                                       int st0 = 0) {
    p = p_; stride = stride_; olo = olo_; ohi = ohi_; nst = nst_;
    chunk = st0 >> 6;
    read(chunk, lo, hi);
    read(chunk + 1, nlo, nhi);
  }
  // range of stage st; calls come with st non-decreasing from st0, one chunk
  // at a time
  __device__ __forceinline__ void get(int st, int& l, int& h) {
    if ((st >> 6) != chunk) {
      lo = nlo;
      hi = nhi;
      ++chunk;
      read(chunk + 1, nlo, nhi);
    }
    l = __builtin_amdgcn_readlane(lo, st & 63);
    h = __builtin_amdgcn_readlane(hi, st & 63);
  }
};

}  // namespace qlora
#endif
