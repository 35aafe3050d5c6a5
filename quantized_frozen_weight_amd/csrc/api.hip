// C ABI of libqlora: argument validation, workspace layout, and the kernel
// sequence of each call. Contract and citations: include/qlora.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "outlier.hpp"
#include "qlora.h"

namespace {

using namespace qlora;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline bool fits_int(long long a, long long b) {
  return a > 0 && b > 0 && a * b < (1LL << 31);
}

int check_dtype(int dtype) {
  return (dtype == QLORA_F32 || dtype == QLORA_BF16) ? QLORA_OK : QLORA_EINVAL;
}

int check_shape(int M, int K, int N, int r) {
  if (M < 1 || K < 16 || N < 16 || r < 1 || r > 32) return QLORA_EINVAL;
  if (K % 16 || N % 16) return QLORA_EINVAL;
  if (!fits_int(M, K) || !fits_int(M, N) || !fits_int(K, N)) return QLORA_ERANGE;
  return QLORA_OK;
}

// Validate a layer description (weights only; data pointers are checked by
// the individual calls).
int check_linear(const qlora_linear* L, int M, int dtype) {
  if (L == nullptr) return QLORA_EINVAL;
  int st = check_dtype(dtype);
  if (st) return st;
  st = check_shape(M, L->K, L->N, L->r);
  if (st) return st;
  if (L->fmt != QLORA_W8 && L->fmt != QLORA_W4G128 && L->fmt != QLORA_W8O) return QLORA_EINVAL;
  if (L->fmt == QLORA_W8O) {
    if (dtype != QLORA_BF16) return QLORA_EUNSUPPORTED;
    if (L->N >= (1 << 24)) return QLORA_EUNSUPPORTED;
  }
  if (L->fmt == QLORA_W4G128) {
    if (L->K % 128) return QLORA_EINVAL;
    if (dtype != QLORA_BF16) return QLORA_EUNSUPPORTED;
    if (L->K > 128 * kW4MaxGroups) return QLORA_EUNSUPPORTED;
  }
  if (L->heads < 0 || (L->heads > 1 && L->N % L->heads)) return QLORA_EINVAL;
  if (L->heads > 1 && (L->N / L->heads) % 64) return QLORA_EUNSUPPORTED;
  const void* ptrs[4] = {L->codes, L->scales, L->A, L->B};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return QLORA_EINVAL;
  return QLORA_OK;
}

// Head width of B / dB (and of W at quantization): N for a one-head layer.
inline int head_width(const qlora_linear* L) {
  return L->heads > 1 ? L->N / L->heads : L->N;
}

inline float lora_s(const qlora_linear* L) {
  return L->alpha / (float)L->r;   // one float32 divide
}

struct FwdLayout {
  size_t xq, sx, t, asum, pacc, pcorr, rs, total;
};
FwdLayout fwd_layout(const qlora_linear* L, int M) {
  FwdLayout w{};
  size_t off = 0;
  // activation codes and scales: the int8 product, and the integer forward
  // of 4-bit layers
  w.xq = off; off = align_up(off + (size_t)M * L->K);
  w.sx = off; off = align_up(off + (size_t)M * 4);
  w.t = off; off = align_up(off + (size_t)M * L->r * 4);
  // row sums of the activation codes (affine weights)
  w.asum = off; off = align_up(off + (L->fmt == QLORA_W8O ? (size_t)M * 4 : 0));
  // split contraction of the int8 product (0 bytes when it does not split):
  // int32 partial sums, and the affine weights' partial corrections
  // (4-bit weights: the float32 partial sums of the split 4-bit product)
  const bool w8 = L->fmt == QLORA_W8, w8o = L->fmt == QLORA_W8O;
  const size_t nsplit = (w8 || w8o) ? fwd_split_ints(M, L->N, L->K, w8o)
                                    : fwd_w4_split_floats(M, L->N, L->K);
  w.pacc = off; off = align_up(off + nsplit * 4);
  w.pcorr = off; off = align_up(off + (w8o ? nsplit * 4 : 0));
  // the row pass of long rows split over k (0 bytes for other widths)
  w.rs = off; off = align_up(off + row_split_floats(M, L->K, L->r) * 4);
  w.total = off;
  return w;
}

struct BwdLayout {
  size_t t, u, pB, pA, pdx, pu, rs, total;
};
// Partial sums of dA and dB: one per split of the rows. The fused int8
// backward splits by row block (at least 64 rows), the other paths into at
// most as many splits, so ceil(M / 64) covers both.
inline size_t partial_floats(int M, int r, int C) {
  return (size_t)((M + 63) / 64) * (size_t)r * (size_t)C;
}
BwdLayout bwd_layout(const qlora_linear* L, int M, int dtype) {
  BwdLayout w{};
  size_t off = 0;
  // the partial sums first: they are the only bytes that outlive a call
  // (qlora_bwd_partials_bytes), everything after them is scratch
  w.pB = off; off = align_up(off + partial_floats(M, L->r, L->N) * 4);
  w.pA = off; off = align_up(off + partial_floats(M, L->r, L->K) * 4);
  w.t = off; off = align_up(off + (size_t)M * L->r * 4);
  w.u = off; off = align_up(off + (size_t)M * L->r * 4);
  // split contraction of the bf16 input gradient (0 bytes when it does not split)
  size_t fdx = 0, fu = 0;
  if (dtype == QLORA_BF16) bwd_split_sizes(M, L->K, L->N, L->r, &fdx, &fu);
  w.pdx = off; off = align_up(off + fdx * 4);
  w.pu = off; off = align_up(off + fu * 4);
  // recomputing t over long rows split over k (0 bytes for other widths)
  w.rs = off; off = align_up(off + row_split_floats(M, L->K, L->r) * 4);
  w.total = off;
  return w;
}

inline char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Scratch of qlora_bwd_noalloc: a static device array, one copy per GPU the
// library runs on, held until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory: its device address is taken
// once per device with hipGetSymbolAddress (that device current) and only
// that address is passed to kernels.
constexpr size_t kNoAllocScratch = QLORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) int8_t scratch[kNoAllocScratch];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call
// on that device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return QLORA_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QLORA_OK;
}

// Optional timing marks around a call's main product kernel.
void mark(void* ev, hipStream_t s) {
  if (ev != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(ev), s);
}

// Before a call enqueues anything: a HIP error that earlier work of the
// caller left pending is not ours to clear, and launching on top of it would
// blame it on this call. The call returns QLORA_EHIP, enqueues nothing and
// leaves the error in place for the caller.
int pending_error() {
  return hipPeekAtLastError() == hipSuccess ? QLORA_OK : QLORA_EHIP;
}

// After a call's launches: nothing was pending before them (pending_error),
// so an error now is one of this call's launches; it is reported and
// cleared.
int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QLORA_OK : QLORA_EHIP;
}

// Row-block count of the adapter-gradient partial sums: the fused bf16
// backward's row tile; the other paths split the rows the same way so that
// the combine needs nothing but (L, M, dtype).
int bwd_splits(const qlora_linear* L, int M) {
  const int bm = bwd_row_block(L->fmt, M, L->K, L->N, L->r);
  return (M + bm - 1) / bm;
}

int bwd_check_ws(const qlora_linear* L, int M, int dtype, void* ws, size_t ws_bytes) {
  const BwdLayout w = bwd_layout(L, M, dtype);
  if (ws_bytes < w.total || !ws || !aligned16(ws)) return QLORA_EWORKSPACE;
  return QLORA_OK;
}


}  // namespace

extern "C" {

const char* qlora_status_str(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument";
    case QLORA_EUNSUPPORTED: return "unsupported combination";
    case QLORA_EWORKSPACE: return "workspace too small";
    case QLORA_ERANGE: return "size out of range";
    case QLORA_EHIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int qlora_weight_bytes(int K, int N, int fmt, size_t* codes_bytes,
                       size_t* scale_bytes) {
  if (codes_bytes == nullptr || scale_bytes == nullptr) return QLORA_EINVAL;
  if (K < 16 || N < 16 || K % 16 || N % 16) return QLORA_EINVAL;
  if (!fits_int(K, N)) return QLORA_ERANGE;
  if (fmt == QLORA_W8) {
    *codes_bytes = (size_t)K * N;
    *scale_bytes = (size_t)N * 4;
    return QLORA_OK;
  }
  if (fmt == QLORA_W4G128) {
    if (K % 128) return QLORA_EINVAL;
    *codes_bytes = (size_t)K * N / 2;
    *scale_bytes = (size_t)N * (K / 128) * 2;
    return QLORA_OK;
  }
  if (fmt == QLORA_W8O) {
    *codes_bytes = (size_t)K * N;
    *scale_bytes = w8o_layout(K, N).total;
    return QLORA_OK;
  }
  return QLORA_EINVAL;
}

int qlora_outlier_layout(int K, int N, size_t* rowptr_off, size_t* col_off,
                         size_t* val_off, int32_t* capacity) {
  if (!rowptr_off || !col_off || !val_off || !capacity) return QLORA_EINVAL;
  if (K < 16 || N < 16 || K % 16 || N % 16) return QLORA_EINVAL;
  if (!fits_int(K, N)) return QLORA_ERANGE;
  const W8OLayout L = w8o_layout(K, N);
  *rowptr_off = L.rowptr;
  *col_off = L.col;
  *val_off = L.val;
  *capacity = L.cap;
  return QLORA_OK;
}

int qlora_quantize(const float* W, int K, int N, int fmt, void* codes,
                   void* scales, void* stream) {
  return qlora_quantize_heads(W, 1, K, N, fmt, codes, scales, stream);
}

int qlora_quantize_heads(const float* W, int heads, int K, int N, int fmt,
                         void* codes, void* scales, void* stream) {
  size_t cb, sb;
  int st = qlora_weight_bytes(K, N, fmt, &cb, &sb);
  if (st) return st;
  if (heads < 1 || N % heads) return QLORA_EINVAL;
  if (heads > 1 && (N / heads) % 64) return QLORA_EUNSUPPORTED;
  if (fmt == QLORA_W8O && (heads > 1 || N >= (1 << 24))) return QLORA_EUNSUPPORTED;
  const int hd = N / heads;
  if (!W || !codes || !scales || !aligned16(W) || !aligned16(codes) || !aligned16(scales))
    return QLORA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pending_error()) return QLORA_EHIP;
  if (fmt == QLORA_W8)
    launch_quantize_w8(W, K, N, hd, static_cast<int8_t*>(codes),
                       static_cast<float*>(scales), s);
  else if (fmt == QLORA_W8O)
    launch_quantize_w8o(W, K, N, static_cast<int8_t*>(codes), scales, s);
  else
    launch_quantize_w4(W, K, N, hd, static_cast<uint8_t*>(codes),
                       static_cast<_Float16*>(scales), s);
  return launch_status();
}

int qlora_fwd_workspace(const qlora_linear* L, int M, int dtype, size_t* bytes) {
  if (bytes == nullptr) return QLORA_EINVAL;
  int st = check_linear(L, M, dtype);
  if (st) return st;
  *bytes = fwd_layout(L, M).total;
  return QLORA_OK;
}

int qlora_fwd_timed(const qlora_linear* L, int M, int dtype, const void* x,
                    void* y, float* t_save, void* ws, size_t ws_bytes,
                    void* stream, int repeats, void* ev_start, void* ev_stop) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (repeats < 1) return QLORA_EINVAL;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return QLORA_EINVAL;
  if (t_save && !aligned16(t_save)) return QLORA_EINVAL;
  const FwdLayout w = fwd_layout(L, M);
  if (ws_bytes < w.total || (w.total && (!ws || !aligned16(ws)))) return QLORA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* t = t_save ? t_save : reinterpret_cast<float*>(at(ws, w.t));
  if (pending_error()) return QLORA_EHIP;
  if (L->fmt == QLORA_W8) {
    int8_t* xq = reinterpret_cast<int8_t*>(at(ws, w.xq));
    float* sx = reinterpret_cast<float*>(at(ws, w.sx));
    launch_rowquant(dtype, x, M, L->K, L->A, L->r, xq, sx, t, s, nullptr,
                    reinterpret_cast<float*>(at(ws, w.rs)));
    mark(ev_start, s);
    for (int rep = 0; rep < repeats; ++rep)
      launch_gemm_fwd_w8(dtype, M, L->N, L->K, xq,
                         static_cast<const int8_t*>(L->codes), sx,
                         static_cast<const float*>(L->scales), t, L->B, head_width(L), L->r,
                         lora_s(L), y, nullptr, reinterpret_cast<int32_t*>(at(ws, w.pacc)), s);
    mark(ev_stop, s);
  } else if (L->fmt == QLORA_W8O) {
    int8_t* xq = reinterpret_cast<int8_t*>(at(ws, w.xq));
    float* sx = reinterpret_cast<float*>(at(ws, w.sx));
    float* asum = reinterpret_cast<float*>(at(ws, w.asum));
    launch_rowquant(dtype, x, M, L->K, L->A, L->r, xq, sx, t, s, asum,
                    reinterpret_cast<float*>(at(ws, w.rs)));
    mark(ev_start, s);
    for (int rep = 0; rep < repeats; ++rep)
      launch_gemm_fwd_w8o(M, L->N, L->K, xq, static_cast<const int8_t*>(L->codes), sx, asum,
                          L->scales, t, L->B, head_width(L), L->r, lora_s(L),
                          static_cast<uint16_t*>(y), reinterpret_cast<int32_t*>(at(ws, w.pacc)),
                          reinterpret_cast<float*>(at(ws, w.pcorr)), s);
    mark(ev_stop, s);
  } else {
    launch_lora_down(dtype, x, M, L->K, L->A, L->r, t, s, reinterpret_cast<float*>(at(ws, w.rs)));
    mark(ev_start, s);
    for (int rep = 0; rep < repeats; ++rep)
      launch_gemm_fwd_w4(M, L->N, L->K, static_cast<const uint16_t*>(x),
                         static_cast<const uint8_t*>(L->codes),
                         static_cast<const _Float16*>(L->scales), t, L->B, head_width(L), L->r,
                         lora_s(L), static_cast<uint16_t*>(y),
                         reinterpret_cast<float*>(at(ws, w.pacc)), s);
    mark(ev_stop, s);
  }
  return launch_status();
}

int qlora_fwd(const qlora_linear* L, int M, int dtype, const void* x, void* y,
              float* t_save, void* ws, size_t ws_bytes, void* stream) {
  return qlora_fwd_timed(L, M, dtype, x, y, t_save, ws, ws_bytes, stream, 1,
                         nullptr, nullptr);
}

int qlora_fwd_a8w4(const qlora_linear* L, int M, int dtype, const void* x, void* y,
                   float* t_save, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (L->fmt != QLORA_W4G128) return QLORA_EUNSUPPORTED;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return QLORA_EINVAL;
  if (t_save && !aligned16(t_save)) return QLORA_EINVAL;
  const FwdLayout w = fwd_layout(L, M);
  if (ws_bytes < w.total || !ws || !aligned16(ws)) return QLORA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* t = t_save ? t_save : reinterpret_cast<float*>(at(ws, w.t));
  int8_t* xq = reinterpret_cast<int8_t*>(at(ws, w.xq));
  float* sx = reinterpret_cast<float*>(at(ws, w.sx));
  if (pending_error()) return QLORA_EHIP;
  launch_rowquant(dtype, x, M, L->K, L->A, L->r, xq, sx, t, s, nullptr,
                  reinterpret_cast<float*>(at(ws, w.rs)));
  launch_gemm_fwd_a8w4(M, L->N, L->K, xq, sx, static_cast<const uint8_t*>(L->codes),
                       static_cast<const _Float16*>(L->scales), t, L->B, head_width(L), L->r, lora_s(L),
                       static_cast<uint16_t*>(y), s);
  return launch_status();
}

int qlora_bwd_workspace(const qlora_linear* L, int M, int dtype, size_t* bytes) {
  if (bytes == nullptr) return QLORA_EINVAL;
  int st = check_linear(L, M, dtype);
  if (st) return st;
  *bytes = bwd_layout(L, M, dtype).total;
  return QLORA_OK;
}

int qlora_bwd_partial_timed(const qlora_linear* L, int M, int dtype, const void* x,
                            const void* dy, const float* t_saved, void* dx, void* ws,
                            size_t ws_bytes, void* stream, int repeats, void* ev_start,
                            void* ev_stop) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (repeats < 1) return QLORA_EINVAL;
  if (!x || !dy) return QLORA_EINVAL;
  if (!aligned16(x) || !aligned16(dy)) return QLORA_EINVAL;
  if ((t_saved && !aligned16(t_saved)) || (dx && !aligned16(dx))) return QLORA_EINVAL;
  st = bwd_check_ws(L, M, dtype, ws, ws_bytes);
  if (st) return st;
  const BwdLayout w = bwd_layout(L, M, dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = lora_s(L);
  float* u = reinterpret_cast<float*>(at(ws, w.u));
  if (pending_error()) return QLORA_EHIP;
  const float* t = t_saved;
  if (t == nullptr) {
    float* tw = reinterpret_cast<float*>(at(ws, w.t));
    launch_lora_down(dtype, x, M, L->K, L->A, L->r, tw, s, reinterpret_cast<float*>(at(ws, w.rs)));
    t = tw;
  }
  float* partB = reinterpret_cast<float*>(at(ws, w.pB));
  float* partA = reinterpret_cast<float*>(at(ws, w.pA));
  if (dtype == QLORA_BF16 && dx != nullptr) {
    // one launch: dx, u, and the per-row-block partial sums of dA and dB
    mark(ev_start, s);
    for (int rep = 0; rep < repeats; ++rep)
      launch_bwd_fused(L->fmt, M, L->K, L->N, static_cast<const uint16_t*>(dy),
                       L->codes, L->scales, L->B, head_width(L), L->A, t,
                       static_cast<const uint16_t*>(x), L->r, sc,
                       static_cast<uint16_t*>(dx), partA, partB,
                       reinterpret_cast<float*>(at(ws, w.pdx)),
                       reinterpret_cast<float*>(at(ws, w.pu)), s);
    mark(ev_stop, s);
    return launch_status();
  }
  launch_bwd_rows(dtype, dy, M, L->N, L->B, head_width(L), L->r, nullptr, nullptr, u, s);
  SkinnyJobs sk = make_adapter_grad_jobs(M, L->r, sc, t, dy, L->N, nullptr, partB,
                                         u, x, L->K, nullptr, partA);
  sk.nsplit = bwd_splits(L, M);
  sk.rows_per_split = (M + sk.nsplit - 1) / sk.nsplit;
  sk.rows_per_split = (sk.rows_per_split + 3) / 4 * 4;
  // float32 compute (int8 weights): the adapter-gradient stage 1, then the
  // float32 input gradient; or no input gradient at all
  launch_skinny_stage1(dtype, sk, s);
  mark(ev_start, s);
  if (dx != nullptr)
    for (int rep = 0; rep < repeats; ++rep)
      launch_gemm_dx_f32(M, L->K, L->N, static_cast<const float*>(dy),
                         static_cast<const int8_t*>(L->codes),
                         static_cast<const float*>(L->scales), u, L->A, L->r,
                         sc, static_cast<float*>(dx), s);
  mark(ev_stop, s);
  return launch_status();
}

int qlora_bwd_partial(const qlora_linear* L, int M, int dtype, const void* x,
                      const void* dy, const float* t_saved, void* dx, void* ws,
                      size_t ws_bytes, void* stream) {
  return qlora_bwd_partial_timed(L, M, dtype, x, dy, t_saved, dx, ws, ws_bytes, stream,
                                 1, nullptr, nullptr);
}

namespace {
int finish_check(const qlora_linear* L, int M, int dtype, float* dA, float* dB, void* ws,
                 size_t ws_bytes) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (!dA || !dB || !aligned16(dA) || !aligned16(dB)) return QLORA_EINVAL;
  return bwd_check_ws(L, M, dtype, ws, ws_bytes);
}

// The combine of one layer's partial sums (left in ws by qlora_bwd_partial).
SkinnyJobs finish_jobs(const qlora_linear* L, int M, int dtype, float* dA, float* dB,
                       void* ws) {
  const BwdLayout w = bwd_layout(L, M, dtype);
  SkinnyJobs sk{};
  sk.njobs = 2; sk.M = M; sk.r = L->r; sk.s = lora_s(L);
  sk.nsplit = bwd_splits(L, M);
  sk.partial[0] = reinterpret_cast<float*>(at(ws, w.pB)); sk.C[0] = L->N;
  sk.out[0] = dB; sk.transpose[0] = 0; sk.hd0 = head_width(L);
  sk.partial[1] = reinterpret_cast<float*>(at(ws, w.pA)); sk.C[1] = L->K;
  sk.out[1] = dA; sk.transpose[1] = 1;
  return sk;
}
}  // namespace

int qlora_bwd_finish(const qlora_linear* L, int M, int dtype, float* dA, float* dB,
                     void* ws, size_t ws_bytes, void* stream) {
  const int st = finish_check(L, M, dtype, dA, dB, ws, ws_bytes);
  if (st) return st;
  if (pending_error()) return QLORA_EHIP;
  launch_skinny_stage2(finish_jobs(L, M, dtype, dA, dB, ws), static_cast<hipStream_t>(stream));
  return launch_status();
}

int qlora_bwd_partials_bytes(const qlora_linear* L, int M, int dtype, size_t* bytes) {
  if (!bytes) return QLORA_EINVAL;
  const int st = check_linear(L, M, dtype);
  if (st) return st;
  *bytes = bwd_layout(L, M, dtype).t;
  return QLORA_OK;
}

int qlora_bwd_finish_batch(const qlora_finish_item* items, int count, void* stream) {
  if (!items || count < 1) return QLORA_EINVAL;
  for (int i = 0; i < count; ++i) {
    const qlora_finish_item& it = items[i];
    const int st = finish_check(it.L, it.M, it.dtype, it.dA, it.dB, it.ws, it.ws_bytes);
    if (st) return st;
  }
  if (pending_error()) return QLORA_EHIP;
  SkinnyJobs sk[kFinishBatch];
  for (int i0 = 0; i0 < count; i0 += kFinishBatch) {
    const int n = count - i0 < kFinishBatch ? count - i0 : kFinishBatch;
    for (int i = 0; i < n; ++i) {
      const qlora_finish_item& it = items[i0 + i];
      sk[i] = finish_jobs(it.L, it.M, it.dtype, it.dA, it.dB, it.ws);
    }
    launch_finish_batch(sk, n, static_cast<hipStream_t>(stream));
  }
  return launch_status();
}

int qlora_bwd_timed(const qlora_linear* L, int M, int dtype, const void* x,
                    const void* dy, const float* t_saved, void* dx, float* dA,
                    float* dB, void* ws, size_t ws_bytes, void* stream,
                    int repeats, void* ev_start, void* ev_stop) {
  // both halves are validated before either is enqueued
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (!dA || !dB || !aligned16(dA) || !aligned16(dB)) return QLORA_EINVAL;
  st = qlora_bwd_partial_timed(L, M, dtype, x, dy, t_saved, dx, ws, ws_bytes, stream,
                               repeats, ev_start, ev_stop);
  if (st) return st;
  return qlora_bwd_finish(L, M, dtype, dA, dB, ws, ws_bytes, stream);
}

int qlora_bwd(const qlora_linear* L, int M, int dtype, const void* x,
              const void* dy, const float* t_saved, void* dx, float* dA,
              float* dB, void* ws, size_t ws_bytes, void* stream) {
  return qlora_bwd_timed(L, M, dtype, x, dy, t_saved, dx, dA, dB, ws, ws_bytes,
                         stream, 1, nullptr, nullptr);
}

const char* qlora_bwd_main_kernel(const qlora_linear* L, int M, int dtype) {
  if (check_linear(L, M, dtype)) return nullptr;
  if (dtype == QLORA_BF16) return bwd_fused_kernel_name(L->fmt, M, L->K, L->N, L->r);
  return "gemm_dx_f32_kernel";
}

int qlora_bwd_noalloc(const qlora_linear* L, int M, int dtype, const void* x,
                      const void* dy, const float* t_saved, void* dx, float* dA,
                      float* dB, void* stream) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (bwd_layout(L, M, dtype).total > kNoAllocScratch) return QLORA_EWORKSPACE;
  if (pending_error()) return QLORA_EHIP;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return qlora_bwd(L, M, dtype, x, dy, t_saved, dx, dA, dB, ws, kNoAllocScratch, stream);
}

int qlora_merge(const qlora_linear* L, void* codes_out, void* scales_out,
                void* stream) {
  int st = check_linear(L, 1, QLORA_BF16);
  if (st) return st;
  if (L->fmt != QLORA_W8) return QLORA_EUNSUPPORTED;
  if (!codes_out || !scales_out || !aligned16(codes_out) || !aligned16(scales_out))
    return QLORA_EINVAL;
  const size_t cb = (size_t)L->N * L->K, sb = (size_t)L->N * 4;
  auto overlaps = [](const void* a, size_t na, const void* b, size_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
  };
  if (overlaps(codes_out, cb, L->codes, cb) || overlaps(codes_out, cb, L->scales, sb) ||
      overlaps(scales_out, sb, L->codes, cb) || overlaps(scales_out, sb, L->scales, sb) ||
      overlaps(codes_out, cb, scales_out, sb))
    return QLORA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pending_error()) return QLORA_EHIP;
  launch_merge_w8(static_cast<const int8_t*>(L->codes), static_cast<const float*>(L->scales),
                  L->A, L->B, head_width(L), L->K, L->N, L->r, lora_s(L),
                  static_cast<int8_t*>(codes_out), static_cast<float*>(scales_out), s);
  return launch_status();
}

int qlora_quantize_rows(const void* x, int M, int K, int dtype, int8_t* xq,
                        float* sx, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (M < 1 || K < 16 || K % 16) return QLORA_EINVAL;
  if (!fits_int(M, K)) return QLORA_ERANGE;
  if (!x || !xq || !sx || !aligned16(x) || !aligned16(xq) || !aligned16(sx))
    return QLORA_EINVAL;
  if (pending_error()) return QLORA_EHIP;
  launch_rowquant(dtype, x, M, K, nullptr, 1, xq, sx, nullptr,
                  static_cast<hipStream_t>(stream));
  return launch_status();
}

int qlora_fwd_acc(const qlora_linear* L, int M, int dtype, const void* x,
                  int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(L, M, dtype);
  if (st) return st;
  if (L->fmt != QLORA_W8 && L->fmt != QLORA_W8O) return QLORA_EUNSUPPORTED;
  if (!x || !acc || !aligned16(x) || !aligned16(acc)) return QLORA_EINVAL;
  const FwdLayout w = fwd_layout(L, M);
  if (ws_bytes < w.total || !ws || !aligned16(ws)) return QLORA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* xq = reinterpret_cast<int8_t*>(at(ws, w.xq));
  float* sx = reinterpret_cast<float*>(at(ws, w.sx));
  if (pending_error()) return QLORA_EHIP;
  launch_rowquant(dtype, x, M, L->K, nullptr, 1, xq, sx, nullptr, s);
  // the integer product alone: no scale is read
  launch_gemm_fwd_w8(dtype, M, L->N, L->K, xq,
                     static_cast<const int8_t*>(L->codes), sx, nullptr, nullptr, L->B,
                     head_width(L), L->r, 0.f, nullptr, acc, nullptr, s);
  return launch_status();
}

}  // extern "C"
