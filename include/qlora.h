/*
 * libqlora -- a linear layer with a frozen quantized weight and a trainable
 * low-rank (LoRA) adapter, forward and backward, on AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed (sources are cited by page title and section):
 *
 *   y  = x . deq(W) + s . (x A) B,          s = alpha / r
 *
 *   - "Parameter-efficient fine-tuning of GPT-2 with LoRA" (keras-io),
 *     "LoRA equation" and "Create LoRA layer": the adapter output (x A) B is
 *     added to the frozen layer's output, scaled by alpha / rank; the original
 *     layer is frozen.
 *   - "Introduce QLoRA-like technique" (keras PR), "Highlights": the frozen
 *     kernel is stored as int8 while the adapter is trained in float.
 *   - keras-llm-light README, "Weights quantization": the adapter weights are
 *     kept in fp32; "Simplified Int4Variable quantization": two 4-bit values
 *     per byte.
 *   - "How to fine-tune the 4-bit model?" (GPTQ-for-LLaMa issue): a 4-bit
 *     frozen matrix under an fp32 rank-4 adapter; gradients need the product
 *     with the transposed quantized matrix.
 *
 * Readings where the pages give no formula (int8 format QLORA_W8):
 *   weight scale sw[n] = absmax_k |W[k,n]| / 127 (one per output channel);
 *   codes q[n,k] = round-half-even(W[k,n] * (127 / absmax)) in [-127, 127];
 *   activations are quantized the same way with one scale per row of x
 *   (sx[m]), and the base product is the exact int32 sum of code products,
 *   rescaled by sx[m] * sw[n].
 * 4-bit format QLORA_W4G128: one fp16 scale per 128 consecutive inputs of an
 *   output channel, sc = f16(absmax / 7), codes round-half-even(W * (1/sc)) in
 *   [-7, 7]; the forward multiplies x (not quantized) by the dequantized weight.
 * Outlier-compensated int8 format QLORA_W8O (keras-llm-light README,
 *   "Simplified Int8Variable quantization": the weight is cut at its 0.1th and
 *   99.9th percentiles, the clipped weight stored as 8-bit codes of an affine
 *   grid reconstructed as bias + value * scale, and the elements outside the
 *   cut kept as fp16 values at their positions): one cut, bias and scale per
 *   weight tensor; lo and hi are the nearest-rank percentiles (the elements
 *   of ascending rank ceil(n / 1000) and ceil(999 n / 1000) among n = K N);
 *   d = fl32(hi - lo), scale = fl32(d / 255), bias = lo, grid index
 *   v = clamp(round-half-even(fl32(fl32(clip(W, lo, hi) - lo) * fl32(255 / d))),
 *   0, 255) (scale 0 and v = 0 if d is 0 or not finite or 255 / d
 *   overflows); outliers are the elements < lo or > hi, kept as fp16
 *   (round-half-even). The layer is reconstructed as Wr = lo + v * scale with
 *   the outliers written over it; the forward quantizes x per row as for
 *   QLORA_W8 and adds the product of the quantized rows with Wr.
 * Backward: the activation quantizer is passed straight through,
 *   dx = dy . deq(W)^T + s (dy B^T) A^T,  dA = s x^T (dy B^T),  dB = s (x A)^T dy,
 *   and the frozen weight receives no gradient (there is no dW argument).
 *
 * Layouts (all row-major, all pointers are DEVICE memory owned by the caller):
 *   W      float32 [K, N]                 (input to qlora_quantize only)
 *   codes  QLORA_W8:     int8  [N, K]     (output channel major, K contiguous)
 *          QLORA_W4G128: uint8 [N, K/2]   (byte j holds k = 2j in the low
 *                                          nibble, 2j+1 in the high nibble,
 *                                          two's complement)
 *          QLORA_W8O:    int8  [N, K]     (v - 128)
 *   scales QLORA_W8:     float32 [N]
 *          QLORA_W4G128: float16 [N, K/128]
 *          QLORA_W8O:    a side buffer of qlora_weight_bytes' scale_bytes:
 *                        a qlora_outlier_header at offset 0, then the
 *                        outlier list at the offsets that
 *                        qlora_outlier_layout gives, then arrays the library
 *                        uses internally
 *   x, dx  [M, K] in the compute dtype;  y, dy  [M, N] in the compute dtype
 *   A, dA  float32 [K, r];               B, dB  float32 [r, N]
 *   t      float32 [M, r]  (t = x A, unscaled; saved by the forward)
 *   Multi-head layers ("Parameter-efficient fine-tuning of GPT-2 with LoRA",
 *   "Create LoRA layer": the attention projections are EinsumDense layers and
 *   the adapter's B keeps their per-head output shape; "Introduce QLoRA-like
 *   technique": frozen int8 EinsumDense kernels): with heads > 1 the N
 *   outputs are heads x hd (n = head * hd + d, hd = N / heads) and
 *     W      float32 [heads, K, hd]       (input to qlora_quantize_heads)
 *     B, dB  float32 [heads, r, hd]
 *   while codes, scales, A, dA, x, y, dx and dy keep the layouts above. A
 *   projection whose heads are on the input side ([heads, hd, N] kernels) is
 *   a plain layer with K = heads * hd.
 *
 * Conventions shared by every entry point:
 *   - The library never allocates, frees or synchronizes. Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and the call returns
 *     immediately. Scratch memory is passed in as `ws` of `ws_bytes`, sized by
 *     the matching *_workspace query; it may be reused between calls that are
 *     ordered on one stream.
 *   - Arguments are validated before anything is launched; a non-OK status
 *     means nothing was enqueued, except QLORA_EHIP from a launch the
 *     runtime rejected (earlier launches of the same call may then be
 *     queued). Device faults surface at the caller's next synchronization.
 *   - A HIP error that earlier work on the calling thread left pending
 *     (hipPeekAtLastError) is neither cleared nor blamed on the library: a
 *     call that would launch returns QLORA_EHIP at once, enqueues nothing
 *     and leaves the error for the caller to read with hipGetLastError.
 *   - Constraints: 1 <= M, 16 <= K, 16 <= N, K % 16 == 0, N % 16 == 0,
 *     1 <= r <= 32, all pointers 16-byte aligned; QLORA_W4G128 needs
 *     K % 128 == 0 and the bf16 compute dtype (EINVAL / EUNSUPPORTED
 *     otherwise), and qlora_fwd / qlora_bwd take K <= 16384 for it (the
 *     products keep one block's fp16 scales in LDS; EUNSUPPORTED above);
 *     QLORA_W8O needs the bf16 compute dtype and N < 2^24
 *     (EUNSUPPORTED otherwise).
 *   - Outputs (y, t, dx, dA, dB) are overwritten, never accumulated into.
 *     codes, scales, A and B are only read by qlora_fwd / qlora_bwd.
 *   - Non-finite x or dy propagate into the outputs; nothing is checked on
 *     the hot path.
 *   - Results do not depend on how the work is split across the GPU: every
 *     reduction has a fixed order, so repeated calls give identical bytes.
 *   - The library holds no mutable global state; calls on different streams
 *     may run concurrently as long as their buffers do not overlap.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_EINVAL = 1,       /* bad pointer, size, alignment or enum */
  QLORA_EUNSUPPORTED = 2, /* valid but not implemented (e.g. W4 with f32) */
  QLORA_EWORKSPACE = 3,   /* ws smaller than the *_workspace query */
  QLORA_ERANGE = 4,       /* size products overflow the index range */
  QLORA_EHIP = 5          /* a kernel launch was rejected by the runtime, or
                             a HIP error was already pending (see below) */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;
typedef enum { QLORA_W8 = 0, QLORA_W4G128 = 1, QLORA_W8O = 2 } qlora_wfmt;

/* One frozen layer with its adapter. All pointers are device memory owned by
 * the caller and only read by the library. */
typedef struct {
  int32_t K, N, r;        /* in-features, out-features, adapter rank */
  float alpha;            /* s = alpha / r, computed as one float32 divide */
  int32_t fmt;            /* qlora_wfmt */
  const void* codes;      /* see "Layouts" */
  const void* scales;     /* see "Layouts" */
  const float* A;         /* [K, r] */
  const float* B;         /* [r, N], or [heads, r, N / heads] */
  int32_t heads;          /* 0 or 1: one head; else N / heads must be a
                             multiple of 64 (EUNSUPPORTED otherwise) */
} qlora_linear;

/* The public head of a QLORA_W8O side buffer (device memory, offset 0),
 * written by qlora_quantize. */
typedef struct {
  float lo, hi;           /* the cut: lower and upper nearest-rank percentile */
  float scale;            /* grid step; the grid's bias is lo */
  int32_t nnz;            /* outliers stored */
} qlora_outlier_header;

/* Human-readable name of a status code (static string, never NULL). */
const char* qlora_status_str(int status);

/* Bytes needed for the codes and scales of a K x N weight in format fmt.
 * Host-only arithmetic; usable without a GPU. */
int qlora_weight_bytes(int K, int N, int fmt, size_t* codes_bytes,
                       size_t* scale_bytes);

/* Where a QLORA_W8O side buffer keeps its outlier list (byte offsets from
 * the buffer's start), in compressed-row form over W [K, N]: the outliers of
 * weight row k are entries [rowptr[k], rowptr[k + 1]) in increasing n, with
 *   rowptr int32 [K + 1] at *rowptr_off,
 *   col    int32 [nnz]   at *col_off   (the output index n),
 *   val    fp16  [nnz]   at *val_off   (the kept value),
 * nnz <= *capacity = 2 floor(K N / 1000) + 2. Host-only arithmetic; the
 * shape rules of qlora_weight_bytes apply. */
int qlora_outlier_layout(int K, int N, size_t* rowptr_off, size_t* col_off,
                         size_t* val_off, int32_t* capacity);

/* Quantize a float32 weight W [K, N] into codes and scales (format above).
 * One-time preparation of the frozen weight ("Introduce QLoRA-like
 * technique", benchmark.py: model.quantize("int8")). Channels (W8) or groups
 * (W4G128) whose abs-max is 0 -- or so small that the inverse scale
 * overflows (W8) -- get scale 0 and zero codes; a non-finite abs-max, or an
 * fp16 scale overflow (W4G128), stores a NaN scale and zero codes so that
 * the NaN reaches every output that uses it. QLORA_W8O: W must be finite
 * (with a NaN or infinite element the cut and codes are unspecified; no
 * write leaves the side buffer); scales is the side buffer, and its whole
 * size is written (the part past the outlier lists is scratch of this
 * call). W is only read. */
int qlora_quantize(const float* W, int K, int N, int fmt, void* codes,
                   void* scales, void* stream);

/* qlora_quantize for a multi-head weight W [heads, K, N / heads] (see
 * Layouts): the same codes and scales as qlora_quantize of the equivalent
 * [K, N] matrix. heads must divide N and N / heads be a multiple of 64
 * (EINVAL / EUNSUPPORTED otherwise); heads = 1 is qlora_quantize. QLORA_W8O
 * takes heads = 1 only (EUNSUPPORTED otherwise). */
int qlora_quantize_heads(const float* W, int heads, int K, int N, int fmt,
                         void* codes, void* scales, void* stream);

/* Workspace needed by qlora_fwd / qlora_fwd_acc for M rows. Layers whose
 * product has few 128 x 128 output tiles (at most 128) over a long
 * contraction also keep there the per-split partial sums of the product, 4
 * bytes per output per split (int32 for int8 weights, float32 for 4-bit
 * ones; 32 MiB for 512 rows of a 16384 -> 2048 layer). */
int qlora_fwd_workspace(const qlora_linear* L, int M, int dtype,
                        size_t* bytes);

/* Forward ("LoRA equation"): y [M, N] = x . deq(W) + s (x A) B, rounded once
 * to the compute dtype. For QLORA_W8, x is quantized per row and the base
 * product is an int8 x int8 -> int32 sum rescaled by sx[m] * sw[n]. If t_save
 * is not NULL, t = x A (float32 [M, r]) is written there for the backward. */
int qlora_fwd(const qlora_linear* L, int M, int dtype, const void* x, void* y,
              float* t_save, void* ws, size_t ws_bytes, void* stream);

/* Integer forward of a QLORA_W4G128 layer with int8 activations, the
 * alternative to qlora_fwd's dequantized bf16 product ("Simplified
 * Int4Variable quantization": two 4-bit codes per byte; "How to fine-tune the
 * 4-bit model?": narrow weights raise the arithmetic intensity). x is
 * quantized per row exactly as for QLORA_W8 layers (xq, sx); then
 *   y[m, n] = sx[m] sum_g sc[n, g] (sum_{k in group g} xq[m, k] q[n, k])
 *             + s (t B)[m, n],
 * each group's sum an exact int32, the weighting and the sum over groups in
 * float32, y rounded once to bf16. t_save as for qlora_fwd. The workspace is
 * qlora_fwd_workspace's. QLORA_W8 layers -> QLORA_EUNSUPPORTED (their
 * qlora_fwd already is the integer product); bf16 activations only. The
 * backward is qlora_bwd's (the activation quantizer is passed straight
 * through). */
int qlora_fwd_a8w4(const qlora_linear* L, int M, int dtype, const void* x,
                   void* y, float* t_save, void* ws, size_t ws_bytes,
                   void* stream);

/* Workspace needed by qlora_bwd for M rows. In bf16, layers whose input
 * gradient has few 128 x 128 output tiles (at most 128) over a long
 * contraction (N of at least 2048) also keep there the per-split partial
 * products of dx, 4 bytes per output per split (32 MiB for 512 rows of a
 * 2048 -> 16384 layer). */
int qlora_bwd_workspace(const qlora_linear* L, int M, int dtype,
                        size_t* bytes);

/* Backward of qlora_fwd for the output gradient dy [M, N]:
 *   u  = dy B^T                                   (float32, internal)
 *   dB = s t^T dy          float32 [r, N]
 *   dA = s x^T u           float32 [K, r]
 *   dx = dy deq(W)^T + s u A^T   [M, K] in the compute dtype (skipped if NULL)
 * t_saved is the t written by qlora_fwd; pass NULL to recompute it from x.
 * The frozen weight gets no gradient ("Why does LoRA reduce memory
 * footprint?": only the adapter is trained). */
int qlora_bwd(const qlora_linear* L, int M, int dtype, const void* x,
              const void* dy, const float* t_saved, void* dx, float* dA,
              float* dB, void* ws, size_t ws_bytes, void* stream);

/* qlora_bwd for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the kernels' scratch is a static device array of
 * QLORA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (the one piece of mutable global state of the
 * library), its address looked up on the first call on each device. The
 * call allocates and frees nothing. Layers whose backward needs more
 * scratch than that (qlora_bwd_workspace) return QLORA_EWORKSPACE before
 * anything is enqueued. All calls on one GPU share the array and it keeps
 * the last call's contents (nothing in it needs to start at zero): calls
 * that can overlap on one GPU -- other streams, other threads -- race, so
 * order them on one stream. Otherwise the same arguments, results (bitwise
 * those of qlora_bwd) and errors as qlora_bwd. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int qlora_bwd_noalloc(const qlora_linear* L, int M, int dtype, const void* x,
                      const void* dy, const float* t_saved, void* dx, float* dA,
                      float* dB, void* stream);

/* qlora_bwd in two calls, for callers that take the adapter gradients off the
 * path that carries dx to the next layer (for instance onto a second stream,
 * the way weight gradients are usually overlapped with the rest of a
 * backward pass). Same arithmetic, bitwise the same results:
 *   - qlora_bwd_partial writes dx (skipped if NULL) and leaves fixed-order
 *     per-row-block partial sums of dB and dA in ws;
 *   - qlora_bwd_finish adds those partial sums, in row-block order, times s,
 *     into dB and dA.
 * Both take the same L, M, dtype and workspace (qlora_bwd_workspace bytes).
 * The caller orders them: finish must run after partial's work on ws has
 * completed, and nothing else may write ws in between. Arguments and errors
 * as for qlora_bwd; each call validates its own arguments. */
int qlora_bwd_partial(const qlora_linear* L, int M, int dtype, const void* x,
                      const void* dy, const float* t_saved, void* dx, void* ws,
                      size_t ws_bytes, void* stream);
int qlora_bwd_finish(const qlora_linear* L, int M, int dtype, float* dA,
                     float* dB, void* ws, size_t ws_bytes, void* stream);

/* One layer of qlora_bwd_finish_batch: the arguments of qlora_bwd_finish. */
typedef struct {
  const qlora_linear* L;
  int M;
  int dtype;
  float* dA;          /* [K, r] float32, overwritten */
  float* dB;          /* [r, N] (or per head [heads, r, hd]) float32, overwritten */
  void* ws;           /* that layer's qlora_bwd_partial workspace */
  size_t ws_bytes;
} qlora_finish_item;

/* qlora_bwd_finish for `count` layers (count >= 1) in one launch per 32
 * layers, for a backward pass that runs qlora_bwd_partial layer by layer and
 * takes every adapter gradient ("Why does LoRA reduce memory footprint?":
 * only the adapter's A and B get gradients) at the end. Each layer's dA and
 * dB are bitwise those of its own qlora_bwd_finish (or qlora_bwd): the same
 * sums in the same order. Each item's partial sums -- the first
 * qlora_bwd_partials_bytes bytes of its workspace -- must not overlap any
 * other item's, and must hold that layer's qlora_bwd_partial results,
 * ordered before this call on `stream`; the rest of an item's workspace (its
 * scratch, dead once that qlora_bwd_partial has completed) may overlap other
 * items' partial sums, as the packing described at qlora_bwd_partials_bytes
 * does; items[] is read during the call only (host memory). Every
 * item is validated as by qlora_bwd_finish before anything is enqueued; the
 * first failing item's status is returned (EINVAL also for items == NULL
 * or count < 1). */
int qlora_bwd_finish_batch(const qlora_finish_item* items, int count,
                           void* stream);

/* Bytes at the start of a qlora_bwd workspace (M rows) that hold the partial
 * sums qlora_bwd_partial leaves for qlora_bwd_finish; the rest of the
 * workspace is scratch only while a call runs. So for qlora_bwd_finish_batch
 * a caller that runs the layers' qlora_bwd_partial in the order k = 0, 1, ...
 * may put layer k's workspace at base + the sum of partials_bytes over the
 * layers run before it (instead of a full workspace per layer): each call's
 * scratch then lies only over bytes of layers that have not run yet. The
 * value is a multiple of 256. */
int qlora_bwd_partials_bytes(const qlora_linear* L, int M, int dtype,
                             size_t* bytes);

/* qlora_fwd / qlora_bwd with timing marks, for timing the call's main
 * product kernel live: the int8 or 4-bit forward product; the fused int8
 * backward (dx, u and the adapter-gradient partial sums) or, on the other
 * paths, the input-gradient product. That kernel is launched `repeats` times
 * (>= 1) back to back; every launch rewrites the same outputs from the same
 * inputs, so results are identical to the unmarked call. If not NULL,
 * ev_start and ev_stop (hipEvent_t) are recorded on `stream` immediately
 * before the first and after the last of these launches, so the elapsed
 * time over `repeats` is the kernel's average duration with the cost of the
 * two event records spread over the launches. repeats < 1 -> QLORA_EINVAL. */
int qlora_fwd_timed(const qlora_linear* L, int M, int dtype, const void* x,
                    void* y, float* t_save, void* ws, size_t ws_bytes,
                    void* stream, int repeats, void* ev_start, void* ev_stop);
int qlora_bwd_timed(const qlora_linear* L, int M, int dtype, const void* x,
                    const void* dy, const float* t_saved, void* dx, float* dA,
                    float* dB, void* ws, size_t ws_bytes, void* stream,
                    int repeats, void* ev_start, void* ev_stop);

/* Name of the kernel that qlora_bwd_timed times for this layer, M and
 * dtype (with dx): the fused backward's block shape, or the float32 input
 * gradient. A static string, for benchmarks and profiles to label their
 * timings; NULL for invalid arguments (as qlora_bwd would reject). Host-only
 * arithmetic; usable without a GPU. */
const char* qlora_bwd_main_kernel(const qlora_linear* L, int M, int dtype);

/* Merge the trained adapter into the frozen int8 weight ("Parameter-efficient
 * fine-tuning of GPT-2 with LoRA", "Merge weights and generate text!": the
 * merged kernel is the frozen kernel plus the adapter product; "Introduce
 * QLoRA-like technique", results-table footnote: merging into int8 kernels
 * is lossy, the merged layer's outputs differ from the unmerged ones):
 *   W'[k, n] = float32( q[n, k] sw[n] + s sum_j A[k, j] B[j, n] ),
 * evaluated in float64 with a fixed sequence (exact products, the r terms
 * added in index order, one multiply by s, one add, one rounding), then
 * quantized with the qlora_quantize int8 rule into codes_out int8 [N, K] and
 * scales_out float32 [N] (device memory, 16-byte aligned, not overlapping L's
 * buffers). QLORA_W8 only (QLORA_EUNSUPPORTED otherwise). */
int qlora_merge(const qlora_linear* L, void* codes_out, void* scales_out,
                void* stream);

/* Test hook: the forward's per-row activation quantizer alone. x [M, K] in
 * the compute dtype -> xq int8 [M, K], sx float32 [M]. Same kernel as
 * qlora_fwd. */
int qlora_quantize_rows(const void* x, int M, int K, int dtype, int8_t* xq,
                        float* sx, void* stream);

/* Test hook: the forward's exact int32 product acc [M, N] = xq . codes^T for
 * QLORA_W8 (same quantizer and main loop as qlora_fwd, integer output). */
int qlora_fwd_acc(const qlora_linear* L, int M, int dtype, const void* x,
                  int32_t* acc, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
