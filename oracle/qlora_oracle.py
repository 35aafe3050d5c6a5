"""CPU oracle for the frozen quantized-weight + LoRA linear (forward and backward).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark import this module. The HIP library never calls it, links it
or shares code with it; it exists to say what the right answer is.

It is written to be read against the pages, not to be fast:

* every quantizer step is one IEEE float32 operation done by numpy on float32
  arrays (correctly rounded divide and multiply, ``np.rint`` = round half to
  even), so codes and scales are exact targets;
* every sum is taken in float64 and rounded once at the end;
* the only library primitive is a float64 matrix product.

Sources (page title, then section):

* [QLoRA-like]  keras PR "Introduce QLoRA-like technique": Highlights (frozen
  int8 kernels for Dense/EinsumDense, LoRA trained on top), the results-table
  footnote (merging LoRA into int8 kernels is lossy), ``model.quantize("int8")``
  in benchmark.py, and the remark that the custom-gradient PR had to land first.
* [GPT-2 LoRA]  keras-io "Parameter-efficient fine-tuning of GPT-2 with LoRA":
  "LoRA equation" (output = W0 x + b0 + B A x), "Create LoRA layer" (the
  adapter output is scaled by alpha / rank; B starts at zero; the original
  layer is frozen), "Why does LoRA reduce memory footprint?" (gradients only
  for the trainable adapter), "Merge weights and generate text!" (W = W0 + BA).
* [llm-light]  keras-llm-light README: "Weights quantization" (LoRA weights kept
  in fp32), "Simplified Int4Variable quantization" (two int4 values per int8),
  "Simplified Int8Variable quantization" (percentile cut, affine codes, fp16
  outliers restored by position).
* [4-bit issue]  GPTQ-for-LLaMa issue "How to fine-tune the 4-bit model?": the
  comments on 4-bit frozen weights under an fp32 adapter, the transposed
  product needed for gradients, dequantize-add-requantize to merge.

Readings taken where the pages are silent:

* int8 weight scale = abs-max of the output channel / 127 (a step size),
  codes = round-half-even(w * (127 / absmax)), symmetric range [-127, 127];
* activations: one abs-max scale per row of the flattened [tokens, K] input,
  same rule;
* a channel/row whose abs-max is 0, or so small that 127/absmax overflows,
  gets scale 0 and zero codes; a non-finite abs-max gets a NaN scale and zero
  codes (so the NaN reaches the output instead of being hidden);
* the gradient passes the activation quantizer unchanged (straight-through):
  dx = dy . deq(W)^T + s (dy B^T) A^T, and the frozen weight gets none;
* 4-bit: groups of 128 along K per output channel, fp16 scale =
  f16(absmax / 7), codes = round-half-even(w * (1 / scale)) in [-7, 7] against
  the stored scale, two's-complement nibbles packed along K with the even k in
  the low nibble; the forward multiplies the (unquantized) activations by the
  dequantized weight;
* multi-head layers: output n = head * hd + d; W [heads, K, hd] and B, dB
  [heads, r, hd] are the plain [K, N] and [r, N] arrays with that column map;
* 4-bit integer forward (the alternative): activations quantized per row as
  above, exact int8 x int4 sums per 128-wide group, each weighted by its fp16
  scale, the total by the row scale; adapter term as in the float forward.
* outlier-compensated int8 weights ([llm-light] "Simplified Int8Variable
  quantization"): one nearest-rank cut per tensor at the 0.1th and 99.9th
  percentiles, an affine 255-step grid between the cuts (bias = lower cut),
  the elements outside the cut kept as fp16 values at their positions; the
  layer quantizes its activations per row as the int8 layer does (details
  in that section below).

Layouts: W [K, N] float32 (the pages' kernel orientation); int8 codes [N, K]
(one output channel per row, K contiguous) with scales [N]; 4-bit codes
[N, K/2] bytes with fp16 scales [N, K/128]; x [M, K]; y, dy [M, N];
A [K, r]; B [r, N]; t = x A [M, r].
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

# ---------------------------------------------------------------------------
# Rounding of results to the compute dtype
# ---------------------------------------------------------------------------


def round_f32(v) -> np.ndarray:
    """float64 -> float32, round to nearest even (numpy's cast)."""
    return np.asarray(v, dtype=F64).astype(F32)


def f32_to_bf16_bits(v32) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Written from the format definition: bfloat16 is the upper half of a
    float32, so the 16 dropped bits are rounded into the kept half. NaN stays
    a (quiet) NaN; values past the largest finite bfloat16 round to infinity.
    """
    u = np.ascontiguousarray(v32, dtype=F32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    rounded = np.where(is_nan, ((u >> 16) | 0x0040) & 0xFFFF, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(F32)


def round_to(v64, dtype: str) -> np.ndarray:
    """Round a float64 result once to float32, then (bf16) once more to bf16.

    Returned as float32 values (a bf16 value is exactly representable)."""
    v32 = round_f32(v64)
    if dtype == "f32":
        return v32
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(v32))
    raise ValueError(dtype)


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / rank ([GPT-2 LoRA] "Create LoRA layer"), one float32 divide."""
    return float(F32(alpha) / F32(r))


# ---------------------------------------------------------------------------
# Symmetric abs-max int8 quantization (weights per output channel, activations
# per row). [QLoRA-like] "Highlights" and benchmark.py's quantize("int8").
# ---------------------------------------------------------------------------


def _absmax_quantize(v: np.ndarray, axis: int, qmax: int):
    """Quantize float32 ``v`` along ``axis`` (the reduced axis) to [-qmax, qmax].

    Returns (codes int8 with v's shape, scale float32 with the other axis).
    Each step is a single float32 operation:
      a     = max |v|                 (exact)
      inv   = fl32(qmax / a)
      scale = fl32(a / qmax)
      q     = clamp(rint(fl32(v * inv)), -qmax, qmax)
    """
    v = np.asarray(v, dtype=F32)
    a = np.max(np.abs(v), axis=axis)
    qm = F32(qmax)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = qm / a
        scale = a / qm
        prod = v * np.expand_dims(inv, axis)
        q = np.clip(np.rint(prod), -qmax, qmax)
    nonfinite = ~np.isfinite(a)
    empty = (~nonfinite) & ((a == 0) | ~np.isfinite(inv))
    dead = np.expand_dims(nonfinite | empty, axis)
    q = np.where(dead, 0, q)
    scale = np.where(empty, F32(0), scale)
    scale = np.where(nonfinite, F32(np.nan), scale).astype(F32)
    return q.astype(np.int8), scale


def quantize_w8(W) -> tuple[np.ndarray, np.ndarray]:
    """Frozen weight W [K, N] -> (codes int8 [N, K], sw float32 [N])."""
    q, sw = _absmax_quantize(np.asarray(W, dtype=F32), axis=0, qmax=127)
    return np.ascontiguousarray(q.T), sw


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Activations x [M, K] (float32 values) -> (xq int8 [M, K], sx float32 [M])."""
    return _absmax_quantize(np.asarray(x, dtype=F32), axis=1, qmax=127)


def dequant_w8(codes, sw) -> np.ndarray:
    """deq(W)[k, n] = codes[n, k] * sw[n], exact in float64, shape [K, N]."""
    return (np.asarray(codes, dtype=F64) * np.asarray(sw, F64)[:, None]).T


def int8_acc(xq, codes) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * codes[n, k] as int64, exact.

    Computed with a float64 product: every term and every partial sum is an
    integer of magnitude <= K * 127 * 127 < 2**31 < 2**53, so no rounding can
    happen in any summation order. The bound is asserted.
    """
    a = np.asarray(xq, dtype=F64) @ np.asarray(codes, dtype=F64).T
    K = np.asarray(xq).shape[1]
    assert K * 127 * 127 < 2 ** 31, "int32 accumulator could overflow"
    return a.astype(np.int64)


# ---------------------------------------------------------------------------
# Forward: y = x deq(W) + s (x A) B     ([GPT-2 LoRA] "LoRA equation",
# "Create LoRA layer"; quantized base product per [QLoRA-like] "Highlights")
# ---------------------------------------------------------------------------


def lora_down(x, A) -> np.ndarray:
    """t = x A in float64 (unscaled), [M, r]."""
    return np.asarray(x, F64) @ np.asarray(A, F64)


def fwd_w8_f64(x, codes, sw, A, B, alpha: float):
    """Unrounded forward. Returns (y64 [M, N], t64 [M, r], xq, sx, acc).

    The base term is the integer product rescaled by the row and channel
    scales; the adapter term is the float LoRA branch scaled by alpha/r.
    """
    x = np.asarray(x, F32)
    xq, sx = quantize_rows(x)
    acc = int8_acc(xq, codes)
    t = lora_down(x, A)
    s = lora_scale(alpha, np.asarray(A).shape[1])
    base = acc.astype(F64) * np.asarray(sx, F64)[:, None] * np.asarray(sw, F64)[None, :]
    y = base + s * (t @ np.asarray(B, F64))
    return y, t, xq, sx, acc


def fwd_w8(x, codes, sw, A, B, alpha: float, dtype: str):
    """Forward rounded to the compute dtype: (y, t as float32)."""
    y, t, *_ = fwd_w8_f64(x, codes, sw, A, B, alpha)
    return round_to(y, dtype), round_f32(t)


# ---------------------------------------------------------------------------
# Backward. Only the adapter is trainable ([GPT-2 LoRA] "Why does LoRA reduce
# memory footprint?", "Create LoRA layer": the original layer is frozen), so
# the outputs are dA, dB and the input gradient dx; there is no dW.
# ---------------------------------------------------------------------------


def bwd_f64(x, dy, Wdeq, A, B, alpha: float):
    """Unrounded gradients for y = x Wdeq + s (x A) B with loss gradient dy.

    Wdeq [K, N] is the dequantized frozen weight (the quantizer of x is passed
    straight through). Returns (dx64 [M,K], dA64 [K,r], dB64 [r,N], u64 [M,r]).
    """
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    A = np.asarray(A, F64)
    B = np.asarray(B, F64)
    s = lora_scale(alpha, A.shape[1])
    t = x @ A                    # [M, r]
    u = dy @ B.T                 # [M, r]  gradient reaching the adapter's middle
    dB = s * (t.T @ dy)          # [r, N]
    dA = s * (x.T @ u)           # [K, r]
    dx = dy @ np.asarray(Wdeq, F64).T + s * (u @ A.T)
    return dx, dA, dB, u


def bwd(x, dy, Wdeq, A, B, alpha: float, dtype: str):
    """Gradients rounded: dx to the compute dtype, dA and dB to float32."""
    dx, dA, dB, _ = bwd_f64(x, dy, Wdeq, A, B, alpha)
    return round_to(dx, dtype), round_f32(dA), round_f32(dB)


# ---------------------------------------------------------------------------
# 4-bit weights: two signed 4-bit codes per byte ([llm-light] "Simplified
# Int4Variable quantization"), one fp16 scale per 128 inputs of an output
# channel; the weight is dequantized to float before the product, as the
# [4-bit issue] comments describe.
# ---------------------------------------------------------------------------

GROUP = 128


def quantize_w4(W):
    """W [K, N] float32 -> (packed uint8 [N, K/2], scales float16 [N, K/128]).

    Per (channel n, group g of 128 consecutive k):
      a   = max |W| over the group
      s16 = f16(fl32(a / 7))          (round to nearest even, may overflow)
      sc  = float(s16)
      q   = clamp(rint(fl32(W * fl32(1 / sc))), -7, 7)   (0 when sc == 0)
    A group whose abs-max is not finite, or whose scale overflows fp16, is
    stored with a NaN scale and zero codes.
    """
    W = np.asarray(W, dtype=F32)
    K, N = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    Wg = np.ascontiguousarray(W.T).reshape(N, G, GROUP)
    a = np.max(np.abs(Wg), axis=2)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        s16 = (a / F32(7)).astype(np.float16)
        sc = s16.astype(F32)
        inv = F32(1) / sc
        q = np.clip(np.rint(Wg * inv[:, :, None]), -7, 7)
    bad = ~np.isfinite(a) | ~np.isfinite(sc)
    zero = (~bad) & (sc == 0)
    q = np.where((bad | zero)[:, :, None], 0, q).astype(np.int8).reshape(N, K)
    s16 = np.where(bad, np.float16(np.nan), s16).astype(np.float16)
    return pack_nibbles(q), s16


def pack_nibbles(q) -> np.ndarray:
    """int8 codes [N, K] in [-8, 7] -> bytes [N, K/2]; even k in the low nibble."""
    q = np.asarray(q, dtype=np.int16)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """bytes [N, K/2] -> int8 codes [N, K], two's-complement nibbles."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_w4(packed, scales) -> np.ndarray:
    """deq4[k, n] = q[n, k] * scale[n, k // 128], exact in float64, [K, N]."""
    q = unpack_nibbles(packed).astype(F64)
    sc = np.asarray(scales, dtype=np.float16).astype(F64)
    N, K = q.shape
    return (q.reshape(N, K // GROUP, GROUP) * sc[:, :, None]).reshape(N, K).T


def fwd_w4_f64(x, packed, scales, A, B, alpha: float):
    """Unrounded 4-bit forward: y = x deq4(W) + s (x A) B; returns (y64, t64)."""
    x64 = np.asarray(x, F64)
    t = lora_down(x64, A)
    s = lora_scale(alpha, np.asarray(A).shape[1])
    y = x64 @ dequant_w4(packed, scales) + s * (t @ np.asarray(B, F64))
    return y, t


def fwd_w4(x, packed, scales, A, B, alpha: float, dtype: str):
    y, t = fwd_w4_f64(x, packed, scales, A, B, alpha)
    return round_to(y, dtype), round_f32(t)


# ---------------------------------------------------------------------------
# Multi-head layouts ([GPT-2 LoRA] "Create LoRA layer": the attention
# projections are EinsumDense layers whose output is [heads, head_dim], and
# the adapter's B keeps that per-head output shape; [QLoRA-like] Highlights:
# frozen int8 EinsumDense kernels). Output n of the layer is head n // hd,
# position n % hd; the layer itself is the plain one on the mapped tensors.
# ---------------------------------------------------------------------------


def heads_to_plain(T) -> np.ndarray:
    """[heads, rows, hd] -> [rows, heads * hd] (column n = head * hd + d)."""
    T = np.asarray(T)
    H, rows, hd = T.shape
    return np.transpose(T, (1, 0, 2)).reshape(rows, H * hd)


def plain_to_heads(T, heads: int) -> np.ndarray:
    """[rows, N] -> [heads, rows, N / heads]; inverse of heads_to_plain."""
    T = np.asarray(T)
    rows, N = T.shape
    return np.ascontiguousarray(np.transpose(T.reshape(rows, heads, N // heads), (1, 0, 2)))


# ---------------------------------------------------------------------------
# Integer forward of the 4-bit layer with int8 activations: an alternative to
# the dequantized float product above. The activations are quantized per row
# with the int8 rule; each 128-wide group of the contraction is an exact
# integer sum of int8 x int4 products, and each group's sum is weighted by
# its fp16 scale. ([llm-light] "Simplified Int4Variable quantization": two
# int4 codes per byte; [4-bit issue]: narrow frozen weights under a float
# adapter and the arithmetic intensity they buy; [QLoRA-like] Highlights: the
# int8 x int8 integer product the int8 path already uses.)
# ---------------------------------------------------------------------------


def int4_group_acc(xq, packed) -> np.ndarray:
    """acc[g, m, n] = sum over k in group g of xq[m, k] * q[n, k], int64, exact."""
    q = unpack_nibbles(packed).astype(np.int64)          # [N, K]
    xq = np.asarray(xq).astype(np.int64)                 # [M, K]
    N, K = q.shape
    G = K // GROUP
    acc = np.empty((G, xq.shape[0], N), np.int64)
    for g in range(G):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        acc[g] = xq[:, ks] @ q[:, ks].T
    return acc


def fwd_a8w4_f64(x, packed, scales, A, B, alpha: float):
    """Unrounded integer 4-bit forward. Returns (y64, t64, xq, sx):
    y[m, n] = sx[m] * sum_g sc[n, g] acc[g, m, n] + s sum_j t[m, j] B[j, n]."""
    x32 = np.asarray(x, F32)
    xq, sx = quantize_rows(x32)
    acc = int4_group_acc(xq, packed).astype(F64)          # exact in float64
    sc = np.asarray(scales, dtype=np.float16).astype(F64)  # [N, G]
    base = np.einsum("gmn,ng->mn", acc, sc)
    t = lora_down(x32.astype(F64), A)
    s = lora_scale(alpha, np.asarray(A).shape[1])
    y = sx.astype(F64)[:, None] * base + s * (t @ np.asarray(B, F64))
    return y, t, xq, sx


def fwd_a8w4(x, packed, scales, A, B, alpha: float, dtype: str):
    y, t, _, _ = fwd_a8w4_f64(x, packed, scales, A, B, alpha)
    return round_to(y, dtype), round_f32(t)


# ---------------------------------------------------------------------------
# Merge of a trained adapter into the frozen weight ([GPT-2 LoRA] "Merge
# weights and generate text!"; lossy when the result is re-quantized per the
# [QLoRA-like] results-table footnote and the [4-bit issue] comments).
# ---------------------------------------------------------------------------


def merged_weight_w8(codes, sw, A, B, alpha: float) -> np.ndarray:
    """The adapter folded into the frozen weight, as float32 [K, N]
    ([GPT-2 LoRA] "Merge weights and generate text!": the merged kernel is
    the frozen kernel plus the adapter product; here scaled by s as in the
    forward):

        W'[k, n] = fl32( deq(W)[k, n] + s * sum_j A[k, j] B[j, n] )

    evaluated in float64 with a fixed operation sequence: deq = q * sw and
    every A B product are exact in float64; the r products are added in
    index order; then one multiply by s, one add, and one rounding to
    float32."""
    A64 = np.asarray(A, F64)
    B64 = np.asarray(B, F64)
    K, r = A64.shape
    acc = np.zeros((K, B64.shape[1]), F64)
    for j in range(r):
        acc = acc + A64[:, j:j + 1] * B64[j:j + 1, :]
    s = F64(lora_scale(alpha, r))
    return (dequant_w8(codes, sw) + s * acc).astype(F32)


def merge_w8(codes, sw, A, B, alpha: float):
    """Merge the adapter into the int8 weight: W' (merged_weight_w8),
    re-quantized with the same per-channel int8 rule. Lossy: the merged codes
    are W' rounded to its own channel grid ([QLoRA-like] results-table
    footnote: merging LoRA into int8 kernels changes the outputs)."""
    return quantize_w8(merged_weight_w8(codes, sw, A, B, alpha))

# ---------------------------------------------------------------------------
# Outlier-compensated int8 weights ([llm-light] "Simplified Int8Variable
# quantization"): the weight is cut at its 0.1th and 99.9th percentiles, the
# clipped weight is stored as 8-bit codes of an affine grid (a bias and a
# step, reconstructed as bias + value * scale in float32), and the elements
# outside the cut are kept exactly, as fp16 values at their (row, column),
# written over the reconstruction before the layer is used.
#
# Readings (the section gives the three steps and the reconstruction code but
# no formulas for the cut or the grid):
# * one cut, one bias and one scale per weight tensor (the section's memory
#   table shows each 2048 x 16384 kernel barely above its size in bytes, and
#   same-shaped kernels of different sizes, i.e. data-dependent outlier
#   counts rather than per-channel arrays);
# * "99.9 percentile cutoff" as two nearest-rank percentiles of all K*N
#   elements, lo = P(0.1) and hi = P(99.9): P(q) is the smallest element x
#   with at least q percent of the elements <= x, i.e. the element of 1-based
#   rank ceil(q n / 100) in ascending order;
# * outliers are the elements < lo ("min") and > hi ("max");
# * the grid spans [lo, hi] in 255 steps: bias = lo, scale = fl32(d / 255)
#   with d = fl32(hi - lo), value = clamp(rint(fl32(fl32(clip(w) - lo) *
#   fl32(255 / d))), 0, 255) -- the same multiply-by-inverse form as the int8
#   rule; if d is 0 or not finite, or 255 / d overflows, scale is 0 and every
#   value 0;
# * the layer itself is the int8 layer's: activations quantized per row, the
#   base product sx[m] * sum_k xq[m, k] Wr[k, n] with Wr the reconstructed
#   weight; the gradient passes the quantizers (dx = dy Wr^T + s u A^T).
# W must be finite (no rule is stated for NaN or infinite weights).
# ---------------------------------------------------------------------------

OUTLIER_TAIL = (1, 1000)   # each tail holds 1/1000 of the elements (0.1 %)


def nearest_rank_index(n: int, num: int, den: int) -> int:
    """0-based ascending position of the nearest-rank percentile 100 num/den
    of n elements: rank ceil(num n / den), at least 1, in exact integers."""
    rank = -(-num * n // den)
    return max(rank, 1) - 1


def quantize_w8o(W) -> dict:
    """W [K, N] float32 -> the outlier-compensated int8 weight:

      lo, hi, scale   float32 scalars (bias = lo)
      value           uint8 [K, N], the clipped weight's grid index
      rows, cols      int64 [nnz], outlier positions in row-major (k, n) order
      vals            float16 [nnz], the outliers' values
    """
    W = np.asarray(W, dtype=F32)
    n = W.size
    num, den = OUTLIER_TAIL
    v = np.sort(W.ravel())
    lo = F32(v[nearest_rank_index(n, num, den)])
    hi = F32(v[nearest_rank_index(n, den - num, den)])
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        d = F32(hi - lo)
        inv = F32(255) / d
        scale = d / F32(255)
    if not (d > 0 and np.isfinite(d) and np.isfinite(inv)):
        inv, scale = F32(0), F32(0)
    clipped = np.minimum(np.maximum(W, lo), hi)
    value = np.clip(np.rint((clipped - lo) * inv), 0, 255).astype(np.uint8)
    rows, cols = np.nonzero((W < lo) | (W > hi))
    return dict(lo=lo, hi=hi, scale=F32(scale), value=value, rows=rows, cols=cols,
                vals=W[rows, cols].astype(np.float16))


def dequant_w8o(q) -> np.ndarray:
    """The reconstructed weight Wr [K, N] float32, as the section's code does
    it: bias + float(value) * scale in float32 (a multiply, then an add),
    then every outlier position overwritten with its fp16 value."""
    Wr = q["lo"] + q["value"].astype(F32) * q["scale"]
    Wr = np.asarray(Wr, dtype=F32).copy()
    Wr[q["rows"], q["cols"]] = q["vals"].astype(F32)
    return Wr


def w8o_device_codes(q) -> np.ndarray:
    """The codes as the library stores them: int8 [N, K] = value - 128
    (the same grid index, offset to the signed range of the int8 products)."""
    return np.ascontiguousarray((q["value"].astype(np.int16) - 128).astype(np.int8).T)


def fwd_w8o_f64(x, q, A, B, alpha: float):
    """Unrounded forward of the outlier-compensated layer. Returns
    (y64, t64, xq, sx): y = sx[m] sum_k xq[m, k] Wr[k, n] + s (x A) B."""
    x32 = np.asarray(x, F32)
    xq, sx = quantize_rows(x32)
    Wr = dequant_w8o(q).astype(F64)
    base = np.asarray(sx, F64)[:, None] * (xq.astype(F64) @ Wr)
    t = lora_down(x32.astype(F64), A)
    s = lora_scale(alpha, np.asarray(A).shape[1])
    return base + s * (t @ np.asarray(B, F64)), t, xq, sx


def fwd_w8o(x, q, A, B, alpha: float, dtype: str):
    y, t, _, _ = fwd_w8o_f64(x, q, A, B, alpha)
    return round_to(y, dtype), round_f32(t)
