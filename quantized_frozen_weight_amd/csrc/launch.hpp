// Internal launchers (one per kernel family). Shapes are validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skinny.hpp"

namespace qlora {

// dtype: 0 = float32, 1 = bfloat16 (matches qlora_dtype)

// hd: head width of W's storage ([heads, K, hd]; N for a plain [K, N]), and
// of B's ([heads, r, hd]) in the launches below
void launch_quantize_w8(const float* W, int K, int N, int hd, int8_t* codes,
                        float* scales, hipStream_t st);
void launch_quantize_w4(const float* W, int K, int N, int hd, uint8_t* packed,
                        _Float16* scales, hipStream_t st);
// Outlier-compensated int8 weight (outlier.hpp): codes int8 [N, K] and the
// side buffer (w8o_layout(K, N).total bytes); W is a plain [K, N].
void launch_quantize_w8o(const float* W, int K, int N, int8_t* codes, void* side,
                         hipStream_t st);
// int8 weight with the adapter merged in, re-quantized (r <= 32); the
// outputs must not overlap the inputs.
void launch_merge_w8(const int8_t* codes, const float* sw, const float* A,
                     const float* B, int hd, int K, int N, int r, float s,
                     int8_t* codes_out, float* scales_out, hipStream_t st);

// asum (optional): float32 [M] row sums of xq
// scratch (optional): row_split_floats(M, K, r) floats; rows of 4097 to
// 16384 entries with t wanted then take two launches split over k instead of
// one that stages the whole adapter in every block
size_t row_split_floats(int M, int K, int r);
void launch_rowquant(int dtype, const void* x, int M, int K, const float* A,
                     int r, int8_t* xq, float* sx, float* t, hipStream_t st,
                     float* asum = nullptr, float* scratch = nullptr);
void launch_lora_down(int dtype, const void* x, int M, int K, const float* A,
                      int r, float* t, hipStream_t st, float* scratch = nullptr);

// y = acc * sx[m] * sw[n] + s * t B   (acc_out != nullptr: write int32 acc).
// Shapes with few output tiles and a long contraction split it when pacc is
// given (fwd_split_ints(M, N, K, false) int32, 0 when the shape does not
// split): the exact partial sums go there and a second launch adds them.
size_t fwd_split_ints(int M, int N, int K, bool affine);
void launch_gemm_fwd_w8(int dtype, int M, int N, int K, const int8_t* xq,
                        const int8_t* codes, const float* sx, const float* sw,
                        const float* t, const float* B, int hd, int r, float s,
                        void* y, int32_t* acc_out, int32_t* pacc, hipStream_t st);
// Outlier-compensated int8 weight (outlier.hpp) with int8 activations:
// y = sx[m] (c acc + b' asum[m] + corr) + s t B (bf16 y). Split like the
// int8 product when pacc and pcorr are given (fwd_split_ints(M, N, K, true)
// int32 and as many floats).
void launch_gemm_fwd_w8o(int M, int N, int K, const int8_t* xq, const int8_t* codes,
                         const float* sx, const float* asum, const void* side,
                         const float* t, const float* B, int hd, int r, float s,
                         uint16_t* y, int32_t* pacc, float* pcorr, hipStream_t st);
// 4-bit weights: the products hold the scales of up to this many 128-wide k
// groups per block in LDS (K <= 16384).
constexpr int kW4MaxGroups = 128;

// y = x deq4(W) + s * t B   (bf16 x and y). Shapes with few 128-row tiles
// and a long contraction split it when pacc is given
// (fwd_w4_split_floats(M, N, K) floats, 0 when the shape does not split):
// the float32 partial sums go there and a second launch adds them.
size_t fwd_w4_split_floats(int M, int N, int K);
// 4-bit weights with int8 activations: exact int8 x int4 sums per 128-wide
// group, weighted by the group's fp16 scale, times sx[m], plus s t B (bf16 y)
void launch_gemm_fwd_a8w4(int M, int N, int K, const int8_t* xq, const float* sx,
                          const uint8_t* packed, const _Float16* scales,
                          const float* t, const float* B, int hd, int r, float s,
                          uint16_t* y, hipStream_t st);
void launch_gemm_fwd_w4(int M, int N, int K, const uint16_t* x,
                        const uint8_t* packed, const _Float16* scales,
                        const float* t, const float* B, int hd, int r, float s,
                        uint16_t* y, float* pacc, hipStream_t st);

// u = dy B^T (float32 [M, r]); if dys != nullptr also dys = bf16(dy * sw[n]).
void launch_bwd_rows(int dtype, const void* dy, int M, int N, const float* B, int hd,
                     int r, const float* sw, uint16_t* dys, float* u,
                     hipStream_t st);

// Adapter gradients dB = s t^T dy ([r, N]) and dA = s x^T u (stored [K, r]):
// stage 1 writes per-split partial sums (partB / partA hold
// skinny_nsplit_host(M) * r * N / K floats), stage 2 adds them in order.
// Stage 1 normally rides along with the input-gradient launch.
SkinnyJobs make_adapter_grad_jobs(int M, int r, float s, const float* t,
                                  const void* dy, int N, float* dB, float* partB,
                                  const float* u, const void* x, int K, float* dA,
                                  float* partA);
void launch_skinny_stage1(int dtype, const SkinnyJobs& p, hipStream_t st);
void launch_skinny_stage2(const SkinnyJobs& p, hipStream_t st);
// stage 2 of n layers, kFinishBatch per launch; each output bitwise as
// launch_skinny_stage2 of its own job
void launch_finish_batch(const SkinnyJobs* jobs, int n, hipStream_t st);

// bf16 backward, int8 (fmt 0: codes [N, K], scales float [N]), 4-bit
// (fmt 1: packed [N, K/2], scales fp16 [N, K/128]) or outlier-compensated
// int8 (fmt 2) weights: dx = dy deq(W)^T + s u A^T with u = dy B^T computed
// on the way, plus per-row-block partial sums of dA (partA [blocks, r, K])
// and dB (partB [blocks, r, N]); blocks = ceil(M / bwd_row_block(...)).
// Shapes with few output tiles and a long contraction split it: the partial
// products go to pdx and the partial u to pu (sizes from bwd_split_sizes,
// both 0 when the shape does not split; the pointers are then unused), and
// a second launch adds them.
int bwd_row_block(int fmt, int M, int K, int N, int r);
// Name of the fused backward kernel (or kernels) launch_bwd_fused uses for
// this shape (static string).
const char* bwd_fused_kernel_name(int fmt, int M, int K, int N, int r);
void bwd_split_sizes(int M, int K, int N, int r, size_t* pdx_floats, size_t* pu_floats);
void launch_bwd_fused(int fmt, int M, int K, int N, const uint16_t* dy,
                      const void* codes, const void* scales, const float* B, int hd,
                      const float* A, const float* t, const uint16_t* x, int r,
                      float s, uint16_t* dx, float* partA, float* partB,
                      float* pdx, float* pu, hipStream_t st);
// dx = dy (codes * sw)^T + s u A^T in float32
void launch_gemm_dx_f32(int M, int K, int N, const float* dy,
                        const int8_t* codes, const float* sw, const float* u,
                        const float* A, int r, float s, float* dx,
                        hipStream_t st);
}  // namespace qlora
