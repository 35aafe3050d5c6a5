// Adapter-gradient reductions: the standalone stage-1 launch (used when no
// input-gradient product runs alongside), and stage 2, which adds the
// per-split partial sums in split order and scales by s. See skinny.hpp.
#include "launch.hpp"
#include "skinny.hpp"

namespace qlora {

namespace {

template <typename T, int R>
__global__ __launch_bounds__(256) void skinny_stage1_kernel(SkinnyJobs p) {
  __shared__ float red[4 * (R < 4 ? R : 4) * kSkCols];
  skinny_partial_block<T, R>(p, blockIdx.x, red);
}

// out = s * sum over splits (split order fixed); one thread per (job, j, c),
// NS loads in flight at a time (NS: the split count rounded up to 8, 16 or 32,
// so no load is wasted on a clamped duplicate).
// What stage 2 reads of a SkinnyJobs (the batched launch carries only this).
struct Stage2Job {
  float* partial[2];
  float* out[2];
  int C[2];
  int transpose[2];
  int hd0, njobs, r, nsplit;
  float s;
};

inline Stage2Job stage2_job(const SkinnyJobs& p) {
  Stage2Job q{};
  for (int i = 0; i < 2; ++i) {
    q.partial[i] = p.partial[i]; q.out[i] = p.out[i];
    q.C[i] = p.C[i]; q.transpose[i] = p.transpose[i];
  }
  q.hd0 = p.hd0; q.njobs = p.njobs; q.r = p.r; q.nsplit = p.nsplit; q.s = p.s;
  return q;
}

template <int NS, typename J>
__device__ __forceinline__ void stage2_elem(const J& p, long e0) {
  const long n0 = (long)p.r * p.C[0];
  const int job = e0 < n0 ? 0 : 1;
  const long e = job ? e0 - n0 : e0;
  if (job == 1 && (p.njobs < 2 || e >= (long)p.r * p.C[1])) return;
  const int C = p.C[job];
  const int j = (int)(e / C), c = (int)(e % C);
  const float* __restrict__ base = p.partial[job] + (long)j * C + c;
  const long stride = (long)p.r * C;
  float sum = 0.f;
  for (int k0 = 0; k0 < p.nsplit; k0 += NS) {
    float v[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      v[k] = base[(k0 + k < p.nsplit ? k0 + k : k0) * stride];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (k0 + k < p.nsplit) sum += v[k];
  }
  const float out = p.s * sum;
  if (p.transpose[job]) p.out[job][(long)c * p.r + j] = out;
  else p.out[job][head_index(j, c, p.r, job == 0 ? p.hd0 : C)] = out;
}

template <int NS>
__global__ __launch_bounds__(256) void skinny_stage2_kernel(SkinnyJobs p) {
  stage2_elem<NS, SkinnyJobs>(p, (long)blockIdx.x * 256 + threadIdx.x);
}

// Stage 2 of several layers in one launch. Block b belongs to item i with
// bstart[i] <= b < bstart[i + 1] and is block b - bstart[i] of that item's
// own stage-2 grid, so every output is the same sum in the same order as in
// a launch of its own.
struct FinishBatch {   // kernel arguments: kept under 4 KiB
  Stage2Job job[kFinishBatch];
  int bstart[kFinishBatch + 1];
  int n;
};
static_assert(sizeof(FinishBatch) <= 4096, "kernel arguments");

template <int NS>
__global__ __launch_bounds__(256) void finish_batch_kernel(FinishBatch fb) {
  const int b = blockIdx.x;
  int i = 0;
  while (i + 1 < fb.n && b >= fb.bstart[i + 1]) ++i;   // block-uniform
  stage2_elem<NS, Stage2Job>(fb.job[i], (long)(b - fb.bstart[i]) * 256 + threadIdx.x);
}

template <typename T>
void stage1_dispatch(const SkinnyJobs& p, hipStream_t st) {
  const int r = p.r, blocks = p.blocks();
  if (r <= 1) skinny_stage1_kernel<T, 1><<<blocks, 256, 0, st>>>(p);
  else if (r <= 2) skinny_stage1_kernel<T, 2><<<blocks, 256, 0, st>>>(p);
  else if (r <= 4) skinny_stage1_kernel<T, 4><<<blocks, 256, 0, st>>>(p);
  else if (r <= 8) skinny_stage1_kernel<T, 8><<<blocks, 256, 0, st>>>(p);
  else if (r <= 16) skinny_stage1_kernel<T, 16><<<blocks, 256, 0, st>>>(p);
  else skinny_stage1_kernel<T, 32><<<blocks, 256, 0, st>>>(p);
}

}  // namespace

SkinnyJobs make_adapter_grad_jobs(int M, int r, float s, const float* t,
                                  const void* dy, int N, float* dB, float* partB,
                                  const float* u, const void* x, int K, float* dA,
                                  float* partA) {
  SkinnyJobs p{};
  p.njobs = 2;
  p.M = M; p.r = r; p.s = s;
  p.nsplit = skinny_nsplit_host(M);
  const int rps = (M + p.nsplit - 1) / p.nsplit;
  p.rows_per_split = (rps + 3) / 4 * 4;
  p.P[0] = t; p.Q[0] = dy; p.C[0] = N; p.out[0] = dB; p.transpose[0] = 0;
  p.partial[0] = partB; p.ncb[0] = (N + kSkCols - 1) / kSkCols; p.hd0 = N;
  p.P[1] = u; p.Q[1] = x; p.C[1] = K; p.out[1] = dA; p.transpose[1] = 1;
  p.partial[1] = partA; p.ncb[1] = (K + kSkCols - 1) / kSkCols;
  return p;
}

void launch_skinny_stage1(int dtype, const SkinnyJobs& p, hipStream_t st) {
  if (dtype == 0) stage1_dispatch<F32>(p, st);
  else stage1_dispatch<BF16>(p, st);
}

namespace {
int stage2_blocks(const SkinnyJobs& p) {
  const long total = (long)p.r * p.C[0] + (p.njobs > 1 ? (long)p.r * p.C[1] : 0);
  return (int)((total + 255) / 256);
}
}  // namespace

void launch_skinny_stage2(const SkinnyJobs& p, hipStream_t st) {
  const dim3 grid((unsigned)stage2_blocks(p));
  if (p.nsplit <= 8) skinny_stage2_kernel<8><<<grid, 256, 0, st>>>(p);
  else if (p.nsplit <= 16) skinny_stage2_kernel<16><<<grid, 256, 0, st>>>(p);
  else skinny_stage2_kernel<kSkMaxSplit><<<grid, 256, 0, st>>>(p);
}

void launch_finish_batch(const SkinnyJobs* jobs, int n, hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kFinishBatch) {
    FinishBatch fb{};
    fb.n = n - i0 < kFinishBatch ? n - i0 : kFinishBatch;
    int maxsplit = 1;
    fb.bstart[0] = 0;
    for (int i = 0; i < fb.n; ++i) {
      fb.job[i] = stage2_job(jobs[i0 + i]);
      fb.bstart[i + 1] = fb.bstart[i] + stage2_blocks(jobs[i0 + i]);
      maxsplit = jobs[i0 + i].nsplit > maxsplit ? jobs[i0 + i].nsplit : maxsplit;
    }
    const dim3 grid((unsigned)fb.bstart[fb.n]);
    if (maxsplit <= 8) finish_batch_kernel<8><<<grid, 256, 0, st>>>(fb);
    else if (maxsplit <= 16) finish_batch_kernel<16><<<grid, 256, 0, st>>>(fb);
    else finish_batch_kernel<kSkMaxSplit><<<grid, 256, 0, st>>>(fb);
  }
}

}  // namespace qlora
