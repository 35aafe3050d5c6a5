// MFMA products of the frozen-weight layer.
//
// Forward, int8 weights: acc[m, n] = sum_k xq[m, k] q[n, k] on
// v_mfma_i32_16x16x64_i8 (exact int32), fused epilogue
//     y[m, n] = fma(s, sum_j t[m, j] B[j, n], float(acc) * (sx[m] * sw[n]))
// ("Parameter-efficient fine-tuning of GPT-2 with LoRA", "LoRA equation":
// the adapter branch is added to the frozen layer's output; "Create LoRA
// layer": scaled by alpha / rank; "Introduce QLoRA-like technique",
// "Highlights": the frozen kernel is int8).
//
// Forward, 4-bit weights: y = x deq4(W) + s t B on v_mfma_f32_16x16x32_bf16;
// the nibbles are unpacked, scaled by their fp16 group scale and rounded to
// bf16 on the way into LDS ("How to fine-tune the 4-bit model?": dequantize
// in place at operand load, feeding the matrix unit).
//
// Input gradient: dx[m, k] = sum_n g[m, n] W'[k, n] + s sum_j u[m, j] A[k, j]
// with the straight-through estimator for the activation quantizer. For
// int8 weights g = bf16(dy * sw) (channel scale folded into the gradient rows
// by the row pass) and W' = q, the raw codes, exact in bf16; for 4-bit
// weights g = dy and W' = bf16(q * scale). The weight is stored [N, K] (K
// contiguous) while this product contracts over n, so every block transposes
// its [64 n x BN k] code slice while widening it to bf16 into LDS ([k][n]);
// this is the transposed quantized product "How to fine-tune the 4-bit
// model?" names as what adapter training needs. The same launch carries the
// first stage of the adapter-gradient reductions (skinny.hpp) as extra
// blocks, since both only need the row pass's outputs.
//
// Block = 4 waves in a 2 x 2 grid; a wave owns (BM/2) x (BN/2) outputs as
// 16 x 16 MFMA blocks. Operands are staged in LDS with the contraction axis
// contiguous and rows padded by 16 bytes, so the 16 rows an MFMA operand read
// touches fall in distinct banks. Global loads run D slices ahead in
// registers, and the epilogue's operands (t or u, B or A^T, row and channel
// scales) are fetched at kernel start, so a block waits on memory about
// once per D slices. 64 x 64 tiles are used when 128 x 128 tiles would leave
// most of the 256 compute units idle.
#include "common.hpp"
#include "launch.hpp"
#include "skinny.hpp"

namespace qlora {

namespace {

constexpr int kCUs = 256;
constexpr int kMaxR = 32;

// Tuning knobs (compile-time): slices in flight for the 64 x 64 and
// 128 x 128 tiles, and whether the adapter-gradient stage 1 rides along
// with the input-gradient launch.
#ifndef QLORA_D_SMALL
#define QLORA_D_SMALL 8
#endif
#ifndef QLORA_D_BIG
#define QLORA_D_BIG 2
#endif
#ifndef QLORA_FUSE_STAGE1
#define QLORA_FUSE_STAGE1 1
#endif
#ifndef QLORA_BIG_TILE_MIN
#define QLORA_BIG_TILE_MIN (kCUs - 16)
#endif

// Epilogue operands in LDS: ts [BM][r], qs [r][BN], rsv [BM], csv [BN].
template <int BM, int BN> struct Epi {
  static constexpr int kFloats = BM * kMaxR + kMaxR * BN + BM + BN;
  static constexpr int NT = BM * kMaxR / 256;     // t entries per thread (bound)
  static constexpr int NQ = kMaxR * BN / 256;
  float t[NT], q[NQ], rs, cs;

  // P float32 [M, r]; Q(j, n) = Q[j * ldj + n * ldn]; rsrc/csrc optional.
  __device__ __forceinline__ void load(int M, int N, int m0, int n0, int r, const float* __restrict__ P,
                       const float* __restrict__ Q, long ldj, long ldn,
                       const float* __restrict__ rsrc, const float* __restrict__ csrc) {
    // Loads run unconditionally from clamped addresses and are masked
    // afterwards: branches around loads make the compiler wait for every
    // outstanding load at each join. A clamped address stays next to the
    // real one, so masked lanes of different blocks do not pile onto one
    // cache line (lanes of one instruction that share a line coalesce).
    const int tid = threadIdx.x;
    const int nt = BM * r, nq = r * BN;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = tid + 256 * i;
      const int ec = e < nt ? e : nt - 1;
      const int gm = m0 + ec / r;
      const float v = P[(long)(gm < M ? gm : M - 1) * r + ec % r];
      t[i] = (e < nt && gm < M) ? v : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 256 * i;
      const int ec = e < nq ? e : nq - 1;
      const int gn = n0 + ec % BN;
      const float v = Q[(long)(ec / BN) * ldj + (long)(gn < N ? gn : N - 1) * ldn];
      q[i] = (e < nq && gn < N) ? v : 0.f;
    }
    if (rsrc != nullptr) {
      const int im = m0 + (tid < BM ? tid : BM - 1), in = n0 + (tid < BN ? tid : BN - 1);
      const float a = rsrc[im < M ? im : M - 1], b = csrc[in < N ? in : N - 1];
      rs = (tid < BM && im < M) ? a : 0.f;
      cs = (tid < BN && in < N) ? b : 0.f;
    } else {
      rs = cs = 0.f;
    }
  }
  __device__ __forceinline__ void store(float* E, int r) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = tid + 256 * i;
      if (e < BM * r) E[e] = t[i];
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 256 * i;
      if (e < r * BN) E[BM * kMaxR + e] = q[i];
    }
    if (tid < BM) E[BM * kMaxR + kMaxR * BN + tid] = rs;
    if (tid < BN) E[BM * kMaxR + kMaxR * BN + BM + tid] = cs;
  }
};

// Apply the epilogue to the wave's FM x FN grid of 16 x 16 accumulator blocks
// (lane holds rows 4 (lane / 16) + ii of column lane % 16 of each block).
template <int BM, int BN, typename OutT, typename AccT, int FM, int FN>
__device__ __forceinline__ void epilogue(const AccT (&acc)[FM][FN], const float* E,
                                         int M, int N, int m0, int n0, int wm, int wn,
                                         int r, float s, bool scaled,
                                         OutT* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const float* ts = E;
  const float* qs = E + BM * kMaxR;
  const float* rsv = qs + kMaxR * BN;
  const float* csv = rsv + BM;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int nl = wn * (BN / 2) + j * 16 + (lane & 15);
    const int n = n0 + nl;
    if (n >= N) continue;
    const float csn = scaled ? csv[nl] : 1.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int ml = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
        const int m = m0 + ml;
        if (m >= M) continue;
        float low = 0.f;
        for (int jj = 0; jj < r; ++jj)
          low = __builtin_fmaf(ts[ml * r + jj], qs[jj * BN + nl], low);
        const float base = scaled ? (float)acc[i][j][ii] * (rsv[ml] * csn)
                                  : (float)acc[i][j][ii];
        store_out(out + (long)m * N + n, __builtin_fmaf(s, low, base));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 products (4-bit forward, input gradients). A operand: bf16 rows
// [M, Kc] with the contraction Kc contiguous, staged directly. B operand
// (per kind):
//   kW4Fwd : packed [N, K/2] + fp16 scales -> LDS [n][k]     (contract k)
//   kW8T   : int8 codes [N, K]             -> LDS [k][n]     (contract n)
//   kW4T   : packed [N, K/2] + fp16 scales -> LDS [k][n]     (contract n)
// The block computes output rows m (BM) x columns c (BN); the contraction
// runs in slices of 64.
// ---------------------------------------------------------------------------
enum BKind { kW4Fwd = 0, kW8T = 1, kW4T = 2 };

template <int BN, int KIND> struct BStage;

// 4-bit forward: B tile [BN n][64 k] = BN x 32 bytes; each thread BN/4
// nibbles of one row.
template <int BN> struct BStage<BN, kW4Fwd> {
  static constexpr int NIB = BN / 4;                 // nibbles per thread (16 or 32)
  static constexpr int TPR = 64 / NIB;               // threads per row
  uint32_t w[NIB / 8];
  float sc;
  __device__ __forceinline__ void load(const void* codes, const _Float16* scales, int Kw, int Nw,
                       int c0, int kc0, bool kok) {
    const uint8_t* packed = reinterpret_cast<const uint8_t*>(codes);
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    const int gn = c0 + row, gk = kc0 + part * NIB;
    const bool ok = kok && gn < Nw && gk < Kw;
    const int gnc = gn < Nw ? gn : Nw - 1, gkc = gk < Kw ? gk : Kw - NIB;
    const uint8_t* p = packed + (long)gnc * (Kw / 2) + gkc / 2;
    if constexpr (NIB == 32) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
      w[0] = ok ? v.x : 0u; w[1] = ok ? v.y : 0u; w[2] = ok ? v.z : 0u; w[3] = ok ? v.w : 0u;
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = ok ? v.x : 0u; w[1] = ok ? v.y : 0u;
    }
    const float scv = (float)scales[(long)gnc * (Kw / 128) + gkc / 128];
    sc = ok ? scv : 0.f;
  }
  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* Bs) const {
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
#pragma unroll
    for (int d = 0; d < NIB / 8; ++d) {
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int q0 = ((int)(w[d] << (28 - 8 * p))) >> 28;
        const int q1 = ((int)(w[d] << (24 - 8 * p))) >> 28;
        o[p] = pack_bf16x2((float)q0 * sc, (float)q1 * sc);
      }
      *reinterpret_cast<u32x4*>(&Bs[row * PITCH + part * NIB + d * 8]) =
          u32x4{o[0], o[1], o[2], o[3]};
    }
  }
};

// 4-bit codes, transposed: tile [64 n][BN k] nibbles. Thread: k octet ko
// (one dword of 8 nibbles), NPT consecutive n rows.
template <int BN> struct BStage<BN, kW4T> {
  static constexpr int KO = BN / 8;                  // k octets per row
  static constexpr int NPT = 64 / (256 / KO);        // n rows per thread (2 or 4)
  uint32_t w[NPT];
  float sc[NPT];
  __device__ __forceinline__ void load(const void* codes, const _Float16* scales, int Kw, int Nw,
                       int c0, int n0, bool kok) {
    const uint8_t* packed = reinterpret_cast<const uint8_t*>(codes);
    const int ko = threadIdx.x % KO, ng = threadIdx.x / KO;
    const int gk = c0 + 8 * ko;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int gn = n0 + ng * NPT + i;
      const bool ok = kok && gn < Nw && gk < Kw;
      const int gnc = gn < Nw ? gn : Nw - 1, gkc = gk < Kw ? gk : Kw - 8;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(packed + (long)gnc * (Kw / 2) + gkc / 2);
      const float scv = (float)scales[(long)gnc * (Kw / 128) + gkc / 128];
      w[i] = ok ? v : 0u;
      sc[i] = ok ? scv : 0.f;
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* Bs) const {
    const int ko = threadIdx.x % KO, ng = threadIdx.x / KO;
#pragma unroll
    for (int jk = 0; jk < 8; ++jk) {
      float v[NPT];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int q = ((int)(w[i] << (28 - 4 * jk))) >> 28;
        v[i] = (float)q * sc[i];
      }
      uint16_t* dst = &Bs[(8 * ko + jk) * PITCH + ng * NPT];
      if constexpr (NPT == 4)
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      else
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(v[0], v[1]);
    }
  }
};

struct Bf16Args {
  int M, Cout, Kc;                 // rows, output columns, contraction length
  int Kw, Nw;                      // weight shape for the B loaders
  const uint16_t* g;               // A operand [M, Kc]
  const void* codes;
  const _Float16* scales;
  const float* P; const float* Q; long ldj, ldn;   // low-rank epilogue
  int r; float s;
  uint16_t* out;                   // [M, Cout]
  int tiles_x, tiles;              // output tiles (grid prefix)
};

// One launch: blocks [0, tiles) compute output tiles; blocks past that run
// stage 1 of the adapter-gradient reductions (R = padded rank; sk may be
// empty).
template <int BM, int BN, int D, int KIND, int R>
__global__ __launch_bounds__(256) void bf16_kernel(Bf16Args a, SkinnyJobs sk) {
  constexpr int BKC = 64, PITCH = BKC + 8;           // bf16 elements
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int CA = BM / 32;                        // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * PITCH];
  __shared__ __attribute__((aligned(16))) float E[Epi<BM, BN>::kFloats];
  static_assert(2 * BM * PITCH * 2 >= 4 * (R < 4 ? R : 4) * kSkCols * 4, "LDS for stage 1");

  if ((int)blockIdx.x >= a.tiles) {
    skinny_partial_block<BF16, R>(sk, blockIdx.x - a.tiles, reinterpret_cast<float*>(&As[0][0]));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = (blockIdx.x / a.tiles_x) * BM, c0 = (blockIdx.x % a.tiles_x) * BN;
  const int arow = tid >> 3, acol = (tid & 7) * 8;
  const int M = a.M, Kc = a.Kc;
  const int nk = (Kc + BKC - 1) / BKC;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // same slice schedule as the int8 forward: nkp = nk rounded up to D,
  // slices past the end re-read the block's own last slice (masked), the
  // last D slices issue nothing.
  const int nkp = (nk + D - 1) / D * D;
  u32x4 ra[D][CA];
  BStage<BN, KIND> rb[D];
  auto issue = [&](u32x4 (&av)[CA], BStage<BN, KIND>& b, int kt) {
    const bool kok = kt < nk;
    const int ktc = kok ? kt : nk - 1;
    const int gk = ktc * BKC + acol;
    const int gkc = gk < Kc ? gk : Kc - 8;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int gm = m0 + arow + 32 * i;
      const bool ok = kok && gm < M && gk < Kc;
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.g + (long)(gm < M ? gm : M - 1) * Kc + gkc);
      av[i] = ok ? v : zero;
    }
    b.load(a.codes, a.scales, a.Kw, a.Nw, c0, ktc * BKC, kok);
  };

#pragma unroll
  for (int st = 0; st < D; ++st) issue(ra[st], rb[st], st);
  {
    Epi<BM, BN> ep;
    ep.load(M, a.Cout, m0, c0, a.r, a.P, a.Q, a.ldj, a.ldn, nullptr, nullptr);
    ep.store(E, a.r);
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto slice = [&](int st, bool refill, int kt) {
    const int buf = st & 1;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][(arow + 32 * i) * PITCH + acol]) = ra[st][i];
    rb[st].template store<PITCH>(Bs[buf]);
    __syncthreads();
    if (refill) issue(ra[st], rb[st], kt + D);
#pragma unroll
    for (int kk = 0; kk < BKC / 32; ++kk) {
      const int off = kk * 32 + (lane >> 4) * 8;
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &As[buf][(wm * (BM / 2) + i * 16 + (lane & 15)) * PITCH + off]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[buf][(wn * (BN / 2) + j * 16 + (lane & 15)) * PITCH + off]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  int kt0 = 0;
  for (; kt0 + D < nkp; kt0 += D) {
#pragma unroll
    for (int st = 0; st < D; ++st) slice(st, true, kt0 + st);
  }
#pragma unroll
  for (int st = 0; st < D; ++st) slice(st, false, kt0 + st);
  epilogue<BM, BN, uint16_t>(acc, E, M, a.Cout, m0, c0, wm, wn, a.r, a.s, false, a.out);
}

inline bool big_tiles(int M, int C) {
  return (long)((M + 127) / 128) * ((C + 127) / 128) >= QLORA_BIG_TILE_MIN;
}

template <int BM, int BN, int D, int KIND>
void bf16_launch_r(Bf16Args a, const SkinnyJobs& sk, hipStream_t st) {
  a.tiles_x = (a.Cout + BN - 1) / BN;
  a.tiles = a.tiles_x * ((a.M + BM - 1) / BM);
  const int extra = sk.njobs > 0 ? sk.blocks() : 0;
  const dim3 grid(a.tiles + extra);
  const int r = sk.njobs > 0 ? sk.r : 1;
  if (r <= 4) bf16_kernel<BM, BN, D, KIND, 4><<<grid, 256, 0, st>>>(a, sk);
  else if (r <= 8) bf16_kernel<BM, BN, D, KIND, 8><<<grid, 256, 0, st>>>(a, sk);
  else if (r <= 16) bf16_kernel<BM, BN, D, KIND, 16><<<grid, 256, 0, st>>>(a, sk);
  else bf16_kernel<BM, BN, D, KIND, 32><<<grid, 256, 0, st>>>(a, sk);
}

template <int KIND>
void bf16_launch(const Bf16Args& a, const SkinnyJobs& sk, hipStream_t st) {
  if (big_tiles(a.M, a.Cout)) bf16_launch_r<128, 128, QLORA_D_BIG, KIND>(a, sk, st);
  else bf16_launch_r<64, 64, QLORA_D_SMALL, KIND>(a, sk, st);
}

}  // namespace

void launch_gemm_fwd_w4(int M, int N, int K, const uint16_t* x,
                        const uint8_t* packed, const _Float16* scales,
                        const float* t, const float* B, int r, float s,
                        uint16_t* y, hipStream_t st) {
  Bf16Args a{};
  a.M = M; a.Cout = N; a.Kc = K; a.Kw = K; a.Nw = N;
  a.g = x; a.codes = packed; a.scales = scales;
  a.P = t; a.Q = B; a.ldj = N; a.ldn = 1; a.r = r; a.s = s; a.out = y;
  SkinnyJobs none{};
  bf16_launch<kW4Fwd>(a, none, st);
}

void launch_gemm_dx_w4(int M, int K, int N, const uint16_t* dy,
                       const uint8_t* packed, const _Float16* scales,
                       const float* u, const float* A, int r, float s,
                       uint16_t* dx, const SkinnyJobs* sk, hipStream_t st) {
  Bf16Args a{};
  a.M = M; a.Cout = K; a.Kc = N; a.Kw = K; a.Nw = N;
  a.g = dy; a.codes = packed; a.scales = scales;
  a.P = u; a.Q = A; a.ldj = 1; a.ldn = r; a.r = r; a.s = s; a.out = dx;
  SkinnyJobs none{};
  bf16_launch<kW4T>(a, sk != nullptr ? *sk : none, st);
}

}  // namespace qlora
