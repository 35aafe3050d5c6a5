// Forward product of the frozen int8 layer on v_mfma_i32_16x16x64_i8.
//
//   acc[m, n] = sum_k xq[m, k] q[n, k]                       (exact int32)
//   y[m, n]   = fma(s, sum_j t[m, j] B[j, n], float(acc) * (sx[m] * sw[n]))
//
// ("Parameter-efficient fine-tuning of GPT-2 with LoRA", "LoRA equation": the
// adapter branch is added to the frozen layer's output; "Create LoRA layer":
// scaled by alpha / rank; "Introduce QLoRA-like technique", "Highlights": the
// frozen kernel is int8 with one scale per output channel.)
//
// Outlier-compensated weights (keras-llm-light README, "Simplified
// Int8Variable quantization"; the format is described in outlier.hpp) use the
// same product with the codes v - 128 of one affine grid for the whole
// weight, so the epilogue becomes
//
//   y[m, n] = sx[m] (c acc[m, n] + b' as[m] + corr[m, n]) + s (t B)[m, n]
//
// with c the grid step, b' = b + 128 c the value of code 0, as[m] the row sum
// of xq (from the row pass), and corr[m, n] = sum over the outliers (k, n) of
// xq[m, k] d (d = value - grid value). The corrections are taken while the
// activation codes of their k are in LDS: wave w owns the 16-column cell
// [16 w, 16 w + 16) of the 64-wide tile over all its rows, one row per lane
// (two for 128-row tiles), and holds the cell's outliers (k_e, n_e, d_e) in
// the stage's 128-wide k block (read one stage ahead, one entry per lane).
// Each entry is broadcast with readlane; every lane gathers xq[m, k_e] from
// the stage's tile and adds xq[m, k_e] d_e into its register for column
// n_e, addressed by the wave-uniform n_e (s_set_gpr_idx). The first eight
// entries of a stage are straight-line code placed ahead of the stage's
// products, so their latency hides behind the matrix work; the rest (rare)
// follow in batches of four. After the loop the 16 columns of every
// row go through LDS to the waves that own the accumulators and are folded
// in: acc' = c acc + corr.
//
// Both operands are K-contiguous int8 rows, so every tile moves straight from
// global memory into the LDS stage ring (ring.hpp) with no conversion. A block
// of 4 waves (2 x 2) owns a BM x BN output tile; a wave owns (BM/2) x (BN/2)
// as 16 x 16 MFMA blocks and reads its operands from the swizzled 128-byte
// rows of the current stage. Tile and depth are picked per shape: 64 x 64 with
// three stages when the grid is about one wave of blocks (latency-bound, so
// depth pays), 128 x 128 or 128 x 64 with two stages for large grids (LDS per
// block then allows several blocks per compute unit). Few tiles over a long
// k axis split it (up to 8 ways, 4 for the affine form): each block leaves
// its exact int32 sums (and the affine form its float corrections) in the
// workspace, and a second launch adds them and applies the epilogue.
#include "launch.hpp"
#include "outlier.hpp"
#include "ring.hpp"

namespace qlora {

namespace {

constexpr int kCUs = 256;

struct I8Args {
  int M, N, K;
  const int8_t* xq;      // [M, K]
  const int8_t* codes;   // [N, K]
  const float* sx;       // [M]
  const float* sw;       // [N]
  const float* t;        // [M, r]
  const float* B;        // [r, N], or [heads, r, hd]
  int hd;                // head width (N: one head)
  int r;
  float s;
  void* y;               // [M, N] float32 or bfloat16
  int32_t* acc_out;      // [M, N] (test hook) or nullptr
  // outlier-compensated weights
  const W8OHeader* w8o;  // grid step and bias
  const float* asum;     // [M] row sums of xq
  const int* fptr;       // forward cells, outlier.hpp
  const u32x2* fent;
  int ng;                // 16-column cells per 128-wide k block
  int tiles_x;
  // split contraction (128 x 128 tiles): the exact int32 partial sums in the
  // accumulator layout, the split count and stages per split
  int32_t* pacc;         // [splits, tiles, 4 waves, FM FN fragments, 64 lanes] int4
  float* pcorr;          // affine: [splits, tiles, 4 waves, CR rows, 16 columns, 64 lanes]
  int splits, nks;
};

template <int BM, int BN, int S, int R, typename OutT, bool ACC_OUT, bool AFF, bool SPLIT = false>
__global__ __launch_bounds__(256) void fwd_i8_kernel(I8Args a) {
  static_assert(!SPLIT || !ACC_OUT, "split: no integer test output");
  constexpr int BK = 128, ASZ = BM * BK, STG = (BM + BN) * BK;
  constexpr int AI = BM / 32, BI = BN / 32, LPS = AI + BI;   // loads per wave per stage
  constexpr int FM = BM / 32, FN = BN / 32;
  static_assert(!AFF || (BK == kW8OFwdCellK && BN == 4 * kW8OFwdCellN),
                "a stage is one forward cell deep; a wave owns one cell's columns");
  // after the loop the ring holds the epilogue operands, then one output
  // staging strip per wave
  constexpr int EPB = (EpiOps<BM, BN, R, true, AFF>::kFloats * 4 + 15) / 16 * 16;
  static_assert(EPB + 4 * epi_strip_bytes<OutT, FN>() <= S * STG, "epilogue fits in the ring");
  __shared__ __attribute__((aligned(1024))) int8_t ring[S * STG];

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int wm = wid >> 1, wn = wid & 1;
  const int M = a.M, N = a.N, K = a.K;
  const int nk = (K + BK - 1) / BK;
  // SPLIT: blocks (split, tile), split-major, renumbered so that the blocks
  // the dispatcher deals to one XCD (every eighth) share one split's k range
  int bid = (int)blockIdx.x, split = 0;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  if constexpr (SPLIT) {
    const int nb = (int)gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    split = bid / tiles;
    bid -= split * tiles;
  }
  int mt, nt;
  if constexpr (SPLIT) {
    mt = bid / a.tiles_x;
    nt = bid % a.tiles_x;
  } else {
    xcd_tile(bid, (M + BM - 1) / BM, a.tiles_x, mt, nt);
  }
  const int m0 = mt * BM, n0 = nt * BN;
  // stages [kt0, kt1) of the contraction
  const int kt0 = SPLIT ? split * a.nks : 0;
  const int kt1 = SPLIT ? (kt0 + a.nks < nk ? kt0 + a.nks : nk) : nk;

  EpiOps<BM, BN, R, true, AFF> ep;
  if constexpr (!ACC_OUT && !SPLIT) ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, a.sx, AFF ? nullptr : a.sw);
  if constexpr (AFF && !SPLIT) ep.load_rows(M, m0, a.asum);

  // AFF: the wave's outlier cell, columns [16 wid, 16 wid + 16) of the tile;
  // entry range of stage kt: [fptr[kt ng + g], fptr[kt ng + g + 1]), empty
  // when the columns are past N
  constexpr int CR = BM / 64;                          // correction rows per lane
  const int g = n0 / kW8OFwdCellN + wid;
  const int gl = g < a.ng ? g : a.ng, gh = g + 1 < a.ng ? g + 1 : a.ng;
  CellRanges cr;
  // one entry per lane from p0 (the list has spare entries past its end)
  auto entries = [&](int p0) { return a.fent[p0 + lane]; };
  float corr[CR][kW8OFwdCellN];                      // [row lane + 64 r][column]
#pragma unroll
  for (int r = 0; r < CR; ++r)
#pragma unroll
    for (int c = 0; c < kW8OFwdCellN; ++c) corr[r][c] = 0.f;

  // Wave wid fills rows [wid * BM/4, (wid + 1) * BM/4) of A and the same
  // share of B; one instruction covers 8 rows (8 lanes of 16 bytes per row).
  // Every stage but a ragged last one loads from a wave-wide base (the
  // stage's first k) plus a fixed 32-bit lane offset; the ragged stage, and
  // every stage of the affine form (whose loop waits for loads by count and
  // must not branch here), compute each lane's address and zero page.
  uint32_t voA[AI], voB[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = wid * (BM / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gm = m0 + row;
    voA[i] = (uint32_t)((long)(gm < M ? gm : M - 1) * K + c * 16);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = wid * (BN / 4) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7), gn = n0 + row;
    voB[i] = (uint32_t)((long)(gn < N ? gn : N - 1) * K + c * 16);
  }
  auto issue = [&](int kt, int slot) {
    int8_t* base = ring + slot * STG;
    if (!AFF && (kt + 1) * BK <= K) {
      const int8_t* xb = a.xq + kt * BK;
      const int8_t* cb = a.codes + kt * BK;
#pragma unroll
      for (int i = 0; i < AI; ++i) lds_dma16(xb + voA[i], base + (wid * (BM / 4) + i * 8) * BK);
#pragma unroll
      for (int i = 0; i < BI; ++i) lds_dma16(cb + voB[i], base + ASZ + (wid * (BN / 4) + i * 8) * BK);
      return;
    }
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int rb = wid * (BM / 4) + i * 8, row = rb + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      const int gk = kt * BK + c * 16, gm = m0 + row;
      const int8_t* src = gk < K ? a.xq + (long)(gm < M ? gm : M - 1) * K + gk : zero_chunk(lane);
      lds_dma16(src, base + rb * BK);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int rb = wid * (BN / 4) + i * 8, row = rb + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      const int gk = kt * BK + c * 16, gn = n0 + row;
      const int8_t* src = gk < K ? a.codes + (long)(gn < N ? gn : N - 1) * K + gk : zero_chunk(lane);
      lds_dma16(src, base + ASZ + rb * BK);
    }
  };

  i32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  // AFF: entries of stage kt (cur) and the ranges of stages kt, kt + 1; the
  // ranges are read before the stage loads so that reading the first entries
  // waits for them alone
  int clo = 0, chi = 0;
  u32x2 cur = u32x2{0u, 0u};
  if constexpr (AFF) cr.init(a.fptr, a.ng, gl, gh, nk, kt0);
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (kt0 + st < kt1) issue(kt0 + st, st);
  if constexpr (AFF) {
    cr.get(kt0, clo, chi);
    cur = entries(clo);
    // (the first stage's entries, like its operands, have landed before the
    // loop starts; the loop then never waits for a load it did not count)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  int slot = 0;
  for (int kt = kt0; kt < kt1; ++kt) {
    wait_stages<LPS, 0, S - 2>(kt1 - 1 - kt);   // stage kt has landed (this wave)
    __builtin_amdgcn_s_barrier();               // ... for every wave; slot kt-1 is free
    // AFF: read ahead (before this iteration's loads enter the queue) the
    // entries of stage kt + 1
    u32x2 nxt = u32x2{0u, 0u};
    int nlo = 0, nhi = 0;
    if constexpr (AFF) {
      cr.get(kt + 1 < kt1 ? kt + 1 : kt, nlo, nhi);
      nxt = entries(nlo);
      // keep this load ahead of the stage loads: it is then waited for by
      // count when the next stage takes it over
      __builtin_amdgcn_sched_barrier(0);
    }
    // (outlier-compensated weights: past the last stage the loads read the
    // zero page into the free slot, so that every iteration queues the same
    // loads and a read-ahead register can be waited for by count)
    if (AFF || kt + S - 1 < kt1) issue(kt + S - 1, slot == 0 ? S - 1 : slot - 1);
    const int8_t* As = ring + slot * STG;
    const int8_t* Bs = As + ASZ;
    // AFF: the stage's first PEEL outliers as straight-line code ahead of the
    // products, so that their gathers and adds hide behind the matrix work;
    // entries past the stage's count add 0
    constexpr int PEEL = 8;
    const int c0 = n0 + 16 * wid;                    // the wave's first column
    if constexpr (AFF) {
      const int cnt = chi - clo;
      uint32_t kn[PEEL];
      float d[PEEL], xv[PEEL][CR];
#pragma unroll
      for (int u = 0; u < PEEL; ++u) {
        kn[u] = (uint32_t)__builtin_amdgcn_readlane((int)cur.x, u);
        d[u] = u < cnt ? __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)cur.y, u)) : 0.f;
        const int kl = (int)(kn[u] & 127);
#pragma unroll
        for (int r = 0; r < CR; ++r) xv[u][r] = (float)As[swz128(64 * r + lane, kl >> 4) + (kl & 15)];
      }
#pragma unroll
      for (int u = 0; u < PEEL; ++u) {
        const int c = ((int)(kn[u] >> 7) - c0) & (kW8OFwdCellN - 1);
#pragma unroll
        for (int r = 0; r < CR; ++r) corr[r][c] = __builtin_fmaf(xv[u][r], d[u], corr[r][c]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < BK / 64; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      i32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(As + swz128(wm * (BM / 2) + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(Bs + swz128(wn * (BN / 2) + j * 16 + (lane & 15), c));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (AFF) {
      // corr[m][n_e - 16 w] += xq[m, k_e] d_e over the stage's outliers of
      // this wave's cell, lane = row m (and m + 64)
      const int cnt = chi - clo;
      auto batch = [&](const u32x2 bat, int q0, int bc) {   // entries q0..bc of a batch
        for (int q = q0; q < bc; q += 4) {
          uint32_t kn[4];
          float d[4], xv[4][CR];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = q + u < 64 ? q + u : 63;
            kn[u] = (uint32_t)__builtin_amdgcn_readlane((int)bat.x, e);
            d[u] = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)bat.y, e));
            const int kl = (int)(kn[u] & 127);
#pragma unroll
            for (int r = 0; r < CR; ++r) xv[u][r] = (float)As[swz128(64 * r + lane, kl >> 4) + (kl & 15)];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (q + u < bc) {                          // uniform
              const int c = ((int)(kn[u] >> 7) - c0) & (kW8OFwdCellN - 1);
#pragma unroll
              for (int r = 0; r < CR; ++r) corr[r][c] = __builtin_fmaf(xv[u][r], d[u], corr[r][c]);
            }
          }
        }
      };
      batch(cur, PEEL, cnt < 64 ? cnt : 64);           // past the peeled ones
      for (int b0 = 64; b0 < cnt; b0 += 64)            // more than 64 in one stage
        batch(a.fent[clo + b0 + lane], 0, cnt - b0 < 64 ? cnt - b0 : 64);
      // the read-ahead entries were queued before this stage's operand loads:
      // all but those loads are done
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
      cur = nxt;
      clo = nlo;
      chi = nhi;
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  if constexpr (SPLIT) {
    // int4 unit ((split tiles + tile) 4 + wave) F + f) 64 + lane for
    // fragment f = i FN + j of F = FM FN: each store writes 1 KB of
    // consecutive bytes
    i32x4* P = reinterpret_cast<i32x4*>(a.pacc) +
               ((long)(split * tiles + bid) * 4 + wid) * (FM * FN * 64) + lane;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) P[(i * FN + j) * 64] = acc[i][j];
    if constexpr (AFF) {
      // the wave's corrections, float unit ((((split tiles + tile) 4 +
      // wave) CR + r) 16 + c) 64 + lane
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the zero-page stage loads past the range
      float* Q = a.pcorr + ((long)(split * tiles + bid) * 4 + wid) * (CR * 16 * 64) + lane;
#pragma unroll
      for (int r = 0; r < CR; ++r)
#pragma unroll
        for (int c = 0; c < kW8OFwdCellN; ++c) Q[(r * 16 + c) * 64] = corr[r][c];
    }
  } else if constexpr (ACC_OUT) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int m = m0 + wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
          const int n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
          if (m < M && n < N) a.acc_out[(long)m * N + n] = acc[i][j][ii];
        }
  } else {
    float* E = reinterpret_cast<float*>(ring);
    __syncthreads();                 // every wave is done with the ring
    if constexpr (AFF) {
      // corrections to the accumulators' owners through LDS ([BM][BN + 4]
      // floats), folded in with the grid step: accf = c acc + corr
      constexpr int CP = BN + 4;
#pragma unroll
      for (int r = 0; r < CR; ++r)
#pragma unroll
        for (int c = 0; c < kW8OFwdCellN; ++c)
          E[(64 * r + lane) * CP + 16 * wid + c] = corr[r][c];
      __syncthreads();
      const float cstep = a.w8o->scale;
      f32x4 accf[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int ml = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + ii;
            const int nl = wn * (BN / 2) + j * 16 + (lane & 15);
            accf[i][j][ii] = __builtin_fmaf(cstep, (float)acc[i][j][ii], E[ml * CP + nl]);
          }
      __syncthreads();
      ep.store(E, M, N, m0, n0, a.r);
      ep.store_rows(E, M, m0, a.w8o->bias_q);
      __syncthreads();
      epilogue_lowrank<BM, BN, R, true, true>(accf, E, M, N, m0, n0, wm * (BM / 2), wn * (BN / 2),
                                              a.s, reinterpret_cast<OutT*>(a.y),
                                              ring + EPB + wid * epi_strip_bytes<OutT, FN>());
    } else {
      ep.store(E, M, N, m0, n0, a.r);
      __syncthreads();
      epilogue_lowrank<BM, BN, R, true>(acc, E, M, N, m0, n0, wm * (BM / 2), wn * (BN / 2),
                                        a.s, reinterpret_cast<OutT*>(a.y),
                                        ring + EPB + wid * epi_strip_bytes<OutT, FN>());
    }
  }
}

// Second launch of the split int8 product, one 512-thread block per 128-row x
// 32-column quarter of a 128 x 128 tile: the int32 partial sums added (exact,
// so the result equals the one-pass product's bit for bit), then the scaled
// low-rank epilogue. Wave v takes rows [16 v, 16 v + 16): fragment row v % 4,
// fragment columns 2 (q % 2) + {0, 1} of the product kernel's wave
// 2 (v / 4) + q / 2 for quarter q; all of a lane's split loads are issued
// before the first add.
template <int R, int NSPL, typename OutT>
__global__ __launch_bounds__(512) void fwd_fixup_kernel(I8Args a) {
  constexpr int BM = 128, HN = 32, FN = 2;
  using Ep = EpiOps<BM, HN, R, true>;
  constexpr int EPB = (Ep::kFloats * 4 + 15) / 16 * 16;
  constexpr int STRIP = epi_strip_bytes<OutT, FN>();
  __shared__ __attribute__((aligned(1024))) int8_t lds[EPB + 8 * STRIP];
  float* E = reinterpret_cast<float*>(lds);

  const int tid = threadIdx.x, lane = tid & 63, v = wave_id();
  const int M = a.M, N = a.N, nsp = a.splits;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  const int tile = (int)blockIdx.x >> 2, q = (int)blockIdx.x & 3;
  const int m0 = (tile / a.tiles_x) * BM, n0 = (tile % a.tiles_x) * 128 + q * HN;

  const int w = 2 * (v >> 2) + (q >> 1), fi = v & 3;
  const i32x4* P = reinterpret_cast<const i32x4*>(a.pacc) + ((long)tile * 4 + w) * (16 * 64) +
                   (fi * 4 + 2 * (q & 1)) * 64 + lane;
  const long pstride = (long)tiles * 4 * 16 * 64;       // int4 units per split
  i32x4 pv[NSPL][FN];
#pragma unroll
  for (int sp = 0; sp < NSPL; ++sp)
#pragma unroll
    for (int j = 0; j < FN; ++j) pv[sp][j] = P[(sp < nsp ? sp : 0) * pstride + j * 64];

  Ep ep;
  if (tid < 256) ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, a.sx, a.sw);
  i32x4 acc[1][FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    acc[0][j] = pv[0][j];
#pragma unroll
    for (int sp = 1; sp < NSPL; ++sp)
      if (sp < nsp) acc[0][j] += pv[sp][j];
  }
  if (tid < 256) ep.store(E, M, N, m0, n0, a.r);
  __syncthreads();
  epilogue_lowrank<BM, HN, R, true>(acc, E, M, N, m0, n0, 16 * v, 0, a.s,
                                    reinterpret_cast<OutT*>(a.y), lds + EPB + v * STRIP);
}

// The same for outlier-compensated weights on 128 x 64 tiles, one 512-thread
// block per tile: the int32 partial sums added (exact), the corrections added
// in split order into LDS ([128][64 + 4] floats, from the product kernel's
// cell layout), then acc' = c acc + corr and the affine epilogue.
template <int R, int NSPL>
__global__ __launch_bounds__(512) void fwd_fixup_aff_kernel(I8Args a) {
  constexpr int BM = 128, BN = 64, FN = 4, CR = 2, CP = BN + 4;
  using Ep = EpiOps<BM, BN, R, true, true>;
  constexpr int EPB = (Ep::kFloats * 4 + 15) / 16 * 16;
  constexpr int CSZ = BM * CP * 4;
  constexpr int STRIP = epi_strip_bytes<uint16_t, FN>();
  __shared__ __attribute__((aligned(1024))) int8_t lds[CSZ + EPB + 8 * STRIP];
  float* C = reinterpret_cast<float*>(lds);
  float* E = reinterpret_cast<float*>(lds + CSZ);

  const int tid = threadIdx.x, lane = tid & 63, v = wave_id();
  const int M = a.M, N = a.N, nsp = a.splits;
  const int tiles = a.tiles_x * ((M + BM - 1) / BM);
  const int tile = (int)blockIdx.x;
  const int m0 = (tile / a.tiles_x) * BM, n0 = (tile % a.tiles_x) * BN;

  // wave v: rows [16 v, 16 v + 16) = fragment row v % 4 of the product
  // kernel's waves 2 (v / 4) + {0, 1} (each 2 fragments of 16 columns)
  const int fi = v & 3;
  i32x4 pv[NSPL][FN];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = 2 * (v >> 2) + h;
    const i32x4* P = reinterpret_cast<const i32x4*>(a.pacc) + ((long)tile * 4 + w) * (8 * 64) +
                     fi * 2 * 64 + lane;
    const long pstride = (long)tiles * 4 * 8 * 64;
#pragma unroll
    for (int sp = 0; sp < NSPL; ++sp)
#pragma unroll
      for (int j = 0; j < 2; ++j) pv[sp][2 * h + j] = P[(sp < nsp ? sp : 0) * pstride + j * 64];
  }
  // corrections: element e = ((w CR + r) 16 + c) 64 + lane of the tile's
  // cells -> row 64 r + lane, column 16 w + c
  constexpr int CE = 4 * CR * 16 * 64 / 512;             // per thread
  float cv[CE][NSPL];
#pragma unroll
  for (int q = 0; q < CE; ++q) {
    const int e = tid + 512 * q;
    const float* Qp = a.pcorr + (long)tile * (4 * CR * 16 * 64) + e;
    const long qstride = (long)tiles * 4 * CR * 16 * 64;
#pragma unroll
    for (int sp = 0; sp < NSPL; ++sp) cv[q][sp] = Qp[(sp < nsp ? sp : 0) * qstride];
  }
  Ep ep;
  if (tid < 256) {
    ep.load(M, N, m0, n0, a.r, a.t, a.B, a.hd, a.sx, nullptr);
    ep.load_rows(M, m0, a.asum);
  }
#pragma unroll
  for (int q = 0; q < CE; ++q) {
    const int e = tid + 512 * q;
    const int ln = e & 63, c = (e >> 6) & 15, r = (e >> 10) & (CR - 1), w = e >> 11;
    float sum = cv[q][0];
#pragma unroll
    for (int sp = 1; sp < NSPL; ++sp)
      if (sp < nsp) sum += cv[q][sp];
    C[(64 * r + ln) * CP + 16 * w + c] = sum;
  }
  i32x4 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    acc[j] = pv[0][j];
#pragma unroll
    for (int sp = 1; sp < NSPL; ++sp)
      if (sp < nsp) acc[j] += pv[sp][j];
  }
  if (tid < 256) {
    ep.store(E, M, N, m0, n0, a.r);
    ep.store_rows(E, M, m0, a.w8o->bias_q);
  }
  __syncthreads();
  const float cstep = a.w8o->scale;
  f32x4 accf[1][FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int ml = 16 * v + (lane >> 4) * 4 + ii, nl = j * 16 + (lane & 15);
      accf[0][j][ii] = __builtin_fmaf(cstep, (float)acc[j][ii], C[ml * CP + nl]);
    }
  epilogue_lowrank<BM, BN, R, true, true>(accf, E, M, N, m0, n0, 16 * v, 0, a.s,
                                          reinterpret_cast<uint16_t*>(a.y), lds + CSZ + EPB + v * STRIP);
}

constexpr int kMaxFwdSplits = 8;

constexpr int kMaxAffSplits = 4;    // the affine fixup holds every split's loads

// Split count and stages per split of the 128 x BN product: only for at
// most 128 tiles over a long contraction, doubling (up to maxsp) while the
// grid stays within two blocks per compute unit and each split keeps at
// least 16 stages of 128 k; a split product then goes on to 4 splits of at
// least 8 stages while the grid stays within one block per compute unit
// (measured: 10-14 % faster at K = 4096 on 64-512 rows; 8 splits of 8
// stages, or a grid of two blocks per compute unit, were 6-8 % slower).
void fwd_split_plan(int M, int N, int K, int BN, int maxsp, int* splits, int* nks) {
  const long tiles = (long)((M + 127) / 128) * ((N + BN - 1) / BN);
  const int nk = (K + 127) / 128;
  int sp = 1;
  if (tiles <= 128) {
    while (sp < maxsp && tiles * sp * 2 <= 2 * kCUs && nk / (sp * 2) >= 16) sp *= 2;
    while (sp > 1 && sp * 2 <= 4 && sp < maxsp && tiles * sp * 2 <= kCUs && nk / (sp * 2) >= 8) sp *= 2;
  }
  *nks = (nk + sp - 1) / sp;
  *splits = (nk + *nks - 1) / *nks;
}

template <typename OutT>
void launch_split(I8Args a, hipStream_t st) {
  constexpr int BM = 128, BN = 128, S = 2;
  a.tiles_x = (a.N + BN - 1) / BN;
  const int tiles = a.tiles_x * ((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles * a.splits)), fgrid((unsigned)(4 * tiles));
  if (a.r <= 4) fwd_i8_kernel<BM, BN, S, 4, OutT, false, false, true><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_i8_kernel<BM, BN, S, 8, OutT, false, false, true><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_i8_kernel<BM, BN, S, 16, OutT, false, false, true><<<grid, 256, 0, st>>>(a);
  else fwd_i8_kernel<BM, BN, S, 32, OutT, false, false, true><<<grid, 256, 0, st>>>(a);
  if (a.splits <= 4) {
    if (a.r <= 4) fwd_fixup_kernel<4, 4, OutT><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 8) fwd_fixup_kernel<8, 4, OutT><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 16) fwd_fixup_kernel<16, 4, OutT><<<fgrid, 512, 0, st>>>(a);
    else fwd_fixup_kernel<32, 4, OutT><<<fgrid, 512, 0, st>>>(a);
  } else {
    if (a.r <= 4) fwd_fixup_kernel<4, kMaxFwdSplits, OutT><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 8) fwd_fixup_kernel<8, kMaxFwdSplits, OutT><<<fgrid, 512, 0, st>>>(a);
    else if (a.r <= 16) fwd_fixup_kernel<16, kMaxFwdSplits, OutT><<<fgrid, 512, 0, st>>>(a);
    else fwd_fixup_kernel<32, kMaxFwdSplits, OutT><<<fgrid, 512, 0, st>>>(a);
  }
}

template <int BM, int BN, int S, typename OutT, bool ACC, bool AFF = false>
void launch_tiles(I8Args a, hipStream_t st) {
  a.tiles_x = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_x * ((a.M + BM - 1) / BM)));
  if (a.r <= 4) fwd_i8_kernel<BM, BN, S, 4, OutT, ACC, AFF><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 8) fwd_i8_kernel<BM, BN, S, 8, OutT, ACC, AFF><<<grid, 256, 0, st>>>(a);
  else if (a.r <= 16) fwd_i8_kernel<BM, BN, S, 16, OutT, ACC, AFF><<<grid, 256, 0, st>>>(a);
  else fwd_i8_kernel<BM, BN, S, 32, OutT, ACC, AFF><<<grid, 256, 0, st>>>(a);
}

template <typename OutT, bool ACC>
void launch_shape(I8Args a, hipStream_t st) {
  if constexpr (!ACC) {
    if (a.pacc != nullptr) {
      fwd_split_plan(a.M, a.N, a.K, 128, kMaxFwdSplits, &a.splits, &a.nks);
      if (a.splits > 1) {
        launch_split<OutT>(a, st);
        return;
      }
    }
  }
  const long t64 = (long)((a.M + 63) / 64) * ((a.N + 63) / 64);
  const long t128 = (long)((a.M + 127) / 128) * ((a.N + 127) / 128);
  const long t192 = (long)((a.M + 127) / 128) * ((a.N + 191) / 192);
  // rounds of two blocks per compute unit, weighted by the work per block:
  // 128 x 192 tiles (1.5 times a 128 x 128 tile's) where N is a multiple of
  // 192 and they take fewer weighted rounds (GPT-2's 2304- and 3072-wide
  // products: 576 and 768 blocks of 128 x 128 in two rounds, 384 and 512 of
  // 128 x 192 in one)
  const long rounds128 = (t128 + 2 * kCUs - 1) / (2 * kCUs), rounds192 = (t192 + 2 * kCUs - 1) / (2 * kCUs);
  if (t64 <= 2 * kCUs) launch_tiles<64, 64, 3, OutT, ACC>(a, st);
  else if (t128 >= 2 * kCUs && a.N % 192 == 0 && 3 * rounds192 < 2 * rounds128)
    launch_tiles<128, 192, 2, OutT, ACC>(a, st);
  else if (t128 >= 2 * kCUs) launch_tiles<128, 128, 2, OutT, ACC>(a, st);
  else launch_tiles<128, 64, 2, OutT, ACC>(a, st);
}

}  // namespace

size_t fwd_split_ints(int M, int N, int K, bool affine) {
  const int bn = affine ? 64 : 128;
  int sp, nks;
  fwd_split_plan(M, N, K, bn, affine ? kMaxAffSplits : kMaxFwdSplits, &sp, &nks);
  if (sp == 1) return 0;
  const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((N + bn - 1) / bn);
  return (size_t)sp * tiles * 128 * (size_t)bn;
}

void launch_gemm_fwd_w8(int dtype, int M, int N, int K, const int8_t* xq,
                        const int8_t* codes, const float* sx, const float* sw,
                        const float* t, const float* B, int hd, int r, float s,
                        void* y, int32_t* acc_out, int32_t* pacc, hipStream_t st) {
  I8Args a{};
  a.M = M; a.N = N; a.K = K; a.xq = xq; a.codes = codes; a.sx = sx; a.sw = sw;
  a.t = t; a.B = B; a.hd = hd; a.r = r; a.s = s; a.y = y; a.acc_out = acc_out;
  a.pacc = pacc;
  if (acc_out != nullptr) launch_shape<float, true>(a, st);
  else if (dtype == 0) launch_shape<float, false>(a, st);
  else launch_shape<uint16_t, false>(a, st);
}

void launch_gemm_fwd_w8o(int M, int N, int K, const int8_t* xq, const int8_t* codes,
                         const float* sx, const float* asum, const void* side,
                         const float* t, const float* B, int hd, int r, float s,
                         uint16_t* y, int32_t* pacc, float* pcorr, hipStream_t st) {
  const W8OLayout L = w8o_layout(K, N);
  const char* sb = static_cast<const char*>(side);
  I8Args a{};
  a.M = M; a.N = N; a.K = K; a.xq = xq; a.codes = codes; a.sx = sx; a.sw = nullptr;
  a.t = t; a.B = B; a.hd = hd; a.r = r; a.s = s; a.y = y; a.acc_out = nullptr;
  a.w8o = reinterpret_cast<const W8OHeader*>(sb);
  a.asum = asum;
  a.fptr = reinterpret_cast<const int*>(sb + L.fptr);
  a.fent = reinterpret_cast<const u32x2*>(sb + L.fent);
  a.ng = L.ng;
  a.pacc = pacc;
  a.pcorr = pcorr;
  if (pacc != nullptr && pcorr != nullptr) {
    fwd_split_plan(M, N, K, 64, kMaxAffSplits, &a.splits, &a.nks);
    if (a.splits > 1) {
      // 128 x 64 tiles over the split contraction, then the fixup per tile
      constexpr int BM = 128, BN = 64, S = 2;
      a.tiles_x = (N + BN - 1) / BN;
      const int tiles = a.tiles_x * ((M + BM - 1) / BM);
      const dim3 grid((unsigned)(tiles * a.splits)), fgrid((unsigned)tiles);
      if (r <= 4) fwd_i8_kernel<BM, BN, S, 4, uint16_t, false, true, true><<<grid, 256, 0, st>>>(a);
      else if (r <= 8) fwd_i8_kernel<BM, BN, S, 8, uint16_t, false, true, true><<<grid, 256, 0, st>>>(a);
      else if (r <= 16) fwd_i8_kernel<BM, BN, S, 16, uint16_t, false, true, true><<<grid, 256, 0, st>>>(a);
      else fwd_i8_kernel<BM, BN, S, 32, uint16_t, false, true, true><<<grid, 256, 0, st>>>(a);
      if (r <= 4) fwd_fixup_aff_kernel<4, kMaxAffSplits><<<fgrid, 512, 0, st>>>(a);
      else if (r <= 8) fwd_fixup_aff_kernel<8, kMaxAffSplits><<<fgrid, 512, 0, st>>>(a);
      else if (r <= 16) fwd_fixup_aff_kernel<16, kMaxAffSplits><<<fgrid, 512, 0, st>>>(a);
      else fwd_fixup_aff_kernel<32, kMaxAffSplits><<<fgrid, 512, 0, st>>>(a);
      return;
    }
  }
  // the correction accumulators take registers: 64 x 64 (three stages) or
  // 128 x 64 (two)
  const long t64 = (long)((M + 63) / 64) * ((N + 63) / 64);
  if (t64 <= 2 * kCUs) launch_tiles<64, 64, 3, uint16_t, false, true>(a, st);
  else launch_tiles<128, 64, 2, uint16_t, false, true>(a, st);
}

}  // namespace qlora
