// Step 1: window score on gfx950.
//
// u[n][t] = AGG_g sum_w softmax_t(scale * <q[n][g][w], k[n][t]>), causal: the
// query at window slot w sits at position T-W+w and sees keys t <= T-W+w.
// Sources: AMS notes, key design 1 (usage of the most recent W queries,
// partly observed suffix filled with the window maximum); SkipKV notes §4.1
// (softmax(QK^T/sqrt(d)) over an observation window, GQA map g(i) =
// floor(i/n)); RefreshKV notes, A6 (max over the query heads of a group).
//
// A column sum of softmax probabilities needs every row's max and sum first,
// and the score matrix (W*G rows x T keys per head) is far too large to keep,
// so the score runs in two passes over the keys, each a bf16 MFMA
// (32x32x16, fp32 accumulate) stream:
//
//   k_rowstats  rows stationary: each wave keeps 64 query rows in registers
//               (the B operand) and the workgroup streams every key of the
//               head through double-buffered LDS tiles.  The accumulator gives
//               each lane one row and 16 keys, so the running max m and sum l
//               of 2^(x-m), x = <q,k>*scale*log2(e), stay lane-local; the two
//               lane halves merge once at the end.  Output: the row
//               normaliser b = m + log2(l) (log2 domain).
//   k_colsum    keys stationary: each wave keeps 64 keys in registers (the B
//               operand) and the workgroup streams the query rows through
//               double-buffered LDS.  The accumulator gives each lane one key
//               and 16 rows, so p = 2^(x - b) summed down the rows is
//               lane-local; the halves merge at the end (per query head for
//               the MAX aggregation).
//   k_fill      positions seen by fewer than W queries take the maximum over
//               the fully observed ones.
//
// Per score element the VALU work is one FMA, one exp2 and one add (plus half
// a max in pass 1).  Both passes are software-pipelined: the MFMAs of one
// 32-wide block are issued interleaved with the softmax arithmetic of the
// previous block, so the matrix cores and the vector ALUs of a SIMD work at
// the same time even within one wave.  The causal mask costs nothing on
// blocks every row sees fully; only blocks reaching past T-W take the masked
// loop.  No atomics: every sum has a fixed order, so u is bitwise
// reproducible.  Blocks are renumbered so that the workgroups of one head
// share an XCD and its L2.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;

// sched_group_barrier masks
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hardware dispatches block b to XCD b % 8.  Renumber so that each XCD runs a
// contiguous range of logical blocks.
__device__ __forceinline__ unsigned xcd_logical_block() {
  const unsigned nb = gridDim.x, b = blockIdx.x;
  const unsigned q = nb / kXcds, r = nb % kXcds;
  const unsigned x = b % kXcds, slot = b / kXcds;
  return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

// Operand layout.  Lane (j = lane & 31, h = lane >> 5) supplies row/column j
// of a 32-wide MFMA operand and, for k-step s, head-dim elements
// [h*D/2 + 8s, h*D/2 + 8s + 8).  Any bijection of the head dimension gives the
// same dot product as long as both operands use it; this one makes a lane's
// share of a row one contiguous run.  Accumulator element r of a 32x32 tile
// is at (row 8(r/4) + 4h + (r%4), column j).
template <int D>
__device__ __forceinline__ void load_rows_op(const u32x4* __restrict__ base, int row, int h,
                                             u32x4 (&op)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) op[s] = base[size_t(row) * (D / 8) + h * (D / 16) + s];
}

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// pass 1: row statistics
// ---------------------------------------------------------------------------
constexpr int kRsWaves = 4;
constexpr int kRsRowBlocks = 2;                         // 32-row blocks per wave
constexpr int kRsRows = kRsWaves * kRsRowBlocks * 32;   // rows per workgroup (256)
constexpr int kRsTile = 64;                             // keys per LDS tile (two 32-key blocks)
constexpr int kRsThreads = 64 * kRsWaves;

// Online max/sum update of one row (this lane's) with 16 new raw dot products.
template <bool MASK>
__device__ __forceinline__ void row_update(f32x16 acc, float c, int t0, int h, int lim, float& m,
                                           float& l) {
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t0 + acc_row(r, h) > lim) acc[r] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(acc[0], acc[1]), acc[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, acc[r]), acc[r + 1]);
  mx = fmaxf(mx, acc[15]);
  const float mn = fmaxf(m, mx);
  // mn is -inf only while every key seen so far is masked (then l stays 0).
  const float nb = mn == -INFINITY ? 0.0f : -mn * c;
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    s0 += fast_exp2(__builtin_fmaf(acc[r], c, nb));
    s1 += fast_exp2(__builtin_fmaf(acc[r + 1], c, nb));
  }
  const float scale = m == -INFINITY ? 0.0f : fast_exp2(__builtin_fmaf(m, c, nb));
  l = __builtin_fmaf(l, scale, s0 + s1);
  m = mn;
}

template <int D>
struct RsCtx {
  u32x4 qop[kRsRowBlocks][D / 16];
  float m[kRsRowBlocks], l[kRsRowBlocks];
  int lim[kRsRowBlocks];
};

// A-operand fragments (one 32-key block) of k-steps 0..D/16-1 from LDS.
template <int D>
__device__ __forceinline__ void load_frags(const u32x4* __restrict__ buf, int blk, int j, int h,
                                           u32x4 (&f)[D / 16]) {
  constexpr int kStride = D / 8 + 1;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = buf[(blk * 32 + j) * kStride + h * (D / 16) + s];
}

// MFMAs of one 32-key block (fragments already in registers) into acc,
// interleaved with the softmax of the previous block (pacc, keys from pt0).
template <int D, bool MASK>
__device__ __forceinline__ void rs_step(RsCtx<D>& cx, const u32x4 (&fa)[D / 16],
                                        f32x16 (&acc)[kRsRowBlocks],
                                        const f32x16 (&pacc)[kRsRowBlocks], int pt0, float c,
                                        int h) {
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) acc[rb] = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
#pragma unroll
    for (int rb = 0; rb < kRsRowBlocks; ++rb) acc[rb] = mfma32(fa[s], cx.qop[rb][s], acc[rb]);
  }
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb)
    row_update<MASK>(pacc[rb], c, pt0, h, cx.lim[rb], cx.m[rb], cx.l[rb]);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kRsRowBlocks, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 15, 0);
  }
}

// One 64-key LDS tile: both blocks' fragments are read up front, then
// MFMA(block 0) || softmax(previous block), MFMA(block 1) || softmax(block 0).
template <int D, bool MASK>
__device__ __forceinline__ void rs_tile(RsCtx<D>& cx, const u32x4* __restrict__ buf,
                                        f32x16 (&accA)[kRsRowBlocks],
                                        f32x16 (&accB)[kRsRowBlocks], int t0, float c, int j,
                                        int h) {
  u32x4 f0[D / 16], f1[D / 16];
  load_frags<D>(buf, 0, j, h, f0);
  load_frags<D>(buf, 1, j, h, f1);
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (D / 16), 0);
  rs_step<D, MASK>(cx, f0, accA, accB, t0 - 32, c, h);
  rs_step<D, MASK>(cx, f1, accB, accA, t0, c, h);
}

template <int D>
__global__ __launch_bounds__(kRsThreads, 2) void k_rowstats(Derived P, const u32x4* __restrict__ q,
                                                            const u32x4* __restrict__ k,
                                                            float* __restrict__ rowb) {
  constexpr int kPerRow = D / 8;        // u32x4 per row
  constexpr int kStride = kPerRow + 1;  // LDS row stride (one pad piece)
  constexpr int kLoads = kRsTile * kPerRow / kRsThreads;
  __shared__ u32x4 ks[2][kRsTile * kStride];

  const int groups = (P.R + kRsRows - 1) / kRsRows;
  const unsigned lb = xcd_logical_block();
  const int n = lb / groups, grp = lb % groups;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int T = P.T, W = P.W, R = P.R;
  const float c = P.c_log2;

  RsCtx<D> cx;
  const int row0 = grp * kRsRows + wave * (kRsRowBlocks * 32);
  const bool wave_active = row0 < R;  // uniform per wave
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) {
    const int r = row0 + rb * 32 + j;
    const int rc = r < R ? r : R - 1;  // padding rows duplicate a real row, never written
    cx.lim[rb] = T - W + rc % W;
    load_rows_op<D>(q + size_t(n) * R * kPerRow, rc, h, cx.qop[rb]);
    cx.m[rb] = -INFINITY;
    cx.l[rb] = 0.0f;
  }

  const u32x4* kn = k + size_t(n) * P.TS * kPerRow;
  const int n_tiles = (T + kRsTile - 1) / kRsTile;
  // Tiles whose every key is seen by every row (t <= T-W) need no mask.
  const int n_full = (T - W + 1) / kRsTile;
  auto fetch = [&](int kt, u32x4 (&pre)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kRsThreads;
      int t = kt * kRsTile + e / kPerRow;
      t = t < T ? t : T - 1;  // rows past T are masked; keep the load in bounds
      pre[i] = kn[size_t(t) * kPerRow + e % kPerRow];
    }
  };
  auto stash = [&](int buf, const u32x4 (&pre)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kRsThreads;
      ks[buf][(e / kPerRow) * kStride + e % kPerRow] = pre[i];
    }
  };

  u32x4 pre[kLoads];
  fetch(0, pre);
  stash(0, pre);
  if (n_tiles > 1) fetch(1, pre);
  __syncthreads();

  // accB starts as a pending block of -inf: its update leaves (m, l) unchanged.
  f32x16 accA[kRsRowBlocks], accB[kRsRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) {
    accA[rb] = f32x16{};
#pragma unroll
    for (int r = 0; r < 16; ++r) accB[rb][r] = -INFINITY;
  }
  int kt = 0;
  // Unmasked tiles: two 32-key blocks each, pipelined across blocks and tiles.
  for (; kt < n_full; ++kt) {
    const u32x4* buf = ks[kt & 1];
    if (wave_active) rs_tile<D, false>(cx, buf, accA, accB, kt * kRsTile, c, j, h);
    // Unconditional (past the end: a clamped reload into the idle buffer) so
    // the loop body stays one basic block for the MFMA/VALU interleave.
    stash((kt + 1) & 1, pre);
    fetch(kt + 2, pre);
    __syncthreads();
  }
  // Tiles that reach past T-W: same pipeline with the causal mask.
  for (; kt < n_tiles; ++kt) {
    const u32x4* buf = ks[kt & 1];
    if (wave_active) rs_tile<D, true>(cx, buf, accA, accB, kt * kRsTile, c, j, h);
    // Unconditional (past the end: a clamped reload into the idle buffer) so
    // the loop body stays one basic block for the MFMA/VALU interleave.
    stash((kt + 1) & 1, pre);
    fetch(kt + 2, pre);
    __syncthreads();
  }
  if (!wave_active) return;
  // Last block still pending in accB (keys from (n_tiles-1)*64 + 32).
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb)
    row_update<true>(accB[rb], c, (n_tiles - 1) * kRsTile + 32, h, cx.lim[rb], cx.m[rb], cx.l[rb]);

  // Merge the two lane halves (same row, different keys) and write b.
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) {
    const float mo = __shfl_xor(cx.m[rb], 32);
    const float lo = __shfl_xor(cx.l[rb], 32);
    const float mm = fmaxf(cx.m[rb], mo);
    float ll = 0.0f;
    if (cx.m[rb] != -INFINITY) ll += cx.l[rb] * fast_exp2((cx.m[rb] - mm) * c);
    if (mo != -INFINITY) ll += lo * fast_exp2((mo - mm) * c);
    const int r = row0 + rb * 32 + j;
    if (h == 0 && r < R) rowb[size_t(n) * R + r] = mm * c + __log2f(ll);
  }
}

// ---------------------------------------------------------------------------
// pass 2: column sums
// ---------------------------------------------------------------------------
constexpr int kCsWaves = 4;
constexpr int kCsKeys = kCsWaves * kScoreKeysPerWave;  // keys per workgroup (256)
constexpr int kCsBatch = 2;                            // 32-row blocks per LDS buffer
constexpr int kCsThreads = 64 * kCsWaves;

template <int D>
struct CsCtx {
  u32x4 kop[2][D / 16];
  float cs0, cs1;
  int key0;  // this lane's first key (second is key0 + 32)
};

// Column sums of one 32-row block's probabilities (accumulators a0/a1, row
// normalisers bblk[0..32) in LDS).
template <bool MASK>
__device__ __forceinline__ void col_update(const f32x16& a0, const f32x16& a1,
                                           const float* __restrict__ bblk, float c, int T, int W,
                                           int wbase, int key0, int h, float& cs0, float& cs1) {
  float b[16];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const f32x4 bb = *reinterpret_cast<const f32x4*>(&bblk[8 * i4 + 4 * h]);
    b[4 * i4 + 0] = bb[0];
    b[4 * i4 + 1] = bb[1];
    b[4 * i4 + 2] = bb[2];
    b[4 * i4 + 3] = bb[3];
  }
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x0 = __builtin_fmaf(a0[r], c, -b[r]);
    float x1 = __builtin_fmaf(a1[r], c, -b[r]);
    if (MASK) {
      const int lim = T - W + wbase + acc_row(r, h);
      x0 = key0 > lim ? -INFINITY : x0;
      x1 = key0 + 32 > lim ? -INFINITY : x1;
    }
    s0 += fast_exp2(x0);
    s1 += fast_exp2(x1);
  }
  cs0 += s0;
  cs1 += s1;
}

template <int D, bool MASK>
__device__ __forceinline__ void cs_step(CsCtx<D>& cx, const u32x4 (&fa)[D / 16], f32x16& a0,
                                        f32x16& a1, const f32x16& p0, const f32x16& p1,
                                        const float* __restrict__ pb, int pwbase, float c, int T,
                                        int W, int h) {
  a0 = f32x16{};
  a1 = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    a0 = mfma32(fa[s], cx.kop[0][s], a0);
    a1 = mfma32(fa[s], cx.kop[1][s], a1);
  }
  col_update<MASK>(p0, p1, pb, c, T, W, pwbase, cx.key0, h, cx.cs0, cx.cs1);
  // The four normaliser reads first, then two MFMAs and ~12 VALU per k-step.
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 12, 0);
  }
}

template <int D, bool MASK>
__device__ void cs_run(CsCtx<D>& cx, u32x4 (*qs)[kCsBatch * 32 * (D / 8 + 1)],
                       const float* __restrict__ bsh, const u32x4* __restrict__ qn, int n_blocks,
                       int n_rb, float c, int T, int W, int j, int h) {
  constexpr int kPerRow = D / 8;
  constexpr int kStride = kPerRow + 1;
  constexpr int kLoads = kCsBatch * 32 * kPerRow / kCsThreads;
  auto fetch = [&](int batch, u32x4 (&pre)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kCsThreads;
      int blk = batch * kCsBatch + e / (32 * kPerRow);
      blk = blk < n_blocks ? blk : n_blocks - 1;
      const int g = blk / n_rb;
      int w = (blk % n_rb) * 32 + (e / kPerRow) % 32;
      w = w < W ? w : W - 1;  // padding slots carry b = +inf, so their rows add 0
      pre[i] = qn[size_t(g * W + w) * kPerRow + e % kPerRow];
    }
  };
  auto stash = [&](int buf, const u32x4 (&pre)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kCsThreads;
      qs[buf][(e / kPerRow) * kStride + e % kPerRow] = pre[i];
    }
  };
  const int n_batches = (n_blocks + kCsBatch - 1) / kCsBatch;
  u32x4 pre[kLoads];
  fetch(0, pre);
  __syncthreads();  // b table ready
  stash(0, pre);
  if (n_batches > 1) fetch(1, pre);
  __syncthreads();

  // (a0B, a1B) start as a pending block of -inf: its column sums add +0.0.
  f32x16 a0A, a1A, a0B, a1B;
  a0A = a1A = f32x16{};
#pragma unroll
  for (int r = 0; r < 16; ++r) a0B[r] = a1B[r] = -INFINITY;
  const int full_batches = n_blocks / kCsBatch;
  int bt = 0;
  for (; bt < full_batches; ++bt) {
    const u32x4* buf = qs[bt & 1];
    const int blk = bt * kCsBatch;
    u32x4 f0[D / 16], f1[D / 16];
    load_frags<D>(buf, 0, j, h, f0);
    load_frags<D>(buf, 1, j, h, f1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (D / 16), 0);
    cs_step<D, MASK>(cx, f0, a0A, a1A, a0B, a1B, bsh + (blk > 0 ? blk - 1 : 0) * 32,
                     ((blk - 1 + n_blocks) % n_rb) * 32, c, T, W, h);
    cs_step<D, MASK>(cx, f1, a0B, a1B, a0A, a1A, bsh + blk * 32, (blk % n_rb) * 32, c, T, W, h);
    stash((bt + 1) & 1, pre);  // unconditional: see k_rowstats
    fetch(bt + 2, pre);
    __syncthreads();
  }
  int last = full_batches * kCsBatch - 1;  // block pending in (a0B, a1B)
  if (bt < n_batches) {                    // odd block count: one more block
    const u32x4* buf = qs[bt & 1];
    const int blk = bt * kCsBatch;
    u32x4 f0[D / 16];
    load_frags<D>(buf, 0, j, h, f0);
    cs_step<D, MASK>(cx, f0, a0A, a1A, a0B, a1B, bsh + (blk > 0 ? blk - 1 : 0) * 32,
                     ((blk - 1 + n_blocks) % n_rb) * 32, c, T, W, h);
    col_update<MASK>(a0A, a1A, bsh + blk * 32, c, T, W, (blk % n_rb) * 32, cx.key0, h, cx.cs0,
                     cx.cs1);
  } else if (last >= 0) {
    col_update<MASK>(a0B, a1B, bsh + last * 32, c, T, W, (last % n_rb) * 32, cx.key0, h, cx.cs0,
                     cx.cs1);
  }
}

template <int D, bool SUM>
__global__ __launch_bounds__(kCsThreads, 2) void k_colsum(Derived P, const u32x4* __restrict__ q,
                                                          const u32x4* __restrict__ k,
                                                          const float* __restrict__ rowb,
                                                          float* __restrict__ u) {
  constexpr int kPerRow = D / 8;
  constexpr int kStride = kPerRow + 1;
  __shared__ u32x4 qs[2][kCsBatch * 32 * kStride];
  __shared__ __align__(16) float bsh[kMaxRows];

  const int chunks = (P.T + kCsKeys - 1) / kCsKeys;
  const unsigned lb = xcd_logical_block();
  const int n = lb / chunks, chunk = lb % chunks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int T = P.T, W = P.W, R = P.R, G = P.G;
  const float c = P.c_log2;
  const int key_base = chunk * kCsKeys + wave * kScoreKeysPerWave;

  // Row blocks enumerate (g, rb) so that no block straddles two query heads:
  // block i covers window slots [rb*32, min(W, rb*32+32)) of head g.
  const int n_rb = (W + 31) / 32;
  const int n_blocks = G * n_rb;
  for (int i = threadIdx.x; i < n_blocks * 32; i += kCsThreads) {
    const int g = i / (n_rb * 32), w = i % (n_rb * 32);
    bsh[i] = w < W ? rowb[size_t(n) * R + g * W + w] : INFINITY;  // +inf: p = 0
  }

  CsCtx<D> cx;
  cx.key0 = key_base + j;
  const u32x4* kn = k + size_t(n) * P.TS * kPerRow;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int t = key_base + kb * 32 + j;
    t = t < T ? t : T - 1;  // keys past T are never written
    load_rows_op<D>(kn, t, h, cx.kop[kb]);
  }
  const u32x4* qn = q + size_t(n) * R * kPerRow;

  if (SUM) {
    cx.cs0 = cx.cs1 = 0.0f;
    // Masking is needed only when some key of this wave lies past T-W (or T).
    const bool mask = key_base + kScoreKeysPerWave - 1 > T - W;
    if (mask) cs_run<D, true>(cx, qs, bsh, qn, n_blocks, n_rb, c, T, W, j, h);
    else cs_run<D, false>(cx, qs, bsh, qn, n_blocks, n_rb, c, T, W, j, h);
    cx.cs0 += __shfl_xor(cx.cs0, 32);
    cx.cs1 += __shfl_xor(cx.cs1, 32);
  } else {
    // MAX over the query heads: one head's blocks at a time.
    float tot0 = -INFINITY, tot1 = -INFINITY;
    for (int g = 0; g < G; ++g) {
      cx.cs0 = cx.cs1 = 0.0f;
      __syncthreads();  // previous head's LDS use done
      cs_run<D, true>(cx, qs, bsh + g * n_rb * 32, qn + size_t(g) * W * kPerRow, n_rb, n_rb, c,
                      T, W, j, h);
      tot0 = fmaxf(tot0, cx.cs0 + __shfl_xor(cx.cs0, 32));
      tot1 = fmaxf(tot1, cx.cs1 + __shfl_xor(cx.cs1, 32));
    }
    cx.cs0 = tot0;
    cx.cs1 = tot1;
  }
  if (h == 0) {
    if (key_base + j < T) u[size_t(n) * T + key_base + j] = cx.cs0;
    if (key_base + 32 + j < T) u[size_t(n) * T + key_base + 32 + j] = cx.cs1;
  }
}

// Positions T-W+1 .. T-1 are seen by fewer than W queries: replace them by
// the maximum usage over the fully observed positions 0 .. T-W.
__global__ __launch_bounds__(256) void k_fill(Derived P, float* __restrict__ u) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int T = P.T, W = P.W;
  float* un = u + size_t(n) * T;
  float m = -INFINITY;
  for (int t = threadIdx.x; t <= T - W; t += 256) m = fmaxf(m, un[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int t = T - W + 1 + threadIdx.x; t < T; t += 256) un[t] = m;
}

}  // namespace

hipError_t launch_score(const Derived& d, const void* q, const void* k, float* u, float* stats,
                        hipStream_t s) {
  const u32x4* qv = static_cast<const u32x4*>(q);
  const u32x4* kv = static_cast<const u32x4*>(k);
  const unsigned g_rs = unsigned((d.R + kRsRows - 1) / kRsRows) * unsigned(d.NH);
  const unsigned g_cs = unsigned((d.T + kCsKeys - 1) / kCsKeys) * unsigned(d.NH);
  if (d.D == 128) {
    k_rowstats<128><<<g_rs, kRsThreads, 0, s>>>(d, qv, kv, stats);
    if (d.head_agg == KVC_AGG_SUM)
      k_colsum<128, true><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
    else
      k_colsum<128, false><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
  } else {
    k_rowstats<64><<<g_rs, kRsThreads, 0, s>>>(d, qv, kv, stats);
    if (d.head_agg == KVC_AGG_SUM)
      k_colsum<64, true><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
    else
      k_colsum<64, false><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
  }
  if (d.W > 1) k_fill<<<d.NH, 256, 0, s>>>(d, u);
  return hipGetLastError();
}

}  // namespace kvc
