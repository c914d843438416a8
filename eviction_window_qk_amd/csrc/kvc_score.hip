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
//               each lane one row and 16 keys, so the sum l of 2^(x-ref),
//               x = <q,k>*scale*log2(e), against a lazily kept reference ref
//               stays lane-local; the two lane halves merge once at the end.
//               Output: the row normaliser b = ref + log2(l) (log2 domain).
//               When a launch has too few heads to fill the chip, each head's
//               keys are split into ranges whose partial normalisers
//               k_rowmerge combines (b = log2 sum_s 2^b_s).
//   k_colsum    keys stationary: each wave keeps 64 keys in registers (the B
//               operand) and the workgroup streams the query rows through
//               double-buffered LDS.  The accumulator gives each lane one key
//               and 16 rows, so p = 2^(x - b) summed down the rows is
//               lane-local; the halves merge at the end (per query head for
//               the MAX aggregation).
//   k_colsum_resident
//               the same column sums with the whole window (queries and
//               normalisers) resident in LDS, each wave walking chunks of
//               keys without barriers: four waves for windows of at most four
//               32-row blocks, twelve (one workgroup per CU) for up to sixteen.
//   k_fill      positions seen by fewer than W queries take the maximum over
//               the fully observed ones.
//
// Per score element the VALU work is one FMA, one exp2 and one add (pass 1
// keeps a lazy reference maximum instead of a running one, so it needs no max
// per element); the exp2 is the costliest of them, and on gfx950 the
// vector ALU port, not the matrix core, bounds both passes.  Each wave issues
// the MFMAs of one 32x32 block and then its softmax arithmetic; three waves
// per SIMD (at most 168 VGPRs) let one wave's MFMAs run under another wave's
// VALU work.  Every (32-row, 32-key) block is classified against the causal
// limits of its rows: blocks no row sees are skipped (MFMAs included), blocks
// every row sees fully take the unmasked update, only the diagonal ones pay
// for the mask.  No atomics: every sum has a fixed order, so u is bitwise
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
// [16s + 8h, 16s + 8h + 8).  Any bijection of the head dimension gives the
// same dot product as long as both operands use it; this one puts the two
// lanes of a row on adjacent 16-byte pieces, so one load instruction of a
// register operand touches 32 cache lines rather than 64 (32 bytes each).
// In LDS (rows padded by one 16-byte piece) the pieces of eight consecutive
// rows still fall in distinct banks.  Accumulator element r of a 32x32 tile
// is at (row 8(r/4) + 4h + (r%4), column j).
template <int D>
__device__ __forceinline__ void load_rows_op(const u32x4* __restrict__ base, int row, int h,
                                             u32x4 (&op)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) op[s] = base[size_t(row) * (D / 8) + 2 * s + h];
}

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Completes the loads of a register-resident MFMA operand here, before the
// main loop.  Without it the compiler waits for them at their first use
// inside the loop on every iteration, and since the vector-memory counter
// retires in order, those waits also wait for the next tile's prefetch.
template <int N>
__device__ __forceinline__ void operand_ready(const u32x4 (&op)[N]) {
#pragma unroll
  for (int s = 0; s < N; ++s) asm volatile("" ::"v"(op[s]));
}

// ---------------------------------------------------------------------------
// pass 1: row statistics
// ---------------------------------------------------------------------------
constexpr int kRsWaves = 4;
constexpr int kRsRowBlocks = 2;                         // 32-row blocks per wave
constexpr int kRsRows = kRsWaves * kRsRowBlocks * 32;   // rows per workgroup (256)
constexpr int kRsTile = 64;                             // keys per LDS tile (two 32-key blocks)
constexpr int kRsThreads = 64 * kRsWaves;

// Sum of 2^(acc*c - m*c) over this lane's 16 dot products, -m*c given as nmc.
__device__ __forceinline__ float exp_sum16(const f32x16& acc, float c, float nmc) {
  float s0 = fast_exp2(__builtin_fmaf(acc[0], c, nmc));
  float s1 = fast_exp2(__builtin_fmaf(acc[1], c, nmc));
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    s0 += fast_exp2(__builtin_fmaf(acc[r], c, nmc));
    s1 += fast_exp2(__builtin_fmaf(acc[r + 1], c, nmc));
  }
  return s0 + s1;
}

// Running sum l of 2^(x*c - ref) over one row (this lane's) with 16 new raw
// dot products x, the reference held as nmc = -ref (log2 units).  The
// reference is not the running maximum: any value works for l as long as no
// term overflows, so the block is summed against the current reference (one
// FMA, one exp2 and one add per element) and the reference is raised only
// when a lane's block sum passes 2^32 (a score 28 log2 units above it): then
// the whole wave takes the block maximum as its new reference and rescales l.
// nmc starts at 2^64, so the first visible block always takes that path;
// masked entries are -inf and add exp2(-inf) = 0.  l stays below 2^18 keys x
// 2^32 per key.  The row normaliser is b = ref + log2(l).
template <bool MASK>
__device__ __forceinline__ void row_update(f32x16 acc, float c, int t0, int h, int lim,
                                           float& nmc, float& l) {
  if (MASK) {
    const int d = lim - t0 - 4 * h;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) > d) acc[r] = -INFINITY;
  }
  const float s = exp_sum16(acc, c, nmc);
  if (__builtin_expect(__any(!(s <= 0x1p32f)), 0)) {
    float mx = fmaxf(acc[0], acc[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, acc[r]), acc[r + 1]);
    const float nb = fminf(nmc, -mx * c);  // -max(ref, block maximum)
    l = __builtin_fmaf(l, fast_exp2(nb - nmc), exp_sum16(acc, c, nb));
    nmc = nb;
  } else {
    l += s;
  }
}

template <int D>
struct RsCtx {
  u32x4 qop[kRsRowBlocks][D / 16];
  float nmc[kRsRowBlocks], l[kRsRowBlocks];  // -reference (log2 units), running sum
  int lim[kRsRowBlocks];
  int lo[kRsRowBlocks], hi[kRsRowBlocks];  // wave-uniform min/max of lim per row block
};

template <int D>
__device__ __forceinline__ void load_frags(const u32x4* __restrict__ buf, int blk, int j, int h,
                                           u32x4 (&f)[D / 16]) {
  constexpr int kStride = D / 8 + 1;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = buf[(blk * 32 + j) * kStride + 2 * s + h];
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return __builtin_amdgcn_readfirstlane(x);
}

template <int D>
__device__ __forceinline__ void rs_update(RsCtx<D>& cx, int rb, const f32x16& acc, int t0,
                                          float c, int h) {
  if (t0 + 31 <= cx.lo[rb])
    row_update<false>(acc, c, t0, h, cx.lim[rb], cx.nmc[rb], cx.l[rb]);
  else
    row_update<true>(acc, c, t0, h, cx.lim[rb], cx.nmc[rb], cx.l[rb]);
}

// One 32-key block: fragments from LDS, MFMAs for the row blocks that see
// any of its keys, then the online update.  Row blocks that see none of the
// keys are skipped (their update would leave m and l unchanged).
template <int D>
__device__ __forceinline__ void rs_block(RsCtx<D>& cx, const u32x4* __restrict__ buf, int blk,
                                         int t0, float c, int j, int h) {
  const bool a0 = t0 <= cx.hi[0], a1 = t0 <= cx.hi[1];
  if (!a0 && !a1) return;
  u32x4 f[D / 16];
  load_frags<D>(buf, blk, j, h, f);
  if (a0 && a1) {
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      acc0 = mfma32(f[s], cx.qop[0][s], acc0);
      acc1 = mfma32(f[s], cx.qop[1][s], acc1);
    }
    rs_update<D>(cx, 0, acc0, t0, c, h);
    rs_update<D>(cx, 1, acc1, t0, c, h);
  } else {
    const int rb = a0 ? 0 : 1;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc = mfma32(f[s], a0 ? cx.qop[0][s] : cx.qop[1][s], acc);
    rs_update<D>(cx, rb, acc, t0, c, h);
  }
}

// NW waves per workgroup: 4 (256 rows); 2 (128 rows) when a head has at most
// 128 query rows, so that no wave idles and more workgroups -- and K tile
// loads -- share a CU (16K-token global event with W*G = 128: 2.03 -> 1.94 ms
// for the score stage).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 2 ? 2 : 3))) void k_rowstats(Derived P, const u32x4* __restrict__ q,
                                                            const u32x4* __restrict__ k,
                                                            float* __restrict__ rowb) {
  // rowb: [NH][R] normalisers, or with P.rs_split > 1 the partial ones
  // [NH][R][rs_split] of key range s = [s*span, min(T, (s+1)*span)).
  constexpr int kPerRow = D / 8;        // u32x4 per row
  constexpr int kStride = kPerRow + 1;  // LDS row stride (one pad piece)
  constexpr int kThreads = 64 * NW;
  constexpr int kRows = NW * kRsRowBlocks * 32;
  constexpr int kLoads = kRsTile * kPerRow / kThreads;
  __shared__ u32x4 ks[2][kRsTile * kStride];

  const int groups = (P.R + kRows - 1) / kRows;
  const int S = P.rs_split;
  const unsigned lb = xcd_logical_block();
  const int n = lb / (groups * S), grp = lb % groups, split = (lb / groups) % S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const Span sp = head_span(P, n);  // real tokens of a left-padded head
  const int T = sp.T, W = P.W, R = P.R;
  const float c = P.c_log2;

  RsCtx<D> cx;
  const int row0 = grp * kRows + wave * (kRsRowBlocks * 32);
  const bool wave_active = row0 < R;  // uniform per wave
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) {
    const int r = row0 + rb * 32 + j;
    const int rc = r < R ? r : R - 1;  // padding rows duplicate a real row, never written
    cx.lim[rb] = T - W + rc % W;
    cx.lo[rb] = wave_min(cx.lim[rb]);
    cx.hi[rb] = wave_max(cx.lim[rb]);
    load_rows_op<D>(q + size_t(n) * R * kPerRow, rc, h, cx.qop[rb]);
    operand_ready(cx.qop[rb]);
    cx.nmc[rb] = 0x1p64f;
    cx.l[rb] = 0.0f;
  }

  // This workgroup's key range: whole tiles, so no tile straddles two ranges.
  // The head splits by its own length (ranges past its count are empty).
  const int S_head = min(score_pass1_splits(R, T), S);  // never above the launch's (T <= P.T)
  const int span = ((T + S_head - 1) / S_head + kRsTile - 1) / kRsTile * kRsTile;
  const int t_lo = split * span;
  const int t_hi = t_lo + span < T ? t_lo + span : T;
  const u32x4* kn = k + (size_t(n) * P.TS + sp.off) * kPerRow;
  const int n_tiles = t_hi > t_lo ? (t_hi - t_lo + kRsTile - 1) / kRsTile : 0;
  // A tile is kRsTile whole key rows, one contiguous run of kRsTile*kPerRow
  // pieces: thread x loads pieces x, x + kThreads, ...  (a uniform tile
  // pointer plus one lane offset).  Only a tile running past T clamps its
  // rows (those keys are masked; the clamp keeps the loads in bounds).
  auto fetch = [&](int kt, u32x4 (&pre)[kLoads]) {
    const int t0 = t_lo + kt * kRsTile;
    const u32x4* tile = kn + size_t(t0) * kPerRow;
    if (t0 + kRsTile <= T) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) pre[i] = tile[threadIdx.x + i * kThreads];
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int e = threadIdx.x + i * kThreads;
        const int row = t0 + e / kPerRow < T ? e / kPerRow : T - 1 - t0;
        pre[i] = tile[row * kPerRow + e % kPerRow];
      }
    }
  };
  auto stash = [&](int buf, const u32x4 (&pre)[kLoads]) {
    u32x4* dst = ks[buf] + (threadIdx.x / kPerRow) * kStride + threadIdx.x % kPerRow;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dst[i * (kThreads / kPerRow) * kStride] = pre[i];
  };

  u32x4 pre[kLoads];
  if (n_tiles > 0) {
    fetch(0, pre);
    stash(0, pre);
    if (n_tiles > 1) fetch(1, pre);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const u32x4* buf = ks[kt & 1];
    if (wave_active) {
      rs_block<D>(cx, buf, 0, t_lo + kt * kRsTile, c, j, h);
      rs_block<D>(cx, buf, 1, t_lo + kt * kRsTile + 32, c, j, h);
    }
    if (kt + 1 < n_tiles) {
      stash((kt + 1) & 1, pre);
      if (kt + 2 < n_tiles) fetch(kt + 2, pre);
    }
    __syncthreads();
  }
  if (!wave_active) return;

  // Merge the two lane halves (same row, different keys) onto the larger
  // reference and write b = ref + log2(l).  Key 0 is visible to every row, so
  // the first key range always has a sum; a half (or a range) that saw no key
  // has l = 0 and nmc = 2^64, and a range with no key gets b = -inf.
#pragma unroll
  for (int rb = 0; rb < kRsRowBlocks; ++rb) {
    const float no = __shfl_xor(cx.nmc[rb], 32);
    const float lo = __shfl_xor(cx.l[rb], 32);
    const float nm = fminf(cx.nmc[rb], no);
    const float ll = cx.l[rb] * fast_exp2(nm - cx.nmc[rb]) + lo * fast_exp2(nm - no);
    const int r = row0 + rb * 32 + j;
    if (h == 0 && r < R) rowb[(size_t(n) * R + r) * S + split] = __log2f(ll) - nm;
  }
}

// Row normaliser from the partial ones of the key ranges: b = M +
// log2(sum_s 2^(b_s - M)), M = max_s b_s (finite: the first range holds key 0,
// which every row sees; a range with no visible key has b_s = -inf and adds
// 2^-inf = 0).  A row's partials are contiguous, so its loads go out together.
__global__ __launch_bounds__(256) void k_rowmerge(Derived P, const float* __restrict__ part,
                                                  float* __restrict__ rowb) {
  const int S = P.rs_split;
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= size_t(P.NH) * P.R) return;
  const float* pn = part + i * S;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < S; ++s) M = fmaxf(M, pn[s]);
  float sum = 0.0f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) sum += fast_exp2(pn[s] - M);
  rowb[i] = M + __log2f(sum);
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

// Column-sum contribution of one 32-row block to one 32-key block (this
// lane's key), normalisers b[] of the block's rows already in registers.
template <bool MASK>
__device__ __forceinline__ void col_update1(const f32x16& a, const float (&b)[16], float c, int lim0,
                                            int key, int h, float& cs) {
  float s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = __builtin_fmaf(a[r], c, -b[r]);
    if (MASK) x = key > lim0 + acc_row(r, h) ? -INFINITY : x;
    const float p = fast_exp2(x);
    if (r == 0) s0 = p;
    else if (r == 1) s1 = p;
    else if (r & 1) s1 += p;
    else s0 += p;
  }
  cs += s0 + s1;
}

// PRIO: the wave runs its softmax arithmetic at raised issue priority
// (s_setprio), so that on a SIMD shared by waves walking keys without
// barriers the one in its VALU phase issues first while the others' MFMAs
// run (128K-token event, twelve-wave resident pass: score stage -1.5 to -2.3 %,
// same bits; no gain, or a loss within noise, for the kernels that meet at a
// barrier after every query batch).
template <int D, bool PRIO = false>
__device__ __forceinline__ void cs_block(CsCtx<D>& cx, const u32x4* __restrict__ buf, int bi,
                                         const float* __restrict__ bblk, int lim_lo, float c,
                                         int kbase, int j, int h) {
  // lim of the block's rows runs over [lim_lo, lim_lo + 31]; keys of block kb
  // are kbase + 32 kb + [0, 32).
  const bool dead0 = kbase > lim_lo + 31, dead1 = kbase + 32 > lim_lo + 31;
  if (dead0) return;  // dead0 implies dead1
  const bool vis0 = kbase + 31 <= lim_lo, vis1 = kbase + 63 <= lim_lo;
  u32x4 f[D / 16];
  load_frags<D>(buf, bi, j, h, f);
  float b[16];
  auto load_b = [&]() {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 bb = *reinterpret_cast<const f32x4*>(&bblk[8 * i4 + 4 * h]);
      b[4 * i4 + 0] = bb[0];
      b[4 * i4 + 1] = bb[1];
      b[4 * i4 + 2] = bb[2];
      b[4 * i4 + 3] = bb[3];
    }
  };
  if (!dead1) {
    f32x16 a0 = f32x16{}, a1 = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      a0 = mfma32(f[s], cx.kop[0][s], a0);
      a1 = mfma32(f[s], cx.kop[1][s], a1);
    }
    load_b();
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    if (vis0) col_update1<false>(a0, b, c, lim_lo, cx.key0, h, cx.cs0);
    else col_update1<true>(a0, b, c, lim_lo, cx.key0, h, cx.cs0);
    if (vis1) col_update1<false>(a1, b, c, lim_lo, cx.key0 + 32, h, cx.cs1);
    else col_update1<true>(a1, b, c, lim_lo, cx.key0 + 32, h, cx.cs1);
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  } else {
    f32x16 a0 = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) a0 = mfma32(f[s], cx.kop[0][s], a0);
    load_b();
    if (vis0) col_update1<false>(a0, b, c, lim_lo, cx.key0, h, cx.cs0);
    else col_update1<true>(a0, b, c, lim_lo, cx.key0, h, cx.cs0);
  }
}

template <int D>
__device__ void cs_run(CsCtx<D>& cx, u32x4 (*qs)[kCsBatch * 32 * (D / 8 + 1)],
                       const float* __restrict__ bsh, const u32x4* __restrict__ qn, int n_blocks,
                       int n_rb, float c, int T, int W, int kbase, int j, int h) {
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
  for (int bt = 0; bt < n_batches; ++bt) {
    const u32x4* buf = qs[bt & 1];
#pragma unroll
    for (int bi = 0; bi < kCsBatch; ++bi) {
      const int blk = bt * kCsBatch + bi;
      if (blk < n_blocks)
        cs_block<D>(cx, buf, bi, bsh + blk * 32, T - W + (blk % n_rb) * 32, c, kbase, j, h);
    }
    if (bt + 1 < n_batches) {
      stash((bt + 1) & 1, pre);
      if (bt + 2 < n_batches) fetch(bt + 2, pre);
    }
    __syncthreads();
  }
}

template <int D, bool SUM>
__global__ __launch_bounds__(kCsThreads, SUM ? 3 : 2) void k_colsum(Derived P, const u32x4* __restrict__ q,
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
  const Span sp = head_span(P, n);  // real tokens of a left-padded head
  const int T = sp.T, W = P.W, R = P.R, G = P.G;
  if (chunk * kCsKeys >= T) return;  // whole workgroup: no real key in this chunk
  const float c = P.c_log2;
  const int key_base = chunk * kCsKeys + wave * kScoreKeysPerWave;

  const int n_rb = (W + 31) / 32;
  const int n_blocks = G * n_rb;
  for (int i = threadIdx.x; i < n_blocks * 32; i += kCsThreads) {
    const int g = i / (n_rb * 32), w = i % (n_rb * 32);
    bsh[i] = w < W ? rowb[size_t(n) * R + g * W + w] : INFINITY;  // +inf: p = 0
  }

  CsCtx<D> cx;
  cx.key0 = key_base + j;
  const u32x4* kn = k + (size_t(n) * P.TS + sp.off) * kPerRow;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int t = key_base + kb * 32 + j;
    t = t < T ? t : T - 1;  // keys past T are never written
    load_rows_op<D>(kn, t, h, cx.kop[kb]);
    operand_ready(cx.kop[kb]);
  }
  const u32x4* qn = q + size_t(n) * R * kPerRow;

  if (SUM) {
    cx.cs0 = cx.cs1 = 0.0f;
    cs_run<D>(cx, qs, bsh, qn, n_blocks, n_rb, c, T, W, key_base, j, h);
    cx.cs0 += __shfl_xor(cx.cs0, 32);
    cx.cs1 += __shfl_xor(cx.cs1, 32);
  } else {
    float tot0 = -INFINITY, tot1 = -INFINITY;
    for (int g = 0; g < G; ++g) {
      cx.cs0 = cx.cs1 = 0.0f;
      __syncthreads();  // previous head's LDS use done
      cs_run<D>(cx, qs, bsh + g * n_rb * 32, qn + size_t(g) * W * kPerRow, n_rb, n_rb, c, T, W,
                key_base, j, h);
      tot0 = fmaxf(tot0, cx.cs0 + __shfl_xor(cx.cs0, 32));
      tot1 = fmaxf(tot1, cx.cs1 + __shfl_xor(cx.cs1, 32));
    }
    cx.cs0 = tot0;
    cx.cs1 = tot1;
  }
  if (h == 0) {
    float* un = u + size_t(n) * P.T + sp.off;
    if (key_base + j < T) un[key_base + j] = cx.cs0;
    if (key_base + 32 + j < T) un[key_base + 32 + j] = cx.cs1;
  }
}

// Pass 2 for heads with at most kResBlocks 32-row blocks (W*G <= 128 after
// padding each query head's window to 32 rows), SUM aggregation, on launches
// with chunks to spare: the whole window (queries and row normalisers) stays
// in LDS, so a workgroup walks cpw consecutive chunks of 64*NW keys of one
// head with no barrier between them instead of re-streaming the queries for
// each chunk (16K-token global event: score stage 1.87 -> 1.76 ms).  The row
// blocks are visited in the same order as in k_colsum, so the sums are
// identical.  Two shapes: four waves and at most four padded 32-row blocks
// (W*G <= 128), several workgroups per CU; and twelve waves and at most
// sixteen blocks (W*G <= 512: 139 KB of queries), one workgroup per CU that
// walks a whole head -- long caches with a few hundred query rows per head,
// whose workgroups would otherwise spend much of their short lives starting
// up (staging the normalisers, loading the key operands, filling the query
// pipeline).
constexpr int kResBlocks = 4;
constexpr int kWideWaves = 12, kWideBlocks = 16;

template <int D, int NW, int NB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void k_colsum_resident(
    Derived P, const u32x4* __restrict__ q, const u32x4* __restrict__ k,
    const float* __restrict__ rowb, float* __restrict__ u, int cpw) {
  constexpr int kPerRow = D / 8;
  constexpr int kStride = kPerRow + 1;
  constexpr int kThreads = 64 * NW;
  constexpr int kChunk = NW * kScoreKeysPerWave;  // keys per chunk
  __shared__ u32x4 qs[NB * 32 * kStride];
  __shared__ __align__(16) float bsh[NB * 32];

  const int chunks = (P.T + kChunk - 1) / kChunk;
  const int groups = (chunks + cpw - 1) / cpw;
  const unsigned lb = xcd_logical_block();
  const int n = lb / groups, grp = lb % groups;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const Span sp = head_span(P, n);  // real tokens of a left-padded head
  const int T = sp.T, W = P.W, R = P.R, G = P.G;
  const int c0 = grp * cpw;
  if (c0 * kChunk >= T) return;  // whole workgroup: no real key in its chunks
  const float c = P.c_log2;
  const int n_rb = (W + 31) / 32;
  const int n_blocks = G * n_rb;  // <= NB (host)

  for (int i = threadIdx.x; i < n_blocks * 32; i += kThreads) {
    const int g = i / (n_rb * 32), w = i % (n_rb * 32);
    bsh[i] = w < W ? rowb[size_t(n) * R + g * W + w] : INFINITY;  // +inf: p = 0
  }
  const u32x4* qn = q + size_t(n) * R * kPerRow;
  for (int e = threadIdx.x; e < n_blocks * 32 * kPerRow; e += kThreads) {
    const int blk = e / (32 * kPerRow);
    const int g = blk / n_rb;
    int w = (blk % n_rb) * 32 + (e / kPerRow) % 32;
    w = w < W ? w : W - 1;  // padding slots carry b = +inf, so their rows add 0
    qs[(e / kPerRow) * kStride + e % kPerRow] = qn[size_t(g * W + w) * kPerRow + e % kPerRow];
  }
  __syncthreads();

  const u32x4* kn = k + (size_t(n) * P.TS + sp.off) * kPerRow;
  float* un = u + size_t(n) * P.T + sp.off;
  for (int ch = c0; ch < c0 + cpw && ch * kChunk < T; ++ch) {
    const int key_base = ch * kChunk + wave * kScoreKeysPerWave;
    CsCtx<D> cx;
    cx.key0 = key_base + j;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int t = key_base + kb * 32 + j;
      t = t < T ? t : T - 1;  // keys past T are never written
      load_rows_op<D>(kn, t, h, cx.kop[kb]);
    }
    cx.cs0 = cx.cs1 = 0.0f;
    for (int blk = 0; blk < n_blocks; ++blk)
      cs_block<D, (NW > kCsWaves)>(cx, qs, blk, bsh + blk * 32, T - W + (blk % n_rb) * 32, c,
                                   key_base, j, h);
    cx.cs0 += __shfl_xor(cx.cs0, 32);
    cx.cs1 += __shfl_xor(cx.cs1, 32);
    if (h == 0) {
      if (key_base + j < T) un[key_base + j] = cx.cs0;
      if (key_base + 32 + j < T) un[key_base + 32 + j] = cx.cs1;
    }
  }
}

// Positions T-W+1 .. T-1 are seen by fewer than W queries: replace them by
// the maximum usage over the fully observed positions 0 .. T-W (positions of
// the head's real tokens).  The padding of a left-padded head gets 0 here,
// also when W = 1 and there is nothing to fill.  One
// workgroup per head; each thread keeps kLoads loads in flight per sweep
// (clamped indices, no branches), so a long cache is not read one load at a
// time (128K-token event: score stage 9.99 -> 9.69 ms).
template <int NT>
__global__ __launch_bounds__(NT) void k_fill(Derived P, float* __restrict__ u) {
  constexpr int kLoads = 8;
  __shared__ float red[NT / 64];
  const int n = blockIdx.x;
  const Span sp = head_span(P, n);
  const int T = sp.T, W = P.W;
  for (int t = threadIdx.x; t < sp.off; t += NT) u[size_t(n) * P.T + t] = 0.0f;  // padding
  if (W <= 1) return;  // every position fully observed (uniform per launch)
  float* un = u + size_t(n) * P.T + sp.off;
  const int last = T - W;  // fully observed: 0 .. last
  float m = -INFINITY;
  for (int t0 = threadIdx.x; t0 <= last; t0 += NT * kLoads) {
    float x[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int t = t0 + i * NT;
      x[i] = un[t <= last ? t : last];  // a clamped copy repeats a value already in the max
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) m = fmaxf(m, x[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
  for (int t = last + 1 + threadIdx.x; t < T; t += NT) un[t] = m;
}

}  // namespace

hipError_t launch_score(const Derived& d, const void* q, const void* k, float* u, float* stats,
                        float* stats_part, hipStream_t s) {
  const u32x4* qv = static_cast<const u32x4*>(q);
  const u32x4* kv = static_cast<const u32x4*>(k);
  const bool small_r = d.R <= 2 * kRsRowBlocks * 32;  // two-wave pass-1 workgroups
  const int rs_rows = small_r ? 2 * kRsRowBlocks * 32 : kRsRows;
  const unsigned g_rs =
      unsigned((d.R + rs_rows - 1) / rs_rows) * unsigned(d.NH) * unsigned(d.rs_split);
  float* rs_out = d.rs_split > 1 ? stats_part : stats;
  const int cs_chunks = (d.T + kCsKeys - 1) / kCsKeys;
  const unsigned g_cs = unsigned(cs_chunks) * unsigned(d.NH);
  const int nb_pad = d.G * ((d.W + 31) / 32);  // padded 32-row blocks per head
  // Small windows (at most kResBlocks padded 32-row blocks) on launches with
  // chunks to spare: queries resident in LDS.
  const bool resident = nb_pad <= kResBlocks && int64_t(cs_chunks) * d.NH >= 8192;
  const int cpw = 8;  // measured: 2, 4, 8, 16, 32 -> 8 fastest
  const unsigned g_res = unsigned((cs_chunks + cpw - 1) / cpw) * unsigned(d.NH);
  // Up to kWideBlocks blocks: one twelve-wave workgroup per CU, each walking
  // its share of a head (at least four 768-key chunks, else the streamed
  // kernel).
  const int w_chunks = (d.T + kWideWaves * kScoreKeysPerWave - 1) / (kWideWaves * kScoreKeysPerWave);
  const int w_groups = d.NH >= 256 ? 1 : (256 + d.NH - 1) / d.NH;  // workgroups per head
  const int w_cpw = (w_chunks + w_groups - 1) / w_groups;
  const bool wide = !resident && d.head_agg == KVC_AGG_SUM && nb_pad <= kWideBlocks && w_cpw >= 4;
  const unsigned g_wide = unsigned((w_chunks + w_cpw - 1) / w_cpw) * unsigned(d.NH);
  if (d.D == 128) {
    if (small_r) k_rowstats<128, 2><<<g_rs, 128, 0, s>>>(d, qv, kv, rs_out);
    else k_rowstats<128, kRsWaves><<<g_rs, kRsThreads, 0, s>>>(d, qv, kv, rs_out);
  } else {
    if (small_r) k_rowstats<64, 2><<<g_rs, 128, 0, s>>>(d, qv, kv, rs_out);
    else k_rowstats<64, kRsWaves><<<g_rs, kRsThreads, 0, s>>>(d, qv, kv, rs_out);
  }
  if (d.rs_split > 1) {
    const size_t rows = size_t(d.NH) * d.R;
    k_rowmerge<<<unsigned((rows + 255) / 256), 256, 0, s>>>(d, stats_part, stats);
  }
  if (d.D == 128) {
    if (wide)
      k_colsum_resident<128, kWideWaves, kWideBlocks><<<g_wide, 64 * kWideWaves, 0, s>>>(d, qv, kv, stats, u, w_cpw);
    else if (d.head_agg == KVC_AGG_SUM)
      resident ? k_colsum_resident<128, kCsWaves, kResBlocks><<<g_res, kCsThreads, 0, s>>>(d, qv, kv, stats, u, cpw)
               : k_colsum<128, true><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
    else
      k_colsum<128, false><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
  } else {
    if (wide)
      k_colsum_resident<64, kWideWaves, kWideBlocks><<<g_wide, 64 * kWideWaves, 0, s>>>(d, qv, kv, stats, u, w_cpw);
    else if (d.head_agg == KVC_AGG_SUM)
      resident ? k_colsum_resident<64, kCsWaves, kResBlocks><<<g_res, kCsThreads, 0, s>>>(d, qv, kv, stats, u, cpw)
               : k_colsum<64, true><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
    else
      k_colsum<64, false><<<g_cs, kCsThreads, 0, s>>>(d, qv, kv, stats, u);
  }
  if (d.W > 1 || d.vlen) {  // the fill, and the zeros on a ragged head's padding
    if (d.T >= 4096)
      k_fill<1024><<<d.NH, 1024, 0, s>>>(d, u);
    else
      k_fill<256><<<d.NH, 256, 0, s>>>(d, u);
  }
  return hipGetLastError();
}

}  // namespace kvc
