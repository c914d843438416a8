// Steps 2 and 3 on gfx950: mass, EMA credit, prefix, cuts, split/merge,
// must-keep and quotas.  One workgroup per head-event (1024 threads for long
// caches, 256 otherwise).
//
// Sources: AMS notes, key design 1 (m_i = (max(u_i,0)+eps)/sum; c <-
// lambda*c + (1-lambda)*m; m_used = normalize(beta*m + (1-beta)*normalize(c));
// small-kernel 1-D average pooling), key design 2 (C(t) = sum_{u<=t} m_u,
// b_k = min{t : C(t) >= k*Delta}, long segments split into near-equal pieces,
// short neighbours merged, masses recounted), key design 3 (must-keep sinks
// and recent suffix first, shorten the suffix when short of budget,
// q_i^min = min(q_min, L_i), T_rem split by segment mass with rounding, clip
// and redistribute).
//
// Every integer decision is bit-identical to a sequential evaluation:
//  - reductions (totals, prefix, segment masses) are unsigned 64-bit
//    fixed-point sums, exact in any order;
//  - each floating-point expression is evaluated one IEEE operation at a time
//    in the written order (contraction is off for this file; division is
//    correctly rounded), non-negative values are truncated toward zero;
//  - usage is held as trunc(ubar * 2^40) + ceil(eps * 2^40), credit and mixed
//    mass as Q44.
#pragma clang fp contract(off)

#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

// Long caches run with 1024 threads per workgroup (one head per CU is then
// enough to keep the loads in flight); short ones with 256.
constexpr int kMaxWaves = 16;
constexpr int kMaxHalo = 31;       // pool_kernel <= 63

// Positions per thread per pass iteration.  The long-cache variant runs one
// workgroup per CU, so each thread keeps 8 loads per array in flight per
// sweep; the short-cache one keeps its LDS small for several workgroups per
// CU.  The scan reads 4 consecutive positions per thread (more measured
// slower: the per-lane runs no longer share cache lines).
template <int NT>
struct Tune {
  static constexpr int kSweep = NT >= 1024 ? 8 : 4;  // pooling tile, EMA sweeps
  static constexpr int kScanItems = 4;               // prefix scan
};
constexpr int kMaxMerged = kMaxThresholds + 1;

// LDS of one workgroup of NT threads (sized by NT so that the short-cache
// variant keeps several workgroups per CU).
template <int NT>
struct Shared {
  static constexpr int kRankStage = 2 * NT;  // segments whose walk data fit LDS
  uint64_t red_u64[kMaxWaves];
  int64_t red_i64[kMaxWaves];
  int merged_a[kMaxMerged];
  int merged_b[kMaxMerged];
  int piece_off[kMaxMerged + 1];
  int cut[kMaxMerged];  // raw cuts e_k (at most kMaxThresholds)
  int n_merged;
  union {
    float tile[NT * Tune<NT>::kSweep + 2 * kMaxHalo];  // pooling input tile with halo
    struct {
      uint64_t m[kRankStage];                // walk order keys (mass)
      int32_t room[kRankStage];              // steps left per segment
    } walk;
  } u;
};

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int64_t wave_max_i64(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Block-wide reductions: every thread must call them (uniform control flow).
template <int NT>
__device__ uint64_t block_sum_u64(uint64_t v, Shared<NT>& sh) {
  v = wave_sum_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_u64[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += sh.red_u64[i];
  return s;
}

template <int NT>
__device__ int64_t block_sum_i64(int64_t v, Shared<NT>& sh) {
  v = wave_sum_i64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_i64[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += sh.red_i64[i];
  return s;
}

template <int NT>
__device__ int64_t block_max_i64(int64_t v, Shared<NT>& sh) {
  v = wave_max_i64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_i64[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t s = sh.red_i64[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) s = sh.red_i64[i] > s ? sh.red_i64[i] : s;
  return s;
}

// Pooled usage at t: centred window of 2h+1, in-range neighbours only.
// Average: fp32 sum in ascending position order from +0.0, one division.
// `tile` holds positions [t_base - h, ...) of the head (only in-range
// positions are ever read).
__device__ __forceinline__ float pooled(const float* __restrict__ tile, int t_base, int T, int t,
                                        int h, int mode) {
  const int lo = t - h < 0 ? 0 : t - h;
  const int hi = t + h > T - 1 ? T - 1 : t + h;
  const float* x = tile + (h - t_base);  // x[j] = u[j]
  if (mode == KVC_POOL_MAX) {
    float m = x[lo];
    for (int j = lo + 1; j <= hi; ++j) m = fmaxf(m, x[j]);
    return m;
  }
  float acc = 0.0f;
  for (int j = lo; j <= hi; ++j) acc = acc + x[j];
  return acc / float(hi - lo + 1);
}

// The same pooled usage at a position whose whole window lies inside the
// cache, for a compile-time half-width H: the window's reads all issue before
// the sum (which keeps its ascending order from +0.0).  The average divides
// by the fixed count n = 2H+1 through its reciprocal y = RN(1/n): with
// q = RN(a*y), RN(q + fma(-n, q, a)*y) is the correctly rounded a/n for every
// float a in [2^-80, 2^100] (no intermediate is subnormal there; checked
// exhaustively against IEEE division for every n <= 63).  Other sums (zero,
// tiny, huge, non-finite) take the division.
template <int H>
__device__ __forceinline__ float pooled_interior(const float* __restrict__ x, int t, int mode) {
  float v[2 * H + 1];
#pragma unroll
  for (int j = 0; j <= 2 * H; ++j) v[j] = x[t - H + j];
  if (mode == KVC_POOL_MAX) {
    float m = v[0];
#pragma unroll
    for (int j = 1; j <= 2 * H; ++j) m = fmaxf(m, v[j]);
    return m;
  }
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j <= 2 * H; ++j) acc = acc + v[j];
  constexpr float n = float(2 * H + 1);
  constexpr float y = 1.0f / n;
  if (acc >= 0x1p-80f && acc <= 0x1p100f) {
    const float q = acc * y;
    return __builtin_fmaf(__builtin_fmaf(-n, q, acc), y, q);
  }
  return acc / n;
}

// a / d correctly rounded, for a >= 0 and a divisor d > 0 that is fixed for
// the whole head (both far from underflow and overflow), from y = RN(1/d)
// taken once: q = RN(a*y) is within one ulp of a/d, the residual a - d*q is
// exact in one FMA, and RN(q + residual*y) is the correctly rounded quotient
// (Markstein's theorem for a reciprocal within half an ulp).  Three fp64
// operations instead of a full division per position.
struct Divisor {
  double d, y;
};
__device__ __forceinline__ Divisor make_divisor(double d) { return Divisor{d, 1.0 / d}; }
__device__ __forceinline__ double div_rn(double a, Divisor D) {
  const double q = a * D.y;
  const double r = __builtin_fma(-D.d, q, a);
  return __builtin_fma(r, D.y, q);
}

// Sum of v over [a, b] (inclusive, may be empty) from the inclusive prefix.
__device__ __forceinline__ uint64_t range_sum(const uint64_t* __restrict__ P, int a, int b) {
  if (a > b) return 0;
  return P[b] - (a > 0 ? P[a - 1] : 0);
}

__device__ __forceinline__ int overlap_len(int a, int b, int c, int e) {
  const int lo = a > c ? a : c, hi = b < e ? b : e;
  return hi >= lo ? hi - lo + 1 : 0;
}

// Does segment x come before segment y in the redistribution order?
// Adding: (mass desc, index asc); removing: (mass asc, index desc).
__device__ __forceinline__ bool precedes(uint64_t mx, int x, uint64_t my, int y, bool adding) {
  if (adding) return mx > my || (mx == my && x < y);
  return mx < my || (mx == my && x > y);
}

// ONE: every head is one raw segment that is not split (no mass thresholds,
// T <= seg_max or no splitting); the host decides it for the whole launch.
template <int NT, bool ONE>
__global__ __launch_bounds__(NT) void k_mass_segment(
    Derived P, const float* __restrict__ u, const uint64_t* __restrict__ credit_in,
    float* __restrict__ score, uint64_t* __restrict__ credit_upd, uint64_t* __restrict__ vp,
    int32_t* __restrict__ seg_start, int32_t* __restrict__ seg_quota, int32_t* __restrict__ n_seg,
    uint64_t* __restrict__ seg_m, int32_t* __restrict__ seg_a, int32_t* __restrict__ seg_f,
    int32_t* __restrict__ seg_q) {
  __shared__ Shared<NT> sh;
  constexpr int kSweep = Tune<NT>::kSweep;
  constexpr int kScanItems = Tune<NT>::kScanItems;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  // A left-padded head runs on its real tokens [off, off + T) only.
  const Span sp = head_span(P, n);
  const int T = sp.T;
  const Keep mk = P.vlen ? must_keep(P.sinks, P.recent, P.K, T) : Keep{P.s_keep, P.r_keep, P.t_keep};
  const float* un = u + size_t(n) * P.T + sp.off;
  float* sc = score + size_t(n) * P.T + sp.off;
  uint64_t* vn = vp + size_t(n) * P.T + sp.off;
  for (int t = tid; t < sp.off; t += NT) {  // padding: score 0, credit 0
    score[size_t(n) * P.T + t] = 0.0f;
    if (P.ema) credit_upd[size_t(n) * P.T + t] = 0;
  }

  // One raw segment (no mass thresholds) that is not split: the prefix C is
  // then only needed for that segment's mass, C(T-1) minus the must-keep
  // positions' share.  Both are exact sums taken during the sweeps below, so
  // the prefix is not built.
  constexpr bool one_seg = ONE;
  const int s_end = mk.s - 1, r_beg = T - mk.r;
  uint64_t mk_part = 0;  // usage of the must-keep positions (one_seg only)

  // The fixed-point usage is a function of the stored pooled score (the same
  // float, so the same integer): later sweeps recompute it from the 4-byte
  // score instead of storing and re-reading an 8-byte copy.
  // Usage outside the documented range (negative, NaN, or past 2^23, which
  // step 1 never produces) is clamped first, so the conversion is always
  // defined; clamping never changes a value in range.
  auto usage_q = [&](float ub) -> uint64_t {
    float nonneg = ub > 0.0f ? ub : 0.0f;  // NaN -> 0
    nonneg = nonneg < 0x1p23f ? nonneg : 0x1p23f;
    return uint64_t(nonneg * 1099511627776.0f) + P.eps_q;  // exact 2^40 scale
  };

  // -- step 2a/2b: pooled score and fixed-point usage w = trunc(ubar*2^40)+e,
  // one tile of NT*kSweep positions (plus the pooling halo) through LDS
  uint64_t part = 0;
  const int h = P.pool_h;
  // Every load of a tile is issued before any is stored: clamped indices
  // instead of branches (slots outside [0, T) hold a copy never read).  The
  // next tile's loads go out before this tile is pooled.  The default
  // pooling kernel (7, half-width 3) runs with its half-width known at
  // compile time, so each interior window is read at once (128K-token event:
  // pooling sweep 87 -> 53 us); edges and other kernels take the loop.
  auto pool_sweep = [&](auto half_width) {
    constexpr int HC = decltype(half_width)::value;  // < 0: only the runtime h
    float tv[kSweep + 1];
    auto load_tile = [&](int t_base) {
#pragma unroll
      for (int k = 0; k <= kSweep; ++k) {
        int t = t_base - h + tid + k * NT;
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
        tv[k] = un[t];
      }
    };
    load_tile(0);
    for (int t_base = 0; t_base < T; t_base += NT * kSweep) {
      const int span = NT * kSweep + 2 * h;  // <= NT * (kSweep + 1): 2h <= 62 < NT
      __syncthreads();  // previous tile consumed
#pragma unroll
      for (int k = 0; k <= kSweep; ++k)
        if (tid + k * NT < span) sh.u.tile[tid + k * NT] = tv[k];
      __syncthreads();
      load_tile(t_base + NT * kSweep);  // past the end: clamped copies, never stored
#pragma unroll
      for (int k = 0; k < kSweep; ++k) {
        const int t = t_base + k * NT + tid;
        if (t < T) {
          float ub;
          if constexpr (HC >= 0) {
            ub = t >= HC && t + HC <= T - 1
                     ? pooled_interior<HC>(sh.u.tile + (HC - t_base), t, P.pool_mode)
                     : pooled(sh.u.tile, t_base, T, t, h, P.pool_mode);
          } else {
            ub = pooled(sh.u.tile, t_base, T, t, h, P.pool_mode);
          }
          sc[t] = ub;
          const uint64_t w = usage_q(ub);
          if (one_seg && (t <= s_end || t >= r_beg)) mk_part += w;
          part += w;
        }
      }
    }
  };
  if (h == 3)
    pool_sweep(std::integral_constant<int, 3>{});
  else
    pool_sweep(std::integral_constant<int, -1>{});
  const uint64_t w_total = block_sum_u64<NT>(part, sh);
  uint64_t v_total = w_total;  // C(T-1)

  // -- step 2c: EMA credit and mixed mass (Q44).  The credit is swept here;
  // the mixed mass v is formed where it is consumed (the prefix scan, or the
  // one-segment sums).
  uint64_t* cu = P.ema ? credit_upd + size_t(n) * P.T + sp.off : nullptr;
  const Divisor wd = make_divisor(double(w_total));
  uint64_t c_total = 0;
  Divisor cd{0.0, 0.0};
  auto mixed = [&](uint64_t w, uint64_t cq) -> uint64_t {
    const double mq = div_rn(double(w), wd);
    const double nc = c_total ? div_rn(double(cq), cd) : 0.0;
    const double mix = (P.beta * mq) + (P.omb * nc);
    return uint64_t(floor(mix * 0x1p44));
  };
  if (P.ema) {
    const uint64_t* ci = credit_in ? credit_in + size_t(n) * P.n_prev : nullptr;
    part = 0;
    // Loads first, clamped (no branches), and one stride ahead of the sweep.
    float sv[kSweep], sv_next[kSweep];
    uint64_t cin[kSweep], cin_next[kSweep];
    auto load_ema = [&](int t0, float (&s_)[kSweep], uint64_t (&c_)[kSweep]) {
#pragma unroll
      for (int k = 0; k < kSweep; ++k) {
        const int t = t0 + k * NT;
        s_[k] = sc[t < T ? t : T - 1];
        c_[k] = 0;
      }
      if (P.n_prev > 0) {
#pragma unroll
        for (int k = 0; k < kSweep; ++k) {
          const int t = t0 + k * NT;
          c_[k] = ci[t < P.n_prev ? t : P.n_prev - 1];
        }
      }
    };
    load_ema(tid, sv, cin);
    for (int t0 = tid; t0 < T; t0 += NT * kSweep) {
      load_ema(t0 + NT * kSweep, sv_next, cin_next);  // past the end: clamped copies, unused
#pragma unroll
      for (int k = 0; k < kSweep; ++k) {
        const int t = t0 + k * NT;
        if (t >= T) continue;
        const double mq = div_rn(double(usage_q(sv[k])), wd);
        const double c = t < P.n_prev ? double(cin[k]) * 0x1p-44 : floor(mq * 0x1p44) * 0x1p-44;
        const double c_new = (P.lam * c) + (P.oml * mq);
        const uint64_t cq = uint64_t(floor(c_new * 0x1p44));
        cu[t] = cq;
        part += cq;
      }
#pragma unroll
      for (int k = 0; k < kSweep; ++k) {
        sv[k] = sv_next[k];
        cin[k] = cin_next[k];
      }
    }
    c_total = block_sum_u64<NT>(part, sh);
    if (c_total) cd = make_divisor(double(c_total));
    if (one_seg) {  // the mixed masses' total and must-keep share
      part = 0;
      mk_part = 0;
      for (int t0 = tid; t0 < T; t0 += NT * kSweep) {
        float sv[kSweep];
        uint64_t cq[kSweep];
#pragma unroll
        for (int k = 0; k < kSweep; ++k) {  // clamped loads (positions past T are skipped below)
          const int t = t0 + k * NT;
          sv[k] = sc[t < T ? t : T - 1];
          cq[k] = cu[t < T ? t : T - 1];
        }
#pragma unroll
        for (int k = 0; k < kSweep; ++k) {
          const int t = t0 + k * NT;
          if (t >= T) continue;
          const uint64_t v = mixed(usage_q(sv[k]), cq[k]);
          if (t <= s_end || t >= r_beg) mk_part += v;
          part += v;
        }
      }
      v_total = block_sum_u64<NT>(part, sh);
    }
  }

  if (T <= P.K) {  // nothing to evict
    if (tid == 0) n_seg[n] = 0;
    return;
  }

  // -- step 2d: inclusive prefix C(t) of v (usage, or the mixed mass with
  // EMA), formed from the stored score (and credit) as the scan reads them
  __syncthreads();
  const uint64_t mk_total = one_seg ? block_sum_u64<NT>(mk_part, sh) : 0;
  if constexpr (!one_seg && NT >= 1024) {
    uint64_t carry = 0;
    const int lane = tid & 63, wave = tid >> 6;
    auto load_tile = [&](int b, float (&s_)[kScanItems], uint64_t (&c_)[kScanItems]) {
#pragma unroll
      for (int i = 0; i < kScanItems; ++i) {  // clamped loads (positions past T are zeroed below)
        const int t0 = b + tid * kScanItems + i;
        const int t = t0 < T ? t0 : T - 1;
        s_[i] = sc[t];
        c_[i] = P.ema ? cu[t] : 0;
      }
    };
    // One tile of NT*kScanItems positions from its loaded score (and credit).
    auto scan_tile = [&](int base, const float (&sv)[kScanItems], const uint64_t (&cq)[kScanItems]) {
      uint64_t x[kScanItems];
      const int i0 = base + tid * kScanItems;
#pragma unroll
      for (int i = 0; i < kScanItems; ++i) {
        const uint64_t w = usage_q(sv[i]);
        x[i] = i0 + i < T ? (P.ema ? mixed(w, cq[i]) : w) : 0;
      }
#pragma unroll
      for (int i = 1; i < kScanItems; ++i) x[i] += x[i - 1];
      uint64_t incl = x[kScanItems - 1];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      __syncthreads();
      if (lane == 63) sh.red_u64[wave] = incl;
      __syncthreads();
      uint64_t wave_off = 0, tile_total = 0;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) {
        wave_off += i < wave ? sh.red_u64[i] : 0;
        tile_total += sh.red_u64[i];
      }
      const uint64_t excl = carry + wave_off + (incl - x[kScanItems - 1]);
#pragma unroll
      for (int i = 0; i < kScanItems; ++i)
        if (i0 + i < T) vn[i0 + i] = x[i] + excl;
      carry += tile_total;
    };
    // Long caches (many tiles): each tile's loads are issued one tile ahead,
    // before the current tile's barriers (128K-token event 498 -> 441 us).
    {
      float sv[kScanItems], sv_next[kScanItems];
      uint64_t cq[kScanItems], cq_next[kScanItems];
      load_tile(0, sv, cq);
      for (int base = 0; base < T; base += NT * kScanItems) {
        load_tile(base + NT * kScanItems, sv_next, cq_next);  // past the end: clamped copies, unused
        scan_tile(base, sv, cq);
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
          sv[i] = sv_next[i];
          cq[i] = cq_next[i];
        }
      }
    }
  }
  if constexpr (!one_seg && NT < 1024) {
    uint64_t carry = 0;
    const int lane = tid & 63, wave = tid >> 6;
    for (int base = 0; base < T; base += NT * kScanItems) {
      uint64_t x[kScanItems];
      const int i0 = base + tid * kScanItems;
      float sv[kScanItems];
      uint64_t cq[kScanItems];
#pragma unroll
      for (int i = 0; i < kScanItems; ++i) {  // clamped loads, then the values
        const int t = i0 + i < T ? i0 + i : T - 1;
        sv[i] = sc[t];
        cq[i] = P.ema ? cu[t] : 0;
      }
#pragma unroll
      for (int i = 0; i < kScanItems; ++i) {
        const uint64_t w = usage_q(sv[i]);
        x[i] = i0 + i < T ? (P.ema ? mixed(w, cq[i]) : w) : 0;
      }
#pragma unroll
      for (int i = 1; i < kScanItems; ++i) x[i] += x[i - 1];
      uint64_t incl = x[kScanItems - 1];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      __syncthreads();
      if (lane == 63) sh.red_u64[wave] = incl;
      __syncthreads();
      uint64_t wave_off = 0, tile_total = 0;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) {
        wave_off += i < wave ? sh.red_u64[i] : 0;
        tile_total += sh.red_u64[i];
      }
      const uint64_t excl = carry + wave_off + (incl - x[kScanItems - 1]);
#pragma unroll
      for (int i = 0; i < kScanItems; ++i)
        if (i0 + i < T) vn[i0 + i] = x[i] + excl;
      carry += tile_total;
    }
  }
  __syncthreads();
  const uint64_t* Pn = vn;
  const uint64_t V = one_seg ? v_total : Pn[T - 1];

  // -- step 3b: thresholds theta_k = min(V, ceil(k*Delta*V)), cuts e_k =
  // the first t with C(t) >= theta_k.  Each thread first loads one of NT
  // evenly spaced samples of C into LDS; a cut is bracketed between two
  // samples there and bisected inside the bracket, so its search takes
  // 1 + log2(T/NT) dependent loads instead of log2(T).
  const int stride = (T + NT - 1) / NT;
  uint64_t* samp = sh.u.walk.m;  // 2*NT entries; the pooling tile is dead here
  if (!one_seg) {
    const int t = (tid + 1) * stride - 1;
    samp[tid] = Pn[t < T - 1 ? t : T - 1];
  }
  __syncthreads();
  for (int kk = tid; kk < P.n_thr; kk += NT) {
    if (P.seg_fixed > 0) {  // ablation: a cut every seg_fixed positions
      const int64_t e = int64_t(kk + 1) * P.seg_fixed - 1;
      sh.cut[kk] = e < T - 1 ? int(e) : T - 1;  // cuts past the end collapse into T-1
      continue;
    }
    const double x = ceil((double(kk + 1) * P.delta) * double(V));
    uint64_t th = uint64_t(x);
    if (th > V) th = V;
    int lo = 0, hi = NT - 1;  // samp[NT-1] = C(T-1) = V >= th
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (samp[mid] >= th) hi = mid; else lo = mid + 1;
    }
    // C(lo*stride - 1) = samp[lo-1] < th, C(min(T-1, (lo+1)*stride - 1)) >= th
    int a = lo * stride, b = (lo + 1) * stride - 1;
    b = b < T - 1 ? b : T - 1;
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (Pn[mid] >= th) b = mid; else a = mid + 1;
    }
    sh.cut[kk] = a;
  }
  __syncthreads();

  // -- step 3c: raw segments (distinct cuts, plus T-1), greedy forward merge
  if (tid == 0) {
    int nm = 0, prev_end = -1;
    int cur_a = -1, cur_b = -1;
    for (int i = 0; i <= P.n_thr; ++i) {
      const int e = i < P.n_thr ? sh.cut[i] : T - 1;
      if (e <= prev_end) continue;  // equal cuts collapse; cuts are nondecreasing
      const int a = prev_end + 1;
      prev_end = e;
      if (cur_a < 0) {
        cur_a = a;
        cur_b = e;
      } else if (cur_b - cur_a + 1 < P.seg_min) {
        cur_b = e;
      } else {
        sh.merged_a[nm] = cur_a;
        sh.merged_b[nm] = cur_b;
        ++nm;
        cur_a = a;
        cur_b = e;
      }
    }
    if (cur_b - cur_a + 1 < P.seg_min && nm > 0) {
      sh.merged_b[nm - 1] = cur_b;
    } else {
      sh.merged_a[nm] = cur_a;
      sh.merged_b[nm] = cur_b;
      ++nm;
    }
    // -- step 3d: pieces per merged segment
    int off = 0;
    for (int i = 0; i < nm; ++i) {
      sh.piece_off[i] = off;
      const int L = sh.merged_b[i] - sh.merged_a[i] + 1;
      off += (P.seg_max > 0 && L > P.seg_max) ? (L + P.seg_max - 1) / P.seg_max : 1;
    }
    sh.piece_off[nm] = off;
    sh.n_merged = nm;
  }
  __syncthreads();
  const int nm = sh.n_merged;
  const int ns = sh.piece_off[nm];  // <= s_cap by construction

  // -- step 3e: per-segment length, must-keep overlap, mass, floor
  const size_t so = size_t(n) * P.s_cap;
  int64_t f_part = 0;
  uint64_t m_part = 0;
  int64_t own_f = 0, own_a = 0;  // segment tid's floor, room and mass, kept for the wave quota path
  uint64_t own_m = 0;
  for (int s = tid; s < ns; s += NT) {
    int lo = 0, hi = nm - 1;  // merged segment holding piece s
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.piece_off[mid] <= s) lo = mid; else hi = mid - 1;
    }
    const int a = sh.merged_a[lo], b = sh.merged_b[lo];
    const int L = b - a + 1;
    int start = a, len = L;
    if (P.seg_max > 0 && L > P.seg_max) {
      const int np = (L + P.seg_max - 1) / P.seg_max;
      const int base = L / np, extra = L % np;
      const int kq = s - sh.piece_off[lo];
      start = a + kq * base + (kq < extra ? kq : extra);
      len = base + (kq < extra ? 1 : 0);
    }
    const int end = start + len - 1;
    const int kmk = overlap_len(start, end, 0, s_end) + overlap_len(start, end, r_beg, T - 1);
    const int avail = len - kmk;
    uint64_t mass;
    if (one_seg) {  // the segment is [0, T-1]
      mass = V - mk_total;
    } else {
      mass = range_sum(Pn, start, end);
      if (start <= s_end) mass -= range_sum(Pn, start, end < s_end ? end : s_end);
      if (end >= r_beg) mass -= range_sum(Pn, start > r_beg ? start : r_beg, end);
    }
    const int lmin = P.q_min < len ? P.q_min : len;
    int fl = lmin - kmk;
    fl = fl < 0 ? 0 : fl;
    fl = fl < avail ? fl : avail;
    if (P.quota_uniform) mass = 1;  // ablation: every segment weighs the same
    seg_start[so + s] = sp.off + start;
    seg_m[so + s] = mass;
    seg_a[so + s] = avail;
    seg_f[so + s] = fl;
    f_part += fl;
    m_part += mass;
    if (s == tid) {
      own_f = fl;
      own_a = avail;
      own_m = mass;
    }
  }
  const int64_t F = block_sum_i64<NT>(f_part, sh);
  const uint64_t SM = block_sum_u64<NT>(m_part, sh);

  // -- step 3f/3g: quotas.  Up to 64 segments (the common case) one wave does
  // it alone, lane s holding segment s (computed by this same thread in 3e
  // and still in its registers), with wave reductions instead of block-wide
  // ones; the arithmetic is the same as the block-wide version below.
  if (ns <= 64) {
    if (tid < 64) {
      const int s = tid;
      const bool has = s < ns;
      const int64_t fl = has ? own_f : 0, av = has ? own_a : 0;
      const uint64_t ms = has ? own_m : 0;
      int64_t qv = fl;
      if (F <= mk.t_keep) {
        const int64_t t_rem = mk.t_keep - F;
        int64_t add = 0;
        if (has && SM > 0) {
          const double share = double(t_rem) * (double(ms) / double(SM));
          add = int64_t(floor(share + 0.5));
        }
        qv = fl + add < av ? fl + add : av;
        const int64_t D = int64_t(mk.t_keep) - wave_sum_i64(qv);
        if (D != 0) {  // the cyclic walk in closed form, as below
          const bool adding = D > 0;
          const int64_t need = adding ? D : -D;
          const int64_t room = has ? (adding ? av - qv : qv - fl) : 0;
          int64_t lo = 0, hi = wave_max_i64(room);
          while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (wave_sum_i64(room < mid ? room : mid) <= need) lo = mid; else hi = mid - 1;
          }
          const int64_t cyc = lo;
          const int64_t r = need - wave_sum_i64(room < cyc ? room : cyc);
          int64_t delta = room < cyc ? room : cyc;
          int64_t rank = 0;
          for (int o = 0; o < ns; ++o) {  // every lane walks all segments (uniform)
            const int64_t ro = __shfl(room, o);
            const uint64_t mo = __shfl(ms, o);
            rank += (ro > cyc) & precedes(mo, o, ms, s, adding);
          }
          if (room > cyc && rank < r) ++delta;
          qv = adding ? qv + delta : qv - delta;
        }
      }
      if (has) seg_quota[so + s] = int32_t(qv);
      if (s == 0) n_seg[n] = ns;
    }
    return;
  }
  if (F > mk.t_keep) {
    for (int s = tid; s < ns; s += NT) seg_q[so + s] = seg_f[so + s];
  } else {
    const int64_t t_rem = mk.t_keep - F;
    int64_t q_part = 0;
    for (int s = tid; s < ns; s += NT) {
      int64_t add = 0;
      if (SM > 0) {
        const double share = double(t_rem) * (double(seg_m[so + s]) / double(SM));
        add = int64_t(floor(share + 0.5));
      }
      int64_t qv = seg_f[so + s] + add;
      if (qv > seg_a[so + s]) qv = seg_a[so + s];
      seg_q[so + s] = int32_t(qv);
      q_part += qv;
    }
    const int64_t D = int64_t(mk.t_keep) - block_sum_i64<NT>(q_part, sh);
    if (D != 0) {
      // Cyclic walk in closed form: c full cycles give every segment
      // min(room, c); the next, partial cycle gives one more to the first r
      // segments (in walk order) whose room exceeds c.
      const bool adding = D > 0;
      const int64_t need = adding ? D : -D;
      // Rooms and walk keys go to LDS when they fit (the ranks below read
      // every segment once per segment).
      const bool staged = ns <= Shared<NT>::kRankStage;
      if (staged) {
        for (int s = tid; s < ns; s += NT) {
          sh.u.walk.room[s] = adding ? seg_a[so + s] - seg_q[so + s] : seg_q[so + s] - seg_f[so + s];
          sh.u.walk.m[s] = seg_m[so + s];
        }
        __syncthreads();
      }
      auto room_of = [&](int s) -> int64_t {
        if (staged) return sh.u.walk.room[s];
        return adding ? seg_a[so + s] - seg_q[so + s] : seg_q[so + s] - seg_f[so + s];
      };
      auto m_of = [&](int s) -> uint64_t { return staged ? sh.u.walk.m[s] : seg_m[so + s]; };
      int64_t rmax = 0;
      for (int s = tid; s < ns; s += NT) {
        const int64_t room = room_of(s);
        rmax = room > rmax ? room : rmax;
      }
      rmax = block_max_i64<NT>(rmax, sh);
      int64_t lo = 0, hi = rmax;
      while (lo < hi) {  // largest c with sum min(room, c) <= need
        const int64_t mid = (lo + hi + 1) >> 1;
        int64_t sp = 0;
        for (int s = tid; s < ns; s += NT) {
          const int64_t room = room_of(s);
          sp += room < mid ? room : mid;
        }
        if (block_sum_i64<NT>(sp, sh) <= need) lo = mid; else hi = mid - 1;
      }
      const int64_t cyc = lo;
      int64_t sp = 0;
      for (int s = tid; s < ns; s += NT) {
        const int64_t room = room_of(s);
        sp += room < cyc ? room : cyc;
      }
      const int64_t r = need - block_sum_i64<NT>(sp, sh);
      if (staged) {
        // The walk order as one unsigned key per segment: 1 + the mass
        // (adding: larger first) or 1 + (2^63 - 1 - mass) (removing: smaller
        // first), and 0 for a segment whose room the full cycles used up.
        // Masses stay below 2^63 (usage totals are bounded by the window and
        // pooling, mixed masses sum to about 2^44), so no key wraps.  A tie
        // goes to the lower index when adding and to the higher one when
        // removing, so segment s is preceded by o iff key[o] >= key[s] on the
        // winning side of s and key[o] >= key[s] + 1 on the other.  Keys are
        // padded with zeros to whole chunks of 32.
        for (int s = tid; s < ((ns + 31) & ~31); s += NT) {
          uint64_t key = 0;
          if (s < ns && sh.u.walk.room[s] > cyc)
            key = 1 + (adding ? sh.u.walk.m[s] : 0x7fffffffffffffffull - sh.u.walk.m[s]);
          sh.u.walk.m[s] = key;
        }
        __syncthreads();
        const uint64_t* key = sh.u.walk.m;
        const int lane = tid & 63;
        for (int sb = tid - lane; sb < ns; sb += NT) {  // lane s = sb + lane, uniform per wave
          const int s = sb + lane;
          const bool mine = s < ns;
          const int64_t room = mine ? sh.u.walk.room[s] : 0;
          const uint64_t ks = mine ? key[s] : 0;
          const bool part = mine && room > cyc && r > 0;
          const uint64_t t_lo = adding ? ks : ks + 1;  // for o < s
          const uint64_t t_hi = adding ? ks + 1 : ks;  // for o > s
          int rank = 0;
          for (int c = 0; c < ns && __any(part && rank < r); c += 32) {
            if (c + 32 <= sb || c >= sb + 64) {  // the whole chunk lies on one side of every lane
              const uint64_t th = c < sb ? t_lo : t_hi;
#pragma unroll
              for (int i = 0; i < 32; ++i) rank += key[c + i] >= th;
            } else {
#pragma unroll 4
              for (int i = 0; i < 32; ++i) {
                const int o = c + i;
                rank += (o != s) & (key[o] >= (o < s ? t_lo : t_hi));
              }
            }
          }
          int64_t delta = room < cyc ? room : cyc;
          if (part && rank < r) ++delta;
          if (mine) seg_quota[so + s] = int32_t(adding ? seg_q[so + s] + delta : seg_q[so + s] - delta);
        }
      } else {
        // New quotas go to the output array; the ranks read the old rooms,
        // which nothing writes during this loop.
        for (int s = tid; s < ns; s += NT) {
          const int64_t room = room_of(s);
          int64_t delta = room < cyc ? room : cyc;
          if (room > cyc && r > 0) {
            const uint64_t ms = m_of(s);
            int64_t rank = 0;
            for (int o = 0; o < ns && rank < r; ++o)
              if (room_of(o) > cyc && precedes(m_of(o), o, ms, s, adding)) ++rank;
            if (rank < r) ++delta;
          }
          seg_quota[so + s] = int32_t(adding ? seg_q[so + s] + delta : seg_q[so + s] - delta);
        }
      }
      if (tid == 0) n_seg[n] = ns;
      return;
    }
  }
  __syncthreads();
  for (int s = tid; s < ns; s += NT) seg_quota[so + s] = seg_q[so + s];
  if (tid == 0) n_seg[n] = ns;
}

}  // namespace

hipError_t launch_mass_segment(const Derived& d, const float* u, const uint64_t* credit_in,
                               float* score, uint64_t* credit_upd, uint64_t* vp,
                               int32_t* seg_start, int32_t* seg_quota, int32_t* n_seg,
                               uint64_t* seg_m, int32_t* seg_a, int32_t* seg_f, int32_t* seg_q,
                               hipStream_t s) {
  // A ragged head's real length is at most d.T, so d.T <= seg_max covers every head.
  const bool one = d.n_thr == 0 && (d.seg_max <= 0 || d.T <= d.seg_max);
  auto go = [&](auto kernel, int nt) {
    kernel<<<d.NH, nt, 0, s>>>(d, u, credit_in, score, credit_upd, vp, seg_start, seg_quota, n_seg,
                              seg_m, seg_a, seg_f, seg_q);
  };
  if (d.T >= 4096)
    one ? go(k_mass_segment<1024, true>, 1024) : go(k_mass_segment<1024, false>, 1024);
  else
    one ? go(k_mass_segment<256, true>, 256) : go(k_mass_segment<256, false>, 256);
  return hipGetLastError();
}

}  // namespace kvc
