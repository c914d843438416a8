// Step 4 on gfx950: in-segment top-q, union with must-keep, budget repair and
// sorted kept indices.  One workgroup per head-event; the keep set lives as a
// bitmap in LDS.
//
// Sources: AMS notes, key design 3 (last paragraph: union with the must-keep
// set, duplicates counted once; over budget drop low-score non-must-keep
// positions, under budget add high-score unselected ones) and key design 4
// (per-segment top-k on the base score, kept indices sorted).
//
// Ranking is by (score desc, position asc).  Scores become order-preserving
// 32-bit keys (+0 and -0 equal), so "the r best of a set" is exact integer
// work: the largest key tau with at least r members >= tau (found digit by
// digit with histograms, or bit by bit with population counts), then the
// members above tau and the lowest-positioned members equal to tau up to r.
// The result is the unique canonical selection, independent of thread order.
#include "kvc_internal.h"

namespace kvc {
namespace {

// Long caches run with 1024 threads per workgroup, short ones with 256.
constexpr int kMaxWaves = 16;
constexpr int kCached = 16;    // keys per thread kept in registers by the threshold search
constexpr int kWaveSeg = 256;  // segments up to this length: one wave each
constexpr int kPerLane = kWaveSeg / 64;
constexpr int kSmallQuota = 8;  // one-wave segments with quotas up to this walk the top keys

// LDS of one workgroup of NT threads: the keep bitmap (the short-cache
// variant only takes caches below 4096 positions, so its bitmap is small and
// several workgroups share a CU) and, for that variant, the segment starts
// and quotas when they fit (every thread reads each of them once per loop).
template <int NT>
struct Shared {
  static constexpr int kBits = NT >= 1024 ? kMaxT / 32 : 4096 / 32;
  static constexpr int kStage = NT >= 1024 ? 1 : 512;
  // Segments longer than kWaveSeg cover more than 256 positions each: at most
  // T/257 of them (15 below 4096 positions, 1020 at 2^18).
  static constexpr int kLongCap = NT >= 1024 ? 1024 : 16;
  uint32_t bits[kBits];
  uint32_t red[kMaxWaves];
  int32_t long_ids[kLongCap];
  int n_long;
  int32_t seg_s[kStage];
  int32_t seg_q[kStage];
  // Radix threshold search over register-cached keys.  The 256-bin digit
  // histogram is kept in kCopies copies (bin-major, the copy picked by the
  // thread index), folded into hsum after each round: the leading digit of
  // a float key is its sign and high exponent bits, so most of a wave's
  // keys share a bin, and one copy would serialise their LDS atomics (eight
  // copies measured 2x faster on a 16K-position cache).  Then the chosen
  // digit and count, and per (cached slot, wave) the ballot of ties.
  static constexpr int kCopies = NT >= 1024 ? 8 : 4;
  uint32_t hist[256 * kCopies];
  uint32_t hsum[256];
  uint32_t pick[2];
  uint64_t tie_mask[kCached * (NT / 64)];
};

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) == 0) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <class Sh>
__device__ __forceinline__ bool test_bit(const Sh& sh, int t) {
  return (sh.bits[t >> 5] >> (t & 31)) & 1u;
}

template <class Sh>
__device__ __forceinline__ void set_bit(Sh& sh, int t) {
  atomicOr(&sh.bits[t >> 5], 1u << (t & 31));
}

template <class Sh>
__device__ __forceinline__ void clear_bit(Sh& sh, int t) {
  atomicAnd(&sh.bits[t >> 5], ~(1u << (t & 31)));
}

// Block-wide count; every thread must call it.  The wave sum adds across the
// lanes of each 16-lane row with DPP (a butterfly: swap neighbours, pairs,
// half-rows, row halves) and reads the four row sums back, instead of six
// cross-lane shuffles through LDS (measured 20 % faster for the 16K-token
// global select, whose threshold search is 46 of these counts).
template <int NT>
__device__ uint32_t block_count(uint32_t c, Shared<NT>& sh) {
  c += __builtin_amdgcn_update_dpp(0u, c, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
  c += __builtin_amdgcn_update_dpp(0u, c, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
  c += __builtin_amdgcn_update_dpp(0u, c, 0x141, 0xf, 0xf, false);  // row_half_mirror
  c += __builtin_amdgcn_update_dpp(0u, c, 0x140, 0xf, 0xf, false);  // row_mirror
  c = __builtin_amdgcn_readlane(c, 0) + __builtin_amdgcn_readlane(c, 16) +
      __builtin_amdgcn_readlane(c, 32) + __builtin_amdgcn_readlane(c, 48);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = c;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += sh.red[i];
  return __builtin_amdgcn_readfirstlane(s);
}

// The r best positions of {t in [a,b] : pred(t)} are those with key > tau,
// plus those with key == tau and t <= xcut.  Requires 1 <= r < |set|; every
// thread must call it with the same arguments.  tau is the largest key with
// at least r members >= it.  When the range fits, each thread caches its
// candidates' keys in registers (kCached per thread); tau then takes four
// rounds of an 8-bit-digit histogram and xcut one pass over per-wave ballots
// of the ties.  Otherwise tau is found bit by bit and xcut by a binary search
// over positions, each step one block-wide count that re-reads the scores.
template <int NT, class Pred>
__device__ void block_threshold(const float* __restrict__ sc, int a, int b, uint32_t r, Pred pred,
                                Shared<NT>& sh, uint32_t* tau_out, int* xcut_out) {
  uint32_t tau = 0;
  int lo = a, hi = b;
  if (b - a + 1 <= NT * kCached) {
    uint32_t key[kCached];
    uint32_t valid = 0;
#pragma unroll
    for (int i = 0; i < kCached; ++i) {  // clamped loads: all issued before any is used
      const int t = a + int(threadIdx.x) + i * NT;
      const float x = sc[t <= b ? t : b];
      const bool ok = t <= b && pred(t);
      key[i] = ok ? order_key(x) : 0u;
      valid |= ok ? (1u << i) : 0u;
    }
    // tau, eight bits at a time: histogram the digit of the members whose
    // higher digits equal tau's so far, then take the largest digit d with
    // (members above) + (members with digit >= d) >= r.  `above` counts the
    // members already known to be > tau.
    constexpr int kC = Shared<NT>::kCopies;
    const uint32_t copy = threadIdx.x % kC;
    uint32_t above = 0;
    for (int i = int(threadIdx.x); i < 256 * kC; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hi_mask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
#pragma unroll
      for (int i = 0; i < kCached; ++i)
        if (((valid >> i) & 1u) && (key[i] & hi_mask) == tau)
          atomicAdd(&sh.hist[((key[i] >> shift) & 255u) * kC + copy], 1u);
      __syncthreads();
      for (int d = int(threadIdx.x); d < 256; d += NT) {  // fold the copies, clear them for the next round
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          v += sh.hist[d * kC + c];
          sh.hist[d * kC + c] = 0;
        }
        sh.hsum[d] = v;
      }
      __syncthreads();
      if (threadIdx.x < 64) {  // lane l holds digits 4l .. 4l+3
        const int l = int(threadIdx.x);
        const uint32_t h0 = sh.hsum[4 * l], h1 = sh.hsum[4 * l + 1], h2 = sh.hsum[4 * l + 2],
                       h3 = sh.hsum[4 * l + 3];
        uint32_t suf = h0 + h1 + h2 + h3;  // inclusive suffix sum over lanes l..63
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_down(suf, off);
          if (l + off < 64) suf += y;
        }
        // members with digit >= 4l+3, 4l+2, 4l+1, 4l
        const uint32_t c3 = suf - h0 - h1 - h2, c2 = c3 + h2, c1 = c2 + h1, c0 = suf;
        int d = -1;
        uint32_t gt = 0;  // members with digit > d
        if (above + c0 >= r) { d = 4 * l; gt = c1; }
        if (above + c1 >= r) { d = 4 * l + 1; gt = c2; }
        if (above + c2 >= r) { d = 4 * l + 2; gt = c3; }
        if (above + c3 >= r) { d = 4 * l + 3; gt = c3 - h3; }
        const uint64_t m = __ballot(d >= 0);  // lanes with a qualifying digit
        const int top = 63 - __clzll(m);      // the largest digits live in the highest lane
        if (l == top) {
          sh.pick[0] = uint32_t(d);
          sh.pick[1] = above + gt;
        }
      }
      __syncthreads();
      tau |= __builtin_amdgcn_readfirstlane(sh.pick[0]) << shift;
      above = __builtin_amdgcn_readfirstlane(sh.pick[1]);
    }
    // xcut: the need-th tie (key == tau) in ascending position order, i.e.
    // slot-major, then thread order; ties are counted per (slot, wave).
    const uint32_t need = r - above;
    constexpr int kW = NT / 64;
    const int lane = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6;
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
      const uint64_t m = __ballot(((valid >> i) & 1u) && key[i] == tau);
      if (lane == 0) sh.tie_mask[i * kW + wave] = m;
    }
    __syncthreads();
    if (threadIdx.x < 64) {  // one wave finds the group holding the need-th tie
      constexpr int kGroups = kCached * kW;
      constexpr int kPer = (kGroups + 63) / 64;  // consecutive groups per lane
      const int l = int(threadIdx.x);
      uint32_t cnt[kPer];
      uint32_t own = 0;
#pragma unroll
      for (int g = 0; g < kPer; ++g) {
        const int e = l * kPer + g;
        cnt[g] = e < kGroups ? uint32_t(__popcll(sh.tie_mask[e])) : 0u;
        own += cnt[g];
      }
      uint32_t pre = own;  // inclusive prefix over lanes 0..l
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(pre, off);
        if (l >= off) pre += y;
      }
      uint32_t before = pre - own;
      if (before < need && pre >= need) {  // exactly one lane holds it
#pragma unroll
        for (int g = 0; g < kPer; ++g) {
          if (before < need && before + cnt[g] >= need) {
            const int e = l * kPer + g;
            uint64_t m = sh.tie_mask[e];
            for (uint32_t k = need - before; k > 1; --k) m &= m - 1;  // drop the first need-before-1 ties
            const int bit = __ffsll(static_cast<unsigned long long>(m)) - 1;
            const int i = e / kW, w = e % kW;
            sh.pick[0] = uint32_t(a + i * NT + w * 64 + bit);
          }
          before += cnt[g];
        }
      }
    }
    __syncthreads();
    lo = __builtin_amdgcn_readfirstlane(int(sh.pick[0]));
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      uint32_t c = 0;
      for (int t = a + threadIdx.x; t <= b; t += NT)
        c += (pred(t) && order_key(sc[t]) >= cand) ? 1u : 0u;
      if (block_count<NT>(c, sh) >= r) tau = cand;
    }
    uint32_t c = 0;
    for (int t = a + threadIdx.x; t <= b; t += NT)
      c += (pred(t) && order_key(sc[t]) > tau) ? 1u : 0u;
    const uint32_t need = r - block_count<NT>(c, sh);
    while (lo < hi) {
      const int mid = lo + ((hi - lo) >> 1);
      uint32_t e = 0;
      for (int t = a + threadIdx.x; t <= mid; t += NT)
        e += (pred(t) && order_key(sc[t]) == tau) ? 1u : 0u;
      if (block_count<NT>(e, sh) >= need) hi = mid; else lo = mid + 1;
    }
  }
  *tau_out = tau;
  *xcut_out = lo;
}

__device__ __forceinline__ uint32_t wave_count(bool v) { return __popcll(__builtin_amdgcn_ballot_w64(v)); }

// Minimum over the wave's 64 lanes, uniform result (DPP within 16-lane rows,
// then the four row minima read back).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0xb1, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x4e, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x141, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x140, 0xf, 0xf, false)));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, d));
}

// Maximum over the wave's 64 lanes, uniform result (as wave_min_u32).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0xb1, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x4e, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x141, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x140, 0xf, 0xf, false)));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}

// The 1024-thread variant is held to 64 VGPRs so that two workgroups share a
// CU (8 waves per SIMD): one workgroup's barriers and LDS rounds then
// overlap the other's loads (16K-position global select 128 -> 113 us).
template <int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT >= 1024 ? 8 : 1))) void k_select(Derived P, const float* __restrict__ score,
                                                     const int32_t* __restrict__ seg_start,
                                                     const int32_t* __restrict__ seg_quota,
                                                     const int32_t* __restrict__ n_seg,
                                                     int32_t* __restrict__ kept) {
  __shared__ Shared<NT> sh;
  const int n = blockIdx.x;
  // A left-padded head runs on its real tokens [off, off + T) only; kept
  // holds positions of the padded cache.
  const Span sp = head_span(P, n);
  const int T = sp.T, K = P.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* kn = kept + size_t(n) * K;
  if (T <= K) {  // nothing to evict: identity, -1 past T
    for (int j = tid; j < K; j += NT) kn[j] = j < T ? sp.off + j : -1;
    return;
  }
  const float* sc = score + size_t(n) * P.T + sp.off;
  const int nw = (T + 31) >> 5;
  const Keep mk = P.vlen ? must_keep(P.sinks, P.recent, P.K, T) : Keep{P.s_keep, P.r_keep, P.t_keep};
  const int s_keep = mk.s, r_beg = T - mk.r;
  auto must_keep = [&](int t) { return t < s_keep || t >= r_beg; };

  // Segments as given (sanitised to [0,T); empty ones are skipped).
  int ns = n_seg[n];
  ns = ns < 0 ? 0 : (ns > P.s_cap ? P.s_cap : ns);
  const int32_t* ss = seg_start + size_t(n) * P.s_cap;
  const int32_t* sq = seg_quota + size_t(n) * P.s_cap;
  const bool staged = NT < 1024 && ns <= Shared<NT>::kStage;
  for (int w = tid; w < nw; w += NT) sh.bits[w] = 0;
  if (staged)
    for (int i = tid; i < ns; i += NT) {
      sh.seg_s[i] = ss[i];
      sh.seg_q[i] = sq[i];
    }
  __syncthreads();
  for (int t = tid; t < s_keep; t += NT) set_bit(sh, t);
  for (int t = r_beg + tid; t < T; t += NT) set_bit(sh, t);
  auto start_of = [&](int i) { return staged ? sh.seg_s[i] : ss[i]; };
  auto quota_of = [&](int i) {
    const int q = staged ? sh.seg_q[i] : sq[i];
    return q < 0 ? 0 : q;
  };
  auto seg_bounds = [&](int i, int* a, int* b) {  // starts are padded-cache positions
    int s0 = start_of(i) - sp.off, s1 = i + 1 < ns ? start_of(i + 1) - sp.off : T;
    s0 = s0 < 0 ? 0 : (s0 > T ? T : s0);
    s1 = s1 < 0 ? 0 : (s1 > T ? T : s1);
    *a = s0;
    *b = s1 - 1;
  };

  // Long segments: the whole workgroup, one at a time.  They are few, so
  // the threads first list them together (in any order: each one only sets
  // bits of its own range) instead of every wave scanning all segments.
  if (tid == 0) sh.n_long = 0;
  __syncthreads();
  for (int i = tid; i < ns; i += NT) {
    int a, b;
    seg_bounds(i, &a, &b);
    if (b - a + 1 > kWaveSeg) {
      const int slot = atomicAdd(&sh.n_long, 1);
      if (slot < Shared<NT>::kLongCap) sh.long_ids[slot] = i;
    }
  }
  __syncthreads();
  const int n_long = __builtin_amdgcn_readfirstlane(sh.n_long < Shared<NT>::kLongCap ? sh.n_long : Shared<NT>::kLongCap);
  for (int li = 0; li < n_long; ++li) {
    const int i = __builtin_amdgcn_readfirstlane(sh.long_ids[li]);
    int a, b;
    seg_bounds(i, &a, &b);
    a = __builtin_amdgcn_readfirstlane(a);
    b = __builtin_amdgcn_readfirstlane(b);
    const int q = __builtin_amdgcn_readfirstlane(quota_of(i));
    uint32_t c = 0;
    for (int t = a + tid; t <= b; t += NT) c += must_keep(t) ? 0u : 1u;
    const uint32_t avail = block_count<NT>(c, sh);
    if (q == 0 || avail == 0) continue;
    if (uint32_t(q) >= avail) {
      for (int t = a + tid; t <= b; t += NT)
        if (!must_keep(t)) set_bit(sh, t);
      continue;
    }
    uint32_t tau;
    int xcut;
    block_threshold<NT>(sc, a, b, uint32_t(q), [&](int t) { return !must_keep(t); }, sh, &tau, &xcut);
    for (int t = a + tid; t <= b; t += NT) {
      if (must_keep(t)) continue;
      const uint32_t kk = order_key(sc[t]);
      if (kk > tau || (kk == tau && t <= xcut)) set_bit(sh, t);
    }
  }

  // Short segments: one wave each, keys held in registers.  The segment
  // index, bounds and quota are wave-uniform; saying so (readfirstlane)
  // keeps the search in scalar control flow, one compare and one scalar
  // population count per key slot and bit (128K-token select 205 -> 123 us).
  for (int i = __builtin_amdgcn_readfirstlane(wave); i < ns; i += (NT / 64)) {
    int a, b;
    seg_bounds(i, &a, &b);
    a = __builtin_amdgcn_readfirstlane(a);
    b = __builtin_amdgcn_readfirstlane(b);
    const int L = b - a + 1;
    if (L <= 0 || L > kWaveSeg) continue;
    const int q = __builtin_amdgcn_readfirstlane(quota_of(i));
    if (q == 0) continue;
    bool ok[kPerLane];
    uint32_t key[kPerLane];
    uint32_t avail = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {  // clamped loads: all issued before any is used
      const int t = a + lane + 64 * e;
      const float x = sc[t <= b ? t : b];
      ok[e] = t <= b && !must_keep(t);
      key[e] = ok[e] ? order_key(x) : 0u;
      avail += wave_count(ok[e]);
    }
    if (uint32_t(q) >= avail) {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e)
        if (ok[e]) set_bit(sh, a + lane + 64 * e);
      continue;
    }
    // tau: the largest key with at least q members >= it (the q-th largest
    // member key, counted with multiplicity).
    uint32_t tau = 0;
    bool exact = false;
    if (q <= kSmallQuota) {
      // Small quotas walk the distinct member keys from the top: each round
      // takes the largest key below the previous one and counts the members
      // at or above it, so at most q rounds.  A bit-by-bit search needs a
      // round per bit down to where the q-th and (q+1)-th keys part (about 17
      // on float scores), and its rounds cost as much: counting is scalar
      // work either way (ballot population counts), which the SIMD's scalar
      // issue slot limits.  A zero maximum means only zero keys are left
      // (non-members carry 0; a member keyed 0 is then a tie at tau = 0).
      uint32_t bound = 0xffffffffu;
      bool first = true;
      for (int round = 0; round < q; ++round) {
        uint32_t lm = 0;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e)
          if (ok[e] && (first || key[e] < bound) && key[e] > lm) lm = key[e];
        const uint32_t m = wave_max_u32(lm);
        if (m == 0) break;
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) c += wave_count(key[e] >= m);  // m >= 1 > the 0 of non-members
        if (c >= uint32_t(q)) {
          tau = m;
          break;
        }
        bound = m;
        first = false;
      }
    } else {
    // Bit by bit.  Once exactly q members are >= the candidate, tau is their
    // smallest key and the remaining bits need no counting.
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) c += wave_count(key[e] >= cand);  // cand >= 1 > the 0 of non-members
      if (c >= uint32_t(q)) {
        tau = cand;
        if (c == uint32_t(q)) {
          exact = true;
          break;
        }
      }
    }
    }
    if (exact) {
      uint32_t mn = 0xffffffffu;
#pragma unroll
      for (int e = 0; e < kPerLane; ++e)
        if (ok[e] && key[e] >= tau) mn = key[e] < mn ? key[e] : mn;
      tau = wave_min_u32(mn);
    }
    uint32_t gt = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) gt += wave_count(ok[e] && key[e] > tau);
    const uint32_t need = uint32_t(q) - gt;
    // Positions a+lane+64e in ascending order are e-major, lane-minor: walk
    // the ties in that order and take the first `need`.
    uint32_t taken = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const bool tie = ok[e] && key[e] == tau;
      const uint64_t m = __ballot(tie);
      const uint32_t before = __popcll(m & ((uint64_t(1) << lane) - 1));
      const bool take = ok[e] && (key[e] > tau || (tie && taken + before < need));
      if (take) set_bit(sh, a + lane + 64 * e);
      taken += __popcll(m);
    }
  }
  __syncthreads();

  // Budget repair.
  uint32_t c = 0;
  for (int w = tid; w < nw; w += NT) c += __popc(sh.bits[w]);
  const uint32_t n_keep = block_count<NT>(c, sh);
  const uint32_t n_mk = uint32_t(mk.s + mk.r);
  if (n_keep > uint32_t(K)) {
    // Keep the best K - |MK| picks, drop the rest (the lowest-scored first).
    auto is_pick = [&](int t) { return !must_keep(t) && test_bit(sh, t); };
    const uint32_t r = uint32_t(K) - n_mk;
    if (r == 0) {
      __syncthreads();
      for (int t = tid; t < T; t += NT)
        if (!must_keep(t)) clear_bit(sh, t);
    } else {
      uint32_t tau;
      int xcut;
      block_threshold<NT>(sc, 0, T - 1, r, is_pick, sh, &tau, &xcut);
      // Each thread tests and clears only its own positions' bits.
      __syncthreads();
      for (int t = tid; t < T; t += NT) {
        if (must_keep(t) || !test_bit(sh, t)) continue;
        const uint32_t kk = order_key(sc[t]);
        if (!(kk > tau || (kk == tau && t <= xcut))) clear_bit(sh, t);
      }
    }
  } else if (n_keep < uint32_t(K)) {
    // Add the best unselected positions.
    auto is_free = [&](int t) { return !must_keep(t) && !test_bit(sh, t); };
    const uint32_t r = uint32_t(K) - n_keep;
    uint32_t f = 0;
    for (int t = tid; t < T; t += NT) f += is_free(t) ? 1u : 0u;
    const uint32_t n_free = block_count<NT>(f, sh);
    if (r >= n_free) {
      __syncthreads();
      for (int t = tid; t < T; t += NT)
        if (!must_keep(t)) set_bit(sh, t);
    } else {
      uint32_t tau;
      int xcut;
      block_threshold<NT>(sc, 0, T - 1, r, is_free, sh, &tau, &xcut);
      // Each thread tests and sets only its own positions' bits.
      __syncthreads();
      for (int t = tid; t < T; t += NT) {
        if (!is_free(t)) continue;
        const uint32_t kk = order_key(sc[t]);
        if (kk > tau || (kk == tau && t <= xcut)) set_bit(sh, t);
      }
    }
  }
  __syncthreads();

  // Compaction: ascending positions of the set bits.
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = tid * wpt;
  uint32_t cnt = 0;
  for (int w = w0; w < w0 + wpt && w < nw; ++w) cnt += __popc(sh.bits[w]);
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) sh.red[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt;
  for (int i = 0; i < wave; ++i) pos += sh.red[i];
  for (int w = w0; w < w0 + wpt && w < nw; ++w) {
    uint32_t word = sh.bits[w];
    while (word) {
      const int b = __ffs(word) - 1;
      word &= word - 1;
      if (pos < uint32_t(K)) kn[pos] = sp.off + w * 32 + b;
      ++pos;
    }
  }
}

}  // namespace

hipError_t launch_select(const Derived& d, const float* score, const int32_t* seg_start,
                         const int32_t* seg_quota, const int32_t* n_seg, int32_t* kept,
                         hipStream_t s) {
  if (d.T >= 4096)
    k_select<1024><<<d.NH, 1024, 0, s>>>(d, score, seg_start, seg_quota, n_seg, kept);
  else
    k_select<256><<<d.NH, 256, 0, s>>>(d, score, seg_start, seg_quota, n_seg, kept);
  return hipGetLastError();
}

}  // namespace kvc
