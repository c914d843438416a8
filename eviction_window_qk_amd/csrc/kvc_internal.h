// Internal declarations shared by the libkvc translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kUsageShift = 40;        // usage fixed point: trunc(ubar * 2^40)
constexpr int kCreditShift = 44;       // credit and mixed-mass fixed point (Q44)
constexpr int kMaxRows = 4096;         // W * G, and G * ceil(W/32) * 32
constexpr int kMaxT = 1 << 18;         // keep-mask bitmap fits one workgroup's LDS
constexpr int kMaxThresholds = 1024;   // mass cuts per head
constexpr int kScoreKeysPerWave = 64;  // two 32-key MFMA blocks per wave

// Parameters after validation, with every derived quantity the kernels need.
struct Derived {
  int NH, G, D, T, TS, W, K, R;
  int seg_min, seg_max, q_min;
  int sinks, recent;            // requested must-keep sizes
  int s_keep, r_keep, t_keep;   // S', R', budget left after must-keep (at length T)
  int pool_h, pool_mode, head_agg, ema, n_prev;
  int n_thr, s_cap;
  float c_log2;                 // softmax scale * log2(e)
  uint64_t eps_q;               // ceil(eps * 2^40)
  double delta, lam, oml, beta, omb;
  int rs_split;                 // key ranges the row-statistics pass is split into
  int seg_fixed;                // > 0: fixed-length raw segments (ablation)
  int quota_uniform;            // 1: every segment weighs 1 in the quotas (ablation)
  const int32_t* vlen;          // NULL or per-head valid length (device)
};

// A head-event's real tokens: positions [off, off + T) of the padded cache.
struct Span {
  int T, off;
};

__device__ __forceinline__ Span head_span(const Derived& P, int n) {
  if (!P.vlen) return Span{P.T, 0};
  int len = P.vlen[n];
  len = len < P.W ? P.W : (len > P.T ? P.T : len);
  return Span{len, P.T - len};
}

// Must-keep sizes and the budget left for the segments, for a cache of
// length T: sinks first, the recent suffix shrinks when the budget is short.
struct Keep {
  int s, r, t_keep;
};

__host__ __device__ __forceinline__ Keep must_keep(int sinks, int recent, int K, int T) {
  const int s = sinks < K ? (sinks < T ? sinks : T) : (K < T ? K : T);
  int r = recent;
  if (r > K - s) r = K - s;
  if (r > T - s) r = T - s;
  return Keep{s, r, K - s - r};
}

// Key ranges the row-statistics pass splits a head's keys into: whole 64-key
// tiles, about kRangeKeys keys each, for heads with more than 128 query rows
// (at most 128 rows stream K at the copy rate already and are not split).  The
// count depends only on the head's own length and row count, never on the
// launch, so a head's normalisers (and its usage) have the same bits whatever
// other heads share the launch; a launch sizes its partials for its longest
// head, and a shorter head leaves its later ranges empty (partial -inf, which
// adds nothing to the merge).  12 ranges at 131072 keys: with 256 heads of 512
// rows that is 6144 four-wave workgroups, eight rounds at three waves per SIMD
// on the 256 CUs of an MI355X (2, 3, 6 ranges measured slower; 18, 24 no
// faster).  The partial statistics are merged by a log-sum-exp pass.
constexpr int kRangeKeys = 172 * 64;
__host__ __device__ inline int score_pass1_splits(int R, int T) {
  if (R <= 128 || T <= kRangeKeys) return 1;
  int s = (T + kRangeKeys - 1) / kRangeKeys;
  s = s < 64 ? s : 64;
  const int span = ((T + s - 1) / s + 63) / 64 * 64;  // no range left empty
  return (T + span - 1) / span;
}

// Workspace carve-up (byte offsets into the caller's buffer, 256-B aligned).
struct WsLayout {
  size_t stats, stats_part, u, score, cupd, vp, seg_start, seg_quota, n_seg, seg_m, seg_a, seg_f,
      seg_q, total;
};
WsLayout workspace_layout(const Derived& d);

// Launchers (one per translation unit); return the first HIP error.
hipError_t launch_score(const Derived& d, const void* q, const void* k, float* u, float* stats,
                        float* stats_part, hipStream_t s);
hipError_t launch_mass_segment(const Derived& d, const float* u, const uint64_t* credit_in,
                               float* score, uint64_t* credit_upd, uint64_t* vp,
                               int32_t* seg_start, int32_t* seg_quota, int32_t* n_seg,
                               uint64_t* seg_m, int32_t* seg_a, int32_t* seg_f, int32_t* seg_q,
                               hipStream_t s);
hipError_t launch_select(const Derived& d, const float* score, const int32_t* seg_start,
                         const int32_t* seg_quota, const int32_t* n_seg, int32_t* kept,
                         hipStream_t s);
hipError_t launch_gather(const Derived& d, const int32_t* kept, const void* k, const void* v,
                         const uint64_t* credit_upd, void* k_out, void* v_out,
                         uint64_t* credit_out, hipStream_t s);
hipError_t launch_gather_paged(const Derived& d, const int32_t* kept, const void* k_pool,
                               const void* v_pool, const int32_t* table_in, int table_in_blocks,
                               const int32_t* table_out, int table_out_blocks, int kv_heads,
                               int block_size, int64_t n_blocks, void* k_pool_out,
                               void* v_pool_out, const uint64_t* credit_upd,
                               uint64_t* credit_out, hipStream_t s);

hipError_t launch_qc_trigger(int rows, int Hq, int d, const void* q, double* q_ref, double thr,
                             int update, int32_t* full, double* cos_out, hipStream_t s);
hipError_t launch_partial_init(int NH, int K, int T, const int32_t* kept, const float* score,
                               float* ps, int32_t* pp, hipStream_t s);
hipError_t launch_partial_append(int NH, int K, int d, float* ps, int32_t* pp, void* kp, void* vp,
                                 const void* kn, const void* vn, int t_new, int32_t* evicted,
                                 hipStream_t s);
hipError_t launch_full_sync(int NH, int K, int d, const int32_t* pp, const void* kp,
                            const void* vp, int t_from, int t_stride, void* kf, void* vf,
                            hipStream_t s);

}  // namespace kvc
