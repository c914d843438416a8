// libkvc host side: the C ABI of include/kvc.h.  Validates every argument,
// derives the quantities the kernels need (must-keep sizes, thresholds count,
// segment capacity, fixed-point eps), carves the caller's workspace and
// enqueues the kernels.  No allocation, no synchronisation, no global state.
#include <math.h>
#include <string.h>

#include "kvc_internal.h"

namespace kvc {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout workspace_layout(const Derived& d) {
  WsLayout L{};
  const size_t nh = size_t(d.NH), T = size_t(d.T), S = size_t(d.s_cap);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.stats = take(nh * size_t(d.R) * sizeof(float));  // row normalisers
  // per-key-range partial normalisers of a split row-statistics pass
  L.stats_part = take(d.rs_split > 1 ? nh * size_t(d.rs_split) * d.R * sizeof(float) : 0);
  L.u = take(nh * T * sizeof(float));
  L.score = take(nh * T * sizeof(float));
  L.cupd = take(d.ema ? nh * T * sizeof(uint64_t) : 0);
  L.vp = take(nh * T * sizeof(uint64_t));
  L.seg_start = take(nh * S * sizeof(int32_t));
  L.seg_quota = take(nh * S * sizeof(int32_t));
  L.n_seg = take(nh * sizeof(int32_t));
  L.seg_m = take(nh * S * sizeof(uint64_t));
  L.seg_a = take(nh * S * sizeof(int32_t));
  L.seg_f = take(nh * S * sizeof(int32_t));
  L.seg_q = take(nh * S * sizeof(int32_t));
  L.total = off;
  return L;
}

// Number of thresholds k*delta < 1 (k >= 1), evaluated exactly as the cuts
// are: (double)k * delta in fp64.  Returns -1 past the supported maximum.
static int count_thresholds(double delta) {
  int n = 0;
  for (int k = 1; double(k) * delta < 1.0; ++k) {
    if (++n > kMaxThresholds) return -1;
  }
  return n;
}

// Upper bound on the sum of the pooled usage of one head-event (see derive).
static int64_t usage_bound(int W, int G, int pool_kernel, int pool_mode) {
  const int64_t factor = pool_mode == KVC_POOL_MAX ? pool_kernel : 2;
  return factor * int64_t(W) * W * G;
}

static int derive(const kvc_params* p, Derived* d) {
  if (p == nullptr) return KVC_EINVAL;
  if (p->n_heads < 0) return KVC_EINVAL;
  if (p->head_dim != 64 && p->head_dim != 128) return KVC_EUNSUPPORTED;
  if (p->group < 1) return KVC_EINVAL;
  if (p->group > 64) return KVC_EUNSUPPORTED;
  if (p->T < 1 || p->T > kMaxT) return KVC_EINVAL;
  if (p->t_stride < p->T) return KVC_EINVAL;
  if (p->window < 1 || p->window > p->T) return KVC_EINVAL;
  const int64_t rows = int64_t(p->window) * p->group;
  if (rows > kMaxRows) return KVC_EINVAL;
  // Row slots padded per query head to whole 32-row MFMA blocks.
  if (int64_t(p->group) * ((p->window + 31) / 32) * 32 > kMaxRows) return KVC_EINVAL;
  // Fixed-point totals stay below 2^63: step 1's usage sums to at most W*W*G
  // (each of the W*G softmax rows sums to 1, plus W-1 filled positions of at
  // most W*G each), and pooling multiplies that sum by less than 2 (average:
  // each position weighs at most (2h+1)/(h+1) over its windows) or by at most
  // the width (max), so sum(ubar) <= pool_factor*W*W*G < 2^22.
  if (p->pool_kernel < 1 || p->pool_kernel > 63 || (p->pool_kernel & 1) == 0) return KVC_EINVAL;
  if (p->pool_mode != KVC_POOL_AVG && p->pool_mode != KVC_POOL_MAX) return KVC_EINVAL;
  if (usage_bound(p->window, p->group, p->pool_kernel, p->pool_mode) >= (int64_t(1) << 22))
    return KVC_EINVAL;
  if (p->budget < 1) return KVC_EINVAL;
  if (!(p->delta > 0.0) || !isfinite(p->delta)) return KVC_EINVAL;
  const int n_thr = count_thresholds(p->delta);
  if (n_thr < 0) return KVC_EINVAL;
  if (p->seg_min < 1 || p->seg_max < 0) return KVC_EINVAL;
  if (p->q_min < 0 || p->sinks < 0 || p->recent < 0) return KVC_EINVAL;
  if (p->head_agg != KVC_AGG_SUM && p->head_agg != KVC_AGG_MAX) return KVC_EINVAL;
  if (p->ema != 0 && p->ema != 1) return KVC_EINVAL;
  if (!(p->lambda >= 0.0 && p->lambda <= 1.0)) return KVC_EINVAL;
  if (!(p->beta >= 0.0 && p->beta <= 1.0)) return KVC_EINVAL;
  if (!(p->eps > 0.0 && p->eps <= 1.0)) return KVC_EINVAL;
  if (p->n_prev < 0 || p->n_prev > p->T) return KVC_EINVAL;
  if (!p->ema && p->n_prev != 0) return KVC_EINVAL;
  if (!(p->scale >= 0.0f) || !isfinite(p->scale)) return KVC_EINVAL;
  if (p->seg_fixed < 0) return KVC_EINVAL;
  if (p->seg_fixed > 0 && (int64_t(p->T) + p->seg_fixed - 1) / p->seg_fixed > kMaxThresholds + 1)
    return KVC_EINVAL;
  if (p->quota_mode != KVC_QUOTA_MASS && p->quota_mode != KVC_QUOTA_UNIFORM) return KVC_EINVAL;
  if (p->valid_len && (reinterpret_cast<uintptr_t>(p->valid_len) & 3u)) return KVC_EINVAL;
  // Element counts must stay addressable.
  const double elems = double(p->n_heads) * double(p->t_stride) * double(p->head_dim);
  if (elems > 9.0e15) return KVC_EINVAL;

  d->NH = p->n_heads;
  d->G = p->group;
  d->D = p->head_dim;
  d->T = p->T;
  d->TS = p->t_stride;
  d->W = p->window;
  d->K = p->budget;
  d->R = int(rows);
  d->seg_min = p->seg_min;
  d->seg_max = p->seg_max;
  d->q_min = p->q_min;
  d->sinks = p->sinks;
  d->recent = p->recent;
  const Keep mk = must_keep(p->sinks, p->recent, p->budget, p->T);
  d->s_keep = mk.s;
  d->r_keep = mk.r;
  d->t_keep = mk.t_keep;
  d->pool_h = p->pool_kernel / 2;
  d->pool_mode = p->pool_mode;
  d->head_agg = p->head_agg;
  d->ema = p->ema;
  d->n_prev = p->n_prev;
  // Raw cuts before merging: mass thresholds, or every seg_fixed positions.
  const int n_cut =
      p->seg_fixed > 0 ? int((int64_t(p->T) + p->seg_fixed - 1) / p->seg_fixed) - 1 : n_thr;
  d->n_thr = n_cut;
  d->seg_fixed = p->seg_fixed;
  d->rs_split = score_pass1_splits(d->R, d->T);  // sized for the longest head
  d->quota_uniform = p->quota_mode == KVC_QUOTA_UNIFORM ? 1 : 0;
  d->vlen = p->valid_len;
  int64_t cap = int64_t(n_cut) + 1 + (p->seg_max > 0 ? p->T / p->seg_max : 0);
  if (cap > p->T) cap = p->T;
  if (cap < 1) cap = 1;
  d->s_cap = int(cap);
  const double scale = p->scale != 0.0f ? double(p->scale) : 1.0 / sqrt(double(p->head_dim));
  d->c_log2 = float(scale * 1.4426950408889634);  // scale * log2(e)
  if (!(d->c_log2 >= 0x1p-60f)) return KVC_EINVAL;  // scores below 2^-60 of a dot product: rejected
  d->eps_q = uint64_t(ceil(p->eps * 1099511627776.0));  // ceil(eps * 2^40)
  d->delta = p->delta;
  d->lam = p->lambda;
  d->oml = 1.0 - p->lambda;
  d->beta = p->beta;
  d->omb = 1.0 - p->beta;
  return KVC_OK;
}

struct Range {
  const void* p;
  size_t n;
};

static bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = uintptr_t(a.p), b0 = uintptr_t(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Every output must be disjoint from every input and from every other output.
static bool any_alias(const Range* in, int n_in, const Range* out, int n_out) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(out[i], in[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j])) return true;
  }
  return false;
}

static bool aligned(const void* p, size_t a) { return (uintptr_t(p) & (a - 1)) == 0; }

static int launch_status(hipError_t e) {
  if (e != hipSuccess) return KVC_EDEVICE;
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EDEVICE;
}

}  // namespace kvc

using namespace kvc;

extern "C" {

int kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_strerror(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_NOOP: return "no eviction needed: T <= budget (identity copy enqueued)";
    case KVC_EINVAL: return "invalid argument: shape or parameter out of range, NULL pointer, or aliasing outputs";
    case KVC_EALIGN: return "misaligned pointer: bf16 tensors need 16-byte alignment";
    case KVC_EWORKSPACE: return "workspace missing or smaller than kvc_workspace_bytes()";
    case KVC_EUNSUPPORTED: return "unsupported variant: head_dim must be 64 or 128 and group <= 64";
    case KVC_EDEVICE: return "HIP runtime reported a launch error";
    case KVC_ESCRATCH: return "event needs more scratch than kvc_compress_event_noalloc holds (KVC_NOALLOC_SCRATCH_BYTES); use kvc_compress_event with a workspace";
    default: return "unknown status";
  }
}

int kvc_check_params(const kvc_params* p) {
  Derived d;
  return derive(p, &d);
}

size_t kvc_workspace_bytes(const kvc_params* p) {
  Derived d;
  if (derive(p, &d) != KVC_OK) return 0;
  return workspace_layout(d).total;
}

int kvc_segment_capacity(const kvc_params* p) {
  Derived d;
  const int rc = derive(p, &d);
  return rc != KVC_OK ? rc : d.s_cap;
}

int kvc_score_window(const kvc_params* p, const void* q_win, const void* k, float* u, void* ws,
                     size_t ws_bytes, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!q_win || !k || !u) return KVC_EINVAL;
  if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(u, 4)) return KVC_EALIGN;
  const WsLayout L = workspace_layout(d);
  if (!ws || ws_bytes < L.total) return KVC_EWORKSPACE;
  if (!aligned(ws, 256)) return KVC_EALIGN;
  const size_t nh = size_t(d.NH);
  const Range in[] = {{q_win, nh * d.R * d.D * 2}, {k, nh * d.TS * d.D * 2}};
  const Range out[] = {{u, nh * d.T * 4}, {ws, ws_bytes}};
  if (any_alias(in, 2, out, 2)) return KVC_EINVAL;
  char* w = static_cast<char*>(ws);
  return launch_status(launch_score(d, q_win, k, u, reinterpret_cast<float*>(w + L.stats),
                                    reinterpret_cast<float*>(w + L.stats_part),
                                    hipStream_t(stream)));
}

int kvc_mass_segment(const kvc_params* p, const float* u, const uint64_t* credit_in, float* score,
                     uint64_t* credit_upd, int32_t* seg_start, int32_t* seg_quota, int32_t* n_seg,
                     void* ws, size_t ws_bytes, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!u || !score || !seg_start || !seg_quota || !n_seg) return KVC_EINVAL;
  if (d.ema && !credit_upd) return KVC_EINVAL;
  if (d.n_prev > 0 && !credit_in) return KVC_EINVAL;
  if (!aligned(u, 4) || !aligned(score, 4) || !aligned(seg_start, 4) || !aligned(seg_quota, 4) ||
      !aligned(n_seg, 4) || (credit_in && !aligned(credit_in, 8)) ||
      (credit_upd && !aligned(credit_upd, 8)))
    return KVC_EALIGN;
  const WsLayout L = workspace_layout(d);
  if (!ws || ws_bytes < L.total) return KVC_EWORKSPACE;
  if (!aligned(ws, 256)) return KVC_EALIGN;
  const size_t nh = size_t(d.NH), T = size_t(d.T), S = size_t(d.s_cap);
  const Range in[] = {{u, nh * T * 4}, {credit_in, nh * size_t(d.n_prev) * 8}};
  const Range out[] = {{score, nh * T * 4},
                       {d.ema ? credit_upd : nullptr, nh * T * 8},
                       {seg_start, nh * S * 4},
                       {seg_quota, nh * S * 4},
                       {n_seg, nh * 4},
                       {ws, ws_bytes}};
  if (any_alias(in, 2, out, 6)) return KVC_EINVAL;
  char* w = static_cast<char*>(ws);
  rc = launch_status(launch_mass_segment(
      d, u, credit_in, score, d.ema ? credit_upd : nullptr, reinterpret_cast<uint64_t*>(w + L.vp),
      seg_start, seg_quota, n_seg, reinterpret_cast<uint64_t*>(w + L.seg_m),
      reinterpret_cast<int32_t*>(w + L.seg_a), reinterpret_cast<int32_t*>(w + L.seg_f),
      reinterpret_cast<int32_t*>(w + L.seg_q), hipStream_t(stream)));
  if (rc != KVC_OK) return rc;
  return (d.T <= d.K && !d.vlen) ? KVC_NOOP : KVC_OK;
}

int kvc_select(const kvc_params* p, const float* score, const int32_t* seg_start,
               const int32_t* seg_quota, const int32_t* n_seg, int32_t* kept, void* ws,
               size_t ws_bytes, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!score || !seg_start || !seg_quota || !n_seg || !kept) return KVC_EINVAL;
  if (!aligned(score, 4) || !aligned(seg_start, 4) || !aligned(seg_quota, 4) ||
      !aligned(n_seg, 4) || !aligned(kept, 4))
    return KVC_EALIGN;
  const WsLayout L = workspace_layout(d);
  if (!ws || ws_bytes < L.total) return KVC_EWORKSPACE;
  const size_t nh = size_t(d.NH), T = size_t(d.T), S = size_t(d.s_cap);
  const Range in[] = {{score, nh * T * 4}, {seg_start, nh * S * 4}, {seg_quota, nh * S * 4},
                      {n_seg, nh * 4}};
  const Range out[] = {{kept, nh * size_t(d.K) * 4}};
  if (any_alias(in, 4, out, 1)) return KVC_EINVAL;
  rc = launch_status(launch_select(d, score, seg_start, seg_quota, n_seg, kept,
                                   hipStream_t(stream)));
  if (rc != KVC_OK) return rc;
  return (d.T <= d.K && !d.vlen) ? KVC_NOOP : KVC_OK;
}

int kvc_gather_compact(const kvc_params* p, const int32_t* kept, const void* k, const void* v,
                       const uint64_t* credit_upd, void* k_out, void* v_out, uint64_t* credit_out,
                       void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!kept || !k || !v || !k_out || !v_out) return KVC_EINVAL;
  if ((credit_upd == nullptr) != (credit_out == nullptr)) return KVC_EINVAL;
  if (!aligned(kept, 4) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || (credit_upd && !aligned(credit_upd, 8)) ||
      (credit_out && !aligned(credit_out, 8)))
    return KVC_EALIGN;
  const size_t nh = size_t(d.NH), K = size_t(d.K);
  const size_t kv_in = nh * size_t(d.TS) * d.D * 2, kv_out = nh * K * d.D * 2;
  const Range in[] = {{kept, nh * K * 4}, {k, kv_in}, {v, kv_in}, {credit_upd, nh * d.T * 8}};
  const Range out[] = {{k_out, kv_out}, {v_out, kv_out}, {credit_out, nh * K * 8}};
  if (any_alias(in, 4, out, 3)) return KVC_EINVAL;
  return launch_status(
      launch_gather(d, kept, k, v, credit_upd, k_out, v_out, credit_out, hipStream_t(stream)));
}

int kvc_gather_paged(const kvc_params* p, int32_t kv_heads, int32_t block_size, int64_t n_blocks,
                     const int32_t* kept, const void* k_pool, const void* v_pool,
                     const int32_t* table_in, int32_t table_in_blocks, const int32_t* table_out,
                     int32_t table_out_blocks, void* k_pool_out, void* v_pool_out,
                     const uint64_t* credit_upd, uint64_t* credit_out, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (kv_heads < 1 || d.NH % kv_heads != 0 || block_size < 1 || n_blocks < 1) return KVC_EINVAL;
  if (int64_t(table_in_blocks) * block_size < d.T) return KVC_EINVAL;
  if (int64_t(table_out_blocks) * block_size < d.K) return KVC_EINVAL;
  if (!kept || !k_pool || !v_pool || !table_in || !table_out || !k_pool_out || !v_pool_out)
    return KVC_EINVAL;
  if ((credit_upd == nullptr) != (credit_out == nullptr)) return KVC_EINVAL;
  if (!aligned(kept, 4) || !aligned(table_in, 4) || !aligned(table_out, 4) ||
      !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_pool_out, 16) ||
      !aligned(v_pool_out, 16) || (credit_upd && !aligned(credit_upd, 8)) ||
      (credit_out && !aligned(credit_out, 8)))
    return KVC_EALIGN;
  const double pool_elems = double(n_blocks) * kv_heads * block_size * d.D;
  if (pool_elems > 9.0e15) return KVC_EINVAL;
  const size_t nh = size_t(d.NH), K = size_t(d.K), B = nh / size_t(kv_heads);
  const size_t pool = size_t(n_blocks) * size_t(kv_heads) * size_t(block_size) * d.D * 2;
  // The destination pools may be the source pools (new blocks of the same
  // allocation); the index arrays and credit must not overlap any pool.
  const Range in[] = {{kept, nh * K * 4},
                      {table_in, B * size_t(table_in_blocks) * 4},
                      {table_out, B * size_t(table_out_blocks) * 4},
                      {credit_upd, nh * d.T * 8}};
  const Range out[] = {{k_pool_out, pool}, {v_pool_out, pool}, {credit_out, nh * K * 8}};
  if (any_alias(in, 4, out, 3)) return KVC_EINVAL;
  const Range kv_in[] = {{k_pool, pool}, {v_pool, pool}};
  const Range cred_out[] = {{credit_out, nh * K * 8}};
  if (any_alias(kv_in, 2, cred_out, 1)) return KVC_EINVAL;
  if (k_pool_out == v_pool_out) return KVC_EINVAL;
  return launch_status(launch_gather_paged(
      d, kept, k_pool, v_pool, table_in, table_in_blocks, table_out, table_out_blocks, kv_heads,
      block_size, n_blocks, k_pool_out, v_pool_out, credit_upd, credit_out, hipStream_t(stream)));
}

int kvc_qc_trigger(int32_t rows, int32_t heads_q, int32_t head_dim, const void* q, double* q_ref,
                   double threshold, int32_t update_ref, int32_t* full, double* cos_out,
                   void* stream) {
  if (rows < 0 || heads_q < 1 || heads_q > 4096 || (head_dim != 64 && head_dim != 128))
    return KVC_EINVAL;
  if (!std::isfinite(threshold)) return KVC_EINVAL;
  if (rows == 0) return KVC_OK;
  if (!q || !q_ref || !full) return KVC_EINVAL;
  if (!aligned(q, 2) || !aligned(q_ref, 8) || !aligned(full, 4) || (cos_out && !aligned(cos_out, 8)))
    return KVC_EALIGN;
  const size_t r = size_t(rows);
  const Range in[] = {{q, r * heads_q * head_dim * 2}};
  const Range out[] = {{q_ref, r * head_dim * 8}, {full, r * 4}, {cos_out, r * 8}};
  if (any_alias(in, 1, out, 3)) return KVC_EINVAL;
  return launch_status(launch_qc_trigger(rows, heads_q, head_dim, q, q_ref, threshold,
                                         update_ref != 0, full, cos_out, hipStream_t(stream)));
}

int kvc_partial_init(const kvc_params* p, const int32_t* kept, const float* score,
                     float* part_score, int32_t* part_pos, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!kept || !score || !part_score || !part_pos) return KVC_EINVAL;
  if (!aligned(kept, 4) || !aligned(score, 4) || !aligned(part_score, 4) || !aligned(part_pos, 4))
    return KVC_EALIGN;
  const size_t nh = size_t(d.NH), K = size_t(d.K);
  const Range in[] = {{kept, nh * K * 4}, {score, nh * size_t(d.T) * 4}};
  const Range out[] = {{part_score, nh * K * 4}, {part_pos, nh * K * 4}};
  if (any_alias(in, 2, out, 2)) return KVC_EINVAL;
  return launch_status(launch_partial_init(d.NH, d.K, d.T, kept, score, part_score, part_pos,
                                           hipStream_t(stream)));
}

int kvc_partial_append(int32_t n_heads, int32_t K, int32_t head_dim, float* part_score,
                       int32_t* part_pos, void* k_part, void* v_part, const void* k_new,
                       const void* v_new, int32_t t_new, int32_t* evicted, void* stream) {
  if (n_heads < 0 || K < 1 || (head_dim != 64 && head_dim != 128) || t_new < 0) return KVC_EINVAL;
  if (n_heads == 0) return KVC_OK;
  if (!part_score || !part_pos || !k_part || !v_part || !k_new || !v_new || !evicted)
    return KVC_EINVAL;
  if (!aligned(part_score, 4) || !aligned(part_pos, 4) || !aligned(evicted, 4) ||
      !aligned(k_part, 16) || !aligned(v_part, 16) || !aligned(k_new, 16) || !aligned(v_new, 16))
    return KVC_EALIGN;
  const size_t nh = size_t(n_heads), kk = size_t(K), row = size_t(head_dim) * 2;
  const Range in[] = {{k_new, nh * row}, {v_new, nh * row}};
  const Range out[] = {{part_score, nh * kk * 4}, {part_pos, nh * kk * 4}, {k_part, nh * kk * row},
                       {v_part, nh * kk * row}, {evicted, nh * 4}};
  if (any_alias(in, 2, out, 5)) return KVC_EINVAL;
  return launch_status(launch_partial_append(n_heads, K, head_dim, part_score, part_pos, k_part,
                                             v_part, k_new, v_new, t_new, evicted,
                                             hipStream_t(stream)));
}

int kvc_full_sync(int32_t n_heads, int32_t K, int32_t head_dim, const int32_t* part_pos,
                  const void* k_part, const void* v_part, int32_t t_from, int32_t t_stride,
                  void* k_full, void* v_full, void* stream) {
  if (n_heads < 0 || K < 1 || (head_dim != 64 && head_dim != 128) || t_from < 0 || t_stride < 1)
    return KVC_EINVAL;
  if (n_heads == 0) return KVC_OK;
  if (!part_pos || !k_part || !v_part || !k_full || !v_full) return KVC_EINVAL;
  if (!aligned(part_pos, 4) || !aligned(k_part, 16) || !aligned(v_part, 16) ||
      !aligned(k_full, 16) || !aligned(v_full, 16))
    return KVC_EALIGN;
  const size_t nh = size_t(n_heads), row = size_t(head_dim) * 2;
  const Range in[] = {{part_pos, nh * size_t(K) * 4}, {k_part, nh * size_t(K) * row},
                      {v_part, nh * size_t(K) * row}};
  const Range out[] = {{k_full, nh * size_t(t_stride) * row}, {v_full, nh * size_t(t_stride) * row}};
  if (any_alias(in, 3, out, 2)) return KVC_EINVAL;
  return launch_status(launch_full_sync(n_heads, K, head_dim, part_pos, k_part, v_part, t_from,
                                        t_stride, k_full, v_full, hipStream_t(stream)));
}

int kvc_compress_event(const kvc_params* p, const void* q_win, const void* k, const void* v,
                       const uint64_t* credit_in, void* k_out, void* v_out, uint64_t* credit_out,
                       int32_t* kept_out, float* u_out, void* ws, size_t ws_bytes, void* stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != KVC_OK) return rc;
  if (d.NH == 0) return KVC_OK;
  if (!q_win || !k || !v || !k_out || !v_out || !kept_out) return KVC_EINVAL;
  if (d.ema && !credit_out) return KVC_EINVAL;
  if (d.n_prev > 0 && !credit_in) return KVC_EINVAL;
  if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || !aligned(kept_out, 4) || (u_out && !aligned(u_out, 4)) ||
      (credit_in && !aligned(credit_in, 8)) || (credit_out && !aligned(credit_out, 8)))
    return KVC_EALIGN;
  const WsLayout L = workspace_layout(d);
  if (!ws || ws_bytes < L.total) return KVC_EWORKSPACE;
  if (!aligned(ws, 256)) return KVC_EALIGN;
  const size_t nh = size_t(d.NH), T = size_t(d.T), K = size_t(d.K);
  const size_t kv_in = nh * size_t(d.TS) * d.D * 2, kv_out = nh * K * d.D * 2;
  const Range in[] = {{q_win, nh * d.R * d.D * 2},
                      {k, kv_in},
                      {v, kv_in},
                      {credit_in, nh * size_t(d.n_prev) * 8}};
  const Range out[] = {{k_out, kv_out},
                       {v_out, kv_out},
                       {d.ema ? credit_out : nullptr, nh * K * 8},
                       {kept_out, nh * K * 4},
                       {u_out, nh * T * 4},
                       {ws, ws_bytes}};
  if (any_alias(in, 4, out, 6)) return KVC_EINVAL;

  char* w = static_cast<char*>(ws);
  hipStream_t s = hipStream_t(stream);
  float* u = u_out ? u_out : reinterpret_cast<float*>(w + L.u);
  float* score = reinterpret_cast<float*>(w + L.score);
  uint64_t* cupd = d.ema ? reinterpret_cast<uint64_t*>(w + L.cupd) : nullptr;
  int32_t* seg_start = reinterpret_cast<int32_t*>(w + L.seg_start);
  int32_t* seg_quota = reinterpret_cast<int32_t*>(w + L.seg_quota);
  int32_t* n_seg = reinterpret_cast<int32_t*>(w + L.n_seg);

  rc = launch_status(launch_score(d, q_win, k, u, reinterpret_cast<float*>(w + L.stats),
                                  reinterpret_cast<float*>(w + L.stats_part), s));
  if (rc != KVC_OK) return rc;
  rc = launch_status(launch_mass_segment(
      d, u, credit_in, score, cupd, reinterpret_cast<uint64_t*>(w + L.vp), seg_start, seg_quota,
      n_seg, reinterpret_cast<uint64_t*>(w + L.seg_m), reinterpret_cast<int32_t*>(w + L.seg_a),
      reinterpret_cast<int32_t*>(w + L.seg_f), reinterpret_cast<int32_t*>(w + L.seg_q), s));
  if (rc != KVC_OK) return rc;
  rc = launch_status(launch_select(d, score, seg_start, seg_quota, n_seg, kept_out, s));
  if (rc != KVC_OK) return rc;
  rc = launch_status(launch_gather(d, kept_out, k, v, cupd, k_out, v_out,
                                   d.ema ? credit_out : nullptr, s));
  if (rc != KVC_OK) return rc;
  return (d.T <= d.K && !d.vlen) ? KVC_NOOP : KVC_OK;
}

}  // extern "C"
