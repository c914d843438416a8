/*
 * kvc.h -- C ABI of libkvc: the decode-time KV-cache compression event
 * (adaptive mass-segmented selection) on AMD MI355X (gfx950).
 *
 * Sources.  The operation is the event described in the notes on
 * "Adaptive Mass-Segmented KV Compression for Long-Form Reasoning" (AMS):
 * section 整体框架 (overall framework) says selection runs independently for
 * every layer and KV head on the current cache and yields a compact cache of
 * the target budget; 关键设计 1-4 (key designs 1-4) give the mass, the
 * cumulative-mass cuts, the segment quotas and the in-segment selection with
 * gather-and-compact.  The one-segment special case is the max-pooled global
 * top-K of the notes on "RefreshKV: Updating Small KV Cache During Long-form
 * Generation" (A2 method details, prefill stage; A6 appendix, baselines).
 *
 * Conventions shared by every entry point.
 *  - One call covers n_heads independent head-events (layer x batch x KV
 *    head).  Head n's data is the n-th slab of every array.
 *  - Every pointer except `params` and the returned strings is a DEVICE
 *    pointer owned by the caller.  The library allocates no memory, keeps no
 *    state between calls and never synchronises: all work is enqueued on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream) and
 *    completes asynchronously.  Results are deterministic: the same inputs
 *    give the same bits on every run, and a head's results do not depend on
 *    the other heads of the call (a head alone, with T set to its real
 *    length, gives the bits it gets inside a left-padded batch).
 *  - All arguments are validated on the host before anything is enqueued; on
 *    an error return nothing has been launched and no output was touched.
 *  - A call enqueues kernel launches only (no memset, copy or allocation), so
 *    it can be captured into a HIP graph and replayed with new inputs copied
 *    into the captured buffers.
 *  - Return values: KVC_OK (0), KVC_NOOP (1, informational: T <= budget, so
 *    nothing is evicted), negative = error (see kvc_strerror).
 *  - bf16 tensors are raw IEEE bfloat16; q, k, v, k_out, v_out must be
 *    16-byte aligned; fp32/u64/i32 arrays need their natural alignment.
 *  - Outputs may not overlap inputs (KVC_EINVAL).
 *  - Calls that share a workspace or outputs must be ordered on one stream.
 *  - Precondition (not checked): q and k are finite.
 *
 * Array layouts (row-major, innermost last; NH = n_heads, G = group,
 * W = window, d = head_dim, S = kvc_segment_capacity(p)):
 *   q_win      bf16 [NH][G][W][d]     last W queries of the G query heads
 *                                      that share each KV head (post-RoPE);
 *                                      window query w sits at position T-W+w
 *   k, v       bf16 [NH][t_stride][d] cached keys/values, rows >= T unused
 *   u          f32  [NH][T]            window usage (step 1 output)
 *   score      f32  [NH][T]            pooled usage, the base score
 *   credit_in  u64  [NH][n_prev]       carried EMA credit, Q44 fixed point
 *   credit_upd u64  [NH][T]            updated credit per position, Q44
 *   seg_start  i32  [NH][S]            first position of each segment
 *   seg_quota  i32  [NH][S]            positions to pick in each segment
 *   n_seg      i32  [NH]               segments used per head
 *   kept       i32  [NH][budget]       kept positions, ascending; -1 pads the
 *                                      tail only when T < budget
 *   k_out,v_out bf16 [NH][budget][d]   compacted cache (zero rows past T)
 *   credit_out u64  [NH][budget]       credit of the kept positions
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 3

enum kvc_status {
  KVC_OK = 0,
  KVC_NOOP = 1,           /* T <= budget: kept = 0..T-1, identity copy      */
  KVC_EINVAL = -1,        /* a shape or parameter is out of range, a
                             required pointer is NULL, or outputs alias
                             inputs                                          */
  KVC_EALIGN = -2,        /* a pointer is not aligned as required           */
  KVC_EWORKSPACE = -3,    /* ws is NULL or ws_bytes < kvc_workspace_bytes() */
  KVC_EUNSUPPORTED = -4,  /* head_dim or group outside the built variants   */
  KVC_EDEVICE = -5,       /* the HIP runtime reported a launch error        */
  KVC_ESCRATCH = -6       /* kvc_compress_event_noalloc: the event needs more
                             scratch than KVC_NOALLOC_SCRATCH_BYTES          */
};

/* Scratch held on each GPU by kvc_compress_event_noalloc (64 MiB). */
#define KVC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum { KVC_POOL_AVG = 0, KVC_POOL_MAX = 1 };
enum { KVC_AGG_SUM = 0, KVC_AGG_MAX = 1 };
enum { KVC_QUOTA_MASS = 0, KVC_QUOTA_UNIFORM = 1 };

/* Event parameters, named after the pages' quantities.  Field order fixes the
 * layout: 17 int32, one float, four doubles, two int32, then one pointer
 * (120 bytes, no padding). */
typedef struct kvc_params {
  int32_t n_heads;     /* NH independent head-events; 0 = nothing to do      */
  int32_t group;       /* G query heads per KV head, 1..64                   */
  int32_t head_dim;    /* d, 64 or 128                                       */
  int32_t T;           /* valid cached positions per head, 1..2^18           */
  int32_t t_stride;    /* rows allocated per head in k/v (>= T)              */
  int32_t window;      /* W recent queries, 1..T; W*G <= 4096 and
                          G*ceil(W/32)*32 <= 4096 (32-row MFMA blocks per
                          query head); F*W*W*G < 2^22 with F = 2 for
                          average pooling and F = pool_kernel for max
                          pooling keeps the fixed-point usage totals below
                          2^63 (step 1's usage sums to at most W*W*G per
                          head, and pooling multiplies that by < F)        */
  int32_t budget;      /* K positions kept per head, >= 1                    */
  int32_t seg_min;     /* shortest segment after merging (>= 1), e.g. 16     */
  int32_t seg_max;     /* longest segment after splitting, e.g. 256; 0 = none*/
  int32_t q_min;       /* per-segment minimum quota (>= 0), e.g. 1           */
  int32_t sinks;       /* leading must-keep positions (>= 0), e.g. 4         */
  int32_t recent;      /* trailing must-keep positions (>= 0), e.g. 64       */
  int32_t pool_kernel; /* odd pooling width 1..63, e.g. 7                    */
  int32_t pool_mode;   /* KVC_POOL_AVG (AMS) or KVC_POOL_MAX (SnapKV-style)  */
  int32_t head_agg;    /* KVC_AGG_SUM or KVC_AGG_MAX over the G query heads  */
  int32_t ema;         /* 1 = EMA credit on, 0 = off                         */
  int32_t n_prev;      /* credit entries carried per head (0..T; 0 if !ema)  */
  float scale;         /* softmax scale; 0 => 1/sqrt(head_dim); otherwise
                          finite with scale*log2(e) >= 2^-60                 */
  double delta;        /* target segment mass Delta in (0, inf); >= 1 => no
                          mass cuts; at most 1024 thresholds                 */
  double lambda;       /* EMA decay, [0,1], e.g. 0.9                          */
  double beta;         /* weight of the current mass, [0,1], e.g. 0.9        */
  double eps;          /* mass floor epsilon, (0, 1], e.g. 1e-6              */
  int32_t seg_fixed;   /* 0 = cuts from the cumulative mass (the method);
                          L > 0 = ablation "fixed-length segments" [AMS
                          notes, ablations, Table 7]: raw segments of L
                          positions (the last one shorter), then merge and
                          split as usual; ceil(T/L) <= 1025              */
  int32_t quota_mode;  /* KVC_QUOTA_MASS (the method) or KVC_QUOTA_UNIFORM:
                          ablation "no mass-weighted quota" [same table]:
                          every segment weighs 1 in the share of the
                          remainder and in the redistribution order      */
  const int32_t* valid_len; /* NULL, or a DEVICE array [n_heads] for ragged
                          (left-padded) batches [SkipKV notes, observation 1
                          and §4.1, attention mask M]: head n holds padding
                          at positions [0, T-len) and real tokens at
                          [T-len, T), len = valid_len[n] clamped to [W, T].
                          The event runs on the real tokens only, exactly
                          as on a cache of length len: u, score and
                          credit_upd are 0 on the padding, seg_start and
                          kept are positions of the padded cache, kept
                          holds min(budget, len) positions, and
                          credit_in[n][j] is the credit of position
                          T-len+j (j < min(n_prev, len)).  With valid_len
                          set, KVC_NOOP is never returned: a head with
                          len <= budget gets its identity copy and the
                          call returns KVC_OK.                            */
} kvc_params;

/* Step 1: window score [AMS notes, key design 1: usage of the most recent W
 * queries per cached position, partly observed suffix filled with the window
 * maximum; SkipKV notes §4.1: softmax(QK^T/sqrt(d)) over an observation window
 * with GQA head mapping].
 * u[n][t] = AGG_g sum_{w : T-W+w >= t} softmax_t'(scale*<q[n][g][w], k[n][t']>)
 * over t' <= T-W+w (AGG = sum or max over g of the per-head sums), then
 * u[n][t] = max_{t' <= T-W} u[n][t'] for t > T-W.  fp32 output; bf16 matrix
 * products with fp32 accumulation, fp32 softmax.
 * ws: at least kvc_workspace_bytes(p). */
int kvc_score_window(const kvc_params* p, const void* q_win, const void* k, float* u,
                     void* ws, size_t ws_bytes, void* stream);

/* Step 2 + step 3: mass, prefix and segmentation with quotas [AMS notes, key
 * design 1 (mass eq. m_i = (max(u_i,0)+eps)/sum, EMA eq.), key design 2 (C(t),
 * b_k = min{t : C(t) >= k*Delta}, split/merge to seg_min/seg_max), key
 * design 3 (must-keep sinks + recent suffix, q_i^min = min(q_min, L_i),
 * remainder split by segment mass with rounding, clip and redistribute)].
 * score[n][t] = pooled u (avg or max over pool_kernel in-range neighbours).
 * With ema: credit_in (may be NULL only when n_prev == 0) is the carried
 * credit of positions 0..n_prev-1; credit_upd receives the updated credit of
 * every position (required when ema, ignored otherwise).
 * Outputs seg_start/seg_quota/n_seg as laid out above.  Integer decisions
 * follow an exact fixed-point contract, bit-identical to a sequential
 * evaluation.  Returns KVC_NOOP (n_seg = 0) when T <= budget.
 * Precondition on u (not checked: it lives on the device): finite,
 * non-negative values whose pooled sum per head is at most F*W*W*G (the bound
 * on `window` above) -- which every u written by kvc_score_window satisfies.
 * Out-of-range values are clamped to [0, 2^23] (NaN to 0) before the
 * fixed-point conversion, so any input gives a valid partition, quotas that
 * respect the segment lengths and in-range indices; but a pooled sum past
 * 2^23 wraps the 64-bit fixed-point totals and the cuts and quotas are then
 * not the method's. */
int kvc_mass_segment(const kvc_params* p, const float* u, const uint64_t* credit_in,
                     float* score, uint64_t* credit_upd, int32_t* seg_start,
                     int32_t* seg_quota, int32_t* n_seg, void* ws, size_t ws_bytes,
                     void* stream);

/* Step 4: select [AMS notes, key design 3, last paragraph: union with the
 * must-keep set counting duplicates once, over budget drop low-score picks,
 * under budget add high-score unselected positions; key design 4: per-segment
 * top-k on a base score of shape [B,Hkv,T], kept indices sorted].
 * score: any finite fp32 base score (the pooled usage by default).  In each
 * segment the min(quota, candidates) non-must-keep positions with the largest
 * score are picked, ties to the lower position; the result always holds
 * min(budget, T) positions in ascending order.  Returns KVC_NOOP (kept =
 * 0..T-1, -1 padded) when T <= budget. */
int kvc_select(const kvc_params* p, const float* score, const int32_t* seg_start,
               const int32_t* seg_quota, const int32_t* n_seg, int32_t* kept, void* ws,
               size_t ws_bytes, void* stream);

/* Step 5: gather-and-compact [AMS notes, key design 4: the same kept indices
 * gather K and V into a fixed-length per-head cache; key design 1, last
 * paragraph: the credit follows the kept positions].
 * k_out[n][j] = k[n][kept[n][j]], v_out likewise, credit_out[n][j] =
 * credit_upd[n][kept[n][j]] (both credit pointers NULL, or both set); rows
 * with kept = -1 are zero-filled.  Bitwise copies; no workspace. */
int kvc_gather_compact(const kvc_params* p, const int32_t* kept, const void* k, const void* v,
                       const uint64_t* credit_upd, void* k_out, void* v_out,
                       uint64_t* credit_out, void* stream);

/* Step 5 on a paged cache [AMS notes, key design 4, appendix E paragraph:
 * the runtime allocates new blocks, copies each head's KV from its kept
 * original positions into the new physical slots, swaps the request's block
 * table and frees the old blocks; one compacted slot may hold KV from
 * different original positions in different heads].
 * Pools: k_pool, v_pool (source) and k_pool_out, v_pool_out (destination,
 * may be the same allocations) are bf16 [n_blocks][kv_heads][block_size][d].
 * Head n = b * kv_heads + h (n_heads = B * kv_heads); logical position t of
 * sequence b lives in block table_in[b][t / block_size], slot t % block_size
 * (table_in is i32 [B][table_in_blocks], table_in_blocks >= ceil(T /
 * block_size)).  Slot j of the compacted cache goes to block
 * table_out[b][j / block_size], slot j % block_size (i32 [B][table_out_blocks],
 * table_out_blocks >= ceil(budget / block_size)): for head h it receives the
 * row of position kept[n][j], or zeros where kept is -1.  Blocks named in
 * table_out must not appear in table_in (the copy reads old blocks while
 * writing new ones); no other block is written.  Block ids outside
 * [0, n_blocks) are never dereferenced (the destination row is skipped, a bad
 * source reads as zeros).  credit_upd/credit_out are optional and as in
 * kvc_gather_compact.  Swapping the tables and freeing the old blocks are the
 * caller's; nothing here allocates. */
int kvc_gather_paged(const kvc_params* p, int32_t kv_heads, int32_t block_size, int64_t n_blocks,
                     const int32_t* kept, const void* k_pool, const void* v_pool,
                     const int32_t* table_in, int32_t table_in_blocks, const int32_t* table_out,
                     int32_t table_out_blocks, void* k_pool_out, void* v_pool_out,
                     const uint64_t* credit_upd, uint64_t* credit_out, void* stream);

/* RefreshKV decode-loop pieces [notes on "RefreshKV: Updating Small KV Cache
 * During Long-form Generation", A2 method details: a full cache C_f and a
 * partial cache C_p of K entries per head; every S steps a query comparison
 * per layer (cosine of the current query averaged over the layer's query
 * heads against the one of its last full-attention step, full step when
 * below the threshold s); partial steps append the new token to C_p and drop
 * the entry with the lowest score of the last full step; a full step first
 * writes the tokens decoded with C_p into C_f, then refreshes C_p (the
 * one-segment event on C_f followed by kvc_partial_init)].  The caller runs
 * the loop and decides when to call what. */

/* Query comparison for `rows` (layer, sequence) rows.  q: bf16
 * [rows][heads_q][head_dim], the current token's queries (head_dim 64 or
 * 128).  q_ref: f64 [rows][head_dim], the head sums of each row's last full
 * step (the cosine is scale-invariant, so sums decide as means do); read,
 * and where a row fires and update_ref != 0, overwritten with the current
 * head sum.  full: i32 [rows], 1 where cos < threshold (a zero vector counts
 * as cos = 1).  cos_out: optional f64 [rows].  fp64 arithmetic. */
int kvc_qc_trigger(int32_t rows, int32_t heads_q, int32_t head_dim, const void* q, double* q_ref,
                   double threshold, int32_t update_ref, int32_t* full, double* cos_out,
                   void* stream);

/* C_p bookkeeping after a refresh: part_pos[n][j] = kept[n][j] and
 * part_score[n][j] = score[n][kept[n][j]] (+inf where kept is -1), with
 * kept/score as produced by the event (f32 score [NH][T], i32 kept
 * [NH][budget]); part_score f32 and part_pos i32 are [NH][budget]. */
int kvc_partial_init(const kvc_params* p, const int32_t* kept, const float* score,
                     float* part_score, int32_t* part_pos, void* stream);

/* One partial step for every head: the slot with the lowest part_score
 * (first slot on ties; scores must not be NaN) receives k_new[n], v_new[n]
 * (bf16 [n_heads][head_dim]) in k_part, v_part (bf16 [n_heads][K][head_dim]);
 * its score becomes +inf and its position t_new.  evicted: i32 [n_heads],
 * the slot used. */
int kvc_partial_append(int32_t n_heads, int32_t K, int32_t head_dim, float* part_score,
                       int32_t* part_pos, void* k_part, void* v_part, const void* k_new,
                       const void* v_new, int32_t t_new, int32_t* evicted, void* stream);

/* Full step, first half: every C_p slot with t_from <= part_pos < t_stride
 * is copied to row part_pos of k_full, v_full (bf16 [n_heads][t_stride]
 * [head_dim]); other rows are untouched. */
int kvc_full_sync(int32_t n_heads, int32_t K, int32_t head_dim, const int32_t* part_pos,
                  const void* k_part, const void* v_part, int32_t t_from, int32_t t_stride,
                  void* k_full, void* v_full, void* stream);

/* The whole event, steps 1-5 in one enqueue [AMS notes, overall framework].
 * credit_in/credit_out as above (credit_out required when ema); u_out (may be
 * NULL) receives the step-1 usage.  kept_out receives the kept positions.
 * Equals kvc_score_window -> kvc_mass_segment -> kvc_select ->
 * kvc_gather_compact on the same arguments, bit for bit.
 * The caller keeps counting logical (RoPE) positions from its generation
 * count; the compacted cache changes only the physical slots [AMS notes,
 * key design 4, appendix E paragraph]. */
int kvc_compress_event(const kvc_params* p, const void* q_win, const void* k, const void* v,
                       const uint64_t* credit_in, void* k_out, void* v_out,
                       uint64_t* credit_out, int32_t* kept_out, float* u_out, void* ws,
                       size_t ws_bytes, void* stream);

/* The whole event exactly as kvc_compress_event (same arguments, same
 * results, bit for bit), for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops and harnesses that forbid
 * allocation.  Instead of a workspace argument it uses scratch memory the
 * library holds on each GPU from module load until the process ends: a
 * device array of KVC_NOALLOC_SCRATCH_BYTES.  Events whose
 * kvc_workspace_bytes() exceeds that return KVC_ESCRATCH before anything is
 * enqueued (the Qwen-7B-shaped 1792-head event needs about 29 MB; larger
 * events use kvc_compress_event with a workspace).  Nothing is allocated and
 * nothing is freed.  The GPU is the one `stream` runs on (the current device
 * for the NULL stream); the first call on a GPU looks the array's address up
 * once.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (no call relies on them): calls that overlap in time on
 * one GPU -- different streams, or different host threads without ordering
 * -- race on it and must not be issued. */
int kvc_compress_event_noalloc(const kvc_params* p, const void* q_win, const void* k,
                               const void* v, const uint64_t* credit_in, void* k_out,
                               void* v_out, uint64_t* credit_out, int32_t* kept_out,
                               float* u_out, void* stream);

/* Workspace bytes any entry point above needs for these parameters (0 when
 * the parameters are invalid).  Pure host function. */
size_t kvc_workspace_bytes(const kvc_params* p);

/* Segment capacity S per head: n_cut + 1 + floor(T/seg_max) capped at T,
 * with n_cut = #{k >= 1 : k*delta < 1} (or ceil(T/seg_fixed) - 1 with fixed
 * segments); seg_max = 0 drops the second term.  Returns a negative status
 * for invalid parameters.  Pure host function. */
int kvc_segment_capacity(const kvc_params* p);

/* Validates the parameters alone (no pointers): KVC_OK or the error code.
 * Pure host function. */
int kvc_check_params(const kvc_params* p);

/* Static description of a status code. */
const char* kvc_strerror(int status);

/* KVC_ABI_VERSION of the built library. */
int kvc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
