"""Plain, slow, obviously-correct CPU oracle of one KV-compression event.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, per independent head-event (one layer x batch x KV head),
follows the pages in their own order:

  step 1  window score   -- usage of the last W queries of the G query heads
          [AMS notes, "关键设计 1" (key design 1), first paragraph;
           SkipKV notes, §4.1 "Token重要性得分" (observation window, GQA map);
           RefreshKV notes, "A6 附录" (GQA aggregation over the group)]
  step 2  mass           -- pooling, m_i = (max(u_i,0)+eps)/sum, EMA credit,
                            prefix C(t)
          [AMS notes, key design 1 (mass eq., EMA eq.); key design 2 (C(t))]
  step 3  segmentation + quota -- b_k = min{t : C(t) >= k*Delta}, split/merge,
                            must-keep, q_i^min, mass-proportional remainder,
                            clip and redistribute
          [AMS notes, key design 2 (cut eq.); key design 3 (quota eq.)]
  step 4  select         -- in-segment top-q_i, union with must-keep, repair,
                            sorted kept indices
          [AMS notes, key design 3 last paragraph; key design 4]
  step 5  gather         -- K/V/credit compacted with the same kept indices
          [AMS notes, key design 4; key design 1 last paragraph (credit follows
           the kept positions)]

Precision.  Step 1 runs in fp64 on the exactly widened bf16 inputs (it is the
reference the GPU's fp32 usage is held to).  Steps 2-5 are a heuristic whose
decisions are integers, so they follow one exact arithmetic contract that any
implementation can reproduce bit for bit:

  E1  every reduction (totals, prefix, segment masses) is over unsigned 64-bit
      fixed-point integers (usage scaled by 2^40, credit and mixed mass by 2^44);
  E2  every other operation is one IEEE-754 operation at a time, in the order
      written here (fp32 for pooling, fp64 for the EMA and the quota share),
      with no fused multiply-add and truncation toward zero when a
      non-negative float becomes an integer;
  E3  scalings by powers of two are exact;
  E4  the fixed-point totals cannot overflow: the usage sums to at most W*W*G
      per head (W*G rows summing to 1, plus W-1 filled positions of at most
      W*G), pooling multiplies that by less than F (F = 2 for the average,
      the width for the max), and F*W*W*G < 2^22 is required of the
      parameters.

Where the pages leave a step open, the reading taken is stated at the step
(each one is also listed with its reason in the design notes).  This file has
no dependency on the HIP library and must never gain one.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

POOL_AVG = 0
POOL_MAX = 1
AGG_SUM = 0
AGG_MAX = 1
QUOTA_MASS = 0      # remainder split by segment mass (the method)
QUOTA_UNIFORM = 1   # ablation: the same weight for every segment

USAGE_SHIFT = 40      # usage fixed point: a_t = trunc(ubar_t * 2^40)
CREDIT_SHIFT = 44     # credit / mixed-mass fixed point (Q44)
_TWO_USAGE = float(2 ** USAGE_SHIFT)
_TWO_CREDIT = float(2 ** CREDIT_SHIFT)


@dataclass(frozen=True)
class Params:
    """Event hyper-parameters, named after the pages' own quantities.

    Defaults: Delta = 0.1 and segment lengths 16/256 [AMS notes, key design 2,
    last paragraph]; q_min = 1 and 4 sink tokens [key design 3]; lambda = beta
    = 0.9 [key design 1]; pooling kernel 7 [RefreshKV notes, A6 baselines:
    SnapKV kernel 7].  The recent suffix length (64) and eps (1e-6) are not
    given by the pages and are readings.
    """
    T: int
    window: int
    budget: int
    group: int = 1
    head_dim: int = 128
    delta: float = 0.1
    seg_min: int = 16
    seg_max: int = 256            # 0 => unlimited
    q_min: int = 1
    sinks: int = 4
    recent: int = 64
    pool_kernel: int = 7
    pool_mode: int = POOL_AVG
    head_agg: int = AGG_SUM
    ema: bool = False
    lam: float = 0.9
    beta: float = 0.9
    eps: float = 1e-6
    n_prev: int = 0
    scale: float = 0.0            # 0 => 1/sqrt(head_dim)
    seg_fixed: int = 0            # ablation: > 0 => fixed-length raw segments
    quota_mode: int = QUOTA_MASS  # ablation: QUOTA_UNIFORM => no mass weighting

    def with_(self, **kw) -> "Params":
        return replace(self, **kw)


# ---------------------------------------------------------------------------
# Step 1: window score (fp64)
# ---------------------------------------------------------------------------

def window_usage_unfilled(q: np.ndarray, k: np.ndarray, p: Params) -> np.ndarray:
    """Usage of every cached position by the last W queries, before the fill.

    q: [G, W, d] window queries of the G query heads that share this KV head
       (post-RoPE; any float dtype, widened exactly to fp64).
    k: [>=T, d] cached keys; rows >= T are ignored.
    Returns u [T] fp64.

    [SkipKV notes, §4.1 token importance: softmax(Q K^T / sqrt(d) + M) over an
    observation window of the most recent queries, query head i belongs to KV
    head floor(i/n).]  [AMS notes, key design 1: usage of the most recent W
    decode queries over each cached position.]

    Readings: the W queries sit at absolute positions T-W .. T-1 and each sees
    keys up to its own position (causal mask); s = <q,k> * scale with scale =
    1/sqrt(d); usage sums the probabilities over the W queries, and over the G
    query heads (AGG_SUM) or takes the max over the G per-head sums (AGG_MAX,
    the RefreshKV/SnapKV group aggregation).
    """
    G, W, d = q.shape
    T = p.T
    assert W == p.window and G == p.group and d == k.shape[1]
    scale = p.scale if p.scale != 0.0 else 1.0 / math.sqrt(d)
    k64 = np.asarray(k[:T], dtype=np.float64)
    qpos = T - W + np.arange(W)                       # absolute query positions
    visible = np.arange(T)[None, :] <= qpos[:, None]  # [W, T] causal mask
    per_head = np.empty((G, T), dtype=np.float64)
    for g in range(G):
        s = scale * (np.asarray(q[g], dtype=np.float64) @ k64.T)   # [W, T]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)                                          # masked -> 0
        prob = e / e.sum(axis=1, keepdims=True)
        per_head[g] = prob.sum(axis=0)                             # sum over W
    if p.head_agg == AGG_SUM:
        return per_head.sum(axis=0)
    return per_head.max(axis=0)


def fill_partial(u: np.ndarray, W: int) -> np.ndarray:
    """Positions the causal window only partly observes get the window max.

    [AMS notes, key design 1: the recent suffix is seen by only part of the
    window queries, so missing observations are filled with the window's
    maximum score.]  Reading: positions t in (T-W, T-1] (seen by fewer than W
    queries) are replaced by M = max over the fully observed t <= T-W.
    """
    T = u.shape[0]
    out = u.copy()
    if W > 1:
        out[T - W + 1:] = u[: T - W + 1].max()
    return out


def window_usage(q: np.ndarray, k: np.ndarray, p: Params) -> np.ndarray:
    """Step 1 result: filled usage u [T] in fp64."""
    return fill_partial(window_usage_unfilled(q, k, p), p.window)


# ---------------------------------------------------------------------------
# Step 2: mass (exact contract)
# ---------------------------------------------------------------------------

def pool(u32: np.ndarray, p: Params) -> np.ndarray:
    """1-D pooling of the fp32 usage; returns ubar [T] fp32.

    [AMS notes, key design 1: small-kernel 1-D average pooling along the
    sequence.]  [RefreshKV notes, prefill stage: max pooling over neighbouring
    scores before top-K; A6 baselines: kernel 7.]

    Reading: stride 1, centred window of pool_kernel positions, only in-range
    neighbours count (no zero padding).  Average: fp32 sum in ascending
    position order starting from +0.0, then one correctly rounded fp32
    division by the in-range count.  Max: the maximum over the same window.
    """
    u32 = np.asarray(u32, dtype=np.float32)
    T = u32.shape[0]
    h = p.pool_kernel // 2
    idx = np.arange(T)
    if p.pool_mode == POOL_MAX:
        out = u32.copy()
        for off in range(-h, h + 1):
            j = idx + off
            ok = (j >= 0) & (j < T)
            out[ok] = np.maximum(out[ok], u32[j[ok]])
        return out
    acc = np.zeros(T, dtype=np.float32)
    cnt = np.zeros(T, dtype=np.int64)
    for off in range(-h, h + 1):                       # ascending j = t + off
        j = idx + off
        ok = (j >= 0) & (j < T)
        acc[ok] = acc[ok] + u32[j[ok]]                 # one fp32 add each
        cnt[ok] += 1
    return acc / cnt.astype(np.float32)                # fp32 division


def eps_fixed(eps: float) -> int:
    """e = ceil(eps * 2^40): the eps of the mass equation in usage fixed point."""
    return int(math.ceil(eps * _TWO_USAGE))


def usage_fixed(ubar: np.ndarray, p: Params) -> np.ndarray:
    """w_t = trunc(max(ubar_t, 0) * 2^40) + e  (uint64).

    [AMS notes, key design 1, mass eq.: m_i = (max(u_i,0)+eps) / sum_v
    (max(u_v,0)+eps).]  Here m_t = w_t / sum(w): the numerator and the
    denominator are the page's, in 2^-40 units.
    """
    nonneg = np.maximum(np.asarray(ubar, dtype=np.float32), np.float32(0.0))
    a = (nonneg * np.float32(_TWO_USAGE)).astype(np.uint64)   # exact scale, trunc
    return a + np.uint64(eps_fixed(p.eps))


def _u64_sum(x: np.ndarray) -> int:
    """Exact sum of a uint64 array as a Python int (E1); the guard proves the
    uint64 accumulation cannot have wrapped."""
    if x.size == 0:
        return 0
    assert int(x.max()) * int(x.size) < 2 ** 64, "fixed-point total would overflow"
    return int(np.sum(x, dtype=np.uint64))


def mass_fraction(w: np.ndarray) -> np.ndarray:
    """m_t = w_t / sum(w) in fp64 (the page's mass shares; sum to 1)."""
    return w.astype(np.float64) / float(_u64_sum(w))


def ema_credit(w: np.ndarray, credit_in: np.ndarray | None, p: Params):
    """EMA credit update and the mixed mass used for allocation.

    [AMS notes, key design 1, EMA eq.: c <- lambda*c + (1-lambda)*m;
    m_used = normalize(beta*m + (1-beta)*normalize(c)); the credit changes
    only the mass used for cutting and quotas, never the base score, and it
    must follow the kept positions across events.]

    Readings: credit is stored per position in Q44 fixed point; positions
    t < n_prev carry the previous event's credit, newer positions (and every
    position at the first event) start from their current mass; the update
    runs before the mix.  Returns (v, cq_new): v is the fixed-point mixed mass
    (Q44) the cuts and quotas use, cq_new the carried credit.
    """
    T = w.shape[0]
    mq = mass_fraction(w)                                        # fp64
    init = np.floor(mq * _TWO_CREDIT) * (1.0 / _TWO_CREDIT)      # new positions
    c = init.copy()
    n_prev = p.n_prev
    if n_prev > 0:
        c[:n_prev] = np.asarray(credit_in[:n_prev], dtype=np.uint64).astype(np.float64) \
            * (1.0 / _TWO_CREDIT)
    one_minus_lam = 1.0 - p.lam
    c_new = (p.lam * c) + (one_minus_lam * mq)                   # two products, one add
    cq_new = np.floor(c_new * _TWO_CREDIT).astype(np.uint64)
    cs = _u64_sum(cq_new)
    nc = cq_new.astype(np.float64) / float(cs) if cs > 0 else np.zeros(T)
    one_minus_beta = 1.0 - p.beta
    mix = (p.beta * mq) + (one_minus_beta * nc)
    v = np.floor(mix * _TWO_CREDIT).astype(np.uint64)
    return v, cq_new


def prefix(v: np.ndarray) -> np.ndarray:
    """C(t) = sum_{u <= t} v_u, inclusive, uint64 [AMS notes, key design 2]."""
    return np.cumsum(v, dtype=np.uint64)


# ---------------------------------------------------------------------------
# Step 3: must-keep, segmentation, quotas
# ---------------------------------------------------------------------------

def must_keep(p: Params):
    """Sinks and recent suffix, shrunk to fit the budget.

    [AMS notes, key design 3: 4 sink tokens at the start and a recent suffix
    are kept first; when the remaining budget would be negative the recent
    suffix is shortened and the sinks are protected.]
    Returns (S', R', T_keep); must-keep = [0,S') u [T-R', T).
    """
    T, K = p.T, p.budget
    s = min(p.sinks, K, T)
    r = min(p.recent, K - s, T - s)
    return s, r, K - s - r


def thresholds(V: int, delta: float):
    """theta_k = min(V, ceil(k*Delta*V)) for k = 1, 2, ... while k*Delta < 1.

    [AMS notes, key design 2, cut eq.: thresholds at Delta, 2*Delta, ...]
    """
    out = []
    k = 1
    while float(k) * delta < 1.0:
        th = math.ceil((float(k) * delta) * float(V))
        out.append(min(V, int(th)))
        k += 1
    return out


def raw_cuts(P: np.ndarray, delta: float):
    """Segment end positions from b_k = min{t : C(t) >= k*Delta}.

    Reading: 0-indexed inclusive ends; the position that completes mass
    k*Delta ends segment k; equal cuts (single-position spikes) collapse;
    T-1 always ends the last segment.
    """
    T = P.shape[0]
    V = int(P[-1])
    ends = set()
    for th in thresholds(V, delta):
        ends.add(int(np.searchsorted(P, np.uint64(th), side="left")))
    ends.add(T - 1)
    return sorted(ends)


def fixed_cuts(T: int, length: int):
    """Ablation "fixed-length segments" [AMS notes, ablations, Table 7]: the
    mass-driven cuts are replaced by cuts every `length` positions.  Reading:
    raw segments [0,L), [L,2L), ..., the last one ending at T-1 (possibly
    shorter); merge and split then run exactly as for mass cuts."""
    ends = list(range(length - 1, T - 1, length))
    ends.append(T - 1)
    return ends


def segments_from_ends(ends):
    segs = []
    start = 0
    for e in ends:
        segs.append((start, e))
        start = e + 1
    return segs


def merge_short(segs, seg_min: int):
    """Short adjacent segments are merged [AMS notes, key design 2].

    Reading: scan left to right, the current segment absorbs the next while
    it is shorter than seg_min; a short trailing segment joins its left
    neighbour.  Merging runs before splitting so that both bounds hold.
    """
    out = []
    cur = segs[0]
    for nxt in segs[1:]:
        if cur[1] - cur[0] + 1 < seg_min:
            cur = (cur[0], nxt[1])
        else:
            out.append(cur)
            cur = nxt
    if cur[1] - cur[0] + 1 < seg_min and out:
        out[-1] = (out[-1][0], cur[1])
    else:
        out.append(cur)
    return out


def split_long(segs, seg_max: int):
    """A segment longer than seg_max becomes near-equal pieces [AMS notes,
    key design 2].  Reading: n = ceil(L/seg_max) pieces, the first (L mod n)
    of length floor(L/n)+1, the rest floor(L/n).  seg_max = 0: no limit."""
    if seg_max <= 0:
        return list(segs)
    out = []
    for a, b in segs:
        L = b - a + 1
        if L <= seg_max:
            out.append((a, b))
            continue
        n = -(-L // seg_max)
        base, extra = divmod(L, n)
        s = a
        for i in range(n):
            ln = base + (1 if i < extra else 0)
            out.append((s, s + ln - 1))
            s += ln
    return out


def segment(P: np.ndarray, p: Params):
    """Cuts, then merge, then split: list of inclusive (start, end)."""
    if p.seg_fixed > 0:
        ends = fixed_cuts(P.shape[0], p.seg_fixed)
    else:
        ends = raw_cuts(P, p.delta)
    segs = segments_from_ends(ends)
    segs = merge_short(segs, p.seg_min)
    return split_long(segs, p.seg_max)


def segment_capacity(p: Params) -> int:
    """Upper bound on the number of segments a head can produce."""
    if p.seg_fixed > 0:
        n_raw = -(-p.T // p.seg_fixed)
    else:
        n_raw = len(thresholds(1 << 62, p.delta)) + 1
    cap = n_raw + (p.T // p.seg_max if p.seg_max > 0 else 0)
    return max(1, min(cap, p.T))


def _walk(q, limit, order, D, step):
    """Cyclic walk over `order`, moving each eligible q_i one step toward its
    limit per cycle until D steps are spent (or a cycle moves nothing)."""
    while D > 0:
        if step > 0:
            elig = order[q[order] < limit[order]]
        else:
            elig = order[q[order] > limit[order]]
        if elig.size == 0:
            break
        take = elig if elig.size <= D else elig[:D]
        q[take] += step
        D -= take.size
    return q


def quotas(segs, v: np.ndarray, p: Params):
    """Per-segment quotas q_i [AMS notes, key design 3, quota eq.].

    q_i^min = min(q_min, L_i); T_rem = T_keep - sum q^min;
    q_i = q_i^min + round(T_rem * M_i / sum_j M_j); then clip to the segment
    and redistribute so the total equals the budget.

    Readings (the page gives the formula "ignoring the must-keep correction"):
    must-keep positions already inside a segment count toward its floor,
    floor_i = min(A_i, max(0, min(q_min, L_i) - K_i)) with K_i = |seg_i n MK|
    and A_i = L_i - K_i; M_i is the mass of the segment's non-must-keep
    positions; round = floor(x + 0.5) on the fp64 share; clip to A_i;
    a positive shortfall is handed out one per segment per cycle in
    (M_i desc, i asc) order, an excess taken back one per segment per cycle
    in (M_i asc, i desc) order without going below the floor.  When the
    floors alone exceed T_keep the quotas stay at the floors and the select
    step's over-budget repair drops the lowest-scored picks (the page: floors
    hold only when the budget allows).
    Ablation "no mass-weighted quota" [AMS notes, ablations, Table 7]
    (quota_mode = QUOTA_UNIFORM): every segment weighs 1 instead of M_i, in the
    share and in the redistribution order alike (so ties go by index).
    Returns (q, floor, A, M) as int64 arrays (M as Python-int object array).
    """
    T = p.T
    s, r, t_keep = must_keep(p)
    mk = np.zeros(T, dtype=bool)
    mk[:s] = True
    if r > 0:
        mk[T - r:] = True
    n = len(segs)
    L = np.array([b - a + 1 for a, b in segs], dtype=np.int64)
    Kmk = np.array([int(mk[a:b + 1].sum()) for a, b in segs], dtype=np.int64)
    A = L - Kmk
    if p.quota_mode == QUOTA_UNIFORM:
        M = [1] * n
    else:
        M = [int(np.sum(v[a:b + 1][~mk[a:b + 1]], dtype=np.uint64)) for a, b in segs]
    floor_ = np.minimum(A, np.maximum(0, np.minimum(p.q_min, L) - Kmk))
    F = int(floor_.sum())
    if F > t_keep:
        return floor_.copy(), floor_, A, M
    t_rem = t_keep - F
    SM = sum(M)
    add = np.zeros(n, dtype=np.int64)
    if SM > 0:
        for i in range(n):
            share = float(t_rem) * (float(M[i]) / float(SM))
            add[i] = int(math.floor(share + 0.5))
    q = np.minimum(A, floor_ + add)
    D = t_keep - int(q.sum())
    ids = np.arange(n)
    if D > 0:
        order = np.array(sorted(ids, key=lambda i: (-M[i], i)), dtype=np.int64)
        q = _walk(q, A, order, D, +1)
    elif D < 0:
        order = np.array(sorted(ids, key=lambda i: (M[i], -i)), dtype=np.int64)
        q = _walk(q, floor_, order, -D, -1)
    return q, floor_, A, M


# ---------------------------------------------------------------------------
# Step 4: select
# ---------------------------------------------------------------------------

def _rank_desc(score: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """pos sorted by (score desc, position asc); ties go to the lower index."""
    return pos[np.lexsort((pos, -score[pos]))]


def select(score: np.ndarray, segs, q, p: Params) -> np.ndarray:
    """Kept indices, ascending, length min(budget, T).

    [AMS notes, key design 3 last paragraph: union with must-keep counting
    duplicates once; over budget drop low-score non-must-keep picks; under
    budget add high-score unselected positions.]  [Key design 4: per-segment
    top-k by the base score, kept indices sorted, the same indices for K and
    V.]  Readings: the base score is the pooled usage (any fp32 score works);
    ties go to the lower index everywhere; picks never include must-keep
    positions; a quota above the segment's candidate count takes them all.
    """
    T, K = p.T, p.budget
    if T <= K:
        return np.arange(T, dtype=np.int64)
    score = np.asarray(score, dtype=np.float32)
    s, r, _ = must_keep(p)
    mk = np.zeros(T, dtype=bool)
    mk[:s] = True
    if r > 0:
        mk[T - r:] = True
    keep = mk.copy()
    picked = np.zeros(T, dtype=bool)
    for (a, b), qi in zip(segs, q):
        cand = np.arange(a, b + 1)
        cand = cand[~mk[a:b + 1]]
        top = _rank_desc(score, cand)[: max(0, int(qi))]
        picked[top] = True
    keep |= picked
    n_keep = int(keep.sum())
    if n_keep > K:
        pk = np.flatnonzero(picked)
        # drop in (score asc, index desc) order == keep the best of the picks
        order = _rank_desc(score, pk)
        keep[order[K - int(mk.sum()):]] = False
    elif n_keep < K:
        free = np.flatnonzero(~keep & ~mk)
        keep[_rank_desc(score, free)[: K - n_keep]] = True
    return np.flatnonzero(keep).astype(np.int64)


# ---------------------------------------------------------------------------
# Step 5: gather
# ---------------------------------------------------------------------------

def gather(kept: np.ndarray, k: np.ndarray, v: np.ndarray, credit, budget: int):
    """K_out[j] = K[kept_j], V_out[j] = V[kept_j], credit_out[j] =
    credit[kept_j]: a fixed-length per-head buffer [AMS notes, key design 4;
    key design 1: credit stays aligned with the kept positions].  Slots past
    len(kept) (only when T < budget) are zero and their kept index is -1."""
    d = k.shape[1]
    n = kept.shape[0]
    k_out = np.zeros((budget, d), dtype=k.dtype)
    v_out = np.zeros((budget, d), dtype=v.dtype)
    k_out[:n] = k[kept]
    v_out[:n] = v[kept]
    c_out = None
    if credit is not None:
        c_out = np.zeros(budget, dtype=np.uint64)
        c_out[:n] = credit[kept]
    kept_full = np.full(budget, -1, dtype=np.int64)
    kept_full[:n] = kept
    return kept_full, k_out, v_out, c_out


# ---------------------------------------------------------------------------
# One head-event
# ---------------------------------------------------------------------------

@dataclass
class HeadResult:
    u: np.ndarray | None            # fp64 filled usage (None when given as input)
    u32: np.ndarray                 # fp32 usage steps 2-5 consumed
    score: np.ndarray               # pooled usage ubar, fp32 (the base score)
    w: np.ndarray                   # fixed-point usage incl. eps (uint64)
    v: np.ndarray                   # mass used for cutting (uint64)
    credit_upd: np.ndarray | None   # carried credit per position (uint64 Q44)
    P: np.ndarray                   # prefix of v (uint64)
    segs: list = field(default_factory=list)
    q: np.ndarray | None = None
    kept: np.ndarray | None = None  # [budget] int64, -1 padded
    k_out: np.ndarray | None = None
    v_out: np.ndarray | None = None
    credit_out: np.ndarray | None = None
    noop: bool = False


def mass_and_segments(u32: np.ndarray, credit_in, p: Params) -> HeadResult:
    """Steps 2-3 on an fp32 usage vector."""
    score = pool(u32, p)
    w = usage_fixed(score, p)
    if p.ema:
        v, credit_upd = ema_credit(w, credit_in, p)
    else:
        v, credit_upd = w, None
    P = prefix(v)
    res = HeadResult(u=None, u32=np.asarray(u32, np.float32), score=score, w=w, v=v,
                     credit_upd=credit_upd, P=P)
    if p.T <= p.budget:
        res.noop = True
        return res
    res.segs = segment(P, p)
    res.q = quotas(res.segs, v, p)[0]
    return res


def steps2to5(u32, k, v, credit_in, p: Params) -> HeadResult:
    """Steps 2-5 of one head from its fp32 usage (the bit-exact contract)."""
    res = mass_and_segments(u32, credit_in, p)
    if res.noop:
        kept = np.arange(p.T, dtype=np.int64)
    else:
        kept = select(res.score, res.segs, res.q, p)
    res.kept, res.k_out, res.v_out, res.credit_out = gather(
        kept, np.asarray(k)[: p.T], np.asarray(v)[: p.T], res.credit_upd, p.budget)
    return res


def event(q, k, v, credit_in, p: Params) -> HeadResult:
    """Whole event for one head: fp64 step 1, rounded once to fp32, then the
    exact steps 2-5 [AMS notes, overall framework: one independent selection
    per layer and KV head producing a compact budget-length cache]."""
    u = window_usage(q, k, p)
    res = steps2to5(u.astype(np.float32), k, v, credit_in, p)
    res.u = u
    return res


# ---------------------------------------------------------------------------
# Ragged (left-padded) multi-batch events
# ---------------------------------------------------------------------------
#
# In a multi-batch decode the prompts of one batch have different lengths and
# are left-padded to the longest one; the attention mask M keeps the padding
# out of the attention scores, and padding that stays in the compressed cache
# eats its budget [SkipKV notes, observation 1; §4.1 token importance with the
# mask M; §5 B' = B - Delta_pad].  Reading: a head-event with valid length
# len holds padding at positions [0, T-len) and real tokens at [T-len, T); the
# event runs on the real tokens only, exactly as on a cache of length len
# (padding takes no part in the softmax, the masses, the must-keep set or the
# budget), and its indices are reported in the padded cache's positions.

def valid_length(p: Params, length: int) -> int:
    """Valid positions of a left-padded head-event, clamped to [W, T]: the
    window queries are the last W positions and are always real tokens."""
    return int(min(max(int(length), p.window), p.T))


def _to_absolute(res: HeadResult, off: int, T: int) -> HeadResult:
    """Re-express a head result computed on positions [off, T) in the padded
    cache's positions: per-position arrays get zeros on the padding, segments
    and kept indices move by off (kept keeps its -1 padding)."""
    def pad(x, dtype):
        if x is None:
            return None
        out = np.zeros(T, dtype=dtype)
        out[off:] = x
        return out
    res.u = pad(res.u, np.float64)
    res.u32 = pad(res.u32, np.float32)
    res.score = pad(res.score, np.float32)
    res.w = pad(res.w, np.uint64)
    res.v = pad(res.v, np.uint64)
    res.credit_upd = pad(res.credit_upd, np.uint64)
    res.segs = [(a + off, b + off) for a, b in res.segs]
    if res.kept is not None:
        res.kept = np.where(res.kept >= 0, res.kept + off, -1).astype(np.int64)
    return res


def _ragged_params(p: Params, length: int):
    Tn = valid_length(p, length)
    return Tn, p.T - Tn, p.with_(T=Tn, n_prev=min(p.n_prev, Tn))


def steps2to5_ragged(u32, k, v, credit_in, p: Params, length: int) -> HeadResult:
    """Steps 2-5 of a left-padded head-event; u32, k and v span all T
    positions, credit_in holds the credit of the first n_prev real tokens."""
    Tn, off, pn = _ragged_params(p, length)
    ci = None if credit_in is None or pn.n_prev == 0 else np.asarray(credit_in)[: pn.n_prev]
    res = steps2to5(np.asarray(u32)[off:p.T], np.asarray(k)[off:p.T], np.asarray(v)[off:p.T],
                    ci, pn)
    return _to_absolute(res, off, p.T)


def window_usage_ragged(q, k, p: Params, length: int) -> np.ndarray:
    """Step 1 of a left-padded head-event: fp64 usage over all T positions,
    zero on the padding."""
    Tn, off, pn = _ragged_params(p, length)
    u = np.zeros(p.T, dtype=np.float64)
    u[off:] = window_usage(q, np.asarray(k)[off:p.T], pn)
    return u


def event_ragged(q, k, v, credit_in, p: Params, length: int) -> HeadResult:
    """Whole event for one left-padded head-event."""
    u = window_usage_ragged(q, k, p, length)
    res = steps2to5_ragged(u.astype(np.float32), k, v, credit_in, p, length)
    res.u = u
    return res


# ---------------------------------------------------------------------------
# Paged-KV compaction
# ---------------------------------------------------------------------------
#
# [AMS notes, key design 4, appendix E paragraph] The selection is separate
# from the paged storage layout: the runtime allocates new blocks, copies each
# head's KV from its kept original positions into the new physical slots, swaps
# the request's block table and frees the old blocks.  One compacted slot may
# hold KV from different original positions in different heads.  Layout read
# here: a pool of blocks [n_blocks][kv_heads][block_size][d]; logical position t
# of sequence b lives in block table[b][t // block_size], slot t % block_size.

def gather_paged(kept: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                 table_in: np.ndarray, table_out: np.ndarray, kv_heads: int):
    """Compacted copy into new blocks of the same pools.

    kept [B*kv_heads][K] (-1 = empty slot), head n = b*kv_heads + h; returns new
    pools where slot j of sequence b's compacted cache (block table_out[b][j //
    bs], slot j % bs) holds, for head h, the row of logical position
    kept[n][j] (zeros for -1); blocks not named in table_out are unchanged."""
    n_blocks, H, bs, d = k_pool.shape
    assert H == kv_heads
    k_new, v_new = k_pool.copy(), v_pool.copy()
    NH, K = kept.shape
    for n in range(NH):
        b, h = divmod(n, kv_heads)
        for j in range(K):
            dst = int(table_out[b][j // bs]), j % bs
            t = int(kept[n][j])
            if t < 0:
                k_new[dst[0], h, dst[1]] = 0
                v_new[dst[0], h, dst[1]] = 0
                continue
            src = int(table_in[b][t // bs]), t % bs
            k_new[dst[0], h, dst[1]] = k_pool[src[0], h, src[1]]
            v_new[dst[0], h, dst[1]] = v_pool[src[0], h, src[1]]
    return k_new, v_new


def read_paged(pool: np.ndarray, table: np.ndarray, b: int, h: int, length: int) -> np.ndarray:
    """Logical rows 0..length-1 of head h of sequence b through its block table."""
    bs = pool.shape[2]
    return np.stack([pool[int(table[b][t // bs]), h, t % bs] for t in range(length)])
