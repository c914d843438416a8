"""The event on a cache split over positions (host check, oracle only).

A head's cache sharded by position, as a sequence-parallel layout would hold
it, still gives the one-device result when the shards exchange a few small
messages:

- step 1 [AMS notes, key design 1; SkipKV notes §4.1]: per-shard row
  statistics (max, sum) merged by log-sum-exp give every row's softmax
  normaliser; each shard then sums its own columns; the tail fill takes the
  maximum of the shards' maxima.  Agrees with the oracle to fp64 rounding.
- step 2 [AMS notes, key design 1]: pooling needs half a pooling window of
  neighbours from the adjacent shards; the fixed-point usage is elementwise;
  the EMA and the mix need only the head's two totals (sum of usage, sum of
  updated credit), which are exact u64 sums of the shards' partial sums.
- step 3 [AMS notes, key designs 2-3]: the prefix is each shard's local
  prefix plus the exact sum of the shards before it, so every shard finds
  the cuts that fall in its range; segment masses come from prefix values
  at segment ends.
- step 4 [AMS notes, key designs 3-4]: with feasible floors each segment's
  picks depend only on that segment's scores, so a segment is selected by
  the shard that owns its first position with its scores gathered.

Steps 2-4 are compared bit for bit with the oracle's one-head evaluation.
"""
import numpy as np
import pytest

from oracle import ams


def _shards(T, n, rng):
    cuts = np.sort(rng.choice(np.arange(1, T), n - 1, replace=False))
    b = [0, *cuts.tolist(), T]
    return [(b[i], b[i + 1]) for i in range(n)]


@pytest.mark.parametrize("agg", [ams.AGG_SUM, ams.AGG_MAX])
@pytest.mark.parametrize("n_shards", [2, 3, 7])
def test_window_score_from_per_shard_row_statistics(agg, n_shards):
    rng = np.random.default_rng(10 * n_shards + agg)
    G, W, d, T = 3, 16, 32, 400
    q = rng.standard_normal((G, W, d))
    k = rng.standard_normal((T, d)) * 1.5
    p = ams.Params(T=T, window=W, group=G, head_dim=d, budget=100, head_agg=agg)
    ref = ams.window_usage(q, k, p)
    scale = 1.0 / np.sqrt(d)
    S = np.einsum("gwd,td->gwt", q, k) * scale
    lim = (T - W + np.arange(W))[None, :, None]                 # query w sees keys t <= T-W+w
    vis = np.arange(T)[None, None, :] <= lim
    shards = _shards(T, n_shards, rng)
    # per-shard row statistics, merged by log-sum-exp
    m = np.full((G, W), -np.inf)
    parts = []
    for a, b in shards:
        s = np.where(vis[:, :, a:b], S[:, :, a:b], -np.inf)
        ms = s.max(axis=2)
        ls = np.where(np.isfinite(ms), np.exp(s - np.where(np.isfinite(ms), ms, 0)[..., None]).sum(axis=2), 0)
        parts.append((ms, ls))
        m = np.maximum(m, ms)
    l = sum(np.where(np.isfinite(ms), ls * np.exp(ms - m), 0.0) for ms, ls in parts)
    # each shard sums its own columns with the merged normalisers
    u = np.zeros(T)
    for a, b in shards:
        pr = np.where(vis[:, :, a:b], np.exp(S[:, :, a:b] - m[..., None]) / l[..., None], 0.0)
        per_g = pr.sum(axis=1)                                  # [G, b-a]
        u[a:b] = per_g.sum(axis=0) if agg == ams.AGG_SUM else per_g.max(axis=0)
    # tail fill: the maximum of the shards' maxima over the fully observed positions
    last = T - W
    fill = max(u[a:min(b, last + 1)].max() for a, b in shards if a <= last)
    u[last + 1:] = fill
    np.testing.assert_allclose(u, ref, rtol=1e-12, atol=0)


def _sharded_steps2to3(u32, credit_in, p, shards):
    """Steps 2-3 evaluated shard by shard with only the messages listed in
    the module docstring; returns (score, credit_upd, v, P, cuts)."""
    T = u32.shape[0]
    h = p.pool_kernel // 2
    score, w = [], []
    for a, b in shards:
        lo, hi = max(0, a - h), min(T, b + h)               # half a pooling window from the neighbours
        sc = ams.pool(u32[lo:hi], p)[a - lo:b - lo]
        score.append(sc)
        w.append(ams.usage_fixed(sc, p))
    W_tot = sum(int(x.sum(dtype=np.uint64)) for x in w)     # exact: each partial is below 2^64
    if p.ema:
        two44 = float(2 ** 44)
        cq, mq = [], []
        for (a, b), ws in zip(shards, w):
            m = ws.astype(np.float64) / float(W_tot)
            c = np.floor(m * two44) * (1.0 / two44)
            if p.n_prev > a:
                n = min(b, p.n_prev) - a
                c[:n] = credit_in[a:a + n].astype(np.float64) * (1.0 / two44)
            cq.append(np.floor(((p.lam * c) + ((1.0 - p.lam) * m)) * two44).astype(np.uint64))
            mq.append(m)
        cs = sum(int(x.sum(dtype=np.uint64)) for x in cq)
        v = []
        for m, c in zip(mq, cq):
            nc = c.astype(np.float64) / float(cs) if cs > 0 else np.zeros(len(c))
            v.append(np.floor(((p.beta * m) + ((1.0 - p.beta) * nc)) * two44).astype(np.uint64))
        credit_upd = np.concatenate(cq)
    else:
        v, credit_upd = w, None
    # prefix: local prefix plus the exact total of the shards before
    P, off = [], 0
    for vs in v:
        P.append(np.cumsum(vs, dtype=np.uint64) + np.uint64(off))
        off += int(vs.sum(dtype=np.uint64))
    V = off
    # cuts: a shard owns the threshold its range crosses
    cuts = {T - 1}
    for th in ams.thresholds(V, p.delta):
        for i, ((a, b), Ps) in enumerate(zip(shards, P)):
            before = int(P[i - 1][-1]) if i else 0           # the prefix just before the shard
            if before < th <= int(Ps[-1]):
                cuts.add(a + int(np.searchsorted(Ps, np.uint64(th), side="left")))
                break
    return (np.concatenate(score), credit_upd, np.concatenate(v), np.concatenate(P),
            sorted(cuts))


CASES = [
    # (label, T, K, n_shards, overrides)
    ("avg", 3000, 500, 4, {}),
    ("max_pool_many_shards", 2500, 300, 9, dict(pool_mode=ams.POOL_MAX)),
    ("ema_fresh", 4000, 700, 5, dict(ema=True)),
    ("ema_carried", 3500, 600, 3, dict(ema=True, n_prev=2000)),
    ("fine_cuts", 3000, 800, 6, dict(delta=0.02, seg_min=4, seg_max=64)),
    ("tiny_shards", 600, 100, 40, dict(delta=0.05)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_steps_2_to_4_on_shards_equal_the_head(case):
    label, T, K, n_shards, over = case
    rng = np.random.default_rng(sum(map(ord, label)))
    u32 = (rng.random(T) ** 4 * 3.0).astype(np.float32)
    p = ams.Params(T=T, window=16, group=2, budget=K, **over)
    credit_in = None
    if p.n_prev:
        r = rng.random(p.n_prev) + 1e-3
        credit_in = np.floor(r / r.sum() * 2.0 ** 44).astype(np.uint64)
    ref = ams.mass_and_segments(u32, credit_in, p)
    shards = _shards(T, n_shards, rng)
    score, credit_upd, v, P, cuts = _sharded_steps2to3(u32, credit_in, p, shards)
    np.testing.assert_array_equal(score.view(np.uint32), ref.score.view(np.uint32))
    if p.ema:
        np.testing.assert_array_equal(credit_upd, ref.credit_upd)
    np.testing.assert_array_equal(v, ref.v)
    np.testing.assert_array_equal(P, ref.P)
    assert cuts == ams.raw_cuts(ref.P, p.delta)
    # segment masses from prefix values at segment ends (must-keep excluded)
    _, _, _, M = ams.quotas(ref.segs, ref.v, p)
    s, r, _ = ams.must_keep(p)
    mk = np.zeros(T, dtype=bool)
    mk[:s] = True
    if r:
        mk[T - r:] = True
    keep_v = np.where(mk, np.uint64(0), ref.v)
    Pk = np.cumsum(keep_v, dtype=np.uint64)
    for (a, b), Mi in zip(ref.segs, M):
        assert int(Pk[b]) - (int(Pk[a - 1]) if a else 0) == int(Mi)
    # step 4: with feasible floors each segment's picks come from its own scores
    kept = ams.select(ref.score, ref.segs, ref.q, p)
    kept_set = set(int(x) for x in kept if x >= 0)
    floors = ams.quotas(ref.segs, ref.v, p)[1]
    if int(np.sum(floors)) <= K - s - r:
        for (a, b), qi in zip(ref.segs, ref.q):
            cand = [t for t in range(a, b + 1) if not mk[t]]
            order = sorted(cand, key=lambda t: (-float(ref.score[t]), t))
            assert set(order[:int(qi)]) == {t for t in cand if t in kept_set}, (label, a, b)
