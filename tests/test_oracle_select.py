"""Pins for the oracle's segmentation, quotas, select and gather (steps 3-5):
the page's worked example, brute-force enumeration, library top-K, closed
forms and invariants, plus a loop restatement over random tiny cases."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import ams, loops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _run(u, p):
    return ams.steps2to5(np.asarray(u, np.float32), np.zeros((p.T, 2), np.uint16),
                         np.zeros((p.T, 2), np.uint16), None, p)


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_worked_example(case):
    pr = dict(case["params"])
    p = ams.Params(**pr)
    res = _run(case["u"], p)
    assert [b for _, b in res.segs] == case["segment_ends"]
    kept = res.kept[res.kept >= 0]
    assert len(kept) == p.budget
    per_seg = [int(np.sum((kept >= a) & (kept <= b))) for a, b in res.segs]
    assert per_seg == case["kept_per_segment"]
    if "quotas" in case:
        assert list(map(int, res.q)) == case["quotas"]
        assert list(map(int, kept)) == case["kept"]
    if "global_top8_kept_in_second_segment" in case:
        score = np.asarray(case["u"], np.float32)
        top = np.argsort(-score, kind="stable")[: p.budget]
        assert int(np.sum((top >= 4) & (top <= 7))) == case["global_top8_kept_in_second_segment"]


def test_uniform_mass_cuts_every_T_delta():
    # Delta = 1/8 is exact in fp64: uniform mass cuts every T*Delta positions.
    T = 96
    v = np.full(T, 12345, dtype=np.uint64)
    assert ams.raw_cuts(ams.prefix(v), 0.125) == list(range(11, 96, 12))
    # Delta = 0.1 is not exact (fp64 3*0.1 > 0.3): a threshold that falls
    # exactly on a prefix value may move one position right, never more.
    T = 100
    v = np.full(T, 12345, dtype=np.uint64)
    ends = ams.raw_cuts(ams.prefix(v), 0.1)
    assert len(ends) == 10 and ends[-1] == 99
    assert all(abs(e - (10 * (i + 1) - 1)) <= 1 for i, e in enumerate(ends))


def test_delta_at_least_one_means_one_segment():
    v = np.arange(1, 51, dtype=np.uint64)
    assert ams.raw_cuts(ams.prefix(v), 1.0) == [49]
    assert ams.thresholds(10 ** 6, 1.0) == []


def test_spike_collapses_cuts():
    # one position holding > 3*Delta of the mass ends several thresholds at once
    v = np.ones(40, dtype=np.uint64) * 10
    v[20] = 10 ** 6
    ends = ams.raw_cuts(ams.prefix(v), 0.1)
    assert ends.count(20) == 1 and ends[-1] == 39 and len(ends) == 2


def test_cut_definition_by_linear_scan():
    rng = np.random.default_rng(0)
    for _ in range(20):
        T = int(rng.integers(5, 200))
        v = rng.integers(0, 1000, size=T).astype(np.uint64)
        v[0] += 1
        P = ams.prefix(v)
        V = int(P[-1])
        for th in ams.thresholds(V, 0.13):
            t = next(i for i in range(T) if int(P[i]) >= th)
            assert t in ams.raw_cuts(P, 0.13)


@given(st.lists(st.integers(1, 300), min_size=1, max_size=30), st.integers(1, 40), st.integers(0, 400))
@settings(max_examples=200, deadline=None)
def test_merge_split_partition_and_bounds(lengths, seg_min, seg_max):
    if seg_max and seg_max < 2 * seg_min:
        seg_max = 2 * seg_min
    ends = list(np.cumsum(lengths) - 1)
    T = int(ends[-1]) + 1
    segs = ams.split_long(ams.merge_short(ams.segments_from_ends(ends), seg_min), seg_max)
    assert segs[0][0] == 0 and segs[-1][1] == T - 1
    for (a, b), (c, _) in zip(segs, segs[1:]):
        assert c == b + 1
    for a, b in segs:
        L = b - a + 1
        if T >= seg_min:
            assert L >= seg_min
        if seg_max:
            assert L <= seg_max
    if seg_max:
        assert len(segs) >= math.ceil(T / seg_max)
    n_thr_cap = len(lengths) + (T // seg_max if seg_max else 0)
    assert len(segs) <= n_thr_cap


def test_split_longer_pieces_first():
    assert ams.split_long([(0, 9)], 4) == [(0, 3), (4, 6), (7, 9)]


def test_merge_tail_joins_left():
    assert ams.merge_short([(0, 9), (10, 12)], 5) == [(0, 12)]
    assert ams.merge_short([(0, 1), (2, 3), (4, 20)], 5) == [(0, 20)]
    assert ams.merge_short([(0, 2)], 5) == [(0, 2)]


def _quota_case(masses, t_keep, L=10):
    n = len(masses)
    T = n * L
    segs = [(i * L, i * L + L - 1) for i in range(n)]
    v = np.zeros(T, dtype=np.uint64)
    for i, m in enumerate(masses):
        v[i * L] = m
    p = ams.Params(T=T, window=1, budget=t_keep, sinks=0, recent=0, seg_min=1, seg_max=0)
    return ams.quotas(segs, v, p)[0]


def test_quota_hand_cases():
    # three equal masses, T_rem = 4: round(4/3) = 1 each, the spare slot goes
    # to the first segment in (mass desc, index asc) order -> adds (2,1,1)
    assert list(_quota_case([7, 7, 7], 3 + 4)) == [3, 2, 2]
    # two equal masses, T_rem = 1: both round 0.5 up, the excess comes back
    # from the last segment in (mass asc, index desc) order -> adds (1, 0)
    assert list(_quota_case([5, 5], 2 + 1)) == [2, 1]
    # proportional split 3:1 of T_rem = 8 -> adds (6, 2)
    assert list(_quota_case([3, 1], 2 + 8)) == [7, 3]


def test_quota_excess_never_goes_below_a_floor():
    # masses 1:5:5:5, floors 1 each, T_rem = 2: shares 0.125 -> 0 and 0.625 -> 1
    # three times, one slot too many.  The excess comes back in (mass asc,
    # index desc) order from segments still above their floor: the light
    # segment sits at its floor and is passed over, the last heavy one gives
    # the slot back [AMS notes, key design 3: clip and redistribute, floors
    # held while the budget allows] -> (1, 2, 2, 1), not (0, 2, 2, 2)
    assert list(_quota_case([1, 5, 5, 5], 4 + 2)) == [1, 2, 2, 1]


def test_quota_clip_and_redistribute():
    # the heavy segment (length 10) asks for more than it has; the rest goes
    # to the others in mass order
    q = _quota_case([1000, 1, 1], 20)
    assert q[0] == 10 and sum(q) == 20 and all(1 <= x <= 10 for x in q)


def _rand_case(rng, T_max=60, ema=None):
    T = int(rng.integers(8, T_max))
    K = int(rng.integers(1, T + 3))
    p = ams.Params(T=T, window=int(rng.integers(1, 5)), budget=K,
                   delta=float(rng.choice([0.05, 0.1, 0.25, 0.3, 1.0])),
                   seg_min=int(rng.integers(1, 6)), seg_max=int(rng.choice([0, 6, 10, 16])),
                   q_min=int(rng.integers(0, 3)), sinks=int(rng.integers(0, 5)),
                   recent=int(rng.integers(0, 9)), pool_kernel=int(rng.choice([1, 3, 7])),
                   pool_mode=int(rng.integers(0, 2)),
                   ema=bool(rng.integers(0, 2)) if ema is None else ema,
                   lam=float(rng.choice([0.0, 0.5, 0.9])), beta=float(rng.choice([0.5, 0.9, 1.0])))
    if p.seg_max and p.seg_max < 2 * p.seg_min:
        p = p.with_(seg_max=2 * p.seg_min)
    u = (rng.random(T) ** 3 * rng.choice([1.0, 10.0, 100.0])).astype(np.float32)
    if rng.random() < 0.3:
        u[rng.integers(0, T, size=T // 3)] = u[0]        # ties
    n_prev = int(rng.integers(0, T + 1)) if p.ema else 0
    p = p.with_(n_prev=n_prev)
    cin = rng.integers(0, 2 ** 42, size=T).astype(np.uint64)
    return u, cin, p


@pytest.mark.parametrize("seed", range(150))
def test_numpy_equals_loops_random(seed):
    rng = np.random.default_rng(1000 + seed)
    u, cin, p = _rand_case(rng)
    res = ams.steps2to5(u, np.zeros((p.T, 1), np.uint16), np.zeros((p.T, 1), np.uint16), cin, p)
    sc = loops.pool(u, p)
    v, cq = loops.mass_v(sc, cin, p)
    assert list(map(int, res.v)) == v
    if p.T <= p.budget:
        assert res.noop
        return
    segs = loops.segments(v, p)
    assert [tuple(s) for s in res.segs] == [tuple(s) for s in segs]
    q = loops.quotas(segs, v, p)
    assert list(map(int, res.q)) == q
    kept = loops.select(sc, segs, q, p)
    assert list(map(int, res.kept[res.kept >= 0])) == kept


@pytest.mark.parametrize("seed", range(60))
def test_quota_invariants(seed):
    rng = np.random.default_rng(5000 + seed)
    u, cin, p = _rand_case(rng, T_max=120)
    if p.T <= p.budget:
        return
    r = ams.mass_and_segments(u, cin, p)
    q, fl, A, M = ams.quotas(r.segs, r.v, p)
    s, rr, t_keep = ams.must_keep(p)
    assert np.all(q >= fl) and np.all(q <= A)
    if fl.sum() <= t_keep:
        assert q.sum() == t_keep
        mk = np.zeros(p.T, bool)
        mk[:s] = True
        if rr:
            mk[p.T - rr:] = True
        for (a, b), qi in zip(r.segs, q):
            L = b - a + 1
            assert qi + mk[a:b + 1].sum() >= min(p.q_min, L)
    kept = r.kept if r.kept is not None else ams.select(r.score, r.segs, q, p)
    assert len(kept) == p.budget and np.all(np.diff(kept) > 0)


def test_quota_share_within_one_without_clipping():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(1, 12))
        masses = rng.integers(1, 10 ** 6, size=n)
        L = 1000
        t_keep = int(rng.integers(n, 4 * n + 40))
        q = _quota_case(list(map(int, masses)), t_keep, L=L)
        t_rem = t_keep - n
        share = t_rem * masses / masses.sum()
        # rounding moves each share by <= 1/2; the total rounding error is
        # <= n/2 < n, so the redistribution walk moves a segment at most once
        assert np.all(np.abs(q - 1 - share) <= 1.5 + 1e-9)
        assert q.sum() == t_keep


def _brute_force_kept(score, segs, q, mk, K):
    """Among subsets containing MK with exactly q_i non-MK members per segment,
    the one with the largest score sum, ties to the lexicographically smallest
    index vector."""
    choices = []
    for (a, b), qi in zip(segs, q):
        cand = [t for t in range(a, b + 1) if t not in mk]
        choices.append(list(itertools.combinations(cand, int(qi))))
    best = None
    for combo in itertools.product(*choices):
        sel = sorted(set(mk) | set(x for c in combo for x in c))
        key = (-float(np.sum(score[sel].astype(np.float64))), sel)
        if best is None or key < best:
            best = key
    return best[1]


@pytest.mark.parametrize("seed", range(40))
def test_select_brute_force(seed):
    rng = np.random.default_rng(9000 + seed)
    T = int(rng.integers(6, 13))
    K = int(rng.integers(2, T))
    p = ams.Params(T=T, window=1, budget=K, delta=float(rng.choice([0.2, 0.34, 0.5])),
                   seg_min=1, seg_max=int(rng.choice([0, 3, 5])), q_min=1,
                   sinks=int(rng.integers(0, 2)), recent=int(rng.integers(0, 3)), pool_kernel=1)
    u = rng.integers(0, 4, size=T).astype(np.float32) / 4     # many ties
    r = ams.mass_and_segments(u, None, p)
    s, rr, t_keep = ams.must_keep(p)
    if r.q.sum() != t_keep:
        return                                              # infeasible floors
    mk = set(range(s)) | set(range(T - rr, T))
    kept = ams.select(r.score, r.segs, r.q, p)
    assert list(kept) == _brute_force_kept(r.score, r.segs, r.q, mk, K)


@pytest.mark.parametrize("seed", range(10))
def test_one_segment_mode_is_global_topk(seed):
    rng = np.random.default_rng(seed)
    T, K = 500, 64
    p = ams.Params(T=T, window=1, budget=K, delta=1.0, seg_min=1, seg_max=0, sinks=0, recent=0,
                   pool_mode=ams.POOL_MAX)
    u = (rng.integers(0, 50, size=T) / 7).astype(np.float32)
    res = _run(u, p)
    assert len(res.segs) == 1
    score = ams.pool(u, p)
    ref = np.sort(np.argsort(-score, kind="stable")[:K])
    np.testing.assert_array_equal(res.kept, ref)


def test_streaming_llm_special_case():
    # budget = sinks + recent: no quota is left, the cache keeps 4 sinks and
    # the K-4 most recent tokens
    T, K = 100, 20
    p = ams.Params(T=T, window=1, budget=K, sinks=4, recent=16)
    res = _run(np.random.default_rng(1).random(T), p)
    np.testing.assert_array_equal(res.kept, np.r_[0:4, 84:100])


def test_recent_shrinks_before_sinks():
    p = ams.Params(T=100, window=1, budget=10, sinks=4, recent=64)
    assert ams.must_keep(p) == (4, 6, 0)
    p = ams.Params(T=100, window=1, budget=3, sinks=4, recent=64)
    assert ams.must_keep(p) == (3, 0, 0)


def test_infeasible_floors_repair_drops_lowest_picks():
    # 6 segments with floor 1 but only 3 free slots: keep the 3 best picks
    T = 60
    u = np.zeros(T, np.float32)
    best = [5, 15, 25, 35, 45, 55]
    vals = [0.5, 0.9, 0.2, 0.9, 0.1, 0.7]
    for t, x in zip(best, vals):
        u[t] = x
    u += np.float32(0.01)
    p = ams.Params(T=T, window=1, budget=3, delta=1.0, seg_min=1, seg_max=10, sinks=0,
                   recent=0, pool_kernel=1)
    res = _run(u, p)
    assert len(res.segs) == 6 and list(res.q) == [1] * 6
    np.testing.assert_array_equal(res.kept, [15, 35, 55])


def test_noop_when_cache_within_budget():
    p = ams.Params(T=10, window=2, budget=16)
    k = np.arange(20, dtype=np.uint16).reshape(10, 2)
    res = ams.steps2to5(np.ones(10, np.float32), k, k + 1, None, p)
    assert res.noop
    np.testing.assert_array_equal(res.kept, np.r_[0:10, [-1] * 6])
    np.testing.assert_array_equal(res.k_out[:10], k)
    assert np.all(res.k_out[10:] == 0)


def test_gather_is_row_indexing():
    rng = np.random.default_rng(3)
    k = rng.integers(0, 65535, size=(30, 8)).astype(np.uint16)
    v = rng.integers(0, 65535, size=(30, 8)).astype(np.uint16)
    c = rng.integers(0, 2 ** 44, size=30).astype(np.uint64)
    kept = np.array([0, 3, 4, 17, 29])
    kf, ko, vo, co = ams.gather(kept, k, v, c, 5)
    for j, t in enumerate(kept):
        assert ko[j].tobytes() == k[t].tobytes() and vo[j].tobytes() == v[t].tobytes()
        assert co[j] == c[t]
    kf, ko, _, _ = ams.gather(np.arange(5), k, v, None, 5)
    np.testing.assert_array_equal(ko, k[:5])


def test_segment_capacity_bounds_every_case():
    rng = np.random.default_rng(77)
    for _ in range(40):
        u, cin, p = _rand_case(rng, T_max=400)
        if p.T <= p.budget:
            continue
        r = ams.mass_and_segments(u, cin, p)
        assert len(r.segs) <= ams.segment_capacity(p)


# ---------------------------------------------------------------------------
# Cut threshold: b_k = min{t : C(t) >= k*Delta} on the normalised cumulative
# mass C(t) = P(t)/V [AMS notes, key design 2, cut equation]
# ---------------------------------------------------------------------------

def test_cut_threshold_rounds_up_between_prefix_values():
    # P = [2, 3, 10], Delta = 0.25: C = [0.2, 0.3, 1.0]. C(0) = 0.2 < 0.25 and
    # C(1) = 0.3 >= 0.25, so the first cut is position 1 (a threshold taken as
    # floor(0.25 * 10) = 2 would wrongly cut at 0); 0.5 and 0.75 are first
    # reached at position 2.
    P = np.array([2, 3, 10], dtype=np.uint64)
    assert ams.thresholds(10, 0.25) == [3, 5, 8]
    assert ams.raw_cuts(P, 0.25) == [1, 2]


@pytest.mark.parametrize("delta", [0.25, 0.125, 0.375, 0.0625, 0.1875, 0.5])
def test_cuts_equal_exact_rational_definition(delta):
    # Dyadic Delta: k*Delta and (k*Delta)*V are exact in fp64, so the cuts must
    # equal the page's real-valued definition evaluated in exact rationals.
    from fractions import Fraction
    rng = np.random.default_rng(int(delta * 1e4))
    for _ in range(40):
        T = int(rng.integers(2, 60))
        v = rng.integers(0, 50, size=T).astype(np.uint64)
        v[int(rng.integers(0, T))] += 1
        P = ams.prefix(v)
        V = int(P[-1])
        want = set()
        k = 1
        while k * Fraction(delta) < 1:
            target = k * Fraction(delta)
            want.add(next(t for t in range(T) if Fraction(int(P[t]), V) >= target))
            k += 1
        want.add(T - 1)
        assert ams.raw_cuts(P, delta) == sorted(want)


# ---------------------------------------------------------------------------
# Under-budget repair: when the picks and must-keep fall short of the budget,
# the highest-scored unselected positions are added [AMS notes, key design 3,
# last paragraph]; reachable when a caller supplies short quotas
# ---------------------------------------------------------------------------

def test_under_budget_repair_adds_highest_scores():
    # one segment of 10, no must-keep, budget 4, caller quota 1: the pick is
    # position 1 (0.9); the repair adds the three best of the rest (0.8, 0.7,
    # 0.6 at 3, 5, 7), not the three worst.
    p = ams.Params(T=10, window=1, budget=4, delta=1.0, seg_min=1, seg_max=0, sinks=0,
                   recent=0, pool_kernel=1)
    score = np.array([0.1, 0.9, 0.3, 0.8, 0.2, 0.7, 0.05, 0.6, 0.4, 0.5], np.float32)
    kept = ams.select(score, [(0, 9)], [1], p)
    assert list(kept) == [1, 3, 5, 7]
    # with must-keep ends (sink 0, recent 9) the one free slot takes 3
    p2 = p.with_(sinks=1, recent=1)
    assert list(ams.select(score, [(0, 9)], [1], p2)) == [0, 1, 3, 9]


@pytest.mark.parametrize("seed", range(30))
def test_under_budget_repair_brute_force(seed):
    # Short caller quotas on tiny caches: the kept set must be must-keep, the
    # per-segment picks, and then the (K - #kept) unselected non-must-keep
    # positions with the largest score sum (ties: smallest index vector).
    rng = np.random.default_rng(4200 + seed)
    T = int(rng.integers(6, 13))
    K = int(rng.integers(3, T))
    p = ams.Params(T=T, window=1, budget=K, delta=float(rng.choice([0.2, 0.34, 0.5])),
                   seg_min=1, seg_max=int(rng.choice([0, 3, 5])), q_min=0,
                   sinks=int(rng.integers(0, 2)), recent=int(rng.integers(0, 3)), pool_kernel=1)
    score = (rng.integers(0, 5, size=T) / 4).astype(np.float32)      # many ties
    r = ams.mass_and_segments(score, None, p)
    s, rr, t_keep = ams.must_keep(p)
    q = np.array([int(rng.integers(0, qi + 1)) for qi in r.q])       # short quotas
    if q.sum() >= t_keep:
        q[:] = 0
    mk = set(range(s)) | set(range(T - rr, T))
    picks = set()
    for (a, b), qi in zip(r.segs, q):
        cand = [t for t in range(a, b + 1) if t not in mk]
        picks |= set(sorted(cand, key=lambda t: (-score[t], t))[:qi])
    base = mk | picks
    free = [t for t in range(T) if t not in base]
    best = None
    for combo in itertools.combinations(free, K - len(base)):
        key = (-float(np.sum(score[list(combo)].astype(np.float64))), list(combo))
        if best is None or key < best:
            best = key
    want = sorted(base | set(best[1]))
    assert list(ams.select(score, r.segs, q, p)) == want
