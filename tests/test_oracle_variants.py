"""Pins for the oracle's ablation variants and its ragged (left-padded)
events: hand-derived closed forms, independence properties and the padding
semantics checked against a direct masked-softmax evaluation on the padded
arrays."""
import numpy as np
import pytest

from oracle import ams


def _steps(u, p):
    return ams.steps2to5(np.asarray(u, np.float32), np.zeros((p.T, 2), np.uint16),
                         np.zeros((p.T, 2), np.uint16), None, p)


# ---------------------------------------------------------------------------
# fixed-length segments
# ---------------------------------------------------------------------------

def test_fixed_cuts_closed_form():
    assert ams.fixed_cuts(64, 16) == [15, 31, 47, 63]
    assert ams.fixed_cuts(70, 16) == [15, 31, 47, 63, 69]
    assert ams.fixed_cuts(10, 16) == [9]
    assert ams.fixed_cuts(16, 16) == [15]


def test_fixed_segments_merge_tail_and_split():
    v = np.ones(70, np.uint64)
    P = ams.prefix(v)
    p = ams.Params(T=70, window=8, budget=8, seg_min=16, seg_max=256, seg_fixed=16)
    # the 6-long tail is shorter than seg_min and joins its left neighbour
    assert ams.segment(P, p) == [(0, 15), (16, 31), (32, 47), (48, 69)]
    p2 = p.with_(seg_min=4, seg_max=8)
    assert ams.segment(P, p2) == [(0, 7), (8, 15), (16, 23), (24, 31), (32, 39), (40, 47),
                                  (48, 55), (56, 63), (64, 69)]


@pytest.mark.parametrize("seed", range(5))
def test_fixed_segments_ignore_mass(seed):
    rng = np.random.default_rng(seed)
    p = ams.Params(T=300, window=8, budget=40, seg_fixed=32, seg_min=16, seg_max=256)
    segs = [ams.segment(ams.prefix(rng.integers(1, 1 << 40, 300, dtype=np.uint64)), p)
            for _ in range(3)]
    assert segs[0] == segs[1] == segs[2]
    assert segs[0] == [(i * 32, i * 32 + 31) for i in range(8)] + [(256, 299)]


def test_fixed_segments_capacity():
    for T, L, smax in [(70, 16, 256), (70, 16, 8), (1000, 7, 0), (1024, 1024, 256)]:
        p = ams.Params(T=T, window=4, budget=8, seg_fixed=L, seg_min=1, seg_max=smax)
        segs = ams.segment(ams.prefix(np.ones(T, np.uint64)), p)
        assert len(segs) <= ams.segment_capacity(p)


# ---------------------------------------------------------------------------
# uniform (not mass-weighted) quotas
# ---------------------------------------------------------------------------

def test_uniform_quota_hand_case():
    # 4 segments of 16, no must-keep, budget 10: floors 1 each, T_rem = 6,
    # share 1.5 rounds to 2 -> 3 each = 12; the excess 2 comes back one per
    # segment in (weight asc, index desc) order = segments 3 then 2.
    p = ams.Params(T=64, window=8, budget=10, seg_min=4, seg_max=16, sinks=0, recent=0,
                   seg_fixed=16, quota_mode=ams.QUOTA_UNIFORM)
    v = np.arange(1, 65, dtype=np.uint64)
    segs = ams.segment(ams.prefix(v), p)
    assert list(ams.quotas(segs, v, p)[0]) == [3, 3, 2, 2]


def test_uniform_quota_clip_then_index_order():
    # segments of 16, 16, 4, 16 (seg_min 4): floors 1, T_rem = 36, share 9 ->
    # [10, 10, 4 (clipped from 10), 10] = 34; the shortfall 6 goes one per
    # segment per cycle to the segments with room, in index order.
    p = ams.Params(T=52, window=4, budget=40, seg_min=4, seg_max=16, sinks=0, recent=0,
                   quota_mode=ams.QUOTA_UNIFORM)
    segs = [(0, 15), (16, 31), (32, 35), (36, 51)]
    v = np.ones(52, np.uint64)
    q = ams.quotas(segs, v, p)[0]
    assert list(q) == [12, 12, 4, 12]


@pytest.mark.parametrize("seed", range(5))
def test_uniform_quota_ignores_mass(seed):
    rng = np.random.default_rng(seed)
    p = ams.Params(T=400, window=8, budget=200, seg_fixed=50, quota_mode=ams.QUOTA_UNIFORM)
    segs = ams.segment(ams.prefix(np.ones(400, np.uint64)), p)
    qs = [tuple(ams.quotas(segs, rng.integers(1, 1 << 44, 400, dtype=np.uint64), p)[0])
          for _ in range(3)]
    assert qs[0] == qs[1] == qs[2]
    assert sum(qs[0]) == ams.must_keep(p)[2]


def test_mass_mode_is_default_and_differs():
    v = np.ones(64, np.uint64)
    v[:16] = 1000
    p = ams.Params(T=64, window=8, budget=12, seg_min=4, seg_max=16, sinks=0, recent=0,
                   seg_fixed=16)
    segs = ams.segment(ams.prefix(v), p)
    qm = list(ams.quotas(segs, v, p)[0])
    qu = list(ams.quotas(segs, v, p.with_(quota_mode=ams.QUOTA_UNIFORM))[0])
    assert qm[0] > qm[1] and qu == [3, 3, 3, 3]


# ---------------------------------------------------------------------------
# ragged (left-padded) events
# ---------------------------------------------------------------------------

def _head(rng, T, G, W, d):
    q = rng.standard_normal((G, W, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    return q, k, v


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_ragged_full_length_is_the_plain_event():
    rng = np.random.default_rng(1)
    p = ams.Params(T=200, window=16, budget=48, group=2, head_dim=8, seg_min=4, seg_max=32)
    q, k, v = _head(rng, 200, 2, 16, 8)
    a = ams.event(q, k, _bits(v), None, p)
    b = ams.event_ragged(q, k, _bits(v), None, p, 200)
    np.testing.assert_array_equal(a.u, b.u)
    assert a.segs == b.segs
    np.testing.assert_array_equal(a.kept, b.kept)
    np.testing.assert_array_equal(a.v_out, b.v_out)


@pytest.mark.parametrize("pad", [1, 17, 63])
def test_ragged_padding_never_leaks(pad):
    # Padding rows hold huge garbage; the result must equal the event on the
    # real tokens alone, shifted by the pad count.
    rng = np.random.default_rng(pad)
    T, G, W, d = 180, 2, 12, 8
    p = ams.Params(T=T, window=W, budget=40, group=G, head_dim=d, seg_min=4, seg_max=32,
                   ema=True)
    q, k, v = _head(rng, T, G, W, d)
    k[:pad] = 1e3 * rng.standard_normal((pad, d))
    v[:pad] = 7.0
    res = ams.event_ragged(q, k, _bits(v), None, p, T - pad)
    ref = ams.event(q, k[pad:], _bits(v[pad:]), None, p.with_(T=T - pad))
    np.testing.assert_array_equal(res.u[:pad], 0.0)
    np.testing.assert_array_equal(res.u[pad:], ref.u)
    np.testing.assert_array_equal(res.credit_upd[:pad], 0)
    np.testing.assert_array_equal(res.credit_upd[pad:], ref.credit_upd)
    assert res.segs == [(a + pad, b + pad) for a, b in ref.segs]
    np.testing.assert_array_equal(res.kept, np.where(ref.kept >= 0, ref.kept + pad, -1))
    np.testing.assert_array_equal(res.v_out, ref.v_out)


def test_ragged_step1_equals_masked_softmax():
    # The pad mask M of a batched decode: pad keys get -inf before the
    # softmax; rows are the window queries, the causal limit as usual.
    rng = np.random.default_rng(7)
    T, G, W, d, pad = 96, 3, 8, 16, 21
    p = ams.Params(T=T, window=W, budget=32, group=G, head_dim=d)
    q, k, _ = _head(rng, T, G, W, d)
    u = ams.window_usage_ragged(q, k, p, T - pad)
    s = np.einsum("gwd,td->gwt", q, k) / np.sqrt(d)
    pos = np.arange(T)
    for w in range(W):
        s[:, w, pos > T - W + w] = -np.inf
    s[:, :, :pad] = -np.inf
    e = np.exp(s - s.max(axis=2, keepdims=True))
    a = (e / e.sum(axis=2, keepdims=True)).sum(axis=(0, 1))
    seen = np.minimum(W, T - pos)        # queries that see position t
    full = a[pad:T - W + 1].max()
    want = np.where(seen < W, full, a)
    want[:pad] = 0.0
    np.testing.assert_allclose(u, want, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("length", [5, 40, 120, 200])
def test_ragged_budget_invariants(length):
    rng = np.random.default_rng(length)
    T, W, K = 200, 8, 48
    p = ams.Params(T=T, window=W, budget=K, seg_min=4, seg_max=32)
    u = rng.random(T).astype(np.float32)
    res = ams.steps2to5_ragged(u, np.zeros((T, 2), np.uint16), np.zeros((T, 2), np.uint16),
                               None, p, length)
    Tn = max(length, W)
    off = T - Tn
    kept = res.kept[res.kept >= 0]
    assert len(kept) == min(K, Tn)
    assert kept.min() >= off and np.all(np.diff(kept) > 0)
    s, r, _ = ams.must_keep(p.with_(T=Tn))
    assert set(range(off, off + s)) | set(range(T - r, T)) <= set(kept.tolist())
    np.testing.assert_array_equal(res.score[:off], 0.0)


@pytest.mark.parametrize("length", [20, 37, 60])
def test_ragged_carried_credit_covers_only_real_tokens(length):
    # credit_in[j] belongs to real token j [AMS notes, key design 1: credit
    # follows the kept positions]; a head shorter than the carried credit is
    # the plain event on its real tokens with the first `length` credits
    rng = np.random.default_rng(length)
    T, W, K, n_prev = 120, 8, 16, 37
    p = ams.Params(T=T, window=W, budget=K, seg_min=4, seg_max=16, ema=True, n_prev=n_prev)
    u = (rng.random(T) ** 2).astype(np.float32)
    r = rng.random(n_prev) + 1e-3
    credit = np.floor(r / r.sum() * 2.0 ** 44).astype(np.uint64)
    z = np.zeros((T, 2), np.uint16)
    res = ams.steps2to5_ragged(u, z, z, credit, p, length)
    off = T - length
    ref = ams.steps2to5(u[off:], z[off:], z[off:], credit[:min(n_prev, length)],
                        p.with_(T=length, n_prev=min(n_prev, length)))
    np.testing.assert_array_equal(res.credit_upd[off:], ref.credit_upd)
    np.testing.assert_array_equal(res.credit_upd[:off], 0)
    np.testing.assert_array_equal(res.kept, np.where(ref.kept >= 0, ref.kept + off, -1))
    np.testing.assert_array_equal(res.credit_out, ref.credit_out)


def test_ragged_clamps_short_lengths_to_the_window():
    rng = np.random.default_rng(3)
    p = ams.Params(T=64, window=16, budget=8, seg_min=4, seg_max=16)
    u = rng.random(64).astype(np.float32)
    z = np.zeros((64, 2), np.uint16)
    a = ams.steps2to5_ragged(u, z, z, None, p, 3)
    b = ams.steps2to5_ragged(u, z, z, None, p, 16)
    np.testing.assert_array_equal(a.kept, b.kept)


def test_uniform_quota_weighs_unequal_segments_alike():
    # Convention for "no mass-weighted quota": every segment weighs 1, not its
    # length.  Segments of 10 and 30 positions, floors 1 each, T_rem = 4:
    # equal weights give shares (2, 2); length weights would give (1, 3).
    p = ams.Params(T=40, window=4, budget=6, seg_min=1, seg_max=0, sinks=0, recent=0,
                   quota_mode=ams.QUOTA_UNIFORM)
    segs = [(0, 9), (10, 39)]
    v = np.arange(1, 41, dtype=np.uint64)
    assert list(ams.quotas(segs, v, p)[0]) == [3, 3]
    # T_rem = 5: shares 2.5 round up to 3 each (one too many); the excess comes
    # back from the higher index first (equal weights, index desc).  Length
    # weights would give (2, 5).
    assert list(ams.quotas(segs, v, p.with_(budget=7))[0]) == [4, 3]
