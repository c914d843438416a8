"""Pins for the oracle's mass step (pooling, fixed-point mass, EMA, prefix)."""
import math

import numpy as np
import pytest
import torch

from oracle import ams, loops


def _p(T, **kw):
    return ams.Params(T=T, window=4, budget=max(1, T // 4), **kw)


@pytest.mark.parametrize("seed,T", [(0, 50), (1, 7), (2, 3), (3, 1000)])
def test_avg_pool_matches_torch(seed, T):
    rng = np.random.default_rng(seed)
    u = (rng.random(T) * rng.choice([1e-6, 1.0, 30.0], size=T)).astype(np.float32)
    got = ams.pool(u, _p(T))
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(u)[None, None], 7, 1, 3,
                                         count_include_pad=False)[0, 0].numpy()
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -21, atol=0)


@pytest.mark.parametrize("seed,T,k", [(0, 50, 7), (1, 9, 3), (2, 2, 7), (3, 64, 5)])
def test_max_pool_matches_torch_exactly(seed, T, k):
    u = np.random.default_rng(seed).random(T).astype(np.float32)
    got = ams.pool(u, _p(T, pool_mode=ams.POOL_MAX, pool_kernel=k))
    ref = torch.nn.functional.max_pool1d(torch.from_numpy(u)[None, None], k, 1, k // 2)[0, 0].numpy()
    np.testing.assert_array_equal(got, ref)


def test_avg_pool_of_dyadic_constant_is_constant():
    u = np.full(40, 0.75, dtype=np.float32)
    np.testing.assert_array_equal(ams.pool(u, _p(40)), u)


def test_avg_pool_edges_count_in_range_only():
    u = np.zeros(10, dtype=np.float32)
    u[0] = 4.0
    got = ams.pool(u, _p(10))
    # t=0 sees j in [0,3] (4 values), t=3 sees [0,6] (7 values), t=4 does not see 0
    assert got[0] == np.float32(1.0) and got[3] == np.float32(4.0) / np.float32(7.0)
    assert got[4] == 0.0


def test_pool_loops_agree():
    rng = np.random.default_rng(9)
    for mode in (0, 1):
        u = rng.random(23).astype(np.float32)
        p = _p(23, pool_mode=mode)
        np.testing.assert_array_equal(ams.pool(u, p), np.array(loops.pool(u, p), dtype=np.float32))


@pytest.mark.parametrize("seed", range(3))
def test_mass_is_the_pages_equation(seed):
    # m_i = (max(u_i,0)+eps)/sum(max(u_v,0)+eps), evaluated directly in fp64,
    # agrees with the fixed-point mass to the 2^-40 quantum; sum m = 1; m > 0.
    rng = np.random.default_rng(seed)
    T = 300
    ubar = (rng.random(T) ** 4 * 50).astype(np.float32)
    ubar[::17] = 0.0
    p = _p(T)
    m = ams.mass_fraction(ams.usage_fixed(ubar, p))
    num = np.maximum(ubar.astype(np.float64), 0.0) + p.eps
    exact = num / num.sum()
    np.testing.assert_allclose(m, exact, rtol=1e-6)
    assert abs(m.sum() - 1.0) < T * 2.0 ** -52
    assert np.all(m > 0)


def test_eps_quantum():
    assert ams.eps_fixed(1e-6) == 1099512          # ceil(1e-6 * 2^40)
    w = ams.usage_fixed(np.array([0.0, 1.0, 2.0 ** -40, 3.5], dtype=np.float32), _p(4))
    assert list(map(int, w)) == [1099512, 2 ** 40 + 1099512, 1 + 1099512, 7 * 2 ** 39 + 1099512]


def test_negative_usage_counts_as_zero():
    # m_i = (max(u_i, 0) + eps) / sum [AMS notes, key design 1, mass equation]:
    # a negative (or negative-zero) usage adds exactly the eps quantum, the
    # same as a zero usage; its magnitude does not count
    w = ams.usage_fixed(np.array([-1.0, -0.0, 0.0, -2.0 ** -30, 2.0], dtype=np.float32), _p(5))
    assert list(map(int, w)) == [1099512, 1099512, 1099512, 1099512, 2 ** 41 + 1099512]


def test_prefix_is_sequential_sum():
    rng = np.random.default_rng(4)
    v = rng.integers(0, 2 ** 50, size=500).astype(np.uint64)
    P = ams.prefix(v)
    run = 0
    for t in range(500):
        run += int(v[t])
        assert int(P[t]) == run


def _w(seed, T):
    rng = np.random.default_rng(seed)
    ubar = (rng.random(T) * 5).astype(np.float32)
    return ams.usage_fixed(ubar, _p(T))


def test_ema_lambda_zero_credit_is_current_mass():
    T = 64
    w = _w(0, T)
    cin = np.random.default_rng(1).integers(0, 2 ** 40, size=T).astype(np.uint64)
    p = _p(T, ema=True, lam=0.0, n_prev=T)
    _, cq = ams.ema_credit(w, cin, p)
    mq = w.astype(np.float64) / float(int(w.sum()))
    np.testing.assert_array_equal(cq, np.floor(mq * 2.0 ** 44).astype(np.uint64))


def test_ema_lambda_one_keeps_credit():
    T = 64
    w = _w(2, T)
    cin = np.random.default_rng(3).integers(0, 2 ** 44, size=T).astype(np.uint64)
    p = _p(T, ema=True, lam=1.0, n_prev=40)
    _, cq = ams.ema_credit(w, cin, p)
    np.testing.assert_array_equal(cq[:40], cin[:40])


def test_ema_beta_one_uses_current_mass_only():
    T = 64
    w = _w(4, T)
    cin = np.random.default_rng(5).integers(0, 2 ** 44, size=T).astype(np.uint64)
    v, _ = ams.ema_credit(w, cin, _p(T, ema=True, beta=1.0, n_prev=T))
    mq = w.astype(np.float64) / float(int(w.sum()))
    np.testing.assert_array_equal(v, np.floor(mq * 2.0 ** 44).astype(np.uint64))


def test_ema_first_event_is_identity_up_to_quantum():
    # n_prev = 0: every position starts from its current mass, so the credit
    # equals the mass and the mixed mass equals it too (to the Q44 quantum).
    T = 200
    w = _w(6, T)
    v, cq = ams.ema_credit(w, None, _p(T, ema=True))
    mq = w.astype(np.float64) / float(int(w.sum()))
    assert np.max(np.abs(cq.astype(np.float64) * 2.0 ** -44 - mq)) < 2 * 2.0 ** -44
    mix = v.astype(np.float64) / float(int(v.sum()))
    np.testing.assert_allclose(mix, mq, rtol=1e-9)


def test_ema_matches_real_valued_equation():
    # c <- lam*c + (1-lam)*m ; m_used = normalize(beta*m + (1-beta)*normalize(c))
    T = 128
    w = _w(7, T)
    rng = np.random.default_rng(8)
    cin = (rng.random(T) * 2.0 ** 38).astype(np.uint64)
    p = _p(T, ema=True, lam=0.8, beta=0.7, n_prev=100)
    v, cq = ams.ema_credit(w, cin, p)
    m = w.astype(np.float64) / float(int(w.sum()))
    c = np.where(np.arange(T) < 100, cin.astype(np.float64) * 2.0 ** -44, m)
    c_new = 0.8 * c + 0.2 * m
    used = 0.7 * m + 0.3 * c_new / c_new.sum()
    used /= used.sum()
    np.testing.assert_allclose(cq.astype(np.float64) * 2.0 ** -44, c_new, rtol=1e-9, atol=2.0 ** -43)
    np.testing.assert_allclose(v.astype(np.float64) / float(int(v.sum())), used, rtol=1e-9)


def test_ema_constant_mass_converges_to_mass():
    T = 50
    w = _w(9, T)
    cq = np.random.default_rng(10).integers(0, 2 ** 44, size=T).astype(np.uint64)
    p = _p(T, ema=True, lam=0.5, n_prev=T)
    for _ in range(80):
        _, cq = ams.ema_credit(w, cq, p)
    mq = w.astype(np.float64) / float(int(w.sum()))
    assert np.max(np.abs(cq.astype(np.float64) * 2.0 ** -44 - mq)) < 1e-12


@pytest.mark.parametrize("ema", [False, True])
def test_mass_loops_agree(ema):
    rng = np.random.default_rng(11)
    T = 40
    ubar = (rng.random(T) * 3).astype(np.float32)
    cin = rng.integers(0, 2 ** 43, size=T).astype(np.uint64)
    p = _p(T, ema=ema, n_prev=25 if ema else 0, lam=0.6, beta=0.75)
    w = ams.usage_fixed(ubar, p)
    v, cq = ams.ema_credit(w, cin, p) if ema else (w, None)
    lv, lcq = loops.mass_v(ubar, cin, p)
    assert list(map(int, v)) == lv
    if ema:
        assert list(map(int, cq)) == lcq


def test_overflow_bound_for_largest_workload():
    # E4: sum(ubar) <= F*W^2*G (F = 2 average, the width for max pooling) and
    # F*W^2*G*2^40 + T*e < 2^63 for every workload
    for W, G, T, F in [(32, 1, 1024, 2), (128, 7, 768, 2), (128, 7, 1536, 2), (32, 4, 16384, 7),
                       (128, 4, 131072, 2)]:
        assert F * W * W * G < 2 ** 22
        assert F * W * W * G * 2 ** 40 + T * ams.eps_fixed(1e-6) < 2 ** 63
    assert math.ceil(1e-6 * 2 ** 40) == 1099512


@pytest.mark.parametrize("mode,width", [(ams.POOL_AVG, 7), (ams.POOL_AVG, 1), (ams.POOL_AVG, 63),
                                        (ams.POOL_MAX, 7), (ams.POOL_MAX, 63)])
def test_pooled_usage_sum_bound(mode, width):
    # The bound the parameters are checked against: the filled usage sums to
    # at most W*W*G, and pooling multiplies that by less than 2 (average) or by
    # at most the width (max).  The extreme case is every query attending to
    # one key (its usage W*G, copied by the fill into W-1 positions).
    rng = np.random.default_rng(width)
    W, G, T, d = 8, 3, 200, 16
    F = width if mode == ams.POOL_MAX else 2
    p = ams.Params(T=T, window=W, budget=16, group=G, head_dim=d, pool_kernel=width,
                   pool_mode=mode)
    for trial in range(4):
        k = rng.standard_normal((T, d))
        q = rng.standard_normal((G, W, d))
        if trial >= 2:                     # one key dominates every row
            k[int(rng.integers(0, T - W))] = 40.0 * np.sign(q.sum(axis=(0, 1)))
        u = ams.window_usage(q, k, p)
        assert u.sum() <= W * W * G * (1 + 1e-12)
        assert float(ams.pool(u.astype(np.float32), p).astype(np.float64).sum()) <= \
            F * W * W * G * (1 + 1e-6)
