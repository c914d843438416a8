"""Pins for the oracle's window score (step 1), independent of its own code.

Each test fixes the result by something other than the oracle: a closed form,
a library routine, an invariant of softmax, or a pure-Python triple loop.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import ams, loops
from eviction_window_qk_amd import synth


def _params(T, W, G, d, agg=ams.AGG_SUM, **kw):
    return ams.Params(T=T, window=W, budget=max(1, T // 4), group=G, head_dim=d, head_agg=agg, **kw)


def _rand(seed, G, W, T, d, kscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, W, d))
    k = rng.standard_normal((T, d)) * kscale
    return q, k


def test_single_query_is_one_softmax_row():
    # G = W = 1: the one query sits at T-1 and sees every key, so the usage is
    # exactly one softmax row (library routine) with scale 1/sqrt(d).
    T, d = 37, 16
    q, k = _rand(1, 1, 1, T, d, kscale=2.0)
    p = _params(T, 1, 1, d)
    u = ams.window_usage(q, k, p)
    ref = scipy.special.softmax((q[0, 0] @ k.T) / math.sqrt(d))
    np.testing.assert_allclose(u, ref, rtol=1e-12, atol=0)


def test_explicit_scale_is_used():
    T, d = 20, 8
    q, k = _rand(2, 1, 1, T, d)
    p = _params(T, 1, 1, d, scale=0.37)
    u = ams.window_usage(q, k, p)
    np.testing.assert_allclose(u, scipy.special.softmax(0.37 * (q[0, 0] @ k.T)), rtol=1e-12)


@pytest.mark.parametrize("T,W,G", [(10, 4, 1), (33, 8, 3), (64, 1, 2), (17, 17, 1)])
def test_identical_keys_closed_form(T, W, G):
    # All keys equal => each query spreads 1 uniformly over the keys it sees:
    # query w (position T-W+w) gives 1/(T-W+w+1) to every t <= T-W+w.
    d = 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((G, W, d))
    k = np.tile(rng.standard_normal(d), (T, 1))
    p = _params(T, W, G, d)
    u0 = ams.window_usage_unfilled(q, k, p)
    expect = np.zeros(T)
    for w in range(W):
        last = T - W + w
        expect[: last + 1] += G / (last + 1)
    np.testing.assert_allclose(u0, expect, rtol=1e-12)
    u = ams.window_usage(q, k, p)
    full = G * sum(1.0 / (T - W + w + 1) for w in range(W))
    np.testing.assert_allclose(u[: T - W + 1], full, rtol=1e-12)
    np.testing.assert_allclose(u[T - W + 1:], full, rtol=1e-12)  # fill = window max


@pytest.mark.parametrize("seed", range(4))
def test_rows_sum_to_one(seed):
    # Each causal softmax row sums to 1, so before the fill sum_t u_t = W*G.
    G, W, T, d = 3, 9, 50, 16
    q, k = _rand(seed, G, W, T, d, kscale=3.0)
    u0 = ams.window_usage_unfilled(q, k, _params(T, W, G, d))
    assert abs(u0.sum() - W * G) < 1e-10


def test_causal_tail_counts():
    # The last position is seen only by the last query: with identical keys
    # its unfilled usage is G/T; position T-W is seen by all W queries.
    G, W, T, d = 2, 5, 12, 4
    q = np.ones((G, W, d))
    k = np.ones((T, d))
    u0 = ams.window_usage_unfilled(q, k, _params(T, W, G, d))
    assert abs(u0[T - 1] - G / T) < 1e-14
    assert abs(u0[T - W] - G * sum(1 / (T - W + w + 1) for w in range(W))) < 1e-14


def test_group_aggregation_sum_vs_max():
    G, W, T, d = 4, 6, 30, 8
    q, k = _rand(5, G, W, T, d, kscale=2.0)
    us = ams.window_usage_unfilled(q, k, _params(T, W, G, d, ams.AGG_SUM))
    um = ams.window_usage_unfilled(q, k, _params(T, W, G, d, ams.AGG_MAX))
    assert np.all(um <= us + 1e-15)
    assert np.all(um * G >= us - 1e-12)
    q1 = q[:1]
    u1s = ams.window_usage_unfilled(q1, k, _params(T, W, 1, d, ams.AGG_SUM))
    u1m = ams.window_usage_unfilled(q1, k, _params(T, W, 1, d, ams.AGG_MAX))
    np.testing.assert_array_equal(u1s, u1m)   # G = 1: SUM == MAX


def test_group_member_order_matters_only_through_rows():
    # Swapping the query heads permutes nothing in u (sum/max over g).
    G, W, T, d = 3, 4, 20, 8
    q, k = _rand(6, G, W, T, d)
    p = _params(T, W, G, d)
    np.testing.assert_allclose(ams.window_usage(q, k, p), ams.window_usage(q[::-1], k, p), rtol=1e-13)


def test_fill_rule():
    u = np.array([0.1, 0.5, 0.2, 0.3, 0.05, 0.01, 0.02])
    out = ams.fill_partial(u, 3)          # T=7, fully seen t <= 4
    np.testing.assert_array_equal(out, [0.1, 0.5, 0.2, 0.3, 0.05, 0.5, 0.5])
    np.testing.assert_array_equal(ams.fill_partial(u, 1), u)


@pytest.mark.parametrize("seed,G,W,T,d,agg", [(0, 1, 3, 9, 4, 0), (1, 2, 4, 13, 5, 0),
                                              (2, 3, 2, 7, 3, 1), (3, 2, 6, 6, 2, 1)])
def test_numpy_equals_triple_loop(seed, G, W, T, d, agg):
    q, k = _rand(seed, G, W, T, d, kscale=1.5)
    p = _params(T, W, G, d, agg)
    a = ams.window_usage(q, k, p)
    b = loops.fill(loops.usage_unfilled(q.tolist(), k.tolist(), p), W)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_bf16_inputs_widen_exactly():
    wl = synth.WORKLOADS["tiny"]
    hd = synth.gen_head(wl, 0)
    kf = synth.bf16_bits_to_f32(hd["k"])
    # bf16 -> fp32 -> fp64 is exact; re-rounding gives the same bits back
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(kf), hd["k"])
    assert np.all((kf.view(np.uint32) & 0xFFFF) == 0)
