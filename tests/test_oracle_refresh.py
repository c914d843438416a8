"""Pins for the RefreshKV decode-loop oracle: cosine closed forms and a library
cosine, the trigger's reference-update rule, the page's statement that a
never-refreshed partial cache is SnapKV (the surviving prompt tokens are the
top-(K - m) by score), and the sync round trip."""
import numpy as np
import pytest
from scipy.spatial import distance

from oracle import refresh


def test_cosine_closed_forms():
    a = np.array([1.0, 2.0, -3.0])
    assert refresh.cosine(a, 2.5 * a) == pytest.approx(1.0, abs=1e-15)
    assert refresh.cosine(a, -a) == pytest.approx(-1.0, abs=1e-15)
    assert refresh.cosine(np.array([1.0, 0.0]), np.array([0.0, 3.0])) == 0.0
    assert refresh.cosine(np.zeros(3), a) == 1.0


@pytest.mark.parametrize("seed", range(5))
def test_cosine_equals_library(seed):
    rng = np.random.default_rng(seed)
    a, b = rng.standard_normal(128), rng.standard_normal(128)
    assert refresh.cosine(a, b) == pytest.approx(1.0 - distance.cosine(a, b), abs=1e-12)


def test_head_sum_and_head_mean_decide_alike():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((50, 7, 64))
    ref = rng.standard_normal((50, 64))
    full, cos, _ = refresh.qc_trigger(q, ref, 0.1)
    cos_mean = np.array([1.0 - distance.cosine(q[i].mean(axis=0), ref[i]) for i in range(50)])
    np.testing.assert_allclose(cos, cos_mean, atol=1e-12)
    np.testing.assert_array_equal(full, cos_mean < 0.1)


def test_trigger_updates_reference_only_when_it_fires():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 3, 16))
    ref = np.stack([refresh.head_sum(q[0]), -refresh.head_sum(q[1]),
                    rng.standard_normal(16), np.zeros(16)])
    full, cos, new = refresh.qc_trigger(q, ref, 0.5)
    assert not full[0] and full[1] and not full[3]          # same query; opposite; zero reference
    np.testing.assert_array_equal(new[0], ref[0])
    np.testing.assert_array_equal(new[1], refresh.head_sum(q[1]))
    assert cos[0] == pytest.approx(1.0, abs=1e-12) and cos[1] == pytest.approx(-1.0, abs=1e-12)


def test_trigger_only_strictly_below_the_threshold():
    # [RefreshKV notes, A2: a layer whose similarity falls below s takes a full
    # step] cos((3,4), (4,3)) = 24/25 exactly: at s = 0.96 the row is not below
    # the threshold, at the next double above it is
    q = np.array([[[3.0, 4.0]]])
    ref = np.array([[4.0, 3.0]])
    full, cos, _ = refresh.qc_trigger(q, ref, 0.96)
    assert cos[0] == 0.96 and not full[0]
    full, _, _ = refresh.qc_trigger(q, ref, np.nextafter(0.96, 1.0))
    assert full[0]


def test_untriggered_steps_keep_comparing_with_the_last_full_step():
    # the reference is the query of the layer's last full step: a step that
    # does not trigger leaves it in place, so a slow drift is measured from
    # the last full step, not from the previous token
    ref = np.array([[1.0, 0.0]])
    full1, _, ref1 = refresh.qc_trigger(np.array([[[1.0, 0.1]]]), ref, 0.75)    # cos 0.995
    assert not full1[0]
    np.testing.assert_array_equal(ref1, ref)
    full2, cos2, ref2 = refresh.qc_trigger(np.array([[[0.7, 0.7]]]), ref1, 0.75)
    assert cos2[0] == pytest.approx(np.sqrt(0.5), abs=1e-15)    # against (1, 0), not (1, 0.1)
    assert full2[0]
    np.testing.assert_array_equal(ref2[0], [0.7, 0.7])


@pytest.mark.parametrize("seed", range(4))
def test_never_refreshed_partial_cache_is_snapkv(seed):
    # After m partial steps without a refresh, the prompt tokens still in C_p
    # are the top-(K - m) of the full step's scores (ties to the lower slot),
    # and all m new tokens are present.
    rng = np.random.default_rng(seed)
    K, m, d = 32, 11, 4
    kept = np.sort(rng.choice(500, K, replace=False))
    score = rng.random(500).astype(np.float32)
    score[kept[3]] = score[kept[9]]                           # a tie
    sc, pos = refresh.partial_init(kept, score)
    kp, vp = np.zeros((K, d)), np.zeros((K, d))
    for i in range(m):
        refresh.partial_append(sc, pos, kp, vp, np.full(d, i), np.full(d, -i), 500 + i)
    survivors = sorted(p for p in pos if p < 500)
    order = sorted(range(K), key=lambda j: (-score[kept[j]], -j))[:K - m]
    assert survivors == sorted(int(kept[j]) for j in order)
    assert sorted(p for p in pos if p >= 500) == list(range(500, 500 + m))


def test_partial_init_gathers_scores():
    score = np.arange(10, dtype=np.float32) * 0.5
    sc, pos = refresh.partial_init(np.array([1, 4, 9, -1]), score)
    np.testing.assert_array_equal(sc, [0.5, 2.0, 4.5, np.inf])
    np.testing.assert_array_equal(pos, [1, 4, 9, -1])


def test_full_sync_round_trip():
    rng = np.random.default_rng(3)
    K, d, T0 = 16, 8, 100
    kf, vf = rng.standard_normal((120, d)), rng.standard_normal((120, d))
    kf0 = kf.copy()
    kept = np.sort(rng.choice(T0, K, replace=False))
    sc, pos = refresh.partial_init(kept, rng.random(T0).astype(np.float32))
    kp, vp = kf[kept].copy(), vf[kept].copy()
    new_k = rng.standard_normal((5, d))
    for i in range(5):
        refresh.partial_append(sc, pos, kp, vp, new_k[i], -new_k[i], T0 + i)
    refresh.full_sync(pos, kp, vp, kf, vf, T0)
    np.testing.assert_array_equal(kf[T0:T0 + 5], new_k)
    np.testing.assert_array_equal(vf[T0:T0 + 5], -new_k)
    np.testing.assert_array_equal(kf[:T0], kf0[:T0])


def test_partial_append_tie_takes_first_slot():
    # Convention (the page leaves ties open): among equal lowest scores the
    # first slot is evicted.
    sc = np.array([0.5, 0.2, 0.9, 0.2, 0.2], np.float32)
    pos = np.array([10, 11, 12, 13, 14])
    kp, vp = np.zeros((5, 2)), np.zeros((5, 2))
    slot = refresh.partial_append(sc, pos, kp, vp, np.ones(2), -np.ones(2), 99)
    assert slot == 1 and pos[1] == 99 and sc[1] == np.inf
    slot = refresh.partial_append(sc, pos, kp, vp, np.ones(2), -np.ones(2), 100)
    assert slot == 3 and list(pos) == [10, 99, 12, 100, 14]
