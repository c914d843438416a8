"""Pins for the oracle's paged-KV compaction: reading the compacted blocks back
through the new block table must give the contiguous gather of the logical
cache, and no block outside the new table may change."""
import numpy as np
import pytest

from oracle import ams


def _setup(seed, B=3, H=2, T=37, bs=8, d=4, K=13, spare=6):
    rng = np.random.default_rng(seed)
    nb_in = -(-T // bs)
    nb_out = -(-K // bs)
    n_blocks = B * (nb_in + nb_out) + spare
    perm = rng.permutation(n_blocks)
    table_in = perm[:B * nb_in].reshape(B, nb_in)
    table_out = perm[B * nb_in:B * (nb_in + nb_out)].reshape(B, nb_out)
    k_pool = rng.integers(0, 1 << 16, (n_blocks, H, bs, d), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, (n_blocks, H, bs, d), dtype=np.uint16)
    kept = np.stack([np.sort(rng.choice(T, K, replace=False)) for _ in range(B * H)])
    return k_pool, v_pool, table_in, table_out, kept, (B, H, T, bs, d, K)


@pytest.mark.parametrize("seed", range(4))
def test_paged_equals_contiguous_gather(seed):
    k_pool, v_pool, tin, tout, kept, (B, H, T, bs, d, K) = _setup(seed)
    kn, vn = ams.gather_paged(kept, k_pool, v_pool, tin, tout, H)
    for n in range(B * H):
        b, h = divmod(n, H)
        k_log = ams.read_paged(k_pool, tin, b, h, T)
        v_log = ams.read_paged(v_pool, tin, b, h, T)
        _, k_ref, v_ref, _ = ams.gather(kept[n], k_log, v_log, None, K)
        np.testing.assert_array_equal(ams.read_paged(kn, tout, b, h, K), k_ref)
        np.testing.assert_array_equal(ams.read_paged(vn, tout, b, h, K), v_ref)


def test_paged_leaves_other_blocks_alone():
    k_pool, v_pool, tin, tout, kept, (B, H, T, bs, d, K) = _setup(9)
    kn, vn = ams.gather_paged(kept, k_pool, v_pool, tin, tout, H)
    untouched = np.setdiff1d(np.arange(k_pool.shape[0]), tout.ravel())
    np.testing.assert_array_equal(kn[untouched], k_pool[untouched])
    np.testing.assert_array_equal(vn[untouched], v_pool[untouched])


def test_paged_empty_slots_are_zero_and_heads_differ():
    k_pool, v_pool, tin, tout, kept, (B, H, T, bs, d, K) = _setup(3)
    kept = kept.copy()
    kept[1, -3:] = -1
    kn, _ = ams.gather_paged(kept, k_pool, v_pool, tin, tout, H)
    rows = ams.read_paged(kn, tout, 0, 1, K)
    np.testing.assert_array_equal(rows[-3:], 0)
    # same compacted slot, different heads, different original positions
    assert kept[0, 0] != kept[1, 0] or kept[0, 1] != kept[1, 1]
