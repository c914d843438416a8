"""GPU parity on the method's degenerate inputs, same acceptance as
tests/test_gpu_parity.py: all keys zero (every softmax uniform, so the usage is
flat and the mass cuts, quotas and selection run on exact ties everywhere),
a window as long as the cache (every position only partly observed), a
one-position cache, and a budget of one."""
import numpy as np
import pytest

from eviction_window_qk_amd import synth
from test_gpu_parity import _pd, _run_case

DEGENERATE = [
    # (label, NH, G, W, d, T, K, overrides, zero_keys)
    ("zero_keys", 2, 2, 16, 64, 300, 100, {}, True),
    ("zero_keys_ema", 2, 2, 16, 64, 300, 100, dict(ema=True), True),
    ("zero_keys_one_segment", 2, 2, 16, 64, 300, 100,
     dict(delta=1.0, seg_min=1, seg_max=0, sinks=0, recent=0, pool_mode=1), True),
    ("window_eq_T", 2, 2, 64, 64, 64, 20, {}, False),
    ("T1", 2, 1, 1, 64, 1, 1, dict(seg_min=1, sinks=0, recent=0), False),
    ("budget_1", 2, 2, 8, 64, 200, 1, {}, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", DEGENERATE, ids=[c[0] for c in DEGENERATE])
def test_degenerate(case):
    label, NH, G, W, d, T, K, over, zero_keys = case
    q, k, v = synth.random_small(sum(map(ord, label)), NH, G, W, d, T)
    if zero_keys:
        k[:] = 0
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, **over)
    u_gpu, u_ref, ev = _run_case(pd, q, k, v, label=label)
    if zero_keys:  # flat usage: every position scores the same
        assert np.ptp(u_ref, axis=1).max() < 1e-12 * u_ref.max()
