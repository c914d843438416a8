"""GPU parity of the quota redistribution on heads with more than 64 segments.

After the mass-weighted shares are rounded and clipped, the quotas still miss
the budget by some D; the cyclic walk hands the shortfall out (D > 0, order:
mass descending, index ascending) or takes the excess back (D < 0, order:
mass ascending, index descending) [AMS notes, key design 3].  Up to 64
segments one wave does this; past that the whole workgroup does, with the
walk data staged in LDS when the segment count allows (2 x the thread count)
and read from the workspace otherwise.  These cases drive kvc_mass_segment
directly from host-made usage (non-negative, pooled sums far inside the
documented bound) so that they reach every one of those paths in both
directions, with distinct masses, equal masses (ties decided by index) and
the uniform-weight ablation (every mass 1).  Steps 2-5 must match the oracle
bit for bit on the same usage.
"""
import numpy as np
import pytest

from eviction_window_qk_amd import synth
from oracle import ams
from parity_utils import check_steps2to5, oracle_params
from test_gpu_parity import _pd

# (label, T, seg_max, budgets, quota_mode): one launch per budget, four heads
# each (usage patterns below).  Segment counts: T / seg_max at least.
CASES = [
    ("nt1024_staged", 8192, 16, (1500, 2601), 0),       # ~520 segments, 1024 threads
    ("nt1024_staged_uniform", 8192, 16, (1500, 2211), 1),
    ("nt256_staged", 3000, 8, (700, 1111), 0),          # ~380 segments, 256 threads
    ("nt256_staged_uniform", 3000, 8, (700, 990), 1),
    ("nt256_workspace", 3000, 4, (1300, 1900), 0),      # ~750 segments > 512: not staged
    ("nt1024_workspace", 40000, 16, (9000, 13001), 0),  # ~2500 segments > 2048: not staged
]
PATTERNS = ("random", "constant", "steps", "spiky")
D_HEAD = 64


def _usage(pattern: str, T: int, seed: int) -> np.ndarray:
    """Non-negative usage summing to at most 32 (the bound is F*W*W*G = 1024
    for W = 16, G = 2 with average pooling)."""
    rng = np.random.default_rng(seed)
    if pattern == "random":
        u = rng.random(T) ** 4
    elif pattern == "constant":  # equal masses for equal-length segments
        u = np.ones(T)
    elif pattern == "steps":  # piecewise constant: runs of equal masses
        u = np.repeat(rng.integers(1, 4, size=(T + 511) // 512).astype(np.float64), 512)[:T]
    else:  # mostly tiny, a few large spikes
        u = np.full(T, 1e-3)
        u[rng.integers(0, T, size=T // 200)] = 1.0
    return (u * (32.0 / u.sum())).astype(np.float32)


def _case_inputs(label, T, seg_max, budget, quota_mode):
    pd = _pd(group=2, window=16, head_dim=D_HEAD, T=T, budget=budget, delta=0.05, seg_min=4,
             seg_max=seg_max, q_min=1, sinks=4, recent=64, quota_mode=quota_mode)
    seed = sum(map(ord, label)) + budget
    u32 = np.stack([_usage(pat, T, seed + i) for i, pat in enumerate(PATTERNS)])
    _, k, v = synth.random_small(seed, len(PATTERNS), 1, 1, D_HEAD, T)
    return pd, u32, k, v


def _walks(pd, u32):
    """(segment count, sign of D) of every walk the oracle takes on these heads."""
    seen = []
    orig = ams._walk

    def rec(q, limit, order, D, step):
        seen.append((len(order), step))
        return orig(q, limit, order, D, step)

    ams._walk = rec
    try:
        op = oracle_params(pd)
        for n in range(u32.shape[0]):
            ams.mass_and_segments(u32[n], None, op)
    finally:
        ams._walk = orig
    return seen


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cases_reach_both_walk_directions(case):
    """The inputs really take the block-wide walk both ways (checked on the
    oracle, so the GPU cases below cannot quietly stop covering it)."""
    label, T, seg_max, budgets, quota_mode = case
    signs = set()
    for K in budgets:
        pd, u32, _, _ = _case_inputs(label, T, seg_max, K, quota_mode)
        signs |= {step for ns, step in _walks(pd, u32) if ns > 64}
    assert signs == {1, -1}, (label, signs)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_quota_walk_many_segments(case):
    label, T, seg_max, budgets, quota_mode = case
    for K in budgets:
        pd, u32, k, v = _case_inputs(label, T, seg_max, K, quota_mode)
        print(f"[case] quota walk {label} T={T} seg_max={seg_max} K={K} quota_mode={quota_mode}",
              flush=True)
        out = check_steps2to5(pd, u32, k, v, None, range(u32.shape[0]))
        assert (out["n_seg"] > 64).all(), out["n_seg"]
