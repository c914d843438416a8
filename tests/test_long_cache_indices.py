"""Data-dependent index ranges of the long-cache mass/segment and select
workgroups, replayed on the CPU for usage that did not come from the score
stage (random u = 3 r^4, r uniform, on 131072-position caches with EMA credit,
and spiky variants).

The GPU kernels' integer decisions equal the oracle's bit for bit (the GPU
tests check every head of every workload), so the oracle's prefix C(t),
segments and quotas are the values the kernels index with.  What is replayed
here is the kernels' own index arithmetic on those values:
  - the two-level cut search: one prefix sample per thread at
    (tid + 1) * stride - 1 (clamped to T - 1), the bracket [lo*stride,
    min((lo+1)*stride - 1, T - 1)] around the first sample >= the threshold,
    and the bisection inside it (1024 threads for caches of 4096 positions or
    more, 256 below);
  - the merged-segment table (at most 1025 entries in LDS) and the piece
    count against the segment capacity the host allocates for;
  - select's long-segment list (at most 1024 entries in LDS), its register
    cache bound and the positions its short-segment waves touch.
Every index must stay inside the array it addresses."""
import numpy as np
import pytest

from oracle import ams

K_MAX_MERGED = 1025
K_LONG_CAP = 1024
K_WAVE_SEG = 256


def _usage(rng, T, kind):
    if kind == "r4":
        return (3.0 * rng.random(T) ** 4).astype(np.float32)
    u = (rng.random(T) * 1e-3).astype(np.float32)            # near-flat with spikes
    u[rng.integers(0, T, size=64)] = 50.0
    return u


def _replay_cuts(P, th_list, T, NT):
    stride = (T + NT - 1) // NT
    samp_idx = np.minimum((np.arange(NT) + 1) * stride - 1, T - 1)
    assert samp_idx.min() >= 0 and samp_idx.max() <= T - 1
    samp = P[samp_idx]
    cuts = []
    for th in th_list:
        lo = int(np.searchsorted(samp, np.uint64(th), side="left"))   # first sample >= th
        assert 0 <= lo <= NT - 1
        a, b = lo * stride, min((lo + 1) * stride - 1, T - 1)
        assert 0 <= a <= b <= T - 1, (a, b)
        while a < b:
            mid = (a + b) >> 1
            assert 0 <= mid <= T - 1
            if P[mid] >= th:
                b = mid
            else:
                a = mid + 1
        cuts.append(a)
    return cuts


@pytest.mark.parametrize("seed,kind", [(5, "r4"), (6, "r4"), (7, "spiky")])
def test_long_cache_index_ranges(seed, kind):
    rng = np.random.default_rng(seed)
    T, K = 131072, 4096
    p = ams.Params(T=T, window=128, budget=K, group=4, ema=True)
    s_cap = ams.segment_capacity(p)
    for head in range(3):
        u = _usage(rng, T, kind)
        r = ams.mass_and_segments(u, None, p)
        P = r.P
        V = int(P[-1])
        assert V < 2 ** 64
        ths = ams.thresholds(V, p.delta)
        assert len(ths) <= K_MAX_MERGED - 1
        for NT in (1024, 256):
            cuts = _replay_cuts(P, ths, T, NT)
            # the replayed search finds the oracle's cuts (b_k = min{t : C(t) >= theta_k})
            assert sorted(set(cuts) | {T - 1}) == ams.raw_cuts(P, p.delta)
        merged = ams.merge_short(ams.segments_from_ends(ams.raw_cuts(P, p.delta)), p.seg_min)
        assert len(merged) <= K_MAX_MERGED
        segs = r.segs
        assert len(segs) <= s_cap
        starts = [a for a, _ in segs]
        assert starts[0] == 0 and all(0 <= a < T for a in starts)
        # select: long segments listed in LDS, short ones one wave each
        lens = [b - a + 1 for a, b in segs]
        assert sum(L > K_WAVE_SEG for L in lens) <= K_LONG_CAP
        for (a, b), L in zip(segs, lens):
            if L <= K_WAVE_SEG:
                t = a + np.arange(64)[:, None] + 64 * np.arange(K_WAVE_SEG // 64)[None, :]
                clamped = np.minimum(t, b)
                assert clamped.min() >= 0 and clamped.max() <= T - 1
        assert len(r.q) == len(segs) and np.all(np.asarray(r.q) >= 0)
