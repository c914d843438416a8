"""Host replay of the block-wide quota walk's rank count (no GPU).

After the full cycles of the quota redistribution, the partial cycle gives
one more step to the first r segments, in walk order, whose room exceeds the
cycle count [AMS notes, key design 3: clip and redistribute].  The walk order
is (mass desc, index asc) when adding and (mass asc, index desc) when
removing.  The mass kernel counts each segment's rank on one unsigned key per
segment: 0 for a segment without room left, else 1 + mass (adding) or
1 + (2^63 - 1 - mass) (removing); segment o precedes s iff key[o] >= key[s]
on the side of s that wins ties (lower indices when adding, higher when
removing) and key[o] >= key[s] + 1 on the other.  The kernel reads the keys in
chunks of 32 that lie wholly on one side of a wave's 64 segments, and a wave
stops once none of its segments can still be among the first r.  This test
replays exactly that loop structure in NumPy and compares the set of segments
that get the extra step with the direct definition, on random cases with
many ties, masses up to 2^63 - 1, both directions and every r.
"""
import numpy as np
import pytest

TOP = (1 << 63) - 1


def _direct(m, room, cyc, r, adding):
    ns = len(m)
    elig = room > cyc
    out = np.zeros(ns, dtype=bool)
    if r <= 0:
        return out
    order = sorted((i for i in range(ns) if elig[i]),
                   key=(lambda i: (-int(m[i]), i)) if adding else (lambda i: (int(m[i]), -i)))
    out[order[:r]] = True
    return out


def _replay(m, room, cyc, r, adding):
    ns = len(m)
    pad = (ns + 31) & ~31
    key = np.zeros(pad, dtype=np.uint64)
    for s in range(ns):
        if room[s] > cyc:
            key[s] = np.uint64(1 + (int(m[s]) if adding else TOP - int(m[s])))
    out = np.zeros(ns, dtype=bool)
    for sb in range(0, ns, 64):  # one wave: lanes s = sb .. sb + 63
        s = np.arange(sb, sb + 64)
        mine = s < ns
        ks = np.where(mine, key[np.minimum(s, ns - 1)], np.uint64(0))
        part = mine & (room[np.minimum(s, ns - 1)] > cyc) & (r > 0)
        one = np.uint64(1)
        t_lo = ks if adding else ks + one  # thresholds for o < s
        t_hi = ks + one if adding else ks  # and for o > s
        rank = np.zeros(64, dtype=np.int64)
        c = 0
        while c < ns and np.any(part & (rank < r)):
            ch = key[c:c + 32]
            if c + 32 <= sb or c >= sb + 64:  # the whole chunk on one side of every lane
                th = t_lo if c < sb else t_hi
                rank += (ch[None, :] >= th[:, None]).sum(axis=1)
            else:
                o = np.arange(c, c + 32)
                th = np.where(o[None, :] < s[:, None], t_lo[:, None], t_hi[:, None])
                rank += ((o[None, :] != s[:, None]) & (ch[None, :] >= th)).sum(axis=1)
            c += 32
        got = part & (rank < r)
        out[s[mine]] = got[mine]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_folded_keys_pick_the_walk_prefix(seed):
    rng = np.random.default_rng(seed)
    for case in range(60):
        ns = int(rng.integers(65, 700))
        adding = bool(rng.integers(0, 2))
        cyc = int(rng.integers(0, 4))
        mode = case % 4
        if mode == 0:
            m = rng.integers(0, 5, size=ns).astype(np.uint64)           # many ties, zeros
        elif mode == 1:
            m = rng.integers(0, TOP, size=ns, dtype=np.uint64)          # the full range
        elif mode == 2:
            m = (TOP - rng.integers(0, 3, size=ns)).astype(np.uint64)   # next to 2^63 - 1
        else:
            m = np.ones(ns, dtype=np.uint64)                            # uniform weights
        room = rng.integers(0, 6, size=ns)
        r = int(rng.integers(0, ns + 2))
        np.testing.assert_array_equal(_replay(m, room, cyc, r, adding),
                                      _direct(m, room, cyc, r, adding),
                                      err_msg=f"seed {seed} case {case} ns={ns} adding={adding}")
