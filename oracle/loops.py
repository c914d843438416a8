"""Pure-Python loop restatement of the event for tiny shapes (T <= ~64).

TEST INFRASTRUCTURE ONLY.  It restates every step of ``oracle.ams`` with
explicit scalar loops (Python floats are IEEE fp64; fp32 steps use NumPy fp32
scalars, one operation at a time) so that a vectorisation slip in the NumPy
oracle -- a wrong mask, an off-by-one in a prefix, a transposed operand --
shows up as a disagreement.  It shares no helper with ``oracle.ams``; only the
parameter record is common.  Sources are the same passages cited there.
"""
from __future__ import annotations

import math

import numpy as np


def usage_unfilled(q, k, p):
    """sum over g, w of softmax_t(scale*<q_gw, k_t>), t <= T-W+w (triple loop)."""
    G, W, d = len(q), len(q[0]), len(k[0])
    T = p.T
    scale = p.scale if p.scale != 0.0 else 1.0 / math.sqrt(d)
    per_g = []
    for g in range(G):
        col = [0.0] * T
        for w in range(W):
            last = T - W + w
            s = []
            for t in range(last + 1):
                acc = 0.0
                for j in range(d):
                    acc += float(q[g][w][j]) * float(k[t][j])
                s.append(acc * scale)
            mx = max(s)
            ex = [math.exp(x - mx) for x in s]
            tot = sum(ex)
            for t in range(last + 1):
                col[t] += ex[t] / tot
        per_g.append(col)
    if p.head_agg == 0:
        return [sum(per_g[g][t] for g in range(G)) for t in range(T)]
    return [max(per_g[g][t] for g in range(G)) for t in range(T)]


def fill(u, W):
    T = len(u)
    out = list(u)
    if W > 1:
        mx = max(u[: T - W + 1])
        for t in range(T - W + 1, T):
            out[t] = mx
    return out


def pool(u32, p):
    T = len(u32)
    h = p.pool_kernel // 2
    out = []
    for t in range(T):
        if p.pool_mode == 1:
            best = None
            for j in range(t - h, t + h + 1):
                if 0 <= j < T:
                    best = u32[j] if best is None else max(best, u32[j])
            out.append(np.float32(best))
        else:
            acc = np.float32(0.0)
            cnt = 0
            for j in range(t - h, t + h + 1):
                if 0 <= j < T:
                    acc = np.float32(acc + np.float32(u32[j]))
                    cnt += 1
            out.append(np.float32(acc / np.float32(cnt)))
    return out


def mass_v(score, credit_in, p):
    """Returns (v list of ints, credit list of ints or None)."""
    e = int(math.ceil(p.eps * 2.0 ** 40))
    w = []
    for x in score:
        y = np.float32(max(np.float32(x), np.float32(0.0)) * np.float32(2.0 ** 40))
        w.append(int(y) + e)          # y is integral-or-truncated: int() truncates
    if not p.ema:
        return w, None
    W = sum(w)
    mq = [float(x) / float(W) for x in w]
    c = []
    for t in range(len(w)):
        if t < p.n_prev:
            c.append(float(int(credit_in[t])) * 2.0 ** -44)
        else:
            c.append(math.floor(mq[t] * 2.0 ** 44) * 2.0 ** -44)
    oml = 1.0 - p.lam
    cq = [int(math.floor(((p.lam * c[t]) + (oml * mq[t])) * 2.0 ** 44)) for t in range(len(w))]
    cs = sum(cq)
    omb = 1.0 - p.beta
    v = []
    for t in range(len(w)):
        nc = float(cq[t]) / float(cs) if cs > 0 else 0.0
        v.append(int(math.floor(((p.beta * mq[t]) + (omb * nc)) * 2.0 ** 44)))
    return v, cq


def segments(v, p):
    T = len(v)
    P = []
    run = 0
    for x in v:
        run += x
        P.append(run)
    V = P[-1]
    ends = []
    k = 1
    while float(k) * p.delta < 1.0:
        th = min(V, int(math.ceil((float(k) * p.delta) * float(V))))
        t = 0
        while P[t] < th:
            t += 1
        if t not in ends:
            ends.append(t)
        k += 1
    if T - 1 not in ends:
        ends.append(T - 1)
    ends.sort()
    segs = []
    start = 0
    for e in ends:
        segs.append([start, e])
        start = e + 1
    merged = []
    i = 0
    while i < len(segs):
        a, b = segs[i]
        while b - a + 1 < p.seg_min and i + 1 < len(segs):
            i += 1
            b = segs[i][1]
        merged.append([a, b])
        i += 1
    if len(merged) > 1 and merged[-1][1] - merged[-1][0] + 1 < p.seg_min:
        last = merged.pop()
        merged[-1][1] = last[1]
    out = []
    for a, b in merged:
        L = b - a + 1
        if p.seg_max <= 0 or L <= p.seg_max:
            out.append((a, b))
            continue
        n = (L + p.seg_max - 1) // p.seg_max
        s = a
        for j in range(n):
            ln = L // n + (1 if j < L % n else 0)
            out.append((s, s + ln - 1))
            s += ln
    return out


def mk_set(p):
    T, K = p.T, p.budget
    s = min(p.sinks, K, T)
    r = min(p.recent, K - s, T - s)
    return set(range(s)) | set(range(T - r, T)), K - s - r


def quotas(segs, v, p):
    mk, t_keep = mk_set(p)
    L = [b - a + 1 for a, b in segs]
    Km = [sum(1 for t in range(a, b + 1) if t in mk) for a, b in segs]
    A = [L[i] - Km[i] for i in range(len(segs))]
    M = [sum(v[t] for t in range(a, b + 1) if t not in mk) for a, b in segs]
    fl = [min(A[i], max(0, min(p.q_min, L[i]) - Km[i])) for i in range(len(segs))]
    if sum(fl) > t_keep:
        return list(fl)
    t_rem = t_keep - sum(fl)
    SM = sum(M)
    q = []
    for i in range(len(segs)):
        add = 0 if SM == 0 else int(math.floor(float(t_rem) * (float(M[i]) / float(SM)) + 0.5))
        q.append(min(A[i], fl[i] + add))
    D = t_keep - sum(q)
    n = len(segs)
    if D > 0:
        order = sorted(range(n), key=lambda i: (-M[i], i))
        while D > 0:
            moved = False
            for i in order:
                if D == 0:
                    break
                if q[i] < A[i]:
                    q[i] += 1
                    D -= 1
                    moved = True
            if not moved:
                break
    elif D < 0:
        order = sorted(range(n), key=lambda i: (M[i], -i))
        while D < 0:
            moved = False
            for i in order:
                if D == 0:
                    break
                if q[i] > fl[i]:
                    q[i] -= 1
                    D += 1
                    moved = True
            if not moved:
                break
    return q


def select(score, segs, q, p):
    T, K = p.T, p.budget
    if T <= K:
        return list(range(T))
    mk, _ = mk_set(p)

    def better(i, j):  # i ranks before j
        return score[i] > score[j] or (score[i] == score[j] and i < j)

    def top(cands, n):
        chosen = []
        rest = list(cands)
        for _ in range(min(n, len(rest))):
            best = rest[0]
            for c in rest[1:]:
                if better(c, best):
                    best = c
            chosen.append(best)
            rest.remove(best)
        return chosen

    picks = []
    for (a, b), qi in zip(segs, q):
        picks += top([t for t in range(a, b + 1) if t not in mk], max(0, qi))
    kept = set(mk) | set(picks)
    if len(kept) > K:
        keep_picks = top(picks, K - len(mk))
        kept = set(mk) | set(keep_picks)
    elif len(kept) < K:
        free = [t for t in range(T) if t not in kept]
        kept |= set(top(free, K - len(kept)))
    return sorted(kept)
