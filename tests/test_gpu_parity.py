"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Step 1 (window score) is held to the fp64 oracle within 2e-3 relative (plus a
1e-30 absolute floor for fp32 exp underflow).  Steps 2-5 run on the oracle's
own fp32 usage and must match it bit for bit: pooled score, credit, segment
starts, quotas, kept indices, compacted K/V and credit.  The whole event must
equal the stage entry points run in sequence, and repeat bit for bit.
"""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import synth
from oracle import ams
from parity_utils import (assert_usage_close, check_event_consistency, check_kept_valid,
                          check_steps2to5, dev_bf16, dev_u64, kvc_params, oracle_params, widen)
from eviction_window_qk_amd import kvc

pytestmark = pytest.mark.gpu

BASE = dict(synth.WORKLOADS["tiny"].params)


def _pd(**kw):
    d = dict(BASE)
    d.update(kw)
    return d


def _run_case(pd, q, k, v, credit_in=None, n_prev=0, t_stride=0, heads=None, label=""):
    NH = q.shape[0]
    T = pd["T"]
    heads = range(NH) if heads is None else heads
    print(f"[case] {label} NH={NH} G={pd['group']} W={pd['window']} d={pd['head_dim']} T={T} "
          f"K={pd['budget']} ema={pd.get('ema')} n_prev={n_prev}", flush=True)
    p = kvc_params(pd, NH, n_prev, t_stride)
    op = oracle_params(pd, n_prev)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    u_gpu = kvc.score_window(p, dq, dk).cpu().numpy()
    u_ref = np.zeros((NH, T), dtype=np.float64)
    for n in range(NH):
        u_ref[n] = ams.window_usage(widen(q[n]), widen(k[n, :T]), op)
    for n in heads:
        assert_usage_close(u_gpu[n], u_ref[n], f"{label} head {n}")
    check_steps2to5(pd, u_ref.astype(np.float32), k, v, credit_in, heads, n_prev, t_stride,
                    dk=dk, dv=dv)
    dci = dev_u64(credit_in) if (credit_in is not None and n_prev > 0) else None
    ev = check_event_consistency(pd, dq, dk, dv, dci, NH, n_prev, t_stride)
    check_kept_valid(ev["kept"].cpu().numpy(), pd, T)
    return u_gpu, u_ref, ev


def test_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    q, k, v = synth.gen_heads(wl, [0])
    _run_case(wl.event_params(), q, k, v, label="tiny")


SMALL = [
    # (label, NH, G, W, d, T, K, overrides, key_scale)
    ("ragged", 3, 2, 8, 64, 100, 40, {}, 1.0),
    ("w1", 2, 1, 1, 128, 300, 50, {}, 1.0),
    ("multi_chunk", 2, 3, 40, 128, 1000, 200, {}, 2.0),
    ("peaky", 2, 2, 16, 64, 513, 64, {}, 6.0),
    ("one_segment", 2, 4, 32, 128, 600, 100,
     dict(delta=1.0, seg_min=1, seg_max=0, sinks=0, recent=0, pool_mode=1), 1.0),
    ("agg_max", 2, 4, 16, 64, 300, 60, dict(head_agg=1), 1.5),
    ("tiny_T", 2, 2, 3, 64, 5, 2, dict(seg_min=1, seg_max=2, sinks=1, recent=0), 1.0),
    ("noop", 2, 2, 4, 64, 20, 32, {}, 1.0),
    ("equal_T_K", 1, 1, 4, 64, 64, 64, {}, 1.0),
    ("short_budget", 2, 2, 8, 64, 200, 10, {}, 1.0),     # must-keep shrinks the recent suffix
    ("infeasible_floors", 2, 2, 8, 64, 400, 90, dict(seg_min=4, seg_max=8, recent=64), 1.0),
    ("fine_delta", 2, 2, 16, 64, 900, 300, dict(delta=0.01, seg_min=2, seg_max=64), 1.0),
    ("q_min_3", 2, 2, 16, 64, 700, 150, dict(q_min=3, pool_kernel=3), 1.0),
    ("long_segments", 1, 2, 16, 64, 5000, 700, dict(seg_max=0, delta=0.3, seg_min=600), 1.0),
    # a 1024-token cache (whole 64-key tiles), 120 query rows (not a multiple of the 256-row
    # pass-1 workgroup), and a cache one position past a 256-key pass-2 chunk boundary
    ("t1024_whole_tiles", 2, 2, 64, 128, 1024, 300, {}, 2.0),
    ("rows_120", 2, 3, 40, 128, 777, 200, {}, 1.0),
    ("t1025_chunk_edge", 2, 3, 40, 128, 1025, 200, {}, 1.0),
    # one unsplit segment (no mass cuts): its mass is the total less the must-keep share
    ("one_segment_must_keep", 2, 4, 32, 128, 600, 100,
     dict(delta=1.0, seg_min=1, seg_max=0, sinks=4, recent=32), 1.0),
    ("one_segment_within_seg_max", 2, 2, 16, 64, 400, 80, dict(delta=1.0, seg_max=512), 1.0),
    ("one_segment_uniform", 2, 2, 16, 64, 300, 60,
     dict(delta=1.0, seg_max=0, quota_mode=1, sinks=2, recent=8), 1.0),
    ("one_segment_ema", 2, 2, 16, 64, 700, 150, dict(delta=1.0, seg_max=0, ema=True), 1.0),
    ("one_segment_long", 1, 2, 16, 64, 5000, 700, dict(delta=1.0, seg_min=1, seg_max=0), 1.0),
    # long caches (1024-thread fill, mass/segment and select) with the MAX head
    # aggregation and with max-pooling
    ("agg_max_long", 1, 4, 16, 64, 5000, 600, dict(head_agg=1), 1.5),
    ("max_pool_long", 1, 2, 16, 64, 6000, 800, dict(pool_mode=1), 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case):
    label, NH, G, W, d, T, K, over, ks = case
    q, k, v = synth.random_small(sum(map(ord, label)), NH, G, W, d, T, key_scale=ks)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, **over)
    _run_case(pd, q, k, v, label=label)


def test_t_stride_larger_than_T():
    NH, G, W, d, T, K, TS = 2, 2, 8, 64, 150, 50, 192
    q, k, v = synth.random_small(7, NH, G, W, d, T, t_stride=TS)
    k[:, T:] = 0x7F80  # +inf bits past T: must never be read
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    _run_case(pd, q, k, v, t_stride=TS, label="t_stride")


@pytest.mark.parametrize("n_prev", [0, 37, 120])
def test_ema_credit(n_prev):
    NH, G, W, d, T, K = 3, 2, 16, 64, 200, 120
    q, k, v = synth.random_small(11 + n_prev, NH, G, W, d, T)
    rng = np.random.default_rng(n_prev)
    credit = (rng.random((NH, max(n_prev, 1))) * 2.0 ** 37).astype(np.uint64)[:, :n_prev]
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, ema=True, lam=0.9, beta=0.9)
    _run_case(pd, q, k, v, credit_in=credit if n_prev else None, n_prev=n_prev,
              label=f"ema{n_prev}")


@pytest.mark.parametrize("T", [300, 4500])
def test_ema_credit_one_segment(T):
    """EMA with carried credit when the cache is one unsplit segment, for both
    workgroup sizes of the mass/segment kernel."""
    NH, G, W, d, K, n_prev = 2, 2, 16, 64, T // 4, 50
    q, k, v = synth.random_small(7 + T, NH, G, W, d, T)
    rng = np.random.default_rng(T)
    credit = (rng.random((NH, n_prev)) * 2.0 ** 37).astype(np.uint64)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, ema=True, delta=1.0, seg_max=0,
             sinks=4, recent=16)
    _run_case(pd, q, k, v, credit_in=credit, n_prev=n_prev, label=f"ema_one_segment_{T}")


def test_ema_credit_long_cache():
    """EMA with carried credit on a cache long enough (>= 4096) for the
    1024-thread mass/segment and select workgroups."""
    NH, G, W, d, T, K, n_prev = 2, 2, 16, 64, 5000, 600, 600
    q, k, v = synth.random_small(4242, NH, G, W, d, T, key_scale=2.0)
    rng = np.random.default_rng(17)
    credit = (rng.random((NH, n_prev)) * 2.0 ** 37).astype(np.uint64)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, ema=True, lam=0.9, beta=0.9)
    _run_case(pd, q, k, v, credit_in=credit, n_prev=n_prev, label="ema_long")


def test_qwen7b_shape_heads():
    wl = synth.WORKLOADS["qwen7b_t768"]
    heads = [0, 1, 777, 1791]
    q, k, v = synth.gen_heads(wl, heads)
    _run_case(wl.event_params(), q, k, v, label="qwen7b_t768 sampled")


def test_llama8b_global_heads():
    wl = synth.WORKLOADS["llama8b_global_t16k"]
    q, k, v = synth.gen_heads(wl, [3, 1000])
    _run_case(wl.event_params(), q, k, v, label="llama8b_global sampled")


def test_qwen7b_ema_event_chain():
    """Event 0 on a fresh 1536-token cache, then event 1 on the compacted
    cache plus 512 new tokens with the carried credit.  Every input of event 1
    comes from the oracle's event 0 (never from the GPU)."""
    wl = synth.WORKLOADS["qwen7b_t1536_ema"]
    heads = [5, 4000]
    pd = wl.event_params()
    op0 = oracle_params(pd, 0)
    q0, k0, v0 = synth.gen_heads(wl, heads, seed=wl.prior_seed)
    K = wl.budget
    k1 = np.zeros_like(k0)
    v1 = np.zeros_like(v0)
    credit = np.zeros((len(heads), K), dtype=np.uint64)
    for i, n in enumerate(heads):
        u0 = ams.window_usage(widen(q0[i]), widen(k0[i]), op0)
        r0 = ams.steps2to5(u0.astype(np.float32), k0[i], v0[i], None, op0)  # bf16 bits
        fk, fv = synth.fresh_rows(wl, n, wl.T - K, seed=wl.seed)
        k1[i] = np.concatenate([r0.k_out, fk])
        v1[i] = np.concatenate([r0.v_out, fv])
        credit[i] = r0.credit_out
    q1 = np.stack([synth.gen_head(wl, n)["q"] for n in heads])
    _run_case(pd, q1, k1, v1, credit_in=credit, n_prev=K, label="qwen7b_ema event 1")


def test_drift_bursts_head():
    """One head of the 131072-token workload: >= 512 segments, EMA on."""
    wl = synth.WORKLOADS["llama8b_t128k"]
    q, k, v = synth.gen_heads(wl, [77])
    _, _, ev = _run_case(wl.event_params(), q, k, v, label="llama8b_t128k head 77")


def test_kept_drives_gather_of_arbitrary_indices():
    """kvc_gather_compact on caller-chosen indices (including -1 and
    out-of-range values, which give zero rows)."""
    NH, d, T, K = 2, 128, 300, 64
    _, k, v = synth.random_small(3, NH, 1, 1, d, T)
    pd = _pd(group=1, window=1, head_dim=d, T=T, budget=K)
    p = kvc_params(pd, NH)
    rng = np.random.default_rng(0)
    kept = np.sort(rng.choice(T, size=(NH, K), replace=True), axis=1).astype(np.int32)
    kept[0, -3:] = -1
    kept[1, 0] = T + 5
    dk, dv = dev_bf16(k), dev_bf16(v)
    ko, vo, _ = kvc.gather_compact(p, torch.from_numpy(kept).cuda(), dk, dv)
    ko = ko.view(torch.int16).cpu().numpy().view(np.uint16)
    for n in range(NH):
        for j in range(K):
            t = kept[n, j]
            expect = k[n, t] if 0 <= t < T else np.zeros(d, np.uint16)
            np.testing.assert_array_equal(ko[n, j], expect)


@pytest.mark.parametrize("T,K", [(500, 80), (8000, 700), (20000, 1500)])
def test_select_with_caller_quotas_under_budget(T, K):
    """Caller-supplied quotas that sum below the budget: the under-budget
    repair fills with the best unselected positions (oracle select).  The
    three lengths take the 256-thread workgroup, the 1024-thread one with the
    keys in registers, and the 1024-thread one re-reading them."""
    NH = 2
    pd = _pd(group=1, window=1, head_dim=64, T=T, budget=K, seg_max=T // 5, seg_min=16)
    p = kvc_params(pd, NH)
    op = oracle_params(pd)
    rng = np.random.default_rng(5 + T)
    score = (rng.random((NH, T)) * 10).astype(np.float32)
    score[:, ::7] = score[:, :1]                           # ties
    starts = np.arange(0, T, T // 5, dtype=np.int32)[:5]
    S = kvc.segment_capacity(p)
    seg_start = np.zeros((NH, S), np.int32)
    seg_quota = np.zeros((NH, S), np.int32)
    seg_start[:, :5] = starts
    seg_quota[:, :5] = [3, 0, 10, 2, 1]
    n_seg = np.full(NH, 5, np.int32)
    kept = kvc.select(p, torch.from_numpy(score).cuda(), torch.from_numpy(seg_start).cuda(),
                      torch.from_numpy(seg_quota).cuda(), torch.from_numpy(n_seg).cuda())
    kept = kept.cpu().numpy()
    segs = [(int(a), int(b) - 1) for a, b in zip(starts, list(starts[1:]) + [T])]
    for n in range(NH):
        ref = ams.select(score[n], segs, [3, 0, 10, 2, 1], op)
        np.testing.assert_array_equal(kept[n], ref)
