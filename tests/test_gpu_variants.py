"""GPU parity of the ablation variants (fixed-length segments, uniform
quotas, StreamingLLM) and of ragged (left-padded) batches against the CPU
oracle, through the C ABI.  Same bar as the base parity tests: step 1 within
2e-3 relative of the fp64 oracle, steps 2-5 bit for bit on the oracle's fp32
usage, the whole event equal to the stage entry points in sequence."""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import ams
from parity_utils import (assert_usage_close, check_event_consistency, check_kept_valid,
                          check_steps2to5, check_steps2to5_ragged, dev_bf16, dev_u64, kvc_params,
                          oracle_params, widen)

pytestmark = pytest.mark.gpu

BASE = dict(synth.WORKLOADS["tiny"].params)


def _pd(**kw):
    d = dict(BASE)
    d.update(kw)
    return d


def _run_case(pd, q, k, v, label):
    NH, T = q.shape[0], pd["T"]
    print(f"[case] {label} NH={NH} T={T} K={pd['budget']} fixed={pd.get('seg_fixed', 0)} "
          f"quota_mode={pd.get('quota_mode', 0)}", flush=True)
    p = kvc_params(pd, NH)
    op = oracle_params(pd)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    u_gpu = kvc.score_window(p, dq, dk).cpu().numpy()
    u_ref = np.stack([ams.window_usage(widen(q[n]), widen(k[n, :T]), op) for n in range(NH)])
    for n in range(NH):
        assert_usage_close(u_gpu[n], u_ref[n], f"{label} head {n}")
    check_steps2to5(pd, u_ref.astype(np.float32), k, v, None, range(NH), dk=dk, dv=dv)
    ev = check_event_consistency(pd, dq, dk, dv, None, NH)
    check_kept_valid(ev["kept"].cpu().numpy(), pd, T)
    return ev


ABLATIONS = [
    # (label, NH, G, W, d, T, K, overrides)
    ("fixed32", 2, 2, 16, 64, 700, 150, dict(seg_fixed=32)),
    ("fixed_split", 2, 2, 8, 64, 600, 120, dict(seg_fixed=100, seg_max=32, seg_min=8)),
    ("fixed_tail_merge", 1, 1, 4, 64, 70, 20, dict(seg_fixed=16, seg_min=16)),
    ("uniform", 2, 2, 16, 64, 700, 150, dict(quota_mode=1)),
    ("fixed_uniform", 2, 3, 16, 128, 900, 200, dict(seg_fixed=64, quota_mode=1)),
    ("fixed_ema", 2, 2, 16, 64, 500, 120, dict(seg_fixed=40, ema=True)),
    ("streaming_llm", 2, 2, 8, 64, 300, 68, dict(sinks=4, recent=64)),
]


@pytest.mark.parametrize("case", ABLATIONS, ids=[c[0] for c in ABLATIONS])
def test_ablation_variants(case):
    label, NH, G, W, d, T, K, over = case
    q, k, v = synth.random_small(sum(map(ord, label)), NH, G, W, d, T)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, **over)
    ev = _run_case(pd, q, k, v, label)
    if label == "streaming_llm":  # T_keep = 0: the sinks and the recent suffix only
        kept = ev["kept"].cpu().numpy()
        want = np.r_[np.arange(4), np.arange(T - 64, T)]
        for n in range(NH):
            np.testing.assert_array_equal(kept[n], want)


def _run_ragged(pd, q, k, v, lengths, label, credit_in=None, n_prev=0):
    NH, T = q.shape[0], pd["T"]
    print(f"[case] {label} NH={NH} T={T} K={pd['budget']} lengths={list(map(int, lengths))} "
          f"n_prev={n_prev}", flush=True)
    dlen = torch.from_numpy(np.ascontiguousarray(lengths, np.int32)).cuda()
    p = kvc_params(pd, NH, n_prev)
    p.valid_len = dlen
    op = oracle_params(pd, n_prev)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    u_gpu = kvc.score_window(p, dq, dk).cpu().numpy()
    u_ref = np.stack([ams.window_usage_ragged(widen(q[n]), widen(k[n, :T]), op, int(lengths[n]))
                      for n in range(NH)])
    for n in range(NH):
        assert_usage_close(u_gpu[n], u_ref[n], f"{label} head {n}")
    check_steps2to5_ragged(pd, u_ref.astype(np.float32), k, v, credit_in, range(NH), lengths,
                           n_prev)
    dci = dev_u64(credit_in) if (credit_in is not None and n_prev > 0) else None
    ev = check_event_consistency(pd, dq, dk, dv, dci, NH, n_prev, valid_len=dlen)
    # the whole event against the oracle's whole ragged event on one head
    n = int(np.argmin(lengths))
    ci = credit_in[n] if (credit_in is not None and n_prev > 0) else None
    ref = ams.event_ragged(widen(q[n]), widen(k[n, :T]), v[n, :T], ci, op, int(lengths[n]))
    kept = ev["kept"].cpu().numpy()[n]
    assert set(kept[kept >= 0].tolist()) <= set(range(T - max(int(lengths[n]), pd["window"]), T))
    assert len(kept[kept >= 0]) == len(ref.kept[ref.kept >= 0])
    return ev


RAGGED = [
    # (label, NH, G, W, d, T, K, lengths, overrides)
    ("basic", 4, 2, 16, 64, 300, 64, [300, 263, 16, 5], {}),
    ("noop_heads", 4, 2, 8, 64, 200, 64, [200, 64, 50, 65], {}),
    ("multi_chunk", 3, 3, 40, 128, 1000, 200, [1000, 611, 257], {}),
    ("one_segment", 3, 4, 32, 128, 700, 100, [700, 333, 101],
     dict(delta=1.0, seg_min=1, seg_max=0, sinks=0, recent=0, pool_mode=1)),
    ("one_segment_must_keep", 3, 2, 16, 64, 500, 100, [500, 250, 90],
     dict(delta=1.0, seg_max=0, sinks=4, recent=16)),
    ("agg_max", 2, 4, 16, 64, 300, 60, [300, 111], dict(head_agg=1)),
    ("fixed_uniform", 3, 2, 16, 64, 640, 120, [640, 500, 129], dict(seg_fixed=48, quota_mode=1)),
    # T >= 4096: the 1024-thread fill, mass/segment and select workgroups on left-padded heads
    ("long_cache", 3, 2, 16, 64, 5000, 600, [5000, 4100, 700], {}),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_batches(case):
    label, NH, G, W, d, T, K, lengths, over = case
    q, k, v = synth.random_small(sum(map(ord, label)) + 5, NH, G, W, d, T)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, **over)
    _run_ragged(pd, q, k, v, np.array(lengths, np.int32), f"ragged_{label}")


def test_ragged_ema_credit():
    NH, G, W, d, T, K, n_prev = 3, 2, 16, 64, 260, 100, 37
    q, k, v = synth.random_small(99, NH, G, W, d, T)
    rng = np.random.default_rng(5)
    credit = (rng.random((NH, n_prev)) * 2.0 ** 37).astype(np.uint64)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, ema=True)
    _run_ragged(pd, q, k, v, np.array([260, 200, 30], np.int32), "ragged_ema", credit, n_prev)


def test_ragged_qwen7b_shape_heads():
    """Qwen-7B-shaped heads of a left-padded batch: prompts in one batch
    differ by up to 400 tokens."""
    wl = synth.WORKLOADS["qwen7b_t768"]
    heads = [0, 5, 777, 1791]
    q, k, v = synth.gen_heads(wl, heads)
    lengths = synth.batch_valid_lengths(wl, 400, seed=1, heads=heads)
    _run_ragged(wl.event_params(), q, k, v, lengths, "ragged qwen7b_t768 sampled")


def test_ragged_window_one_zeroes_the_padding():
    """W = 1 has no positions to fill, but a left-padded head's usage must still
    be 0 on its padding: the output buffer starts as NaN so that any position
    the kernels leave unwritten fails the comparison."""
    NH, G, W, d, T, K = 3, 4, 1, 64, 300, 40
    lengths = np.array([T, T // 2, 5], np.int32)
    q, k, v = synth.random_small(4242, NH, G, W, d, T)
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    p = kvc_params(pd, NH)
    p.valid_len = torch.from_numpy(lengths).cuda()
    op = oracle_params(pd)
    dq, dk = dev_bf16(q), dev_bf16(k)
    u = torch.full((NH, T), float("nan"), dtype=torch.float32, device="cuda")
    kvc.score_window(p, dq, dk, u=u)
    u_gpu = u.cpu().numpy()
    for n in range(NH):
        u_ref = ams.window_usage_ragged(widen(q[n]), widen(k[n, :T]), op, int(lengths[n]))
        assert_usage_close(u_gpu[n], u_ref, f"W=1 ragged head {n}")
        assert np.all(u_gpu[n, :T - max(int(lengths[n]), W)] == 0.0)
    _run_ragged(pd, q, k, v, lengths, "ragged_window_one")
