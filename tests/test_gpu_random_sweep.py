"""Seeded random sweep of small events on the GPU against the oracle.

Each case draws a shape and a parameter set the host accepts: group size,
window, head dim, cache length (on both sides of the 4096-position switch to
the long-cache kernels), budget (also at or above the cache length), mass
cut spacing, segment bounds, must-keep sizes, pooling kernel and mode, head
aggregation, EMA (fresh, or with credit carried from an earlier event), quota
mode, fixed-length segments, a key/value row stride past the cache length
and, for some cases, a left-padded batch.  Every head is held to the same bars as the hand-picked
parity cases: usage within 2e-3 of the fp64 oracle, steps 2-5 bit for bit on
the oracle's usage, and the whole event equal to the stages run in turn.
"""
import numpy as np
import pytest

from eviction_window_qk_amd import kvc, synth
from oracle import ams
from parity_utils import (assert_usage_close, check_steps2to5_ragged, dev_bf16, kvc_params,
                          oracle_params, widen)
from test_gpu_parity import _pd, _run_case

N_CASES = 1000


def _draw(seed: int):
    """A valid (pd, NH, lengths or None, n_prev, t_stride) for this seed."""
    rng = np.random.default_rng(1000 + seed)
    while True:
        G = int(rng.choice([1, 2, 3, 4, 7, 8]))
        W = int(rng.choice([1, 5, 16, 32, 33, 64, 128]))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(max(W, 40), 9000)) if rng.random() < 0.6 else int(rng.integers(max(W, 8), 600))
        K = int(rng.integers(1, T + 50))
        seg_min = int(rng.choice([1, 4, 16]))
        seg_max = int(rng.choice([0, 2 * seg_min, 64, 256]))
        over = dict(
            group=G, window=W, head_dim=d, T=T, budget=K,
            delta=float(rng.choice([0.1, 0.05, 0.2, 0.3, 1.0])),
            seg_min=seg_min, seg_max=seg_max, q_min=int(rng.integers(0, 3)),
            sinks=int(rng.choice([0, 4])), recent=int(rng.choice([0, 16, 64])),
            pool_kernel=int(rng.choice([1, 3, 7, 9])), pool_mode=int(rng.integers(0, 2)),
            head_agg=int(rng.integers(0, 2)), ema=bool(rng.random() < 0.4),
            quota_mode=int(rng.random() < 0.2),
            seg_fixed=int(rng.choice([0, 0, 0, 8, 48])),
        )
        pd = _pd(**over)
        NH = int(rng.integers(1, 4))
        p = kvc_params(pd, NH)
        if kvc.check_params(p) != 0:
            continue
        lengths = None
        n_prev, t_stride = 0, T
        if rng.random() < 0.3:
            lengths = rng.integers(W, T + 1, size=NH).astype(np.int32)
        else:
            if pd["ema"] and rng.random() < 0.5:
                n_prev = int(rng.integers(1, T + 1))
            if rng.random() < 0.3:
                t_stride = T + int(rng.integers(1, 40))
        if kvc.check_params(kvc_params(pd, NH, n_prev, t_stride)) != 0:
            continue
        return pd, NH, lengths, n_prev, t_stride


def _credit(seed: int, NH: int, n_prev: int) -> np.ndarray:
    """Carried credit like an earlier event's output: Q44 fractions summing to
    about 2^44 per head."""
    rng = np.random.default_rng(5000 + seed)
    r = rng.random((NH, n_prev)) ** 3 + 1e-3
    return np.floor(r / r.sum(axis=1, keepdims=True) * 2.0 ** 44).astype(np.uint64)


def test_sweep_draws_are_varied():
    """The draws reach both kernel sizes, the no-eviction case, every
    pooling/aggregation mode, EMA, the ablations and ragged batches."""
    seen = set()
    for s in range(N_CASES):
        pd, NH, lengths, n_prev, t_stride = _draw(s)
        seen.add("long" if pd["T"] >= 4096 else "short")
        seen.add("noop" if pd["budget"] >= pd["T"] else "evict")
        seen.add(f"pool{pd['pool_mode']}")
        seen.add(f"agg{pd['head_agg']}")
        seen.add("ema" if pd["ema"] else "no_ema")
        if pd["quota_mode"]:
            seen.add("uniform")
        if pd["seg_fixed"]:
            seen.add("fixed")
        if lengths is not None:
            seen.add("ragged")
        if n_prev:
            seen.add("carried_credit")
        if t_stride > pd["T"]:
            seen.add("stride")
    need = {"long", "short", "noop", "evict", "pool0", "pool1", "agg0", "agg1", "ema", "no_ema",
            "uniform", "fixed", "ragged", "carried_credit", "stride"}
    assert need <= seen, need - seen


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_event(seed):
    pd, NH, lengths, n_prev, t_stride = _draw(seed)
    G, W, d, T = pd["group"], pd["window"], pd["head_dim"], pd["T"]
    label = f"sweep {seed}"
    q, k, v = synth.random_small(77000 + seed, NH, G, W, d, T, t_stride=t_stride)
    if lengths is None:
        credit = _credit(seed, NH, n_prev) if n_prev else None
        _run_case(pd, q, k, v, credit_in=credit, n_prev=n_prev, t_stride=t_stride, label=label)
        return
    import torch
    print(f"[case] {label} ragged NH={NH} G={G} W={W} d={d} T={T} K={pd['budget']} "
          f"lengths={lengths.tolist()}", flush=True)
    p = kvc_params(pd, NH)
    p.valid_len = torch.from_numpy(lengths).cuda()
    u = kvc.score_window(p, dev_bf16(q), dev_bf16(k)).cpu().numpy()
    op = oracle_params(pd)
    u_ref = np.zeros((NH, T), dtype=np.float64)
    for n in range(NH):
        u_ref[n] = ams.window_usage_ragged(widen(q[n]), widen(k[n, :T]), op, int(lengths[n]))
        assert_usage_close(u[n], u_ref[n], f"{label} head {n} (len {lengths[n]})")
    check_steps2to5_ragged(pd, u_ref.astype(np.float32), k, v, None, range(NH), lengths)


N_LONG = 30


def _draw_long(seed: int):
    """A valid long-cache case: enough heads and positions for the resident
    and twelve-wave column sums and the split row statistics."""
    rng = np.random.default_rng(3000 + seed)
    while True:
        NH = int(rng.choice([16, 32, 64, 128]))
        T = int(rng.integers(8192, 40000))
        if NH * T > 2_200_000:
            continue
        G = int(rng.choice([1, 2, 4, 8]))
        W = int(rng.choice([16, 32, 64, 128]))
        if seed % 5 == 0:  # a launch with >= 8192 column-sum chunks and a small window: resident pass 2
            NH, T = 128, int(rng.integers(16384, 17000))
            G, W = int(rng.choice([1, 2, 4])), int(rng.choice([16, 32]))
        seg_min = int(rng.choice([4, 16]))
        over = dict(
            group=G, window=W, head_dim=int(rng.choice([64, 128])), T=T,
            budget=int(rng.integers(64, T // 4)),
            delta=float(rng.choice([0.1, 0.05, 1.0])), seg_min=seg_min,
            seg_max=int(rng.choice([0, 4 * seg_min, 256])), q_min=int(rng.integers(0, 3)),
            sinks=4, recent=64, pool_kernel=int(rng.choice([3, 7])),
            pool_mode=int(rng.integers(0, 2)), head_agg=int(rng.random() < 0.25),
            ema=bool(rng.random() < 0.4), quota_mode=int(rng.random() < 0.2),
        )
        pd = _pd(**over)
        if kvc.check_params(kvc_params(pd, NH)) != 0:
            continue
        return pd, NH


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_LONG))
def test_random_long_event(seed):
    import torch
    from parity_utils import check_event_consistency, check_steps2to5
    pd, NH = _draw_long(seed)
    G, W, d, T = pd["group"], pd["window"], pd["head_dim"], pd["T"]
    heads = sorted({0, NH // 2, NH - 1})
    print(f"[case] long sweep {seed}: NH={NH} G={G} W={W} d={d} T={T} K={pd['budget']} "
          f"agg={pd['head_agg']} ema={pd['ema']} sampled heads {heads}", flush=True)
    q, k, v = synth.random_small(88000 + seed, NH, G, W, d, T)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    p = kvc_params(pd, NH)
    u_gpu = kvc.score_window(p, dq, dk).cpu().numpy()
    op = oracle_params(pd)
    u_mix = u_gpu.copy()
    for n in heads:
        u_ref = ams.window_usage(widen(q[n]), widen(k[n, :T]), op)
        assert_usage_close(u_gpu[n], u_ref, f"long sweep {seed} head {n}")
        u_mix[n] = u_ref.astype(np.float32)
    check_steps2to5(pd, u_mix, k, v, None, heads, dk=dk, dv=dv)
    check_event_consistency(pd, dq, dk, dv, None, NH)
