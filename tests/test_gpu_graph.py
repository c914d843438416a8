"""The whole event captured once in a HIP graph and replayed.

kvc_compress_event enqueues kernel launches only (no memset, copy,
allocation or synchronisation), so a decode loop can capture it once and
replay it at every compression step after copying the step's queries, keys,
values and credit into the captured buffers.  Each replay here runs on new
seeded inputs and is compared bit for bit with an eager call on the same
inputs, with eager work and a synchronisation between replays.  The
no-allocation entry point is captured the same way (its scratch address is
looked up once by an eager call before the capture).
"""
import time

import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from parity_utils import kvc_params

pytestmark = pytest.mark.gpu

CASES = [
    # (label, NH, G, W, d, T, K, ema, n_prev, ragged)
    ("short_ema_carried", 8, 4, 32, 128, 3000, 500, True, 1200, False),
    ("long_cache", 4, 2, 64, 64, 9000, 700, False, 0, False),
    ("ragged", 6, 7, 16, 128, 2000, 300, False, 0, True),
]


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _inputs(seed, NH, G, W, d, T, n_prev):
    q, k, v = synth.random_small(seed, NH, G, W, d, T)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    credit = None
    if n_prev:
        rng = np.random.default_rng(seed)
        r = rng.random((NH, n_prev)) + 1e-3
        credit = torch.from_numpy(np.floor(r / r.sum(axis=1, keepdims=True) * 2.0 ** 44)
                                  .astype(np.uint64).view(np.int64))
    return to(q), to(k), to(v), credit


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_captured_event_replays_match_eager(case, noalloc):
    label, NH, G, W, d, T, K, ema, n_prev, ragged = case
    pd = dict(synth.WORKLOADS["tiny"].params, group=G, window=W, head_dim=d, T=T, budget=K,
              ema=ema)
    p = kvc_params(pd, NH, n_prev)
    dev = torch.device("cuda:0")
    if ragged:
        rng = np.random.default_rng(5)
        p.valid_len = torch.from_numpy(rng.integers(W, T + 1, size=NH).astype(np.int32)).to(dev)
    print(f"[case] graph {label} {'noalloc' if noalloc else 'workspace'}: NH={NH} G={G} W={W} "
          f"d={d} T={T} K={K} ema={ema} n_prev={n_prev}", flush=True)
    if noalloc:
        assert kvc.workspace_bytes(p) <= kvc.NOALLOC_SCRATCH_BYTES
    call = kvc.compress_event_noalloc if noalloc else kvc.compress_event

    # Static buffers the graph reads and writes.
    q0, k0, v0, c0 = _inputs(100, NH, G, W, d, T, n_prev)
    sq, sk, sv = q0.to(dev), k0.to(dev), v0.to(dev)
    sc = c0.to(dev) if c0 is not None else None
    ws = None if noalloc else kvc.new_workspace(p, dev)
    out = dict(k_out=torch.empty((NH, K, d), dtype=torch.bfloat16, device=dev),
               v_out=torch.empty((NH, K, d), dtype=torch.bfloat16, device=dev),
               kept=torch.empty((NH, K), dtype=torch.int32, device=dev),
               u=torch.empty((NH, T), dtype=torch.float32, device=dev))
    if ema:
        out["credit_out"] = torch.empty((NH, K), dtype=torch.int64, device=dev)
    kw = {} if noalloc else dict(ws=ws)

    # Eager warm-up on a side stream (also the no-allocation scratch lookup).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(p, sq, sk, sv, sc, out=out, want_u=True, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(p, sq, sk, sv, sc, out=out, want_u=True, **kw)
    torch.cuda.synchronize()

    for rep in range(4):
        q, k, v, c = _inputs(200 + rep, NH, G, W, d, T, n_prev)
        sq.copy_(q)
        sk.copy_(k)
        sv.copy_(v)
        if sc is not None:
            sc.copy_(c)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in out.items()}
        ref = kvc.compress_event(p, sq, sk, sv, sc, want_u=True)  # eager, its own workspace
        torch.cuda.synchronize()
        for key in got:
            assert torch.equal(_bits(got[key]), _bits(ref[key])), (label, rep, key)
    # Replay rate against eager calls on the same stream (information only).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    t_graph = (time.perf_counter() - t0) / 20
    t0 = time.perf_counter()
    for _ in range(20):
        call(p, sq, sk, sv, sc, out=out, want_u=True, **kw)
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / 20
    print(f"[case] graph {label}: 4 replays bit-identical to eager calls; replay {t_graph * 1e6:.1f} us, "
          f"eager {t_eager * 1e6:.1f} us per event", flush=True)
