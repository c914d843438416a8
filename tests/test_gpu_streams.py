"""Events on several streams at once.

The library keeps no state between calls and enqueues on the caller's
stream, so independent events (each with its own workspace and outputs) may
run concurrently on different streams, and may be enqueued from different
host threads.  Two events of different shapes are enqueued back to back on
two streams, and again from two threads, with no synchronisation between
them; every output must equal the same event run alone on one stream, bit
for bit.
"""
import threading

import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from parity_utils import kvc_params

pytestmark = pytest.mark.gpu

EVENTS = [
    # (seed, NH, G, W, d, T, K, ema)
    (11, 64, 4, 32, 128, 4000, 600, True),
    (12, 128, 7, 64, 64, 1500, 256, False),
]


def _prepare(ev, dev):
    seed, NH, G, W, d, T, K, ema = ev
    q, k, v = synth.random_small(seed, NH, G, W, d, T)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    pd = dict(synth.WORKLOADS["tiny"].params, group=G, window=W, head_dim=d, T=T, budget=K, ema=ema)
    p = kvc_params(pd, NH)
    return p, to(q), to(k), to(v)


def _outputs(p, dev):
    NH, K, d, T = p.n_heads, p.budget, p.head_dim, p.T
    o = dict(k_out=torch.empty((NH, K, d), dtype=torch.bfloat16, device=dev),
             v_out=torch.empty((NH, K, d), dtype=torch.bfloat16, device=dev),
             kept=torch.empty((NH, K), dtype=torch.int32, device=dev),
             u=torch.empty((NH, T), dtype=torch.float32, device=dev))
    if p.ema:
        o["credit_out"] = torch.empty((NH, K), dtype=torch.int64, device=dev)
    return o


def _same(a, b):
    for key in a:
        x, y = a[key], b[key]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), key


def test_two_streams_and_two_threads():
    dev = torch.device("cuda:0")
    evs = [_prepare(ev, dev) for ev in EVENTS]
    print(f"[case] streams: events {[(p.n_heads, p.T) for p, *_ in evs]}", flush=True)
    ref = []
    for p, q, k, v in evs:  # alone, one after the other
        ref.append(kvc.compress_event(p, q, k, v, want_u=True))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in evs]
    wss = [kvc.new_workspace(p, dev) for p, *_ in evs]
    for rep in range(3):
        outs = [_outputs(p, dev) for p, *_ in evs]
        torch.cuda.synchronize()
        for (p, q, k, v), s, ws, o in zip(evs, streams, wss, outs):
            kvc.compress_event(p, q, k, v, ws=ws, out=o, want_u=True, stream=s)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            _same(o, r)

    outs = [_outputs(p, dev) for p, *_ in evs]
    errs = []

    def run(i):
        try:
            p, q, k, v = evs[i]
            kvc.compress_event(p, q, k, v, ws=wss[i], out=outs[i], want_u=True, stream=streams[i])
        except Exception as e:  # reported below
            errs.append(e)

    torch.cuda.synchronize()
    th = [threading.Thread(target=run, args=(i,)) for i in range(len(evs))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for o, r in zip(outs, ref):
        _same(o, r)
    print("[case] streams: concurrent events on two streams and from two threads equal the "
          "events run alone", flush=True)
