"""kvc_compress_event_noalloc (library-held scratch, no workspace) against
kvc_compress_event with a caller workspace, through the C ABI: every output
bit for bit, on two calls in a row, the second smaller than the first (the
scratch keeps the first call's contents, which no call may rely on)."""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from parity_utils import dev_bf16, dev_u64, kvc_params

pytestmark = pytest.mark.gpu


def _both(pd, NH, q, k, v, credit=None, n_prev=0):
    p = kvc_params(pd, NH, n_prev)
    assert kvc.workspace_bytes(p) <= kvc.NOALLOC_SCRATCH_BYTES
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    dci = dev_u64(credit) if credit is not None else None
    ref = kvc.compress_event(p, dq, dk, dv, dci, want_u=True)
    got = kvc.compress_event_noalloc(p, dq, dk, dv, dci, want_u=True)
    torch.cuda.synchronize()
    assert got["status"] == ref["status"]
    assert torch.equal(got["u"].view(torch.int32), ref["u"].view(torch.int32))
    assert torch.equal(got["kept"], ref["kept"])
    assert torch.equal(got["k_out"].view(torch.int16), ref["k_out"].view(torch.int16))
    assert torch.equal(got["v_out"].view(torch.int16), ref["v_out"].view(torch.int16))
    if p.ema:
        assert torch.equal(got["credit_out"], ref["credit_out"])
    return got


def test_noalloc_equals_workspace_event_twice_shrinking():
    wl = synth.WORKLOADS["qwen7b_t768"]
    heads = list(range(512))
    q, k, v = synth.gen_heads(wl, heads)
    print(f"[noalloc] call 1: {len(heads)} Qwen-7B-shaped heads, T={wl.T}", flush=True)
    _both(wl.event_params(), len(heads), q, k, v)
    # second call: fewer heads, a shorter cache, EMA credit carried in
    NH, G, W, d, T, K, n_prev = 5, 2, 16, 64, 300, 100, 60
    q2, k2, v2 = synth.random_small(77, NH, G, W, d, T)
    rng = np.random.default_rng(3)
    credit = (rng.random((NH, n_prev)) * 2.0 ** 37).astype(np.uint64)
    pd = dict(synth.WORKLOADS["tiny"].params, group=G, window=W, head_dim=d, T=T, budget=K,
              ema=True)
    print(f"[noalloc] call 2: {NH} heads, T={T}, EMA with {n_prev} carried credits", flush=True)
    _both(pd, NH, q2, k2, v2, credit, n_prev)
    print("[noalloc] both calls bit-identical to the workspace entry point", flush=True)


def test_noalloc_rejects_an_event_past_its_scratch():
    """The 128K-token event needs ~0.8 GB of scratch: rejected on the host
    before any device call or launch."""
    import ctypes
    wl = synth.WORKLOADS["llama8b_t128k"]
    p = kvc.Params.from_dict(wl.event_params(), n_heads=wl.n_heads)
    assert kvc.workspace_bytes(p) > kvc.NOALLOC_SCRATCH_BYTES
    rc = kvc.lib().kvc_compress_event_noalloc(ctypes.byref(p.to_c()), *([None] * 10))
    assert rc == kvc.ESCRATCH


def test_noalloc_sequence_of_varied_events():
    """Ten events in a row through the no-allocation entry point, each a
    different shape and parameter set (seeded draws of the random sweep:
    pooling, aggregation, EMA with and without carried credit, ablations,
    row stride), each bit for bit equal to the workspace entry point: no call
    depends on what an earlier one left in the shared scratch."""
    from test_gpu_random_sweep import _credit, _draw
    done = 0
    seed = 0
    while done < 10:
        pd, NH, lengths, n_prev, t_stride = _draw(seed)
        seed += 1
        if lengths is not None or t_stride != pd["T"]:
            continue
        G, W, d, T = pd["group"], pd["window"], pd["head_dim"], pd["T"]
        q, k, v = synth.random_small(99000 + seed, NH, G, W, d, T)
        credit = _credit(seed, NH, n_prev) if n_prev else None
        print(f"[noalloc] sequence call {done}: NH={NH} G={G} W={W} d={d} T={T} K={pd['budget']} "
              f"ema={pd['ema']} n_prev={n_prev}", flush=True)
        _both(pd, NH, q, k, v, credit, n_prev)
        done += 1
