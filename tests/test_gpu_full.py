"""Full-size events of every workload, in the launch configuration bench.py
times: one kvc_compress_event over all head-events of the workload.

Sampled head-events are checked against the oracle (window score to 2e-3
relative; steps 2-5 bit for bit on the oracle's fp32 usage, fed through the
stage entry points at full size); every head-event is checked by properties
(valid kept lists, K/V rows equal to the gathered input rows); the event equals
the stage entry points run in sequence, bit for bit.
"""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import ams
from parity_utils import (assert_usage_close, check_kept_valid, dev_bf16, dev_u64, gen_all,
                          host_bits, host_u64, kvc_params, oracle_params, widen)

pytestmark = pytest.mark.gpu


def _steps2to5_sampled(pd, p, u_full: torch.Tensor, u_ref32: dict, credit_in, k_bits, v_bits,
                       dk, dv, n_prev, heads):
    """Stage entry points at full size on the GPU's usage with the sampled
    heads' rows replaced by the oracle's fp32 usage; sampled heads must equal
    the oracle bit for bit."""
    op = oracle_params(pd, n_prev)
    u_mix = u_full.clone()
    for n in heads:
        u_mix[n] = torch.from_numpy(u_ref32[n]).cuda()
    dci = dev_u64(credit_in) if credit_in is not None else None
    ws = kvc.new_workspace(p, u_mix.device)
    ms = kvc.mass_segment(p, u_mix, dci, ws=ws)
    kept = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    ko, vo, co = kvc.gather_compact(p, kept, dk, dv, ms.get("credit_upd"))
    torch.cuda.synchronize()
    for n in heads:
        ci = credit_in[n] if credit_in is not None else None
        res = ams.steps2to5(u_ref32[n], k_bits[n, :pd["T"]], v_bits[n, :pd["T"]], ci, op)
        np.testing.assert_array_equal(ms["score"][n].cpu().numpy().view(np.uint32),
                                      res.score.view(np.uint32), err_msg=f"head {n} score")
        ns = len(res.segs)
        assert int(ms["n_seg"][n]) == ns, f"head {n}"
        np.testing.assert_array_equal(ms["seg_start"][n, :ns].cpu().numpy(), [a for a, _ in res.segs])
        np.testing.assert_array_equal(ms["seg_quota"][n, :ns].cpu().numpy(), res.q)
        np.testing.assert_array_equal(kept[n].cpu().numpy(), res.kept, err_msg=f"head {n} kept")
        np.testing.assert_array_equal(host_bits(ko[n]), res.k_out, err_msg=f"head {n} K_out")
        np.testing.assert_array_equal(host_bits(vo[n]), res.v_out, err_msg=f"head {n} V_out")
        if p.ema:
            np.testing.assert_array_equal(host_u64(co[n]), res.credit_out)
    return ms


def _check_event(name, pd, q, k, v, credit_in, n_prev, heads, label):
    NH = q.shape[0]
    T = pd["T"]
    print(f"[full] {label}: NH={NH} T={T} K={pd['budget']} sampled heads {heads}", flush=True)
    p = kvc_params(pd, NH, n_prev)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    dci = dev_u64(credit_in) if credit_in is not None else None
    ws = kvc.new_workspace(p, dq.device)
    ev = kvc.compress_event(p, dq, dk, dv, dci, ws=ws, want_u=True)
    torch.cuda.synchronize()
    # properties on every head-event
    kept = ev["kept"].cpu().numpy()
    check_kept_valid(kept, pd, T)
    idx = ev["kept"].long().clamp(min=0)
    gk = torch.gather(dk.view(torch.int16), 1, idx[:, :, None].expand(-1, -1, dk.shape[2]))
    assert torch.equal(gk, ev["k_out"].view(torch.int16)), "K_out rows != K[kept]"
    gv = torch.gather(dv.view(torch.int16), 1, idx[:, :, None].expand(-1, -1, dv.shape[2]))
    assert torch.equal(gv, ev["v_out"].view(torch.int16)), "V_out rows != V[kept]"
    # the event equals the stage entry points in sequence
    u2 = kvc.score_window(p, dq, dk, ws=ws)
    ms = kvc.mass_segment(p, u2, dci, ws=ws)
    kept2 = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(u2.view(torch.int32), ev["u"].view(torch.int32))
    assert torch.equal(kept2, ev["kept"])
    print(f"[full] {label}: properties and event consistency ok", flush=True)
    # sampled heads against the oracle
    op = oracle_params(pd, n_prev)
    u_gpu = ev["u"].cpu().numpy()
    u_ref32 = {}
    for n in heads:
        u_ref = ams.window_usage(widen(q[n]), widen(k[n, :T]), op)
        assert_usage_close(u_gpu[n], u_ref, f"{label} head {n}")
        u_ref32[n] = u_ref.astype(np.float32)
        print(f"[full] {label}: head {n} usage within tolerance", flush=True)
    _steps2to5_sampled(pd, p, ev["u"], u_ref32, credit_in, k, v, dk, dv, n_prev, heads)
    print(f"[full] {label}: steps 2-5 bit-exact on sampled heads", flush=True)
    return ev


def test_full_tiny():
    q, k, v = synth.gen_heads(synth.WORKLOADS["tiny"], [0])
    _check_event("tiny", synth.WORKLOADS["tiny"].event_params(), q, k, v, None, 0, [0], "tiny")


def test_full_qwen7b_t768():
    name = "qwen7b_t768"
    q, k, v = gen_all(name)
    _check_event(name, synth.WORKLOADS[name].event_params(), q, k, v, None, 0,
                 [0, 613, 1234, 1791], name)


def test_full_qwen7b_t1536_ema_chain():
    """Event 0 on the fresh cache, then event 1 on the compacted cache plus the
    512 tokens since, with the carried credit.  Sampled heads take their event-1
    inputs from the oracle's event 0; the other heads from the GPU's (they are
    checked by properties only)."""
    name = "qwen7b_t1536_ema"
    wl = synth.WORKLOADS[name]
    pd = wl.event_params()
    K, T = wl.budget, wl.T
    heads = [0, 3333, 7167]
    q0, k0, v0 = gen_all(name, seed=wl.prior_seed)
    ev0 = _check_event(name, pd, q0, k0, v0, None, 0, heads[:1], "qwen7b_t1536_ema event 0")
    k_out = host_bits(ev0["k_out"])
    v_out = host_bits(ev0["v_out"])
    credit = host_u64(ev0["credit_out"])
    del ev0
    op0 = oracle_params(pd, 0)
    for n in heads:  # oracle event 0 for the sampled heads
        u0 = ams.window_usage(widen(q0[n]), widen(k0[n]), op0)
        r0 = ams.steps2to5(u0.astype(np.float32), k0[n], v0[n], None, op0)
        k_out[n], v_out[n], credit[n] = r0.k_out, r0.v_out, r0.credit_out
    del q0, k0, v0
    q1, kf, vf = gen_all(name, T=T - K)           # fresh queries and the new tokens
    k1 = np.concatenate([k_out, kf], axis=1)
    v1 = np.concatenate([v_out, vf], axis=1)
    _check_event(name, pd, q1, k1, v1, credit, K, heads, "qwen7b_t1536_ema event 1")


def test_full_llama8b_global_t16k():
    name = "llama8b_global_t16k"
    q, k, v = gen_all(name)
    _check_event(name, synth.WORKLOADS[name].event_params(), q, k, v, None, 0, [0, 1023], name)


def test_full_llama8b_t128k():
    name = "llama8b_t128k"
    q, k, v = gen_all(name, chunk=4)
    ev = _check_event(name, synth.WORKLOADS[name].event_params(), q, k, v, None, 0, [0, 200], name)
    assert int(ev["kept"].shape[1]) == 4096


def test_full_qwen7b_t768_fixed_uniform():
    """The two quota/segment ablations together at full size (the bench's
    --seg-fixed 64 --quota-mode uniform run)."""
    name = "qwen7b_t768"
    q, k, v = gen_all(name)
    pd = synth.WORKLOADS[name].event_params(seg_fixed=64, quota_mode=ams.QUOTA_UNIFORM)
    _check_event(name, pd, q, k, v, None, 0, [0, 999, 1791], "qwen7b_t768 fixed64+uniform")


def test_full_qwen7b_t768_ragged():
    """A left-padded batch at full size (the bench's --ragged 400 run): each
    batch element's prompt is shorter by 0..400 tokens."""
    name = "qwen7b_t768"
    wl = synth.WORKLOADS[name]
    pd = wl.event_params()
    T, K = wl.T, wl.budget
    q, k, v = gen_all(name)
    lengths = synth.batch_valid_lengths(wl, 400, seed=wl.seed)
    heads = [0, 5, 1000, 1791]
    print(f"[full] ragged {name}: lengths {lengths.min()}..{lengths.max()}, heads {heads}",
          flush=True)
    dlen = torch.from_numpy(lengths).cuda()
    p = kvc_params(pd, wl.n_heads)
    p.valid_len = dlen
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    ws = kvc.new_workspace(p, dq.device)
    ev = kvc.compress_event(p, dq, dk, dv, None, ws=ws, want_u=True)
    torch.cuda.synchronize()
    kept = ev["kept"].cpu().numpy()
    for n in range(wl.n_heads):  # properties on every head-event
        L = int(lengths[n])
        row = kept[n][kept[n] >= 0]
        assert len(row) == min(K, L), n
        assert row[0] >= T - L and row[-1] < T and np.all(np.diff(row) > 0), n
    idx = ev["kept"].long().clamp(min=0)
    gk = torch.gather(dk.view(torch.int16), 1, idx[:, :, None].expand(-1, -1, dk.shape[2]))
    assert torch.equal(gk, ev["k_out"].view(torch.int16)), "K_out rows != K[kept]"
    u2 = kvc.score_window(p, dq, dk, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(u2.view(torch.int32), ev["u"].view(torch.int32))
    op = oracle_params(pd)
    u_gpu = ev["u"].cpu().numpy()
    u_mix = ev["u"].clone()
    for n in heads:
        u_ref = ams.window_usage_ragged(widen(q[n]), widen(k[n]), op, int(lengths[n]))
        assert_usage_close(u_gpu[n], u_ref, f"ragged head {n}")
        u_mix[n] = torch.from_numpy(u_ref.astype(np.float32)).cuda()
    ms = kvc.mass_segment(p, u_mix, None, ws=ws)
    kept2 = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    ko, vo, _ = kvc.gather_compact(p, kept2, dk, dv, None)
    torch.cuda.synchronize()
    for n in heads:
        res = ams.steps2to5_ragged(u_mix[n].cpu().numpy(), k[n], v[n], None, op, int(lengths[n]))
        np.testing.assert_array_equal(ms["score"][n].cpu().numpy().view(np.uint32),
                                      res.score.view(np.uint32), err_msg=f"head {n} score")
        ns = len(res.segs)
        assert int(ms["n_seg"][n]) == ns, f"head {n}"
        np.testing.assert_array_equal(ms["seg_start"][n, :ns].cpu().numpy(), [a for a, _ in res.segs])
        np.testing.assert_array_equal(ms["seg_quota"][n, :ns].cpu().numpy(), res.q)
        np.testing.assert_array_equal(kept2[n].cpu().numpy(), res.kept, err_msg=f"head {n} kept")
        np.testing.assert_array_equal(host_bits(ko[n]), res.k_out, err_msg=f"head {n} K_out")
        np.testing.assert_array_equal(host_bits(vo[n]), res.v_out, err_msg=f"head {n} V_out")
    print(f"[full] ragged {name}: sampled heads bit-exact", flush=True)
