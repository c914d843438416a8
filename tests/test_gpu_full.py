"""Full-size events of every workload, in the launch configuration bench.py
times: one kvc_compress_event over all head-events of the workload.

Every head-event's steps 2-5 are checked against the oracle run on the GPU's
own fp32 usage of that event (CPU worker processes): pooled score, credit,
segment starts, quotas, kept indices and carried credit bit for bit, and the
compacted K/V rows equal to K[kept], V[kept] (so, with kept equal to the
oracle's, to the oracle's gather).  The window score is compared with the fp64
oracle on every head of the Qwen-7B and 16K global workloads and on sampled
heads of the others (2e-3 relative); sampled heads also run the stage entry
points on the oracle's own usage, bit for bit.  The event equals the stage
entry points run in sequence, bit for bit.
"""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import ams
import oracle_workers
from parity_utils import (assert_usage_close, check_kept_valid, dev_bf16, dev_u64, gen_all,
                          host_bits, host_u64, kvc_params, oracle_params, widen)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cpu_pool():
    pool = oracle_workers.pool()
    yield pool
    pool.close()
    pool.join()


def _every_head_steps2to5(label, pd, p, u_dev: torch.Tensor, kept_dev: torch.Tensor, credit_in,
                          credit_out_dev, n_prev, pool, lengths=None):
    """Steps 2-5 of every head-event against the oracle fed the GPU's own usage
    u_dev: kvc_mass_segment on u_dev gives the per-head score, credit and
    segment tables (the event computes them identically: the event/stage
    equality is checked separately); kept and the carried credit are the
    event's own outputs."""
    NH, T = u_dev.shape
    dci = dev_u64(credit_in) if (credit_in is not None and n_prev > 0) else None
    ws = kvc.new_workspace(p, u_dev.device)
    ms = kvc.mass_segment(p, u_dev, dci, ws=ws)
    torch.cuda.synchronize()
    u = u_dev.cpu().numpy()
    score = ms["score"].cpu().numpy().view(np.uint32)
    n_seg, starts, quotas = (ms["n_seg"].cpu().numpy(), ms["seg_start"].cpu().numpy(),
                             ms["seg_quota"].cpu().numpy())
    cupd = host_u64(ms["credit_upd"]) if p.ema else None
    kept = kept_dev.cpu().numpy()
    cout = host_u64(credit_out_dev) if p.ema else None
    args = [(pd, n_prev, u[n], None if dci is None else credit_in[n],
             None if lengths is None else int(lengths[n])) for n in range(NH)]
    print(f"[full] {label}: oracle steps 2-5 on the GPU's usage, all {NH} heads", flush=True)
    for n, ref in enumerate(pool.imap(oracle_workers.steps2to5_head, args, chunksize=4)):
        tag = f"{label} head {n}"
        np.testing.assert_array_equal(score[n], ref["score"], err_msg=f"{tag}: pooled score")
        if p.ema:
            np.testing.assert_array_equal(cupd[n], ref["credit_upd"], err_msg=f"{tag}: credit")
            np.testing.assert_array_equal(cout[n], ref["credit_out"], err_msg=f"{tag}: credit_out")
        if ref["noop"]:
            assert n_seg[n] == 0, tag
        else:
            ns = len(ref["starts"])
            assert n_seg[n] == ns, f"{tag}: {n_seg[n]} segments, oracle {ns}"
            np.testing.assert_array_equal(starts[n, :ns], ref["starts"], err_msg=f"{tag}: starts")
            np.testing.assert_array_equal(quotas[n, :ns], ref["quotas"], err_msg=f"{tag}: quotas")
        np.testing.assert_array_equal(kept[n], ref["kept"], err_msg=f"{tag}: kept")
        if (n + 1) % max(1, NH // 4) == 0:
            print(f"[full] {label}: {n + 1}/{NH} heads bit-exact", flush=True)


def _every_head_usage(label, name, u_gpu: np.ndarray, pool, over=None, seed=None):
    """The window score of every head-event against the fp64 oracle (inputs
    regenerated per head in the workers)."""
    NH = u_gpu.shape[0]
    print(f"[full] {label}: fp64 oracle usage, all {NH} heads", flush=True)
    args = [(name, n, over or {}, seed) for n in range(NH)]
    for n, u_ref in enumerate(pool.imap(oracle_workers.usage_head, args, chunksize=4)):
        assert_usage_close(u_gpu[n], u_ref, f"{label} head {n}")
    print(f"[full] {label}: usage within tolerance on every head", flush=True)


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


def _check_event(name, pd, q, k, v, credit_in, n_prev, heads, label, pool, usage_all=False,
                 seed=None):
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
    if usage_all:
        _every_head_usage(label, name, u_gpu, pool, _overrides(name, pd), seed)
    _every_head_steps2to5(label, pd, p, ev["u"], ev["kept"], credit_in, ev.get("credit_out"),
                          n_prev, pool)
    return ev


def _overrides(name, pd):
    """Event parameters of pd that differ from the workload's own."""
    base = synth.WORKLOADS[name].event_params()
    return {k: v for k, v in pd.items() if base.get(k) != v}


def test_full_tiny(cpu_pool):
    q, k, v = synth.gen_heads(synth.WORKLOADS["tiny"], [0])
    _check_event("tiny", synth.WORKLOADS["tiny"].event_params(), q, k, v, None, 0, [0], "tiny",
                 cpu_pool, usage_all=True)


def test_full_qwen7b_t768(cpu_pool):
    name = "qwen7b_t768"
    q, k, v = gen_all(name)
    _check_event(name, synth.WORKLOADS[name].event_params(), q, k, v, None, 0,
                 [0, 613, 1234, 1791], name, cpu_pool, usage_all=True)


def test_full_qwen7b_t1536_ema_chain(cpu_pool):
    """Event 0 on the fresh cache, then event 1 on the compacted cache plus the
    512 tokens since, with the carried credit.  Sampled heads take their event-1
    inputs from the oracle's event 0; the other heads from the GPU's."""
    name = "qwen7b_t1536_ema"
    wl = synth.WORKLOADS[name]
    pd = wl.event_params()
    K, T = wl.budget, wl.T
    heads = [0, 3333, 7167]
    q0, k0, v0 = gen_all(name, seed=wl.prior_seed)
    ev0 = _check_event(name, pd, q0, k0, v0, None, 0, heads[:1], "qwen7b_t1536_ema event 0",
                       cpu_pool, usage_all=True, seed=wl.prior_seed)
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
    _check_event(name, pd, q1, k1, v1, credit, K, heads, "qwen7b_t1536_ema event 1", cpu_pool)


def test_full_llama8b_global_t16k(cpu_pool):
    """The one-segment global top-2048 at full size: the headline SUM over the
    four query heads, then the same inputs with the MAX head aggregation."""
    name = "llama8b_global_t16k"
    q, k, v = gen_all(name)
    pd = synth.WORKLOADS[name].event_params()
    _check_event(name, pd, q, k, v, None, 0, [0, 1023], name, cpu_pool, usage_all=True)
    pd_max = synth.WORKLOADS[name].event_params(head_agg=ams.AGG_MAX)
    _check_event(name, pd_max, q, k, v, None, 0, [0, 511, 1023], f"{name} head_agg=max", cpu_pool,
                 usage_all=True)


def test_full_llama8b_t128k(cpu_pool):
    name = "llama8b_t128k"
    q, k, v = gen_all(name, chunk=4)
    ev = _check_event(name, synth.WORKLOADS[name].event_params(), q, k, v, None, 0, [0, 200], name,
                      cpu_pool, usage_all=True)
    assert int(ev["kept"].shape[1]) == 4096


def test_full_qwen7b_t768_fixed_uniform(cpu_pool):
    """The two quota/segment ablations together at full size (the bench's
    --seg-fixed 64 --quota-mode uniform run)."""
    name = "qwen7b_t768"
    q, k, v = gen_all(name)
    pd = synth.WORKLOADS[name].event_params(seg_fixed=64, quota_mode=ams.QUOTA_UNIFORM)
    _check_event(name, pd, q, k, v, None, 0, [0, 999, 1791], "qwen7b_t768 fixed64+uniform",
                 cpu_pool)


def test_full_qwen7b_t768_ragged(cpu_pool):
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
    _every_head_steps2to5(f"ragged {name}", pd, p, ev["u"], ev["kept"], None, None, 0, cpu_pool,
                          lengths=lengths)
