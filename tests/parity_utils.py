"""Shared helpers for the GPU parity tests: move seeded inputs to the GPU, run
the oracle on the same inputs, compare element by element.

Inputs always come from the seeded generators (eviction_window_qk_amd.synth);
expected values always come from the oracle run on those inputs.  The steps
2-5 comparisons feed the ORACLE's fp32 usage into the HIP entry points, so
both sides take every integer decision on identical fp32 usage.
"""
from __future__ import annotations

import numpy as np
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import ams

# Step-1 acceptance: |u_gpu - u_ref| <= RTOL * u_ref + ATOL (fp64 reference).
RTOL = 2e-3
ATOL = 1e-30


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u64(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint64).view(np.int64)).cuda()


def host_u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_params(pd: dict, n_prev: int = 0) -> ams.Params:
    keys = {f for f in ams.Params.__dataclass_fields__}
    d = {k: v for k, v in pd.items() if k in keys}
    d["n_prev"] = n_prev
    d["ema"] = bool(d.get("ema", False))
    return ams.Params(**d)


def kvc_params(pd: dict, n_heads: int, n_prev: int = 0, t_stride: int = 0) -> kvc.Params:
    return kvc.Params.from_dict(pd, n_heads=n_heads, n_prev=n_prev, t_stride=t_stride)


def widen(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def assert_usage_close(u_gpu: np.ndarray, u_ref: np.ndarray, what: str = ""):
    err = np.abs(u_gpu.astype(np.float64) - u_ref)
    bound = RTOL * np.abs(u_ref) + ATOL
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err / bound))
        raise AssertionError(f"{what}: {int(bad.sum())} usage values out of tolerance; worst at "
                             f"{i}: gpu={u_gpu.flat[i]!r} ref={u_ref.flat[i]!r}")


def check_steps2to5(pd: dict, u32: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                    credit_in: np.ndarray | None, heads, n_prev: int = 0, t_stride: int = 0,
                    dk=None, dv=None):
    """Run kvc_mass_segment -> kvc_select -> kvc_gather_compact on the fp32
    usage u32 [NH,T] and compare the listed heads bit for bit with the oracle
    run on the same usage.  Returns the GPU outputs."""
    NH, T = u32.shape
    p = kvc_params(pd, NH, n_prev, t_stride)
    op = oracle_params(pd, n_prev)
    du = torch.from_numpy(np.ascontiguousarray(u32, np.float32)).cuda()
    dci = dev_u64(credit_in) if (credit_in is not None and n_prev > 0) else None
    dk = dev_bf16(k_bits) if dk is None else dk
    dv = dev_bf16(v_bits) if dv is None else dv
    ws = kvc.new_workspace(p, du.device)
    ms = kvc.mass_segment(p, du, dci, ws=ws)
    kept = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    ko, vo, co = kvc.gather_compact(p, kept, dk, dv, ms.get("credit_upd"))
    torch.cuda.synchronize()
    g_score = ms["score"].cpu().numpy()
    g_nseg = ms["n_seg"].cpu().numpy()
    g_start = ms["seg_start"].cpu().numpy()
    g_quota = ms["seg_quota"].cpu().numpy()
    g_kept = kept.cpu().numpy()
    g_ko, g_vo = host_bits(ko), host_bits(vo)
    g_cu = host_u64(ms["credit_upd"]) if p.ema else None
    g_co = host_u64(co) if p.ema else None
    for n in heads:
        ci = credit_in[n] if (credit_in is not None and n_prev > 0) else None
        res = ams.steps2to5(u32[n], k_bits[n, :T], v_bits[n, :T], ci, op)
        np.testing.assert_array_equal(g_score[n].view(np.uint32), res.score.view(np.uint32),
                                      err_msg=f"head {n}: pooled score")
        if p.ema:
            np.testing.assert_array_equal(g_cu[n], res.credit_upd, err_msg=f"head {n}: credit")
        if res.noop:
            assert g_nseg[n] == 0
        else:
            ns = len(res.segs)
            assert g_nseg[n] == ns, f"head {n}: {g_nseg[n]} segments, oracle {ns}"
            np.testing.assert_array_equal(g_start[n, :ns], [a for a, _ in res.segs],
                                          err_msg=f"head {n}: segment starts")
            np.testing.assert_array_equal(g_quota[n, :ns], res.q, err_msg=f"head {n}: quotas")
        np.testing.assert_array_equal(g_kept[n], res.kept, err_msg=f"head {n}: kept")
        np.testing.assert_array_equal(g_ko[n], res.k_out, err_msg=f"head {n}: K_out")
        np.testing.assert_array_equal(g_vo[n], res.v_out, err_msg=f"head {n}: V_out")
        if p.ema:
            np.testing.assert_array_equal(g_co[n], res.credit_out, err_msg=f"head {n}: credit_out")
    return dict(score=g_score, kept=g_kept, k_out=g_ko, v_out=g_vo, credit_upd=g_cu,
                credit_out=g_co, n_seg=g_nseg)


def check_event_consistency(pd: dict, dq, dk, dv, dci, n_heads: int, n_prev: int = 0,
                            t_stride: int = 0, valid_len=None):
    """kvc_compress_event equals the four stage entry points run in sequence on
    the same arguments, bit for bit, and repeated calls give the same bits."""
    p = kvc_params(pd, n_heads, n_prev, t_stride)
    p.valid_len = valid_len
    ws = kvc.new_workspace(p, dq.device)
    ev = kvc.compress_event(p, dq, dk, dv, dci, ws=ws, want_u=True)
    ev2 = kvc.compress_event(p, dq, dk, dv, dci, ws=ws, want_u=True)
    u = kvc.score_window(p, dq, dk, ws=ws)
    ms = kvc.mass_segment(p, u, dci, ws=ws)
    kept = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    ko, vo, co = kvc.gather_compact(p, kept, dk, dv, ms.get("credit_upd"))
    torch.cuda.synchronize()
    assert torch.equal(ev["u"].view(torch.int32), u.view(torch.int32))
    assert torch.equal(ev2["u"].view(torch.int32), u.view(torch.int32))
    assert torch.equal(ev["kept"], kept) and torch.equal(ev2["kept"], kept)
    assert torch.equal(ev["k_out"].view(torch.int16), ko.view(torch.int16))
    assert torch.equal(ev["v_out"].view(torch.int16), vo.view(torch.int16))
    if p.ema:
        assert torch.equal(ev["credit_out"], co)
    return ev


def check_kept_valid(kept: np.ndarray, pd: dict, T: int):
    """Properties every kept list has: ascending, distinct, in range, holds the
    must-keep set, length min(budget, T)."""
    K = pd["budget"]
    s = min(pd["sinks"], K, T)
    r = min(pd["recent"], K - s, T - s)
    for n in range(kept.shape[0]):
        row = kept[n]
        valid = row[row >= 0]
        assert len(valid) == min(K, T)
        assert np.all(np.diff(valid) > 0) and valid[0] >= 0 and valid[-1] < T
        must = set(range(s)) | set(range(T - r, T))
        assert must <= set(valid.tolist())


def _gen_chunk(args):
    name, heads, seed, T = args
    return synth.gen_heads(synth.WORKLOADS[name], heads, T=T, seed=seed)


def gen_all(name: str, seed=None, T=None, workers: int = 16, chunk: int = 16):
    """Every head-event of a workload (bf16 bits), generated in parallel; prints
    progress so a long generation is visibly alive."""
    import multiprocessing as mp
    import os
    import time
    wl = synth.WORKLOADS[name]
    T = wl.T if T is None else T
    heads = list(range(wl.n_heads))
    chunks = [heads[i:i + chunk] for i in range(0, len(heads), chunk)]
    q = np.empty((wl.n_heads, wl.group, wl.window, wl.head_dim), np.uint16)
    k = np.empty((wl.n_heads, T, wl.head_dim), np.uint16)
    v = np.empty((wl.n_heads, T, wl.head_dim), np.uint16)
    workers = max(1, min(workers, len(os.sched_getaffinity(0))))
    t0 = time.time()
    with mp.get_context("spawn").Pool(workers) as pool:
        for i, (c, (qq, kk, vv)) in enumerate(zip(chunks, pool.imap(
                _gen_chunk, [(name, c, seed, T) for c in chunks]))):
            q[c[0]:c[-1] + 1], k[c[0]:c[-1] + 1], v[c[0]:c[-1] + 1] = qq, kk, vv
            if (i + 1) % max(1, len(chunks) // 8) == 0:
                print(f"[gen] {name}: {c[-1] + 1}/{wl.n_heads} heads, {time.time() - t0:.1f} s",
                      flush=True)
    return q, k, v


def check_steps2to5_ragged(pd: dict, u32: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                           credit_in, heads, lengths: np.ndarray, n_prev: int = 0):
    """As check_steps2to5 for a left-padded batch (valid_len set): the listed
    heads must equal the oracle's ragged steps 2-5 bit for bit, padding
    included (zeros)."""
    NH, T = u32.shape
    dlen = torch.from_numpy(np.ascontiguousarray(lengths, np.int32)).cuda()
    p = kvc.Params.from_dict(pd, n_heads=NH, n_prev=n_prev, valid_len=dlen)
    op = oracle_params(pd, n_prev)
    du = torch.from_numpy(np.ascontiguousarray(u32, np.float32)).cuda()
    dci = dev_u64(credit_in) if (credit_in is not None and n_prev > 0) else None
    dk, dv = dev_bf16(k_bits), dev_bf16(v_bits)
    ws = kvc.new_workspace(p, du.device)
    ms = kvc.mass_segment(p, du, dci, ws=ws)
    kept = kvc.select(p, ms["score"], ms["seg_start"], ms["seg_quota"], ms["n_seg"], ws=ws)
    ko, vo, co = kvc.gather_compact(p, kept, dk, dv, ms.get("credit_upd"))
    torch.cuda.synchronize()
    g_score = ms["score"].cpu().numpy()
    g_nseg, g_start, g_quota = (ms["n_seg"].cpu().numpy(), ms["seg_start"].cpu().numpy(),
                                ms["seg_quota"].cpu().numpy())
    g_kept, g_ko, g_vo = kept.cpu().numpy(), host_bits(ko), host_bits(vo)
    g_cu = host_u64(ms["credit_upd"]) if p.ema else None
    g_co = host_u64(co) if p.ema else None
    for n in heads:
        ci = credit_in[n] if (credit_in is not None and n_prev > 0) else None
        res = ams.steps2to5_ragged(u32[n], k_bits[n, :T], v_bits[n, :T], ci, op, int(lengths[n]))
        tag = f"head {n} (len {int(lengths[n])})"
        np.testing.assert_array_equal(g_score[n].view(np.uint32), res.score.view(np.uint32),
                                      err_msg=f"{tag}: pooled score")
        if p.ema:
            np.testing.assert_array_equal(g_cu[n], res.credit_upd, err_msg=f"{tag}: credit")
        if res.noop:
            assert g_nseg[n] == 0, tag
        else:
            ns = len(res.segs)
            assert g_nseg[n] == ns, f"{tag}: {g_nseg[n]} segments, oracle {ns}"
            np.testing.assert_array_equal(g_start[n, :ns], [a for a, _ in res.segs],
                                          err_msg=f"{tag}: segment starts")
            np.testing.assert_array_equal(g_quota[n, :ns], res.q, err_msg=f"{tag}: quotas")
        np.testing.assert_array_equal(g_kept[n], res.kept, err_msg=f"{tag}: kept")
        np.testing.assert_array_equal(g_ko[n], res.k_out, err_msg=f"{tag}: K_out")
        np.testing.assert_array_equal(g_vo[n], res.v_out, err_msg=f"{tag}: V_out")
        if p.ema:
            np.testing.assert_array_equal(g_co[n], res.credit_out, err_msg=f"{tag}: credit_out")
    return dict(kept=g_kept)
