"""CPU worker functions that run the oracle on many head-events in parallel
for the full-size GPU tests.  Imports only NumPy, the seeded input generator
and the oracle (no torch, no HIP library), so the worker processes never touch
the GPU."""
from __future__ import annotations

import os

import numpy as np

from eviction_window_qk_amd import synth
from oracle import ams


def oracle_params(pd: dict, n_prev: int = 0) -> ams.Params:
    keys = set(ams.Params.__dataclass_fields__)
    d = {k: v for k, v in pd.items() if k in keys}
    d["n_prev"] = n_prev
    d["ema"] = bool(d.get("ema", False))
    return ams.Params(**d)


def steps2to5_head(args):
    """Oracle steps 2-5 of one head on a given fp32 usage row.  Returns the
    integer results and the fp32/u64 arrays the GPU must equal bit for bit;
    the gathered rows follow from `kept` (K_out = K[kept])."""
    pd, n_prev, u_row, credit_row, length = args
    op = oracle_params(pd, n_prev)
    T = pd["T"]
    k0 = np.zeros((T, 1), np.uint16)
    if length is None:
        res = ams.steps2to5(np.asarray(u_row, np.float32), k0, k0, credit_row, op)
    else:
        res = ams.steps2to5_ragged(np.asarray(u_row, np.float32), k0, k0, credit_row, op, length)
    return dict(kept=res.kept, score=res.score.view(np.uint32), credit_upd=res.credit_upd,
                credit_out=res.credit_out, starts=[a for a, _ in res.segs],
                quotas=None if res.q is None else np.asarray(res.q), noop=res.noop)


def usage_head(args):
    """fp64 oracle usage of head-event n of a workload, its inputs regenerated
    here from the seeded generator (optionally with overridden parameters and
    another seed, as for the first event of a chain)."""
    name, n, over, seed = args
    wl = synth.WORKLOADS[name]
    pd = wl.event_params(**over)
    hd = synth.gen_head(wl, n, seed=seed, with_v=False)
    widen = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
    return ams.window_usage(widen(hd["q"]), widen(hd["k"]), oracle_params(pd))


def pool(workers: int = 16):
    """A process pool for these workers, sized to the cores this process may use."""
    import multiprocessing as mp
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    n = max(1, min(workers, len(os.sched_getaffinity(0))))
    return mp.get_context("spawn").Pool(n)
