"""Throughput of the KV-compression event on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-heads N]
                    [--ragged MAX_PAD] [--seg-fixed L] [--quota-mode mass|uniform]

--ragged left-pads each batch element's prompt by 0..MAX_PAD positions (its
real tokens are the last T - pad); --seg-fixed / --quota-mode select the
fixed-length-segment and uniform-quota ablations.  These variants are
reported with their own config keys; the headline is the default run.

One step = one compression event over every head-event of the workload
(all layers x batch x KV heads): window score -> mass/segmentation/quota ->
select -> gather, inputs resident in HBM, outputs preallocated.  W untimed
warm-up events run first, and at least 0.25 s of them (warmup_events in the
output counts them), then exactly K timed events.  The default
workload is the largest one, the Llama-3.1-8B-shaped long-context event
(32 layers x 8 KV heads, G=4, d=128, T=131072, W=128, budget 4096, full AMS
segmentation with EMA credit); --workload picks another (qwen7b_t768,
qwen7b_t1536_ema, llama8b_global_t16k, tiny).  Inputs are seeded synthetic
data (eviction_window_qk_amd.synth).

Prints ONE JSON line:
  value          cached tokens scored per second (n_heads * T / step time)
  roofline       the score stage (the dominant kernels: row statistics,
                 column sums, fill) timed live with HIP events on the launch
                 stream: algorithmic flops (one causal QK^T) / duration against
                 the bf16 dense MFMA peak, or, where the stage's arithmetic
                 intensity is below the ridge (the 16K global workload),
                 algorithmic bytes (one read of K and Q, the write of u) /
                 duration against HBM; mfma_frac is the flop view either way
  cpu_baseline   the CPU oracle (test infrastructure, not tuned) timed on this
                 host's cores on a bounded sample of the same workload, plus
                 the oracle's steps 2-5 on every head of the GPU's own usage
                 (the bit-exact check path) and whether the GPU's kept
                 indices equal it
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-compression throughput: cached tokens scored/sec per GPU; % of roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
SETTLE_S = 0.25                # minimum untimed warm-up before the timed events


def _gen_chunk(args):
    name, heads, seed, T = args
    from eviction_window_qk_amd import synth
    return synth.gen_heads(synth.WORKLOADS[name], heads, T=T, seed=seed)


def generate(name: str, seed=None, workers: int = 16, T=None):
    """All heads of the workload as bf16 bits (host), in parallel chunks
    (T rows of K/V per head, the workload's T by default)."""
    from eviction_window_qk_amd import synth
    wl = synth.WORKLOADS[name]
    heads = list(range(wl.n_heads))
    chunks = [heads[i:i + 64] for i in range(0, len(heads), 64)]
    G, W, d = wl.group, wl.window, wl.head_dim
    T = wl.T if T is None else T
    q = np.empty((wl.n_heads, G, W, d), np.uint16)
    k = np.empty((wl.n_heads, T, d), np.uint16)
    v = np.empty((wl.n_heads, T, d), np.uint16)
    if workers <= 1 or len(chunks) == 1:
        parts = map(_gen_chunk, [(name, c, seed, T) for c in chunks])
    else:
        import multiprocessing as mp
        pool = mp.get_context("spawn").Pool(workers)
        parts = pool.imap(_gen_chunk, [(name, c, seed, T) for c in chunks])
    for c, (qq, kk, vv) in zip(chunks, parts):
        q[c[0]:c[-1] + 1], k[c[0]:c[-1] + 1], v[c[0]:c[-1] + 1] = qq, kk, vv
    if workers > 1 and len(chunks) > 1:
        pool.close()
        pool.join()
    return q, k, v


def algorithmic(wl, lengths=None) -> dict:
    """Per-event algorithmic work (one causal QK^T; bytes of the data each
    stage must move at least once), summed over the heads' real lengths
    (all T unless a ragged batch gives per-head lengths)."""
    G, W, d, K = wl.group, wl.window, wl.head_dim, wl.budget
    Ts = np.full(wl.n_heads, wl.T, dtype=np.float64) if lengths is None else \
        np.asarray(lengths, dtype=np.float64)
    ema = bool(wl.params.get("ema"))
    pairs = W * (Ts - W) + W * (W + 1) / 2.0         # causal (query, key) pairs per head
    kk = np.minimum(Ts, K)
    flops = float(np.sum(2.0 * d * G * pairs))
    b_score = float(np.sum(2.0 * Ts * d + 2.0 * G * W * d + 4.0 * Ts))
    b_mass = float(np.sum(4.0 * Ts + 4.0 * Ts + (8.0 * K + 16.0 * Ts if ema else 0.0)))
    b_select = float(np.sum(4.0 * Ts + 4.0 * K))
    b_gather = float(np.sum(8.0 * kk * d + (16.0 * kk if ema else 0.0)))
    return dict(flops=flops, b_score=b_score, b_mass=b_mass, b_select=b_select,
                b_gather=b_gather, b_total=b_score + b_mass + b_select + b_gather)


def _recorded(kind: str, workload: str):
    """A committed counter record (profiles/<kind>_<workload>.json), or None
    when it is missing or the score kernels have changed since the counters
    were taken (source hash mismatch)."""
    import hashlib
    f = os.path.join(ROOT, "profiles", f"{kind}_{workload}.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    src = os.path.join(ROOT, "eviction_window_qk_amd", "csrc", "kvc_score.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    return rec if rec.get("score_source_sha256_16") == h else None


def recorded_traffic(workload: str):
    """HBM bytes per score-stage launch (FETCH_SIZE + WRITE_SIZE runs)."""
    rec = _recorded("traffic", workload)
    return rec["score_stage_traffic_bytes"] if rec else None


def recorded_mfma(workload: str):
    """rocprofv3 MfmaUtil of the two score passes and the bf16 flops they
    execute per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)."""
    rec = _recorded("mfma", workload)
    if not rec:
        return None
    return {"mfma_busy": rec["mfma_busy"],
            "executed_flops_per_launch": sum(rec["mfma_flops_per_launch"].values())}


def _oracle_head(args):
    name, n = args
    from eviction_window_qk_amd import synth
    from oracle import ams
    wl = synth.WORKLOADS[name]
    hd = synth.gen_head(wl, n)
    pd = wl.event_params()
    keys = set(ams.Params.__dataclass_fields__)
    op = ams.Params(**{k: v for k, v in pd.items() if k in keys})
    q = synth.bf16_bits_to_f32(hd["q"]).astype(np.float64)
    k = synth.bf16_bits_to_f32(hd["k"]).astype(np.float64)
    t0 = time.perf_counter()
    ams.event(q, k, hd["v"], None, op)
    return time.perf_counter() - t0


# Head-events in the default CPU sample: about 10-30 s of single-core oracle
# work per workload (the fp64 window score dominates).
CPU_SAMPLE_HEADS = {"tiny": 64, "qwen7b_t768": 3584, "qwen7b_t1536_ema": 1024,
                    "llama8b_global_t16k": 128, "llama8b_t128k": 32}


def _oracle_steps2to5(args):
    """Oracle steps 2-5 of one head on the GPU's fp32 usage; returns (seconds,
    kept)."""
    pd, n_prev, u_row, credit_row = args
    from oracle import ams
    keys = set(ams.Params.__dataclass_fields__)
    op = ams.Params(**{k: v for k, v in pd.items() if k in keys}).with_(n_prev=n_prev)
    k0 = np.zeros((pd["T"], 1), np.uint16)
    t0 = time.perf_counter()
    res = ams.steps2to5(u_row, k0, k0, credit_row, op)
    return time.perf_counter() - t0, res.kept


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, n_heads: int, cores: int, gpu_u=None, gpu_kept=None, pd=None,
                 n_prev=0, credit=None) -> dict:
    """The oracle, as it stands, on n_heads head-events of the workload (the
    first n_heads, cycling if more than the workload has), and its steps 2-5 on
    the GPU's usage of every head (when given)."""
    import multiprocessing as mp
    from eviction_window_qk_amd import synth
    wl = synth.WORKLOADS[name]
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    heads = [i % wl.n_heads for i in range(n_heads)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_head, [("tiny", 0)] * cores)         # warm the workers
        t0 = time.perf_counter()
        busy = pool.map(_oracle_head, [(name, n) for n in heads])
        wall = time.perf_counter() - t0
        s25 = None
        if gpu_u is not None:
            args = [(pd, n_prev, gpu_u[n], None if credit is None else credit[n])
                    for n in range(gpu_u.shape[0])]
            t1 = time.perf_counter()
            res = pool.map(_oracle_steps2to5, args, chunksize=4)
            wall25 = time.perf_counter() - t1
            exact = all(np.array_equal(kept, gpu_kept[n]) for n, (_, kept) in enumerate(res))
            s25 = {"heads": len(args), "wall_s": wall25, "cpu_s": sum(s for s, _ in res),
                   "tokens_per_s": len(args) * wl.T / wall25, "kept_bit_exact": exact}
    tokens = len(heads) * wl.T
    out = {"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{len(heads)} head-events ({len(heads) / wl.n_heads:.3f} events of {name}, "
                     f"{wl.n_heads} head-events each, T={wl.T}): full oracle event per head (fp64 "
                     f"score + exact steps 2-5), {cores} worker processes x 1 thread; "
                     f"{sum(busy):.1f} s of CPU work in {wall:.1f} s wall",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if s25:
        out["oracle_steps2to5_on_gpu_usage"] = s25
    return out


def refresh_pieces(wl, steps: int, warmup: int) -> dict:
    """Times of the RefreshKV decode-loop pieces at the workload's shape: one
    query comparison over every (layer, sequence) row, one partial step over
    every head, and the full sync of 16 decoded tokens per head."""
    import torch
    from eviction_window_qk_amd import kvc
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(wl.seed)
    rows, Hq, d = wl.layers * wl.batch, wl.kv_heads * wl.group, wl.head_dim
    NH, K, T = wl.n_heads, wl.budget, wl.T
    q = torch.randn((rows, Hq, d), generator=g).to(torch.bfloat16).to(dev)
    q_ref = torch.randn((rows, d), generator=g, dtype=torch.float64).to(dev)
    ps = torch.rand((NH, K), generator=g).to(dev)
    pp = torch.randint(0, T, (NH, K), generator=g, dtype=torch.int32).to(dev)
    kp = torch.randn((NH, K, d), generator=g).to(torch.bfloat16).to(dev)
    vp = torch.randn_like(kp)
    kn = torch.randn((NH, d), generator=g).to(torch.bfloat16).to(dev)
    vn = torch.randn_like(kn)
    kf = torch.zeros((NH, T + 16, d), dtype=torch.bfloat16, device=dev)
    vf = torch.zeros_like(kf)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1000.0  # us

    t_qc = timed(lambda: kvc.qc_trigger(q, q_ref, 0.5, update_ref=False, stream=stream))
    t_app = timed(lambda: kvc.partial_append(ps, pp, kp, vp, kn, vn, T, stream=stream))
    # 16 tokens decoded since the last full step, in random slots of each head
    pp.copy_(torch.randint(0, T, (NH, K), generator=g, dtype=torch.int32).to(dev))
    slots = torch.rand((NH, K), generator=g).argsort(dim=1)[:, :16].to(dev)
    pp.scatter_(1, slots, (T + torch.arange(16, dtype=torch.int32, device=dev)).expand(NH, 16)
                .contiguous())
    t_sync = timed(lambda: kvc.full_sync(pp, kp, vp, kf, vf, T, stream=stream))
    b_qc = rows * Hq * d * 2 + rows * d * 8
    b_app = NH * K * 4 + NH * (2 * d * 2 * 2 + 8)
    b_sync = NH * K * 4 + NH * 16 * d * 2 * 2 * 2
    return {"metric": "RefreshKV decode-loop pieces: us per call", "workload": wl.name,
            "rows": rows, "heads_q": Hq, "n_heads": NH, "budget": K, "head_dim": d,
            "qc_trigger_us": t_qc, "partial_append_us": t_app, "full_sync_us": t_sync,
            "GBs": {"qc_trigger": b_qc / t_qc / 1e3, "partial_append": b_app / t_app / 1e3,
                    "full_sync": b_sync / t_sync / 1e3},
            "steps": steps, "warmup": warmup}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_t128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="head-events in the CPU oracle sample (default: about 10-30 s of "
                         "single-core work for the workload)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--ragged", type=int, default=0, metavar="MAX_PAD",
                    help="left-pad each batch element by 0..MAX_PAD positions (ragged batch)")
    ap.add_argument("--seg-fixed", type=int, default=0, metavar="L",
                    help="ablation: fixed-length raw segments of L positions")
    ap.add_argument("--quota-mode", choices=("mass", "uniform"), default="mass",
                    help="ablation: uniform instead of mass-weighted quotas")
    ap.add_argument("--refresh", action="store_true",
                    help="time the RefreshKV decode-loop pieces (query comparison, partial "
                         "append/evict, full sync) at the workload's shape instead of the event")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="also time the paged compaction (kvc_gather_paged) with BLOCK-token "
                         "blocks of a shuffled pool, driven by the event's kept indices")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (the event is independent per head "
              f"and runs on one GPU's share); --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from eviction_window_qk_amd import kvc, synth

    if not torch.cuda.is_available():
        sys.exit("bench.py: no GPU visible")
    if args.copy_probe:
        # A plain device-to-device copy of known size: what FETCH_SIZE/WRITE_SIZE
        # read for it calibrates the traffic counters.
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        secs = e0.elapsed_time(e1) / 10 * 1e-3
        print(json.dumps({"copy_probe_bytes": args.copy_probe,
                          "copy_read_plus_write_GBs": 2 * args.copy_probe / secs / 1e9}))
        return
    wl = synth.WORKLOADS[args.workload]
    if args.refresh:
        print(json.dumps(refresh_pieces(wl, args.steps, args.warmup)), flush=True)
        return
    cores = min(len(os.sched_getaffinity(0)), 16)
    t_gen = time.perf_counter()
    prior = bool(wl.params.get("ema")) and bool(wl.prior_seed) and not args.ragged
    q, k, v = generate(args.workload, seed=wl.prior_seed if prior else None, workers=cores)
    print(f"[bench] generated {wl.n_heads} head-events in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    ema = bool(wl.params.get("ema"))
    # A workload with a prior event times the second of two: event 0 runs here on
    # the prior cache, event 1 on its compacted K/V plus the T - K tokens decoded
    # since, with its credit.  Other EMA workloads start fresh (no carried credit).
    chained = prior
    n_prev = wl.budget if chained else 0
    credit = None
    if chained:
        p0 = kvc.Params.from_dict(wl.event_params(), n_heads=wl.n_heads)
        ev0 = kvc.compress_event(p0, dq, dk, dv)  # dq, dk, dv: the prior event's inputs
        q1, kf, vf = generate(args.workload, workers=cores, T=wl.T - wl.budget)
        dq = to_dev(q1)
        dk = torch.cat([ev0["k_out"], to_dev(kf)], dim=1)
        dv = torch.cat([ev0["v_out"], to_dev(vf)], dim=1)
        credit = ev0["credit_out"]
        del ev0, q1, kf, vf
        torch.cuda.synchronize()
    variant = {}
    if args.seg_fixed:
        variant["seg_fixed"] = args.seg_fixed
    if args.quota_mode == "uniform":
        variant["quota_mode"] = kvc.QUOTA_UNIFORM
    p = kvc.Params.from_dict(wl.event_params(**variant), n_heads=wl.n_heads, n_prev=n_prev)
    lengths = None
    if args.ragged:
        lengths = synth.batch_valid_lengths(wl, args.ragged, seed=wl.seed)
        p.valid_len = torch.from_numpy(lengths).to(dev)
    ws = kvc.new_workspace(p, dev)
    S = kvc.segment_capacity(p)
    u = torch.empty((wl.n_heads, wl.T), dtype=torch.float32, device=dev)
    out = dict(score=torch.empty((wl.n_heads, wl.T), dtype=torch.float32, device=dev),
               seg_start=torch.empty((wl.n_heads, S), dtype=torch.int32, device=dev),
               seg_quota=torch.empty((wl.n_heads, S), dtype=torch.int32, device=dev),
               n_seg=torch.empty((wl.n_heads,), dtype=torch.int32, device=dev))
    if ema:
        out["credit_upd"] = torch.empty((wl.n_heads, wl.T), dtype=torch.int64, device=dev)
    kept = torch.empty((wl.n_heads, wl.budget), dtype=torch.int32, device=dev)
    k_out = torch.empty((wl.n_heads, wl.budget, wl.head_dim), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty_like(k_out)
    c_out = torch.empty((wl.n_heads, wl.budget), dtype=torch.int64, device=dev) if ema else None
    stream = torch.cuda.current_stream()

    def stages(ev=None):
        if ev:
            ev[0].record(stream)
        kvc.score_window(p, dq, dk, u=u, ws=ws, stream=stream)
        if ev:
            ev[1].record(stream)
        kvc.mass_segment(p, u, credit, ws=ws, stream=stream, out=out)
        if ev:
            ev[2].record(stream)
        kvc.select(p, out["score"], out["seg_start"], out["seg_quota"], out["n_seg"], kept=kept,
                   ws=ws, stream=stream)
        if ev:
            ev[3].record(stream)
        kvc.gather_compact(p, kept, dk, dv, out.get("credit_upd"), k_out=k_out, v_out=v_out,
                           credit_out=c_out, stream=stream)
        if ev:
            ev[4].record(stream)

    ev_out = dict(k_out=k_out, v_out=v_out, kept=kept)
    if ema:
        ev_out["credit_out"] = c_out

    def event():
        kvc.compress_event(p, dq, dk, dv, credit, ws=ws, out=ev_out, stream=stream)

    def timed(fn, steps):
        """Average ms of fn over `steps` calls, bracketed by events on the
        launch stream after a full synchronisation."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # A: the headline -- whole events through the product entry point.  The
    # untimed warm-up is the W events asked for and at least SETTLE_S seconds
    # of them: the first events after start-up run ~10 % slower (clocks, TLB
    # and caches still settling), which a short W would leave in the timing.
    n_warm, t_warm = 0, time.perf_counter()
    while n_warm < args.warmup or time.perf_counter() - t_warm < SETTLE_S:
        event()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()  # keep the wall clock in step with the GPU
    ms = timed(event, args.steps)
    # B: the dominant kernels (score stage) alone, same stream, same data.
    score_ms = timed(lambda: kvc.score_window(p, dq, dk, u=u, ws=ws, stream=stream), args.steps)
    # C: per-stage breakdown (event records between stages; informative only).
    for _ in range(2):
        stages()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        stages(events[i])
    torch.cuda.synchronize()
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in events])
    stage_ms = stage.mean(axis=0)
    # D: the per-event distribution (an event recorded between consecutive
    # events; informative only -- the headline is A's block average).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        event()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per_event = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    event_pct = {"p10": float(np.percentile(per_event, 10)), "median": float(np.median(per_event)),
                 "p90": float(np.percentile(per_event, 90))}

    paged = None
    if args.paged:
        # The same cache as a pool of BLOCK-token blocks [n_blocks, kv_heads, BLOCK, d] in
        # shuffled order; every (layer, batch) pair is one sequence of the pool.
        bs, H = args.paged, wl.kv_heads
        if wl.T % bs or wl.budget % bs:
            sys.exit("bench.py: --paged needs T and budget multiples of BLOCK")
        nseq, nb_in, nb_out = wl.n_heads // H, wl.T // bs, wl.budget // bs
        n_blocks = nseq * (nb_in + nb_out)
        g = torch.Generator().manual_seed(wl.seed)
        perm = torch.randperm(n_blocks, generator=g).to(torch.int32)
        t_in = perm[:nseq * nb_in].view(nseq, nb_in).to(dev)
        t_out = perm[nseq * nb_in:].contiguous().view(nseq, nb_out).to(dev)
        k_pool = torch.empty((n_blocks, H, bs, wl.head_dim), dtype=torch.bfloat16, device=dev)
        v_pool = torch.empty_like(k_pool)
        blocked = lambda x: x.view(nseq, H, nb_in, bs, wl.head_dim).permute(0, 2, 1, 3, 4) \
            .reshape(nseq * nb_in, H, bs, wl.head_dim)
        k_pool[t_in.flatten().long()] = blocked(dk)
        v_pool[t_in.flatten().long()] = blocked(dv)
        gp = lambda: kvc.gather_paged(p, kept, k_pool, v_pool, t_in, t_out, H, stream=stream)
        for _ in range(2):
            gp()
        gp_ms = timed(gp, args.steps)
        b_gp = algorithmic(wl, lengths)["b_gather"]
        paged = {"block": bs, "ms": gp_ms, "achieved_GBs": b_gp / (gp_ms * 1e-3) / 1e9,
                 "frac": b_gp / (gp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    alg = algorithmic(wl, lengths)
    tokens = wl.n_heads * wl.T if lengths is None else int(lengths.sum())
    # The score stage's bound from its own arithmetic intensity: one causal QK^T
    # against one read of K and Q (and the write of u).  Every workload but the
    # 16K global one (128 query rows per head) sits above the ridge.
    score_hbm_bound = alg["b_score"] / (PEAK_HBM_GBS * 1e9) > alg["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    achieved = alg["flops"] / (score_ms * 1e-3) / 1e12
    if score_hbm_bound:
        achieved_gbs = alg["b_score"] / (score_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    t_roof = max(alg["flops"] / (PEAK_BF16_TFLOPS * 1e12), alg["b_total"] / (PEAK_HBM_GBS * 1e9))
    gather_gbs = alg["b_gather"] / (stage_ms[3] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_events": n_warm,
        "ms_per_step": ms,
        "event_ms": event_pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_heads": wl.n_heads, "layers": wl.layers,
                   "batch": wl.batch, "kv_heads": wl.kv_heads, "group": wl.group,
                   "head_dim": wl.head_dim, "T": wl.T, "window": wl.window,
                   "budget": wl.budget, "ema": ema, "seed": wl.seed, "n_prev": n_prev,
                   **({"prior_event_seed": wl.prior_seed} if chained else {}), **variant,
                   **({"ragged_max_pad": args.ragged, "real_tokens": tokens} if args.ragged
                      else {})},
        "roofline": {**roof,
                     "traffic": None if (args.ragged or variant) else recorded_traffic(wl.name),
                     "kernel": "score stage (k_rowstats [+ k_rowmerge] + k_colsum or k_colsum_resident + k_fill)",
                     "algorithmic_flops_per_launch": alg["flops"],
                     "algorithmic_bytes_per_launch": alg["b_score"],
                     "mfma_frac": achieved / PEAK_BF16_TFLOPS},
        "events_per_s": 1000.0 / ms,
        "event_roofline_frac": t_roof / (ms * 1e-3),
        "score_stage_ms": score_ms,
        "stages_ms": {"score": stage_ms[0], "mass_segment": stage_ms[1],
                      "select": stage_ms[2], "gather": stage_ms[3]},
        "gather": {"achieved_GBs": gather_gbs, "frac": gather_gbs / PEAK_HBM_GBS},
    }
    mf = None if (args.ragged or variant) else recorded_mfma(wl.name)
    if mf:  # counter-derived, from profiles/: executed work (two passes) and MFMA busy
        ex = mf["executed_flops_per_launch"] / (score_ms * 1e-3) / 1e12
        line["roofline"].update({"executed_flops_per_launch": mf["executed_flops_per_launch"],
                                 "executed_frac": ex / PEAK_BF16_TFLOPS,
                                 "mfma_busy": mf["mfma_busy"]})
    if paged:
        line["paged_gather"] = paged
    if not args.no_cpu_baseline and not (args.ragged or variant):
        # The GPU's own usage and kept indices of one more event, for the
        # oracle's steps 2-5 (the bit-exact check path).
        ev_u = dict(ev_out, u=u)
        kvc.compress_event(p, dq, dk, dv, credit, ws=ws, out=ev_u, stream=stream)
        torch.cuda.synchronize()
        gpu_u, gpu_kept = u.cpu().numpy(), kept.cpu().numpy()
        cred = credit.cpu().numpy().view(np.uint64) if credit is not None else None
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(
            args.workload, args.cpu_heads or CPU_SAMPLE_HEADS.get(args.workload, 2 * wl.n_heads),
            cores, gpu_u=gpu_u, gpu_kept=gpu_kept, pd=wl.event_params(**variant), n_prev=n_prev,
            credit=cred)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
