"""GPU parity at the limits the host accepts (include/kvc.h): the longest
cache (2^18 positions), the most query rows per KV head (W*G = 4096, G = 64),
the most mass thresholds (1024) and the most fixed segments (1025) -- the
last two also take the segment tables past what the workgroups stage in LDS,
so the global-memory fallbacks of the quota walk and of select run.  Same
acceptance as tests/test_gpu_parity.py: usage within 2e-3 of the fp64 oracle,
steps 2-5 bit for bit on the oracle's usage, the event equal to the stages."""
import pytest

from eviction_window_qk_amd import kvc, synth
from test_gpu_parity import _pd, _run_case

LIMITS = [
    # (label, NH, G, W, d, T, K, overrides)
    ("max_T", 1, 1, 4, 64, 1 << 18, 4096, {}),
    ("max_rows_G64_W64", 2, 64, 64, 128, 1024, 300, {}),
    ("G64_W1", 2, 64, 1, 64, 700, 100, {}),
    ("max_thresholds", 1, 2, 16, 64, 8192, 2000, dict(delta=1.0 / 1025, seg_min=1, seg_max=0)),
    # q_min = 0: no floors, so the quota walk runs over all 1025 segments
    ("max_fixed_segments", 1, 2, 16, 64, 2050, 600, dict(seg_fixed=2, seg_min=1, seg_max=0,
                                                        q_min=0)),
    # about 4100 segments: past what the 1024-thread workgroup stages in LDS
    ("max_T_many_segments", 1, 1, 4, 64, 1 << 18, 8192, dict(seg_max=64)),
    # one segment longer than select's register cache (16 keys x 1024 threads):
    # the threshold search re-reads the scores bit by bit
    ("segment_past_register_cache", 2, 2, 16, 64, 20000, 3000,
     dict(delta=1.0, seg_min=1, seg_max=0)),
    # floors of 1250 segments (q_min = 2) exceed the budget: the over-budget repair
    # runs over a 20000-position cache, also past the register cache
    ("repair_past_register_cache", 1, 2, 16, 64, 20000, 2000,
     dict(seg_min=16, seg_max=16, q_min=2)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", LIMITS, ids=[c[0] for c in LIMITS])
def test_limits(case):
    label, NH, G, W, d, T, K, over = case
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K, **over)
    assert kvc.check_params(kvc.Params(n_heads=NH, T=T, window=W, budget=K, group=G, head_dim=d,
                                       **{k: v for k, v in over.items()})) == 0
    q, k, v = synth.random_small(sum(map(ord, label)), NH, G, W, d, T)
    _run_case(pd, q, k, v, label=label)


def test_segment_counts_reach_the_limits():
    """The two segment-count cases really produce 1025 segments."""
    from oracle import ams
    p = ams.Params(T=2050, window=16, budget=600, seg_fixed=2, seg_min=1, seg_max=0, q_min=0)
    assert ams.segment_capacity(p) == 1025
    p = ams.Params(T=8192, window=16, budget=2000, delta=1.0 / 1025, seg_min=1, seg_max=0)
    assert ams.segment_capacity(p) == 1025


RESIDENT = [
    # (label, NH, G, W, d, T, K, sampled heads): windows of at most four padded 32-row blocks on a
    # launch with >= 8192 column-sum chunks, so pass 2 keeps the queries in LDS and walks 8 chunks
    # per workgroup; the first case ends in a partial chunk and a partial group of chunks
    ("resident_G4_W32", 64, 4, 32, 64, 32768 + 100, 4000, [0, 37, 63]),
    ("resident_G2_W64", 64, 2, 64, 128, 32768, 3000, [0, 63]),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", RESIDENT, ids=[c[0] for c in RESIDENT])
def test_resident_column_sums(case):
    label, NH, G, W, d, T, K, heads = case
    chunks = (T + 255) // 256
    assert NH * chunks >= 8192 and G * ((W + 31) // 32) <= 4
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, v = synth.random_small(sum(map(ord, label)), NH, G, W, d, T)
    _run_case(pd, q, k, v, heads=heads, label=label)


@pytest.mark.gpu
def test_resident_and_streamed_column_sums_agree_bitwise():
    """Pass 2 takes the LDS-resident kernel on a launch with >= 8192 column-sum
    chunks and the streamed one otherwise; both visit the row blocks in the same
    order, so a head's usage has the same bits whichever kernel ran it.  The
    same heads run once inside a 64-head launch (resident) and once alone
    (streamed)."""
    import numpy as np
    import torch
    from parity_utils import dev_bf16, kvc_params
    NH, G, W, d, T, K = 64, 4, 32, 128, 32768, 2000
    assert NH * ((T + 255) // 256) >= 8192 and 4 * ((T + 255) // 256) < 8192
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, _ = synth.random_small(31337, NH, G, W, d, T)
    dq, dk = dev_bf16(q), dev_bf16(k)
    u_all = kvc.score_window(kvc_params(pd, NH), dq, dk)
    for sub in ([0, 1, 2, 3], [40, 63]):
        idx = torch.tensor(sub, device="cuda")
        u_sub = kvc.score_window(kvc_params(pd, len(sub)), dq[idx].contiguous(),
                                 dk[idx].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(u_sub.view(torch.int32), u_all[idx].view(torch.int32)), sub
    print("[case] resident vs streamed column sums: identical bits", flush=True)


@pytest.mark.gpu
def test_resident_column_sums_ragged():
    """A left-padded batch on the LDS-resident pass 2 (its chunk walk stops at
    each head's real length); sampled heads against the oracle."""
    import numpy as np
    import torch
    from oracle import ams
    from parity_utils import (assert_usage_close, check_steps2to5_ragged, dev_bf16, kvc_params,
                              oracle_params, widen)
    NH, G, W, d, T, K = 64, 4, 32, 64, 32768 + 100, 3000
    assert NH * ((T + 255) // 256) >= 8192
    rng = np.random.default_rng(77)
    lengths = rng.integers(W, T + 1, size=NH).astype(np.int32)
    lengths[:4] = [T, 300, W, 16000 + 37]
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, v = synth.random_small(2718, NH, G, W, d, T)
    p = kvc_params(pd, NH)
    p.valid_len = torch.from_numpy(lengths).cuda()
    u = torch.full((NH, T), float("nan"), dtype=torch.float32, device="cuda")
    kvc.score_window(p, dev_bf16(q), dev_bf16(k), u=u)
    u_gpu = u.cpu().numpy()
    op = oracle_params(pd)
    heads = [0, 1, 2, 3, 50]
    for n in heads:
        u_ref = ams.window_usage_ragged(widen(q[n]), widen(k[n, :T]), op, int(lengths[n]))
        assert_usage_close(u_gpu[n], u_ref, f"resident ragged head {n} (len {lengths[n]})")
    assert not np.isnan(u_gpu).any()
    check_steps2to5_ragged(pd, u_gpu, k, v, None, heads, lengths)
    print("[case] resident ragged: sampled heads ok", flush=True)


@pytest.mark.gpu
def test_wide_resident_column_sums_agree_with_streamed():
    """Windows of up to sixteen padded 32-row blocks on long caches take the
    twelve-wave LDS-resident pass 2 (one workgroup per CU walking a share of a
    head); the same heads in a small launch take the streamed kernel.  Their
    usage must have the same bits, and sampled heads match the oracle."""
    import numpy as np
    import torch
    from oracle import ams
    from parity_utils import assert_usage_close, dev_bf16, kvc_params, oracle_params, widen
    NH, G, W, d, T, K = 16, 4, 128, 64, 49152, 2000   # 16 heads x 64 chunks of 768 keys
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, _ = synth.random_small(8080, NH, G, W, d, T)
    dq, dk = dev_bf16(q), dev_bf16(k)
    print(f"[case] wide resident pass 2: NH={NH} G={G} W={W} d={d} T={T}", flush=True)
    u_all = kvc.score_window(kvc_params(pd, NH), dq, dk)
    for sub in ([0, 1], [9, 15]):
        idx = torch.tensor(sub, device="cuda")
        u_sub = kvc.score_window(kvc_params(pd, len(sub)), dq[idx].contiguous(), dk[idx].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(u_sub.view(torch.int32), u_all[idx].view(torch.int32)), sub
    u_gpu = u_all.cpu().numpy()
    op = oracle_params(pd)
    for n in (0, 15):
        assert_usage_close(u_gpu[n], ams.window_usage(widen(q[n]), widen(k[n, :T]), op),
                           f"wide resident head {n}")
    print("[case] wide resident pass 2: identical bits, sampled heads within tolerance", flush=True)


@pytest.mark.gpu
def test_split_rows_and_wide_resident_ragged():
    """A left-padded batch on the long-cache score path: 512 query rows per
    head over 49152 positions split pass 1 into 5 key ranges (merged by
    log-sum-exp) and take the twelve-wave LDS-resident pass 2.  Heads whose
    real length is shorter split into fewer ranges of their own (a head of
    1000 positions into one) and leave the rest empty (their partial
    normaliser is -inf and adds nothing); sampled heads match the oracle's
    masked usage and steps 2-5."""
    import numpy as np
    import torch
    from oracle import ams
    from parity_utils import (assert_usage_close, check_steps2to5_ragged, dev_bf16, kvc_params,
                              oracle_params, widen)
    NH, G, W, d, T, K = 16, 4, 128, 64, 49152, 2000
    rng = np.random.default_rng(4242)
    lengths = rng.integers(W, T + 1, size=NH).astype(np.int32)
    lengths[:4] = [T, 1000, W, 30000 + 17]   # 1000: one range
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, v = synth.random_small(9090, NH, G, W, d, T)
    p = kvc_params(pd, NH)
    p.valid_len = torch.from_numpy(lengths).cuda()
    print(f"[case] split pass 1 + wide pass 2, ragged: NH={NH} G={G} W={W} d={d} T={T}", flush=True)
    u = torch.full((NH, T), float("nan"), dtype=torch.float32, device="cuda")
    kvc.score_window(p, dev_bf16(q), dev_bf16(k), u=u)
    u_gpu = u.cpu().numpy()
    assert not np.isnan(u_gpu).any()
    op = oracle_params(pd)
    heads = [0, 1, 2, 3]
    for n in heads:
        u_ref = ams.window_usage_ragged(widen(q[n]), widen(k[n, :T]), op, int(lengths[n]))
        assert_usage_close(u_gpu[n], u_ref, f"split/wide ragged head {n} (len {lengths[n]})")
    check_steps2to5_ragged(pd, u_gpu, k, v, None, heads, lengths)
    print("[case] split pass 1 + wide pass 2, ragged: sampled heads ok", flush=True)


@pytest.mark.gpu
def test_whole_head_wide_pass_agrees_with_streamed():
    """With 256 heads the twelve-wave pass 2 walks a whole head per workgroup,
    after a pass 1 split into two key ranges.  The same heads launched four at
    a time take the streamed pass 2 (the same two key ranges, merged the same
    way); the usage must have the same bits, and sampled heads match the
    oracle."""
    import numpy as np
    import torch
    from oracle import ams
    from parity_utils import assert_usage_close, dev_bf16, kvc_params, oracle_params, widen
    NH, G, W, d, T, K = 256, 4, 128, 64, 12288, 1000
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, _ = synth.random_small(6060, NH, G, W, d, T)
    dq, dk = dev_bf16(q), dev_bf16(k)
    print(f"[case] whole-head wide pass: NH={NH} G={G} W={W} d={d} T={T}", flush=True)
    u_all = kvc.score_window(kvc_params(pd, NH), dq, dk)
    for sub in ([0, 1, 2, 3], [100, 200, 254, 255]):
        idx = torch.tensor(sub, device="cuda")
        u_sub = kvc.score_window(kvc_params(pd, len(sub)), dq[idx].contiguous(), dk[idx].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(u_sub.view(torch.int32), u_all[idx].view(torch.int32)), sub
    u_gpu = u_all.cpu().numpy()
    op = oracle_params(pd)
    for n in (0, 255):
        assert_usage_close(u_gpu[n], ams.window_usage(widen(q[n]), widen(k[n, :T]), op),
                           f"whole-head wide pass head {n}")
    print("[case] whole-head wide pass: identical bits, sampled heads within tolerance",
          flush=True)
