"""A head's results do not depend on the launch it is in (GPU, through the C ABI).

The kernels pick their launch shape from the whole launch (how many heads,
the padded cache length): how many key ranges the row statistics are split
into, which column-sum kernel runs, the thread count of the mass and select
kernels.  None of these choices may change a head's bits.  Each head of a
left-padded batch is run again alone, as a cache of exactly its real length,
and its usage, kept indices (shifted by the padding), compacted K/V must be
identical bit for bit.
"""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from parity_utils import dev_bf16, kvc_params
from test_gpu_parity import _pd

pytestmark = pytest.mark.gpu

CASES = [
    # (label, NH, G, W, d, T, K, lengths of the checked heads (the rest random), checked heads)
    # six heads, streamed column sums; lengths around the 11008-key range boundary
    ("mixed_lengths", 6, 4, 128, 64, 40000, 2000, [40000, 30000, 11008, 11009, 25000, 128], None),
    # 64 heads: the batch takes the twelve-wave column sums, each head alone the streamed ones
    ("wide_batch", 64, 4, 128, 64, 40000, 3000, [40000, 23456, 11009, 5000], [0, 1, 2, 3]),
]


def _event(pd, NH, q, k, v, lengths=None):
    p = kvc_params(pd, NH)
    if lengths is not None:
        p.valid_len = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    ev = kvc.compress_event(p, dev_bf16(q), dev_bf16(k), dev_bf16(v), want_u=True)
    torch.cuda.synchronize()
    return {key: ev[key].cpu() for key in ("u", "kept", "k_out", "v_out")}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_head_alone_equals_head_in_batch(case):
    label, NH, G, W, d, T, K, fixed, heads = case
    rng = np.random.default_rng(sum(map(ord, label)))
    lengths = rng.integers(W, T + 1, size=NH).astype(np.int32)
    lengths[:len(fixed)] = fixed
    heads = range(NH) if heads is None else heads
    pd = _pd(group=G, window=W, head_dim=d, T=T, budget=K)
    q, k, v = synth.random_small(sum(map(ord, label)) + 7, NH, G, W, d, T)
    print(f"[case] batch invariance {label}: NH={NH} G={G} W={W} d={d} T={T} K={K}", flush=True)
    batch = _event(pd, NH, q, k, v, lengths)
    for n in heads:
        L = int(lengths[n])
        off = T - L
        alone = _event(dict(pd, T=L), 1, q[n:n + 1], k[n:n + 1, off:], v[n:n + 1, off:])
        tag = f"{label} head {n} (length {L})"
        assert torch.equal(batch["u"][n, off:].view(torch.int32), alone["u"][0].view(torch.int32)), tag
        kb, ka = batch["kept"][n], alone["kept"][0]
        assert torch.equal(kb, torch.where(ka >= 0, ka + off, ka)), tag
        assert torch.equal(batch["k_out"][n].view(torch.int16), alone["k_out"][0].view(torch.int16)), tag
        assert torch.equal(batch["v_out"][n].view(torch.int16), alone["v_out"][0].view(torch.int16)), tag
        print(f"[case] {tag}: identical", flush=True)
