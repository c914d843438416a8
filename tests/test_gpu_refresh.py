"""GPU parity of the RefreshKV decode-loop pieces against the oracle: the
query-comparison trigger (fp64 cosine), the partial-cache append/evict over
a run of decode steps, and the full-cache sync.  Inputs are seeded synthetic
(the kept lists and scores of the last refresh are generated, not taken from
the GPU)."""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import refresh
from parity_utils import dev_bf16, host_bits, widen

pytestmark = pytest.mark.gpu


def test_qc_trigger_matches_oracle():
    rows, Hq, d, s = 448, 28, 128, 0.6
    rng = np.random.default_rng(11)
    q = synth.f32_to_bf16_bits(rng.standard_normal((rows, Hq, d), dtype=np.float32))
    qf = widen(q)
    ref = rng.standard_normal((rows, d))
    ref[::7] = np.stack([refresh.head_sum(qf[i]) for i in range(0, rows, 7)])
    ref[1::7] = -np.stack([refresh.head_sum(qf[i]) for i in range(1, rows, 7)])
    ref[2::7] = 0.0
    # rows 3::7 close to the current query (cos near 1), 4::7 a mix (cos ~ 0.6)
    for i in range(3, rows, 7):
        ref[i] = refresh.head_sum(qf[i]) + 0.1 * rng.standard_normal(d)
    for i in range(4, rows, 7):
        cur = refresh.head_sum(qf[i])
        ref[i] = cur + 1.3 * np.linalg.norm(cur) / np.sqrt(d) * rng.standard_normal(d)
    full_o, cos_o, ref_o = refresh.qc_trigger(qf, ref, s)
    dref = torch.from_numpy(ref.copy()).cuda()
    full_g, cos_g = kvc.qc_trigger(dev_bf16(q), dref, s, update_ref=True, want_cos=True)
    torch.cuda.synchronize()
    cos_g = cos_g.cpu().numpy()
    np.testing.assert_allclose(cos_g, cos_o, rtol=0, atol=1e-12)
    clear = np.abs(cos_o - s) > 1e-9          # decisions away from the threshold are unique
    assert clear.sum() > rows - 2
    np.testing.assert_array_equal(full_g.cpu().numpy()[clear].astype(bool), full_o[clear])
    np.testing.assert_array_equal(dref.cpu().numpy()[clear], ref_o[clear])
    assert full_o.any() and (~full_o).any()


def _random_loops(n):
    """Seeded random decode loops: head count, cache budget (one slot up),
    cache length, steps (more steps than slots included, so every slot turns
    over), head dim, empty slots on one head and the spacing of tied scores."""
    rng = np.random.default_rng(909)
    out = []
    for i in range(n):
        K = int(rng.integers(1, 300))
        out.append((f"random{i}", int(rng.integers(1, 40)), K, int(rng.integers(K, 2000)),
                    int(rng.integers(1, 2 * K + 20)), int(rng.choice([64, 128])),
                    int(rng.integers(0, K + 1)), int(rng.choice([1, 3, 50]))))
    return out


LOOPS = [("d128", 24, 64, 700, 40, 128, 5, 50), ("d64", 24, 64, 700, 40, 64, 5, 50)] + _random_loops(60)


@pytest.mark.parametrize("case", LOOPS, ids=[c[0] for c in LOOPS])
def test_partial_loop_and_sync_match_oracle(case):
    label, NH, K, T0, steps, d, n_empty, tie_step = case
    print(f"[case] refresh loop {label}: NH={NH} K={K} T0={T0} steps={steps} d={d}", flush=True)
    rng = np.random.default_rng(sum(map(ord, label)) + d)
    kf = synth.f32_to_bf16_bits(rng.standard_normal((NH, T0 + steps, d), dtype=np.float32))
    vf = synth.f32_to_bf16_bits(rng.standard_normal((NH, T0 + steps, d), dtype=np.float32))
    kept = np.stack([np.sort(rng.choice(T0, K, replace=False)) for _ in range(NH)]).astype(np.int32)
    if n_empty:
        kept[NH // 2, K - n_empty:] = -1                    # a short head: empty slots
    score = rng.random((NH, T0)).astype(np.float32)
    score[:, ::tie_step] = 0.25                             # ties
    new_k = synth.f32_to_bf16_bits(rng.standard_normal((steps, NH, d), dtype=np.float32))
    new_v = synth.f32_to_bf16_bits(rng.standard_normal((steps, NH, d), dtype=np.float32))
    # oracle
    ps_o, pp_o, kp_o, vp_o, ev_o = [], [], [], [], []
    for n in range(NH):
        sc, pos = refresh.partial_init(kept[n], score[n])
        kp = np.where(kept[n][:, None] >= 0, kf[n][np.maximum(kept[n], 0)], 0).astype(np.uint16)
        vp = np.where(kept[n][:, None] >= 0, vf[n][np.maximum(kept[n], 0)], 0).astype(np.uint16)
        evs = [refresh.partial_append(sc, pos, kp, vp, new_k[i, n], new_v[i, n], T0 + i)
               for i in range(steps)]
        ps_o.append(sc), pp_o.append(pos), kp_o.append(kp), vp_o.append(vp), ev_o.append(evs)
    kf_o = kf.copy()
    vf_o = vf.copy()
    for n in range(NH):
        refresh.full_sync(pp_o[n], kp_o[n], vp_o[n], kf_o[n], vf_o[n], T0)
    # GPU
    p = kvc.Params(n_heads=NH, T=T0, window=1, budget=K, head_dim=d)
    dps, dpp = kvc.partial_init(p, torch.from_numpy(kept).cuda(), torch.from_numpy(score).cuda())
    kp0 = np.where(kept[:, :, None] >= 0, np.take_along_axis(kf, np.maximum(kept, 0)[:, :, None], 1), 0)
    vp0 = np.where(kept[:, :, None] >= 0, np.take_along_axis(vf, np.maximum(kept, 0)[:, :, None], 1), 0)
    dkp, dvp = dev_bf16(kp0.astype(np.uint16)), dev_bf16(vp0.astype(np.uint16))
    evs_g = []
    for i in range(steps):
        evs_g.append(kvc.partial_append(dps, dpp, dkp, dvp, dev_bf16(new_k[i]), dev_bf16(new_v[i]),
                                        T0 + i))
    dkf, dvf = dev_bf16(kf), dev_bf16(vf)
    kvc.full_sync(dpp, dkp, dvp, dkf, dvf, T0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.stack([e.cpu().numpy() for e in evs_g], 1), np.array(ev_o))
    np.testing.assert_array_equal(dps.cpu().numpy(), np.stack(ps_o))
    np.testing.assert_array_equal(dpp.cpu().numpy(), np.stack(pp_o))
    np.testing.assert_array_equal(host_bits(dkp), np.stack(kp_o))
    np.testing.assert_array_equal(host_bits(dvp), np.stack(vp_o))
    np.testing.assert_array_equal(host_bits(dkf), kf_o)
    np.testing.assert_array_equal(host_bits(dvf), vf_o)
