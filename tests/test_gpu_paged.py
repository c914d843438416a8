"""GPU parity of the paged-KV compaction (kvc_gather_paged) against the
oracle: every block of the pools, bit for bit, after the copy into new
blocks; plus the event's kept indices driving it at the Qwen-7B shape."""
import numpy as np
import pytest
import torch

from eviction_window_qk_amd import kvc, synth
from oracle import ams
from parity_utils import host_u64

pytestmark = pytest.mark.gpu


def _case(seed, B, H, T, bs, d, K, spare=5, same_pool=True, bad_ids=False, empty=False):
    rng = np.random.default_rng(seed)
    nb_in, nb_out = -(-T // bs), -(-K // bs)
    n_blocks = B * (nb_in + nb_out) + spare
    perm = rng.permutation(n_blocks).astype(np.int32)
    tin = perm[:B * nb_in].reshape(B, nb_in)
    tout = perm[B * nb_in:B * (nb_in + nb_out)].reshape(B, nb_out).copy()
    k_pool = rng.integers(0, 1 << 16, (n_blocks, H, bs, d), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, (n_blocks, H, bs, d), dtype=np.uint16)
    kept = np.stack([np.sort(rng.choice(T, K, replace=False)) for _ in range(B * H)]).astype(np.int32)
    if empty:
        kept[1, -7:] = -1
    if bad_ids:
        tout[0, -1] = -1            # skipped destination
        tout[-1, 0] = n_blocks + 3  # out of range: skipped
    return k_pool, v_pool, tin, tout, kept


def _bits(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


CASES = [
    # (label, B, H, T, bs, d, K, kwargs)
    ("d128_bs16", 5, 4, 300, 16, 128, 100, {}),
    ("d64_bs8_separate", 3, 2, 129, 8, 64, 40, dict(same_pool=False)),
    ("odd_block", 2, 8, 500, 7, 128, 77, dict(empty=True)),
    ("bad_ids", 3, 4, 200, 16, 128, 64, dict(bad_ids=True)),
]


def _random_cases(n):
    """Seeded random layouts: batch size, KV heads, cache length, block size
    (odd sizes and single-slot blocks included), head dim, budget, separate
    output pools, empty kept slots and skipped destination blocks."""
    rng = np.random.default_rng(2024)
    out = []
    for i in range(n):
        T = int(rng.integers(2, 1200))
        kw = dict(same_pool=bool(rng.random() < 0.5), empty=bool(rng.random() < 0.3))
        B = int(rng.integers(2, 6))
        if kw["empty"] or rng.random() < 0.3:
            kw["bad_ids"] = bool(rng.random() < 0.5)
        out.append((f"random{i}", B, int(rng.choice([1, 2, 4, 8])), T,
                    int(rng.choice([1, 2, 3, 7, 8, 16, 32, 64])), int(rng.choice([64, 128])),
                    int(rng.integers(8, T + 1)) if T >= 8 else T, kw))
    return out


CASES += _random_cases(200)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gather_paged_matches_oracle(case):
    label, B, H, T, bs, d, K, kw = case
    print(f"[case] paged {label}", flush=True)
    same = kw.pop("same_pool", True)
    k_pool, v_pool, tin, tout, kept = _case(sum(map(ord, label)), B, H, T, bs, d, K, **kw)
    # -1 destinations are not in the oracle's layout: give it the surviving slots only
    p = kvc.Params(n_heads=B * H, T=T, window=1, budget=K, head_dim=d)
    dk, dv = _bits(k_pool), _bits(v_pool)
    ko = dk if same else torch.zeros_like(dk)
    vo = dv if same else torch.zeros_like(dv)
    base_k = k_pool if same else np.zeros_like(k_pool)
    base_v = v_pool if same else np.zeros_like(v_pool)
    kvc.gather_paged(p, torch.from_numpy(kept).cuda(), dk, dv, torch.from_numpy(tin).cuda(),
                     torch.from_numpy(tout).cuda(), H, k_pool_out=ko, v_pool_out=vo)
    torch.cuda.synchronize()
    n_blocks = k_pool.shape[0]
    ok_rows = np.ones_like(kept, dtype=bool)
    tout_ok = tout.copy()
    # Rows with a skipped destination go to a spare block that neither table
    # names, so the oracle's copy of them cannot land on a real destination.
    spare = min(set(range(n_blocks)) - set(tin.ravel().tolist()) - set(tout.ravel().tolist()))
    for b in range(B):
        for j in range(K):
            blk = tout[b, j // bs]
            if blk < 0 or blk >= n_blocks:
                ok_rows[b * H:(b + 1) * H, j] = False
                tout_ok[b, j // bs] = spare
    want_k, want_v = base_k.copy(), base_v.copy()
    ref_k, ref_v = ams.gather_paged(kept, k_pool, v_pool, tin, tout_ok, H)
    for n in range(B * H):
        b, h = divmod(n, H)
        for j in range(K):
            if ok_rows[n, j]:
                blk, s = tout_ok[b, j // bs], j % bs
                want_k[blk, h, s] = ref_k[blk, h, s]
                want_v[blk, h, s] = ref_v[blk, h, s]
    np.testing.assert_array_equal(_host(ko), want_k)
    np.testing.assert_array_equal(_host(vo), want_v)


def test_gather_paged_credit_and_event_kept():
    """Kept indices from a real event at the Qwen-7B head shape drive the paged
    copy; credit follows them as in the contiguous gather."""
    wl = synth.WORKLOADS["qwen7b_t768"]
    heads = list(range(8))                       # 2 sequences x 4 KV heads
    q, k, v = synth.gen_heads(wl, heads)
    pd = wl.event_params(ema=True)
    p = kvc.Params.from_dict(pd, n_heads=8)
    dq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    dkc = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
    dvc = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
    ev = kvc.compress_event(p, dq, dkc, dvc, None)
    ws = kvc.new_workspace(p, dq.device)
    u = kvc.score_window(p, dq, dkc, ws=ws)
    ms = kvc.mass_segment(p, u, None, ws=ws)
    kept = ev["kept"]
    # paged copy of the same cache: 16-token blocks, shuffled
    H, bs, T, K, d = 4, 16, wl.T, wl.budget, wl.head_dim
    rng = np.random.default_rng(0)
    nb_in, nb_out = T // bs, K // bs
    n_blocks = 2 * (nb_in + nb_out)
    perm = rng.permutation(n_blocks).astype(np.int32)
    tin, tout = perm[:2 * nb_in].reshape(2, nb_in), perm[2 * nb_in:].reshape(2, nb_out)
    kp = np.zeros((n_blocks, H, bs, d), np.uint16)
    vp = np.zeros_like(kp)
    for n in range(8):
        b, h = divmod(n, H)
        for t in range(T):
            kp[tin[b, t // bs], h, t % bs] = k[n, t]
            vp[tin[b, t // bs], h, t % bs] = v[n, t]
    dkp, dvp = _bits(kp), _bits(vp)
    _, _, co = kvc.gather_paged(p, kept, dkp, dvp, torch.from_numpy(tin).cuda(),
                                torch.from_numpy(tout).cuda(), H, credit_upd=ms["credit_upd"])
    torch.cuda.synchronize()
    kh, vh = _host(dkp), _host(dvp)
    ko, vo = _host(ev["k_out"]), _host(ev["v_out"])
    for n in range(8):
        b, h = divmod(n, H)
        np.testing.assert_array_equal(ams.read_paged(kh, tout, b, h, K), ko[n])
        np.testing.assert_array_equal(ams.read_paged(vh, tout, b, h, K), vo[n])
    np.testing.assert_array_equal(host_u64(co), host_u64(ev["credit_out"]))
