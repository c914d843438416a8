"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/kvc.h declares, and its host-side validation (pure host code that
returns before anything is launched) behaves as documented."""
import ctypes
import subprocess
import os
import re
import sys

import pytest

from eviction_window_qk_amd import kvc
from eviction_window_qk_amd import build as kbuild
from oracle import ams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH),
                                reason="libkvc.so not built (python -m eviction_window_qk_amd.build)")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**\s*(kvc_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for fn in ["kvc_score_window", "kvc_mass_segment", "kvc_select", "kvc_gather_compact",
               "kvc_compress_event"]:
        assert fn in names


def test_every_declared_symbol_is_exported():
    exported = kbuild.exported_symbols(kvc.LIB_PATH)
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    L = kvc.lib()
    for n in _declared():
        assert hasattr(L, n)


def test_abi_version_and_strerror():
    assert kvc.abi_version() == kvc.ABI_VERSION == 3
    for code in (0, 1, -1, -2, -3, -4, -5, -6):
        assert kvc.strerror(code) and kvc.strerror(code) != "unknown status"
    assert kvc.strerror(-99) == "unknown status"


def test_noalloc_rejects_events_past_its_scratch():
    # Host-side checks of kvc_compress_event_noalloc return before any device
    # call: invalid parameters, and events needing more than the library's
    # scratch (the 128K-token event needs ~0.8 GB).
    src = open(HEADER).read()
    m = re.search(r"#define\s+KVC_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kvc.NOALLOC_SCRATCH_BYTES
    L = kvc.lib()
    big = _p(n_heads=256, T=131072, window=128, budget=4096, group=4, ema=True).to_c()
    assert kvc.workspace_bytes(_p(n_heads=256, T=131072, window=128, budget=4096, group=4,
                                  ema=True)) > kvc.NOALLOC_SCRATCH_BYTES
    args = [None] * 10
    assert L.kvc_compress_event_noalloc(ctypes.byref(big), *args) == kvc.ESCRATCH
    bad = _p(window=0).to_c()
    assert L.kvc_compress_event_noalloc(ctypes.byref(bad), *args) == -1
    assert kvc.workspace_bytes(_p(n_heads=1792)) <= kvc.NOALLOC_SCRATCH_BYTES


def test_header_version_matches_binding():
    src = open(HEADER).read()
    m = re.search(r"#define\s+KVC_ABI_VERSION\s+(\d+)", src)
    assert m and int(m.group(1)) == kvc.ABI_VERSION


def test_graft_entry_import_check():
    sys.path.insert(0, ROOT)
    import __graft_entry__
    __graft_entry__.check_import()


def test_param_struct_layout(tmp_path):
    assert ctypes.sizeof(kvc._CParams) == 120
    assert kvc._CParams.delta.offset == 72
    assert kvc._CParams.valid_len.offset == 112
    # The binding's field offsets equal the C compiler's for include/kvc.h.
    names = [f for f, _ in kvc._CParams._fields_]
    src = tmp_path / "layout.c"
    body = "".join(
        f'  printf("%s %zu\\n", "{f}", offsetof(kvc_params, {f.rstrip("_")}));\n' for f in names)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kvc.h"\nint main(void) {\n'
                   + body + '  printf("sizeof %zu\\n", sizeof(kvc_params));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(__file__), "..", "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(kvc._CParams)
    for f in names:
        assert int(got[f]) == getattr(kvc._CParams, f).offset, f


def _p(**kw):
    base = dict(n_heads=4, T=768, window=128, budget=256, group=7, head_dim=128)
    base.update(kw)
    return kvc.Params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -4), (dict(group=65), -4), (dict(group=0), -1),
    (dict(T=0), -1), (dict(T=(1 << 18) + 1), -1), (dict(t_stride=100), -1),
    (dict(window=0), -1), (dict(window=769), -1), (dict(budget=0), -1),
    (dict(delta=0.0), -1), (dict(delta=-1.0), -1), (dict(delta=float("nan")), -1),
    (dict(delta=1e-4), -1),                  # > 1024 thresholds
    (dict(seg_min=0), -1), (dict(seg_max=-1), -1), (dict(q_min=-1), -1),
    (dict(sinks=-1), -1), (dict(recent=-1), -1), (dict(pool_kernel=6), -1),
    (dict(pool_kernel=65), -1), (dict(pool_mode=2), -1), (dict(head_agg=3), -1),
    (dict(lam=1.5), -1), (dict(beta=-0.1), -1), (dict(eps=0.0), -1), (dict(eps=2.0), -1),
    (dict(n_prev=5), -1),                    # credit without EMA
    (dict(ema=True, n_prev=769), -1), (dict(scale=-1.0), -1), (dict(scale=1e-20), -1),
    (dict(scale=float("inf")), -1),
    (dict(seg_fixed=-1), -1), (dict(T=4096, seg_fixed=2), -1),  # > 1025 fixed segments
    (dict(quota_mode=2), -1),
    (dict(window=128, group=64), -1),        # W*G > 4096
    (dict(T=2048, window=512, group=8), -1), # W*G = 4096 but 2*W*W*G >= 2^22
    # max pooling multiplies the usage sum by its width: 63*128*128*8 >= 2^22
    (dict(T=2048, window=128, group=8, pool_mode=1, pool_kernel=63), -1),
    (dict(n_heads=-1), -1),
])
def test_invalid_params(kw, code):
    p = _p(**kw)
    assert kvc.check_params(p) == code
    assert kvc.workspace_bytes(p) == 0


def test_usage_bound_depends_on_the_pooling():
    # the same shape passes with average pooling (2*W*W*G < 2^22) and with
    # max pooling of width 7, but not of width 63
    assert kvc.check_params(_p(T=2048, window=128, group=8)) == 0
    assert kvc.check_params(_p(T=2048, window=128, group=8, pool_mode=1, pool_kernel=7)) == 0
    assert kvc.check_params(_p(T=2048, window=128, group=8, pool_mode=1, pool_kernel=63)) == -1


def test_valid_params_for_every_workload():
    from eviction_window_qk_amd import synth
    for name in synth.ORDER:
        wl = synth.WORKLOADS[name]
        p = kvc.Params.from_dict(wl.event_params(), n_heads=wl.n_heads,
                                 n_prev=wl.budget if wl.params.get("ema") else 0)
        assert kvc.check_params(p) == 0, name
        assert kvc.workspace_bytes(p) > 0


def test_segment_capacity_matches_oracle_bound():
    for kw in [dict(), dict(seg_max=0), dict(delta=0.25), dict(delta=1.0, seg_max=0),
               dict(seg_fixed=64), dict(seg_fixed=7, seg_max=0), dict(seg_fixed=1000),
               dict(T=131072, window=128, group=4, budget=4096), dict(T=20, window=4, budget=5,
                                                                    seg_max=2, delta=0.05)]:
        p = _p(**kw)
        o = ams.Params(T=p.T, window=p.window, budget=p.budget, delta=p.delta, seg_min=p.seg_min,
                       seg_max=p.seg_max, seg_fixed=p.seg_fixed)
        assert kvc.segment_capacity(p) == ams.segment_capacity(o)
    assert kvc.segment_capacity(_p(T=131072, window=128, group=4, budget=4096)) == 522


def test_workspace_grows_with_heads():
    assert kvc.workspace_bytes(_p(n_heads=8)) > kvc.workspace_bytes(_p(n_heads=4)) > 0


# --- pointer validation: returns before any launch ---------------------------

FAKE = 1 << 40          # aligned, never dereferenced


def _call_score(p, q=FAKE, k=FAKE + (1 << 32), u=FAKE + (2 << 32), ws=FAKE + (3 << 32), wsb=None):
    c = p.to_c()
    if wsb is None:
        wsb = kvc.workspace_bytes(p)
    return kvc.lib().kvc_score_window(ctypes.byref(c), q, k, u, ws, wsb, None)


def test_null_pointers_rejected():
    p = _p()
    assert _call_score(p, q=None) == -1
    assert _call_score(p, u=None) == -1


def test_misaligned_rejected():
    assert _call_score(_p(), q=FAKE + 2) == -2


def test_small_workspace_rejected():
    p = _p()
    assert _call_score(p, wsb=kvc.workspace_bytes(p) - 1) == -3
    assert _call_score(p, ws=None) == -3


def test_aliasing_rejected():
    assert _call_score(_p(), u=FAKE + 64) == -1          # u overlaps q


def test_zero_heads_is_a_noop_without_pointers():
    p = _p(n_heads=0)
    c = p.to_c()
    assert kvc.lib().kvc_score_window(ctypes.byref(c), None, None, None, None, 0, None) == 0
    assert kvc.lib().kvc_compress_event(ctypes.byref(c), None, None, None, None, None, None, None,
                                        None, None, None, 0, None) == 0


def test_gather_credit_pointers_both_or_neither():
    p = _p()
    c = p.to_c()
    L = kvc.lib()
    a = FAKE
    rc = L.kvc_gather_compact(ctypes.byref(c), a, a + (1 << 32), a + (2 << 32), a + (3 << 32),
                              a + (4 << 32), a + (5 << 32), None, None)
    assert rc == -1


def test_event_rejects_missing_credit_when_ema():
    p = _p(ema=True, n_prev=256)
    c = p.to_c()
    a = FAKE
    L = kvc.lib()
    ws = kvc.workspace_bytes(p)
    # credit_in NULL with n_prev > 0
    rc = L.kvc_compress_event(ctypes.byref(c), a, a + (1 << 32), a + (2 << 32), None,
                              a + (4 << 32), a + (5 << 32), a + (6 << 32), a + (7 << 32), None,
                              a + (8 << 32), ws, None)
    assert rc == -1


def test_binding_rejects_cpu_tensors():
    import torch
    p = _p(n_heads=1)
    q = torch.zeros((1, 7, 128, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 768, 128), dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        kvc.score_window(p, q, k, u=torch.zeros((1, 768)), ws=torch.zeros(8, dtype=torch.uint8))


def _call_paged(p, kv_heads=4, bs=16, n_blocks=4096, tin_blocks=48, tout_blocks=16,
                k_out=FAKE + (5 << 32), v_out=FAKE + (6 << 32)):
    c = p.to_c()
    a = FAKE
    return kvc.lib().kvc_gather_paged(ctypes.byref(c), kv_heads, bs, n_blocks, a,
                                      a + (1 << 32), a + (2 << 32), a + (3 << 32), tin_blocks,
                                      a + (4 << 32), tout_blocks, k_out, v_out, None, None, None)


def test_gather_paged_validation():
    p = _p(n_heads=8, T=768, budget=256)          # 2 sequences x 4 KV heads
    assert _call_paged(p, kv_heads=3) == -1        # n_heads not a multiple of kv_heads
    assert _call_paged(p, tin_blocks=47) == -1     # 47 * 16 < T
    assert _call_paged(p, tout_blocks=15) == -1    # 15 * 16 < budget
    assert _call_paged(p, bs=0) == -1
    assert _call_paged(p, n_blocks=0) == -1
    assert _call_paged(p, k_out=FAKE + (4 << 32)) == -1       # output pool overlaps table_out
    assert _call_paged(p, v_out=FAKE + (5 << 32) + 64) == -1  # the two output pools overlap
    assert _call_paged(p, k_out=FAKE + (5 << 32) + 8) == -2   # misaligned


def test_refresh_pieces_validation():
    L = kvc.lib()
    a = FAKE
    assert L.kvc_qc_trigger(4, 8, 96, a, a + (1 << 32), 0.5, 1, a + (2 << 32), None, None) == -1
    assert L.kvc_qc_trigger(4, 8, 128, a, a + (1 << 32), float("nan"), 1, a + (2 << 32), None,
                            None) == -1
    assert L.kvc_qc_trigger(4, 8, 128, a, a + 8, 0.5, 1, a + (2 << 32), None, None) == -1  # alias
    assert L.kvc_qc_trigger(0, 8, 128, None, None, 0.5, 1, None, None, None) == 0
    assert L.kvc_partial_append(4, 0, 128, a, a, a, a, a, a, 7, a, None) == -1
    assert L.kvc_partial_append(4, 16, 128, a, a + (1 << 32), a + (2 << 32) + 4, a + (3 << 32),
                                a + (4 << 32), a + (5 << 32), 7, a + (6 << 32), None) == -2
    assert L.kvc_full_sync(4, 16, 128, a, a + (1 << 32), a + (2 << 32), -1, 100, a + (3 << 32),
                           a + (4 << 32), None) == -1
