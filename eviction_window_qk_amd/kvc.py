"""Thin Python binding over libkvc (include/kvc.h): argument marshalling only.

Every step of the event runs in the HIP library; this module checks tensor
dtypes, devices, shapes and contiguity, passes raw device pointers and the
current HIP stream, and turns status codes into exceptions.  PyTorch is used
for device memory and streams only.  There is no fallback: if the library is
missing or fails to load, every call raises.

Tensor conventions (see include/kvc.h for the full layouts):
  bf16 data     torch.bfloat16 (or torch.uint16 / torch.int16 bit views)
  u64 credit    torch.int64 holding the unsigned bit pattern
  i32 indices   torch.int32
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

OK, NOOP = 0, 1
ESCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20   # KVC_NOALLOC_SCRATCH_BYTES
POOL_AVG, POOL_MAX = 0, 1
AGG_SUM, AGG_MAX = 0, 1
QUOTA_MASS, QUOTA_UNIFORM = 0, 1


class KvcError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status}: {strerror(status)}")


class _CParams(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32), ("group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("T", ctypes.c_int32), ("t_stride", ctypes.c_int32), ("window", ctypes.c_int32),
        ("budget", ctypes.c_int32), ("seg_min", ctypes.c_int32), ("seg_max", ctypes.c_int32),
        ("q_min", ctypes.c_int32), ("sinks", ctypes.c_int32), ("recent", ctypes.c_int32),
        ("pool_kernel", ctypes.c_int32), ("pool_mode", ctypes.c_int32),
        ("head_agg", ctypes.c_int32), ("ema", ctypes.c_int32), ("n_prev", ctypes.c_int32),
        ("scale", ctypes.c_float), ("delta", ctypes.c_double), ("lambda_", ctypes.c_double),
        ("beta", ctypes.c_double), ("eps", ctypes.c_double),
        ("seg_fixed", ctypes.c_int32), ("quota_mode", ctypes.c_int32),
        ("valid_len", ctypes.c_void_p),
    ]


@dataclass
class Params:
    """Mirror of kvc_params (names follow the pages' quantities)."""
    n_heads: int
    T: int
    window: int
    budget: int
    group: int = 1
    head_dim: int = 128
    t_stride: int = 0          # 0 => T
    delta: float = 0.1
    seg_min: int = 16
    seg_max: int = 256
    q_min: int = 1
    sinks: int = 4
    recent: int = 64
    pool_kernel: int = 7
    pool_mode: int = POOL_AVG
    head_agg: int = AGG_SUM
    ema: bool = False
    lam: float = 0.9
    beta: float = 0.9
    eps: float = 1e-6
    n_prev: int = 0
    scale: float = 0.0
    seg_fixed: int = 0         # ablation: > 0 => fixed-length raw segments
    quota_mode: int = QUOTA_MASS
    valid_len: object = None   # None or int32 device tensor [n_heads] (left padding)

    @classmethod
    def from_dict(cls, d: dict, **over) -> "Params":
        names = {f.name for f in fields(cls)}
        kw = {k: v for k, v in {**d, **over}.items() if k in names}
        return cls(**kw)

    def to_c(self) -> _CParams:
        c = _CParams()
        for f in fields(self):
            v = getattr(self, f.name)
            if f.name == "lam":
                c.lambda_ = float(v)
            elif f.name == "t_stride":
                c.t_stride = int(v) if v else int(self.T)
            elif f.name == "ema":
                c.ema = 1 if v else 0
            elif f.name == "valid_len":
                c.valid_len = None if v is None else _ptr(v, (torch.int32,), (self.n_heads,),
                                                          "valid_len")
            elif f.name in ("delta", "beta", "eps", "scale"):
                setattr(c, f.name, float(v))
            else:
                setattr(c, f.name, int(v))
        return c

    @property
    def stride(self) -> int:
        return self.t_stride or self.T


# The kvc_params layout and entry-point signatures this binding marshals
# (KVC_ABI_VERSION in include/kvc.h); a library of another version is refused.
ABI_VERSION = 3

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkvc.so not found at {LIB_PATH}: build it with "
                           "`python -m eviction_window_qk_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_CParams)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "kvc_score_window": [P, vp, vp, vp, vp, sz, vp],
        "kvc_mass_segment": [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "kvc_select": [P, vp, vp, vp, vp, vp, vp, sz, vp],
        "kvc_gather_compact": [P, vp, vp, vp, vp, vp, vp, vp, vp],
        "kvc_gather_paged": [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, vp, vp, vp, vp,
                             ctypes.c_int32, vp, ctypes.c_int32, vp, vp, vp, vp, vp],
        "kvc_compress_event": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "kvc_compress_event_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "kvc_qc_trigger": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                           ctypes.c_double, ctypes.c_int32, vp, vp, vp],
        "kvc_partial_init": [P, vp, vp, vp, vp, vp],
        "kvc_partial_append": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp,
                               vp, vp, ctypes.c_int32, vp, vp],
        "kvc_full_sync": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp,
                          ctypes.c_int32, ctypes.c_int32, vp, vp, vp],
        "kvc_workspace_bytes": [P],
        "kvc_segment_capacity": [P],
        "kvc_check_params": [P],
        "kvc_strerror": [ctypes.c_int],
        "kvc_abi_version": [],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.kvc_workspace_bytes.restype = ctypes.c_size_t
    L.kvc_strerror.restype = ctypes.c_char_p
    if L.kvc_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.kvc_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild with `python -m eviction_window_qk_amd.build`")
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().kvc_strerror(status).decode()


def abi_version() -> int:
    return lib().kvc_abi_version()


def check_params(p: Params) -> int:
    c = p.to_c()
    return lib().kvc_check_params(ctypes.byref(c))


def workspace_bytes(p: Params) -> int:
    c = p.to_c()
    return int(lib().kvc_workspace_bytes(ctypes.byref(c)))


def segment_capacity(p: Params) -> int:
    c = p.to_c()
    rc = lib().kvc_segment_capacity(ctypes.byref(c))
    if rc < 0:
        raise KvcError(rc, "kvc_segment_capacity")
    return rc


# ---------------------------------------------------------------------------
# tensor plumbing
# ---------------------------------------------------------------------------

_BF16_LIKE = (torch.bfloat16, torch.uint16, torch.int16)


def _ptr(t, dtypes, shape, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, fn: str) -> int:
    if rc < 0:
        raise KvcError(rc, fn)
    return rc


def _device(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor):
            return t.device
    raise ValueError("no tensor argument")


def new_workspace(p: Params, device) -> torch.Tensor:
    n = workspace_bytes(p)
    if n == 0:
        raise KvcError(_check_params_rc(p), "kvc_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_params_rc(p: Params) -> int:
    rc = check_params(p)
    return rc if rc < 0 else -1


def _ws(p, ws, device):
    if ws is None:
        ws = new_workspace(p, device)
    if ws.dtype != torch.uint8 or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace: contiguous uint8 GPU tensor expected")
    return ws


def score_window(p: Params, q, k, u=None, ws=None, stream=None):
    """Step 1.  q [NH,G,W,d] bf16, k [NH,t_stride,d] bf16 -> u [NH,T] fp32."""
    dev = _device(q, k)
    if u is None:
        u = torch.empty((p.n_heads, p.T), dtype=torch.float32, device=dev)
    ws = _ws(p, ws, dev)
    c = p.to_c()
    rc = lib().kvc_score_window(
        ctypes.byref(c),
        _ptr(q, _BF16_LIKE, (p.n_heads, p.group, p.window, p.head_dim), "q_win"),
        _ptr(k, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "k"),
        _ptr(u, (torch.float32,), (p.n_heads, p.T), "u"), ws.data_ptr(), ws.numel(),
        _stream(stream))
    _check(rc, "kvc_score_window")
    return u


def mass_segment(p: Params, u, credit_in=None, ws=None, stream=None, out=None):
    """Steps 2-3.  Returns dict(score, credit_upd, seg_start, seg_quota, n_seg, status)."""
    dev = _device(u)
    S = segment_capacity(p)
    o = dict(out or {})
    o.setdefault("score", torch.empty((p.n_heads, p.T), dtype=torch.float32, device=dev))
    if p.ema:
        o.setdefault("credit_upd", torch.empty((p.n_heads, p.T), dtype=torch.int64, device=dev))
    o.setdefault("seg_start", torch.empty((p.n_heads, S), dtype=torch.int32, device=dev))
    o.setdefault("seg_quota", torch.empty((p.n_heads, S), dtype=torch.int32, device=dev))
    o.setdefault("n_seg", torch.empty((p.n_heads,), dtype=torch.int32, device=dev))
    ws = _ws(p, ws, dev)
    c = p.to_c()
    rc = lib().kvc_mass_segment(
        ctypes.byref(c), _ptr(u, (torch.float32,), (p.n_heads, p.T), "u"),
        _ptr(credit_in, (torch.int64,), (p.n_heads, p.n_prev), "credit_in"),
        _ptr(o["score"], (torch.float32,), (p.n_heads, p.T), "score"),
        _ptr(o.get("credit_upd"), (torch.int64,), (p.n_heads, p.T), "credit_upd"),
        _ptr(o["seg_start"], (torch.int32,), (p.n_heads, S), "seg_start"),
        _ptr(o["seg_quota"], (torch.int32,), (p.n_heads, S), "seg_quota"),
        _ptr(o["n_seg"], (torch.int32,), (p.n_heads,), "n_seg"), ws.data_ptr(), ws.numel(),
        _stream(stream))
    o["status"] = _check(rc, "kvc_mass_segment")
    return o


def select(p: Params, score, seg_start, seg_quota, n_seg, kept=None, ws=None, stream=None):
    """Step 4.  Returns kept [NH, budget] int32 (ascending, -1 padded)."""
    dev = _device(score)
    S = segment_capacity(p)
    if kept is None:
        kept = torch.empty((p.n_heads, p.budget), dtype=torch.int32, device=dev)
    ws = _ws(p, ws, dev)
    c = p.to_c()
    rc = lib().kvc_select(
        ctypes.byref(c), _ptr(score, (torch.float32,), (p.n_heads, p.T), "score"),
        _ptr(seg_start, (torch.int32,), (p.n_heads, S), "seg_start"),
        _ptr(seg_quota, (torch.int32,), (p.n_heads, S), "seg_quota"),
        _ptr(n_seg, (torch.int32,), (p.n_heads,), "n_seg"),
        _ptr(kept, (torch.int32,), (p.n_heads, p.budget), "kept"), ws.data_ptr(), ws.numel(),
        _stream(stream))
    _check(rc, "kvc_select")
    return kept


def gather_compact(p: Params, kept, k, v, credit_upd=None, k_out=None, v_out=None,
                   credit_out=None, stream=None):
    """Step 5.  Returns (k_out, v_out, credit_out)."""
    dev = _device(kept)
    shp = (p.n_heads, p.budget, p.head_dim)
    if k_out is None:
        k_out = torch.empty(shp, dtype=k.dtype, device=dev)
    if v_out is None:
        v_out = torch.empty(shp, dtype=v.dtype, device=dev)
    if credit_upd is not None and credit_out is None:
        credit_out = torch.empty((p.n_heads, p.budget), dtype=torch.int64, device=dev)
    c = p.to_c()
    rc = lib().kvc_gather_compact(
        ctypes.byref(c), _ptr(kept, (torch.int32,), (p.n_heads, p.budget), "kept"),
        _ptr(k, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "k"),
        _ptr(v, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "v"),
        _ptr(credit_upd, (torch.int64,), (p.n_heads, p.T), "credit_upd"),
        _ptr(k_out, _BF16_LIKE, shp, "k_out"), _ptr(v_out, _BF16_LIKE, shp, "v_out"),
        _ptr(credit_out, (torch.int64,), (p.n_heads, p.budget), "credit_out"), _stream(stream))
    _check(rc, "kvc_gather_compact")
    return k_out, v_out, credit_out


def gather_paged(p: Params, kept, k_pool, v_pool, table_in, table_out, kv_heads: int,
                 k_pool_out=None, v_pool_out=None, credit_upd=None, credit_out=None,
                 stream=None):
    """Step 5 on a paged cache: pools [n_blocks, kv_heads, block_size, d],
    tables int32 [B, blocks].  Writes the compacted rows into the blocks of
    table_out of k_pool_out / v_pool_out (default: the source pools
    themselves).  Returns (k_pool_out, v_pool_out, credit_out)."""
    dev = _device(kept)
    n_blocks, H, bs, d = k_pool.shape
    B = p.n_heads // kv_heads
    k_pool_out = k_pool if k_pool_out is None else k_pool_out
    v_pool_out = v_pool if v_pool_out is None else v_pool_out
    if credit_upd is not None and credit_out is None:
        credit_out = torch.empty((p.n_heads, p.budget), dtype=torch.int64, device=dev)
    pshape = (n_blocks, kv_heads, bs, p.head_dim)
    c = p.to_c()
    rc = lib().kvc_gather_paged(
        ctypes.byref(c), kv_heads, bs, n_blocks,
        _ptr(kept, (torch.int32,), (p.n_heads, p.budget), "kept"),
        _ptr(k_pool, _BF16_LIKE, pshape, "k_pool"), _ptr(v_pool, _BF16_LIKE, pshape, "v_pool"),
        _ptr(table_in, (torch.int32,), (B, table_in.shape[1]), "table_in"), table_in.shape[1],
        _ptr(table_out, (torch.int32,), (B, table_out.shape[1]), "table_out"),
        table_out.shape[1],
        _ptr(k_pool_out, _BF16_LIKE, pshape, "k_pool_out"),
        _ptr(v_pool_out, _BF16_LIKE, pshape, "v_pool_out"),
        _ptr(credit_upd, (torch.int64,), (p.n_heads, p.T), "credit_upd"),
        _ptr(credit_out, (torch.int64,), (p.n_heads, p.budget), "credit_out"), _stream(stream))
    _check(rc, "kvc_gather_paged")
    return k_pool_out, v_pool_out, credit_out


def compress_event(p: Params, q, k, v, credit_in=None, ws=None, out=None, want_u=False,
                   stream=None):
    """The whole event.  Returns dict(k_out, v_out, credit_out, kept, u, status)."""
    dev = _device(q, k, v)
    shp = (p.n_heads, p.budget, p.head_dim)
    o = dict(out or {})
    o.setdefault("k_out", torch.empty(shp, dtype=k.dtype, device=dev))
    o.setdefault("v_out", torch.empty(shp, dtype=v.dtype, device=dev))
    o.setdefault("kept", torch.empty((p.n_heads, p.budget), dtype=torch.int32, device=dev))
    if p.ema:
        o.setdefault("credit_out", torch.empty((p.n_heads, p.budget), dtype=torch.int64, device=dev))
    if want_u:
        o.setdefault("u", torch.empty((p.n_heads, p.T), dtype=torch.float32, device=dev))
    ws = _ws(p, ws, dev)
    c = p.to_c()
    rc = lib().kvc_compress_event(
        ctypes.byref(c),
        _ptr(q, _BF16_LIKE, (p.n_heads, p.group, p.window, p.head_dim), "q_win"),
        _ptr(k, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "k"),
        _ptr(v, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "v"),
        _ptr(credit_in, (torch.int64,), (p.n_heads, p.n_prev), "credit_in"),
        _ptr(o["k_out"], _BF16_LIKE, shp, "k_out"), _ptr(o["v_out"], _BF16_LIKE, shp, "v_out"),
        _ptr(o.get("credit_out"), (torch.int64,), (p.n_heads, p.budget), "credit_out"),
        _ptr(o["kept"], (torch.int32,), (p.n_heads, p.budget), "kept"),
        _ptr(o.get("u"), (torch.float32,), (p.n_heads, p.T), "u_out"), ws.data_ptr(),
        ws.numel(), _stream(stream))
    o["status"] = _check(rc, "kvc_compress_event")
    return o


def compress_event_noalloc(p: Params, q, k, v, credit_in=None, out=None, want_u=False,
                           stream=None):
    """The whole event through kvc_compress_event_noalloc (library-held scratch,
    no workspace).  Returns dict(k_out, v_out, credit_out, kept, u, status)."""
    dev = _device(q, k, v)
    shp = (p.n_heads, p.budget, p.head_dim)
    o = dict(out or {})
    o.setdefault("k_out", torch.empty(shp, dtype=k.dtype, device=dev))
    o.setdefault("v_out", torch.empty(shp, dtype=v.dtype, device=dev))
    o.setdefault("kept", torch.empty((p.n_heads, p.budget), dtype=torch.int32, device=dev))
    if p.ema:
        o.setdefault("credit_out", torch.empty((p.n_heads, p.budget), dtype=torch.int64, device=dev))
    if want_u:
        o.setdefault("u", torch.empty((p.n_heads, p.T), dtype=torch.float32, device=dev))
    c = p.to_c()
    rc = lib().kvc_compress_event_noalloc(
        ctypes.byref(c),
        _ptr(q, _BF16_LIKE, (p.n_heads, p.group, p.window, p.head_dim), "q_win"),
        _ptr(k, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "k"),
        _ptr(v, _BF16_LIKE, (p.n_heads, p.stride, p.head_dim), "v"),
        _ptr(credit_in, (torch.int64,), (p.n_heads, p.n_prev), "credit_in"),
        _ptr(o["k_out"], _BF16_LIKE, shp, "k_out"), _ptr(o["v_out"], _BF16_LIKE, shp, "v_out"),
        _ptr(o.get("credit_out"), (torch.int64,), (p.n_heads, p.budget), "credit_out"),
        _ptr(o["kept"], (torch.int32,), (p.n_heads, p.budget), "kept"),
        _ptr(o.get("u"), (torch.float32,), (p.n_heads, p.T), "u_out"), _stream(stream))
    o["status"] = _check(rc, "kvc_compress_event_noalloc")
    return o


# ---------------------------------------------------------------------------
# RefreshKV decode-loop pieces (include/kvc.h documents each call)
# ---------------------------------------------------------------------------

def qc_trigger(q, q_ref, threshold: float, update_ref: bool = True, want_cos: bool = False,
               stream=None):
    """Query comparison: q bf16 [rows, Hq, d], q_ref float64 [rows, d] (updated in
    place where a row fires).  Returns full (int32 [rows]) or (full, cos)."""
    rows, Hq, d = q.shape
    dev = _device(q)
    full = torch.empty((rows,), dtype=torch.int32, device=dev)
    cos = torch.empty((rows,), dtype=torch.float64, device=dev) if want_cos else None
    rc = lib().kvc_qc_trigger(rows, Hq, d, _ptr(q, _BF16_LIKE, (rows, Hq, d), "q"),
                              _ptr(q_ref, (torch.float64,), (rows, d), "q_ref"), float(threshold),
                              1 if update_ref else 0, _ptr(full, (torch.int32,), (rows,), "full"),
                              _ptr(cos, (torch.float64,), (rows,), "cos"), _stream(stream))
    _check(rc, "kvc_qc_trigger")
    return (full, cos) if want_cos else full


def partial_init(p: Params, kept, score, stream=None):
    """C_p bookkeeping after a refresh.  Returns (part_score, part_pos)."""
    dev = _device(kept)
    ps = torch.empty((p.n_heads, p.budget), dtype=torch.float32, device=dev)
    pp = torch.empty((p.n_heads, p.budget), dtype=torch.int32, device=dev)
    c = p.to_c()
    rc = lib().kvc_partial_init(ctypes.byref(c),
                                _ptr(kept, (torch.int32,), (p.n_heads, p.budget), "kept"),
                                _ptr(score, (torch.float32,), (p.n_heads, p.T), "score"),
                                ps.data_ptr(), pp.data_ptr(), _stream(stream))
    _check(rc, "kvc_partial_init")
    return ps, pp


def partial_append(part_score, part_pos, k_part, v_part, k_new, v_new, t_new: int, stream=None):
    """One partial step for every head (in place).  Returns the evicted slots."""
    NH, K, d = k_part.shape
    dev = _device(k_part)
    ev = torch.empty((NH,), dtype=torch.int32, device=dev)
    rc = lib().kvc_partial_append(
        NH, K, d, _ptr(part_score, (torch.float32,), (NH, K), "part_score"),
        _ptr(part_pos, (torch.int32,), (NH, K), "part_pos"),
        _ptr(k_part, _BF16_LIKE, (NH, K, d), "k_part"), _ptr(v_part, _BF16_LIKE, (NH, K, d), "v_part"),
        _ptr(k_new, _BF16_LIKE, (NH, d), "k_new"), _ptr(v_new, _BF16_LIKE, (NH, d), "v_new"),
        int(t_new), ev.data_ptr(), _stream(stream))
    _check(rc, "kvc_partial_append")
    return ev


def full_sync(part_pos, k_part, v_part, k_full, v_full, t_from: int, stream=None):
    """Write the C_p entries decoded since t_from into the full cache (in place)."""
    NH, K, d = k_part.shape
    TS = k_full.shape[1]
    rc = lib().kvc_full_sync(
        NH, K, d, _ptr(part_pos, (torch.int32,), (NH, K), "part_pos"),
        _ptr(k_part, _BF16_LIKE, (NH, K, d), "k_part"), _ptr(v_part, _BF16_LIKE, (NH, K, d), "v_part"),
        int(t_from), TS, _ptr(k_full, _BF16_LIKE, (NH, TS, d), "k_full"),
        _ptr(v_full, _BF16_LIKE, (NH, TS, d), "v_full"), _stream(stream))
    _check(rc, "kvc_full_sync")
