"""Seeded synthetic inputs for the KV-compression event.

This module is the only thing the HIP path and the CPU oracle have in common:
it draws the inputs both consume.  It holds none of the method's arithmetic
(no scores, masses, cuts, quotas or selections) -- only random draws, the
bf16 rounding of inputs and the workload table.

Every head-event n = (layer l, batch b, KV head h) draws from its own stream
``PCG64(SeedSequence([seed, l, b, h]))`` in the fixed order Z_K [T,d],
Z_V [T,d], Z_Q [G,W,d], then the structure draws, so any head can be
regenerated alone (the oracle checks sampled heads of the full-size runs).

Workloads (shapes from the pages' models and schedule; value distributions
are synthetic choices, see the design notes):
  tiny            1 head, G=1, d=64, T=1024, W=32, budget 128, N(0,1)
  qwen7b_t768     Qwen-7B-shaped decode event, 28 layers x B16 x 4 KV heads,
                  G=7, d=128, T=768, W=128, budget 256, key norms LogNormal(0,.5)
  qwen7b_t1536_ema  same shape, B64, T=1536, budget 1024, EMA credit carried
                  from a prior event, ~1% keys x8 (single-position spikes)
  llama8b_global_t16k  Llama-8B-shaped prefill-time global select (one
                  segment), 32 x B4 x 8, G=4, T=16384, W=32, max-pool 7, top 2048
  llama8b_t128k   Llama-8B shape, B1, T=131072, W=128, budget 4096, EMA on,
                  smooth low-frequency key drift plus dense bursts
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Event parameter sets.  Keys mirror the library's parameter record.
_AMS_DEFAULT = dict(delta=0.1, seg_min=16, seg_max=256, q_min=1, sinks=4, recent=64,
                    pool_kernel=7, pool_mode=0, head_agg=0, ema=False, lam=0.9,
                    beta=0.9, eps=1e-6, n_prev=0, scale=0.0)
_ONE_SEGMENT = dict(_AMS_DEFAULT, delta=1.0, seg_min=1, seg_max=0, sinks=0, recent=0,
                    pool_mode=1)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    layers: int
    batch: int
    kv_heads: int
    group: int
    head_dim: int
    T: int
    window: int
    budget: int
    keys: str                     # key value structure, see _keys()
    params: dict = field(default_factory=dict)
    prior_seed: int = 0           # seed of the prior event that seeds the credit

    @property
    def n_heads(self) -> int:
        return self.layers * self.batch * self.kv_heads

    def head_coords(self, n: int):
        """n = (l * batch + b) * kv_heads + h."""
        h = n % self.kv_heads
        lb = n // self.kv_heads
        return lb // self.batch, lb % self.batch, h

    def event_params(self, **over) -> dict:
        d = dict(self.params)
        d.update(T=self.T, window=self.window, budget=self.budget, group=self.group,
                 head_dim=self.head_dim)
        d.update(over)
        return d


WORKLOADS = {
    "tiny": Workload("tiny", 101, 1, 1, 1, 1, 64, 1024, 32, 128, "normal",
                     dict(_AMS_DEFAULT)),
    "qwen7b_t768": Workload("qwen7b_t768", 202, 28, 16, 4, 7, 128, 768, 128, 256,
                            "lognormal", dict(_AMS_DEFAULT)),
    "qwen7b_t1536_ema": Workload("qwen7b_t1536_ema", 303, 28, 64, 4, 7, 128, 1536, 128,
                                 1024, "outliers", dict(_AMS_DEFAULT, ema=True),
                                 prior_seed=3030),
    "llama8b_global_t16k": Workload("llama8b_global_t16k", 404, 32, 4, 8, 4, 128, 16384,
                                    32, 2048, "normal", dict(_ONE_SEGMENT)),
    "llama8b_t128k": Workload("llama8b_t128k", 505, 32, 1, 8, 4, 128, 131072, 128, 4096,
                              "drift_bursts", dict(_AMS_DEFAULT, ema=True)),
}
ORDER = ["tiny", "qwen7b_t768", "qwen7b_t1536_ema", "llama8b_global_t16k", "llama8b_t128k"]


# ---------------------------------------------------------------------------
# bf16 as raw bits (NumPy has no bfloat16)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.
    Inputs are finite by construction."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# per-head draws
# ---------------------------------------------------------------------------

def _rng(seed: int, l: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, l, b, h])))


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _keys(wl: Workload, rng, zk: np.ndarray, zq: np.ndarray, T: int, sinks: int):
    """Key (and, for the drift workload, query) structure draws."""
    d = wl.head_dim
    if wl.keys == "normal":
        return zk, zq
    if wl.keys in ("lognormal", "outliers"):
        r = rng.lognormal(0.0, 0.5, size=T).astype(np.float32)
        k = zk * r[:, None]
        if wl.keys == "outliers":
            spike = rng.random(T) < 0.01
            k = np.where(spike[:, None], k * np.float32(8.0), k)
        return k, zq
    if wl.keys == "drift_bursts":
        a = 0.5 * math.sqrt(d)
        a_d = 0.25 * math.sqrt(d)
        e = _unit(rng, (d,))
        vs = _unit(rng, (4, d))
        periods = rng.uniform(T / 16, T / 2, size=4)
        phases = rng.uniform(0.0, 2.0 * math.pi, size=4)
        lengths = rng.integers(200, 801, size=26)
        free = (T - wl.window - sinks) - int(lengths.sum())
        offs = np.sort(rng.integers(0, max(free, 0) + 1, size=26))
        starts = sinks + offs + np.concatenate([[0], np.cumsum(lengths)[:-1]])
        t = np.arange(T, dtype=np.float64)
        drift = np.zeros((T, d), dtype=np.float64)
        for j in range(4):
            drift += np.sin(2.0 * math.pi * t / periods[j] + phases[j])[:, None] * vs[j][None, :]
        burst = np.zeros(T, dtype=bool)
        for s0, ln in zip(starts, lengths):
            burst[s0:s0 + ln] = True
        k = zk + (a_d * drift + a * burst[:, None] * e[None, :]).astype(np.float32)
        q = zq + np.float32(a) * e.astype(np.float32)
        return k, q
    raise ValueError(wl.keys)


def gen_head(wl: Workload, n: int, T: int | None = None, seed: int | None = None,
             with_q: bool = True, with_v: bool = True):
    """Inputs of head-event n as bf16 bits: q [G,W,d], k [T,d], v [T,d]."""
    T = wl.T if T is None else T
    l, b, h = wl.head_coords(n)
    rng = _rng(wl.seed if seed is None else seed, l, b, h)
    d = wl.head_dim
    zk = rng.standard_normal((T, d), dtype=np.float32)
    zv = rng.standard_normal((T, d), dtype=np.float32)
    zq = rng.standard_normal((wl.group, wl.window, d), dtype=np.float32)
    k, q = _keys(wl, rng, zk, zq, T, wl.params.get("sinks", 4))
    out = {"k": f32_to_bf16_bits(k)}
    if with_v:
        out["v"] = f32_to_bf16_bits(zv)
    if with_q:
        out["q"] = f32_to_bf16_bits(q)
    return out


def gen_heads(wl: Workload, heads, T: int | None = None, seed: int | None = None,
              t_stride: int | None = None):
    """Stacked inputs for a list of heads: q [n,G,W,d], k/v [n,t_stride,d] (bits).
    Rows T..t_stride-1 of k/v are zero."""
    heads = list(heads)
    T = wl.T if T is None else T
    ts = T if t_stride is None else t_stride
    G, W, d = wl.group, wl.window, wl.head_dim
    q = np.empty((len(heads), G, W, d), dtype=np.uint16)
    k = np.zeros((len(heads), ts, d), dtype=np.uint16)
    v = np.zeros((len(heads), ts, d), dtype=np.uint16)
    for i, n in enumerate(heads):
        hd = gen_head(wl, n, T=T, seed=seed)
        q[i], k[i, :T], v[i, :T] = hd["q"], hd["k"], hd["v"]
    return q, k, v


def fresh_rows(wl: Workload, n: int, rows: int, seed: int):
    """`rows` new K/V rows for head n (the tokens generated since the last
    event), drawn with the same key structure as the workload."""
    hd = gen_head(wl, n, T=rows, seed=seed, with_q=False)
    return hd["k"], hd["v"]


def random_small(seed: int, n_heads: int, G: int, W: int, d: int, T: int,
                 key_scale: float = 1.0, t_stride: int | None = None):
    """Small random inputs for parity sweeps: N(0,1) queries, N(0, key_scale^2)
    keys, N(0,1) values, as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, n_heads, G, W, d, T])))
    ts = T if t_stride is None else t_stride
    q = f32_to_bf16_bits(rng.standard_normal((n_heads, G, W, d), dtype=np.float32))
    k = np.zeros((n_heads, ts, d), dtype=np.uint16)
    v = np.zeros((n_heads, ts, d), dtype=np.uint16)
    k[:, :T] = f32_to_bf16_bits(rng.standard_normal((n_heads, T, d), dtype=np.float32)
                                * np.float32(key_scale))
    v[:, :T] = f32_to_bf16_bits(rng.standard_normal((n_heads, T, d), dtype=np.float32))
    return q, k, v


def batch_valid_lengths(wl: Workload, max_pad: int, seed: int, heads=None) -> np.ndarray:
    """Valid lengths of a left-padded batch: batch element b gets a pad count
    drawn uniformly from 0..max_pad, shared by all its layers and KV heads
    (the prompts of one batch differ in length, every layer sees the same
    padding).  Returns int32 [len(heads)] (all heads by default)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.batch, max_pad])))
    pads = rng.integers(0, max_pad + 1, size=wl.batch)
    heads = range(wl.n_heads) if heads is None else heads
    return np.array([wl.T - pads[wl.head_coords(n)[1]] for n in heads], dtype=np.int32)
