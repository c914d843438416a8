"""Oracle of the RefreshKV decode-loop pieces around the compression event.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the notes on "RefreshKV: Updating Small KV Cache During Long-form
Generation", section A2 (method details): the model keeps the full cache C_f
and a partial cache C_p of K entries.
  - Query comparison every S steps: per layer, the cosine similarity between
    the current token's query averaged over the layer's query heads and the
    averaged query of the layer's most recent full-attention step; below the
    threshold s the layer decodes with C_f (a full step), otherwise with C_p.
  - Partial step: the new token's KV enters C_p and, to keep |C_p| = K, the
    entry with the lowest attention score from the last full step leaves.
  - Full step: the KV of the tokens decoded with C_p is first written into
    C_f; then attention over C_f gives fresh scores and C_p is rebuilt from
    the top-K (the compression event in its one-segment mode).
Readings (the page leaves them open; the design notes list them):
  - one decision per (layer, sequence) row; the reference query of a row is
    stored as the sum over its query heads (the cosine is scale-invariant, so
    sum and mean give the same decision) and is replaced by the current sum
    whenever the row triggers;
  - the cosine of a zero vector is taken as 1 (no trigger);
  - a new token gets score +inf in C_p, so tokens decoded since the last full
    step stay until it (they are exactly what the sync writes into C_f);
  - ties in the minimum score go to the lowest slot index.
"""
from __future__ import annotations

import numpy as np


def head_sum(q: np.ndarray) -> np.ndarray:
    """Sum over the query heads of one row, fp64: q [Hq, d] -> [d]."""
    return np.sum(np.asarray(q, dtype=np.float64), axis=0)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """cos(a, b) in fp64; 1 when either vector is zero (nothing to compare)."""
    na = float(np.sqrt(np.dot(a, a)))
    nb = float(np.sqrt(np.dot(b, b)))
    if na == 0.0 or nb == 0.0:
        return 1.0
    return float(np.dot(a, b)) / (na * nb)


def qc_trigger(q: np.ndarray, q_ref: np.ndarray, s: float):
    """Query-comparison step for every row: q [rows, Hq, d] (the current
    token's queries), q_ref [rows, d] (head sums of the last full step).
    Returns (full [rows] bool, cos [rows], new q_ref)."""
    rows = q.shape[0]
    full = np.zeros(rows, dtype=bool)
    cos = np.zeros(rows, dtype=np.float64)
    ref = np.array(q_ref, dtype=np.float64, copy=True)
    for i in range(rows):
        cur = head_sum(q[i])
        cos[i] = cosine(cur, ref[i])
        full[i] = cos[i] < s
        if full[i]:
            ref[i] = cur
    return full, cos, ref


def partial_init(kept: np.ndarray, score: np.ndarray):
    """C_p bookkeeping after a refresh: slot j holds position kept[j] with the
    full step's score of that position (empty slots: -1, +inf)."""
    pos = np.array(kept, dtype=np.int64)
    sc = np.full(pos.shape, np.inf, dtype=np.float32)
    ok = pos >= 0
    sc[ok] = np.asarray(score, dtype=np.float32)[pos[ok]]
    return sc, pos


def partial_append(part_score, part_pos, k_part, v_part, k_new, v_new, t_new: int):
    """One partial step for one head: the lowest-scored slot (first one on
    ties) takes the new token; its score becomes +inf.  Returns the slot."""
    slot = int(np.argmin(part_score))          # argmin returns the first minimum
    k_part[slot] = k_new
    v_part[slot] = v_new
    part_score[slot] = np.inf
    part_pos[slot] = t_new
    return slot


def full_sync(part_pos, k_part, v_part, k_full, v_full, t_from: int):
    """Full step, first half: every C_p entry decoded since the last full step
    (position >= t_from) is written into C_f at its position."""
    for slot, t in enumerate(np.asarray(part_pos)):
        if t >= t_from:
            k_full[t] = k_part[slot]
            v_full[t] = v_part[slot]
