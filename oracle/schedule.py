"""Oracle: the deterministic dispatch/combine schedule. TEST INFRASTRUCTURE ONLY.

What it computes follows [R] "Mixture-of-Kittens: a deterministic MoE
megakernel for NVL72 racks":
  * §"The two API layers and the schedule object": routing decisions are
    materialised once, before any expert math, and the same schedule object is
    passed to forward and backward; it is sized for the worst case by the
    capacity multiplier.
  * §"Tuning the five hyperparameters before production": the capacity
    multiplier is the worst-case fraction of tokens sent to one destination
    (1.0 = all of them), and expert padding makes the true worst case slightly
    larger than 1.0.
  * §"How MoK differs from a general MoE kernel library": the materialised
    plan is deterministic and replayable.

Readings taken where the pages are silent:
  * With every expert on one GPU, the "destination" is an expert: the
    per-expert capacity is C = min(T, ceil(mult * T)) assignments, with
    mult the float32 value in the config evaluated in float64.
  * Assignments beyond an expert's capacity are dropped deterministically:
    the first C in flat order a = t*k + j are kept.
  * Inside an expert's segment rows are in ascending flat order a (token
    order); duplicate ids within a token are separate assignments.
  * Expert ids outside [0, E) are invalid: counted, never dispatched.
  * Each expert segment is padded up to a multiple of P rows (P = 32 by
    default); padding rows have source -1.
  * Minibatch sub-offsets: rows of expert e whose token lies in minibatch b
    are [mb_offsets[b, e], mb_offsets[b+1, e]).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["capacity", "rows_cap", "build_schedule"]


def capacity(T: int, capacity_multiplier: float) -> int:
    """Per-expert capacity C = min(T, ceil(mult * T)); mult is rounded to
    float32 first (the config field's type) and the product is taken in
    float64."""
    m = float(np.float32(capacity_multiplier))
    return int(min(T, math.ceil(m * T)))


def rows_cap(T: int, k: int, E: int, capacity_multiplier: float, expert_pad: int) -> int:
    """Upper bound on the padded expert-contiguous rows:
    sum_e ceil(kept_e / P) * P <= min(T*k, E*C) + E*(P-1)."""
    C = capacity(T, capacity_multiplier)
    return min(T * k, E * C) + E * (expert_pad - 1)


def build_schedule(top_experts: np.ndarray, num_experts: int, capacity_multiplier: float = 1.0,
                   expert_pad: int = 32, minibatch_size: int = 0) -> dict:
    """Build the schedule from top-k expert ids ``int64 [T, k]``.

    Returns a dict of int64 numpy arrays / ints:
      C, rows_cap, counts[E] (valid assignments per expert), kept[E],
      padded[E], offsets[E+1] (exclusive prefix sum of padded),
      row_src[rows_cap] (flat assignment index a = t*k + j of each row, -1 for
      padding and unused rows), slot_row[T*k] (row of each assignment, -1 if
      dropped or invalid), rank[T*k] (position among the expert's valid
      assignments in flat order, -1 if invalid), mb_offsets[n_mb+1, E],
      dropped, invalid, n_mb, minibatch_size.

    Pin: tests/test_oracle_schedule.py checks it against a pure-Python
    dict-of-lists brute force using Python's stable ``sorted`` on random tiny
    cases, against a hand-worked example (tests/golden/schedule_small.txt) and
    against invariants (sum of counts = T*k - invalid, kept + dropped, the
    inverse-map property, sorted segments, no drops at mult 1.0).
    """
    top = np.asarray(top_experts, dtype=np.int64)
    T, k = top.shape
    E, P = int(num_experts), int(expert_pad)
    C = capacity(T, capacity_multiplier)
    Rc = rows_cap(T, k, E, capacity_multiplier, P)

    e = top.reshape(-1)                      # expert of flat assignment a = t*k + j
    a_all = np.arange(T * k, dtype=np.int64)
    valid = (e >= 0) & (e < E)
    invalid = int((~valid).sum())

    # Counts per expert, then each valid assignment's rank among its expert's
    # assignments in flat order: a stable sort by expert keeps flat order
    # inside each expert's group.
    counts = np.bincount(e[valid], minlength=E).astype(np.int64)
    group_start = np.concatenate([[0], np.cumsum(counts)])
    order = np.argsort(np.where(valid, e, E), kind="stable")[: int(valid.sum())]
    rank = np.full(T * k, -1, dtype=np.int64)
    rank[order] = np.arange(order.size, dtype=np.int64) - group_start[e[order]]

    keep = valid & (rank < C)
    dropped = int(valid.sum() - keep.sum())
    kept = np.minimum(counts, C)
    padded = ((kept + P - 1) // P) * P
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    assert offsets[-1] <= Rc

    row_src = np.full(Rc, -1, dtype=np.int64)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    rows = offsets[e[keep]] + rank[keep]
    row_src[rows] = a_all[keep]
    slot_row[keep] = rows

    mb = T if minibatch_size <= 0 else int(minibatch_size)
    n_mb = max(1, -(-T // mb)) if T > 0 else 1
    mb_offsets = np.zeros((n_mb + 1, E), dtype=np.int64)
    tok_of_row = np.where(row_src >= 0, row_src // max(k, 1), -1)
    for b in range(n_mb + 1):
        bound = min(b * mb, T)
        for ex in range(E):
            seg = tok_of_row[offsets[ex]: offsets[ex] + kept[ex]]
            mb_offsets[b, ex] = offsets[ex] + int((seg < bound).sum())

    return dict(T=T, k=k, E=E, P=P, C=C, rows_cap=Rc, counts=counts, kept=kept, padded=padded,
                offsets=offsets, row_src=row_src, slot_row=slot_row, rank=rank,
                mb_offsets=mb_offsets, dropped=dropped, invalid=invalid,
                n_mb=n_mb, minibatch_size=mb)
