"""Capacity-limited dispatch in plain Python/numpy (test infrastructure only).

Sources (titles and sections of the pages these follow):
  [P4] MoE-survey blog page ("six MoE papers"), section 3 (GShard): an expert
       capacity bounds the tokens one expert takes; the gate keeps a running
       counter c_e per expert; a token whose chosen experts are already full
       overflows, its gate vector becomes zero and its representation reaches
       the next layer through the residual connection; local group
       dispatching splits the batch into G groups of S tokens, each with its
       own share of every expert's capacity.  Section 4 (Switch): expert
       capacity = tokens per batch / number of experts x capacity factor.

Readings taken where the pages leave a step open:
  * The capacity C counts (token, expert) assignments per expert and per
    group.  The counter runs over a group's tokens in ascending order; a
    token's K' chosen experts are distinct, so their order inside the token
    does not matter.
  * An assignment that finds its expert full is dropped: the gate of that
    expert becomes 0 for that token, the token's other assignments stand and
    are not renormalised.  A token with every assignment dropped is the
    page's overflowed token: no routed contribution, only the shared experts
    and, when added, the residual.
  * Groups are consecutive runs of S tokens, the last one possibly shorter;
    S = 0 (or S >= T) is one group of the whole batch.
  * capacity_for: C = ceil(factor * S * K' / N'), the Switch formula with the
    batch counted in assignments; for K' = 2 and factor 1 it is GShard's
    2N/(G E) per group.
"""
from __future__ import annotations

import math

import numpy as np


def group_length(T: int, group_size: int) -> int:
    return group_size if 0 < group_size < T else max(T, 1)


def capacity_for(T: int, n_routed: int, top_k: int, factor: float, group_size: int = 0) -> int:
    """Slots per expert per group: ceil(factor * S * K' / N')."""
    S = group_length(T, group_size)
    return max(1, math.ceil(factor * S * top_k / n_routed))


def keep_mask(idx: np.ndarray, n_routed: int, capacity: int, group_size: int = 0) -> np.ndarray:
    """True where assignment (t, j) keeps its slot: [P4] section 3's running
    counter, reset at the start of every group."""
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    S = group_length(T, group_size)
    for g0 in range(0, T, S):
        c = [0] * n_routed
        for t in range(g0, min(g0 + S, T)):
            for j in range(k):
                e = int(idx[t, j])
                if c[e] < capacity:
                    c[e] += 1
                    keep[t, j] = True
    return keep


def dispatch_capacity(idx: np.ndarray, n_routed: int, capacity: int, group_size: int = 0):
    """Per-expert lists of the kept assignments, tokens ascending within an
    expert.  Returns counts [N'] (kept), offsets [N'+1], row_token [kept
    rows], slot_row [T*K'] (row of slot t*K'+j, or -1 when dropped) and the
    keep mask."""
    T, k = idx.shape
    keep = keep_mask(idx, n_routed, capacity, group_size)
    flat = idx.reshape(-1).astype(np.int64)
    kept_slots = np.nonzero(keep.reshape(-1))[0]
    counts = np.bincount(flat[kept_slots], minlength=n_routed).astype(np.int32)
    offsets = np.zeros(n_routed + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = kept_slots[np.argsort(flat[kept_slots], kind="stable")]
    row_token = (order // k).astype(np.int32)
    slot_row = np.full(T * k, -1, dtype=np.int32)
    slot_row[order] = np.arange(order.size, dtype=np.int32)
    return counts, offsets, row_token, slot_row, keep
