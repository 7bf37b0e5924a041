"""Log-sum-exp merge of partial attention states -- oracle side.
TEST INFRASTRUCTURE ONLY.

"Beyond just running: native inference optimisation in vLLM on AMD ROCm",
section "Processing details of the three paths": each context chunk of an
extend produces an output and an LSE; the LSE carries the chunk's softmax
denominator (in log space), which makes the merge numerically stable, and a
chunk with higher attention scores naturally dominates the merged result.

For two states (o1, lse1), (o2, lse2) over disjoint key sets:
  lse = ln(e^lse1 + e^lse2),  o = e^(lse1 - lse) o1 + e^(lse2 - lse) o2.
A state with lse = -inf (no keys) has weight zero.
"""
from __future__ import annotations

import numpy as np


def merge(o1, lse1, o2, lse2):
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    lse = np.logaddexp(lse1, lse2)
    both_empty = ~np.isfinite(lse)
    ref = np.where(both_empty, 0.0, lse)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - ref), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - ref), 0.0)
    o = w1[..., None] * o1 + w2[..., None] * o2
    o = np.where(both_empty[..., None], 0.0, o)
    return o, lse


def merge_all(states):
    """Fold merge() over a list of (o, lse) states, left to right."""
    o, lse = states[0]
    for o2, lse2 in states[1:]:
        o, lse = merge(o, lse, o2, lse2)
    return o, lse
