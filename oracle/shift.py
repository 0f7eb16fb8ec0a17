"""Causal label shift (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The cut-cross-entropy package description (what_it_does) offers optional
token shifting for causal language modelling: the prediction at position s
of a sequence is scored against the label at position s + 1, so the last
position has no label.  Here that position gets the ignore index, which the
loss treats as an ignored row (loss 0, not counted in the mean, gradient 0).
Written as plain loops over the (d0, d1) grid.
"""
from __future__ import annotations

import numpy as np


def shift_targets(targets: np.ndarray, seq_axis: int, ignore_idx: int = -100) -> np.ndarray:
    """(d0, d1) int64 targets, sequence along ``seq_axis`` (0 or 1) -> shifted copy."""
    t = np.asarray(targets, np.int64)
    d0, d1 = t.shape
    out = np.empty_like(t)
    for i0 in range(d0):
        for i1 in range(d1):
            n0, n1 = (i0 + 1, i1) if seq_axis == 0 else (i0, i1 + 1)
            if n0 < d0 and n1 < d1:
                out[i0, i1] = t[n0, n1]
            else:
                out[i0, i1] = ignore_idx
    return out
