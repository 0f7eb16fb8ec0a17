"""Pure-Python (``math`` only) cross-entropy for tiny cases.

TEST INFRASTRUCTURE ONLY (see the package docstring).  A third, independent
statement of the same definitions as the C core, written with Python floats
and explicit loops so the two can be compared on tiny inputs:

    p_v = exp(z_v) / sum_u exp(z_u)          (computed with the max shifted out)
    q_v = (1 - eps) [v = t] + eps / V
    loss = - sum_v q_v log p_v,   grad_v = g (p_v - q_v)

Follows the TransformerEngine cross-entropy API page (I/O Contract) and the
gradient-from-statistics PR (Changes).
"""
from __future__ import annotations

import math


def softmax(z):
    m = max(z)
    e = [math.exp(x - m) for x in z]
    s = sum(e)
    return [x / s for x in e]


def loss_row(z, t, eps=0.0, ignore_idx=-100):
    if t == ignore_idx:
        return 0.0
    V = len(z)
    p = softmax(z)
    total = 0.0
    for v in range(V):
        q = eps / V + ((1.0 - eps) if v == t else 0.0)
        if q != 0.0:
            total -= q * math.log(p[v])
    return total


def grad_row(z, t, g=1.0, eps=0.0, ignore_idx=-100):
    V = len(z)
    if t == ignore_idx:
        return [0.0] * V
    p = softmax(z)
    return [g * (p[v] - (eps / V + ((1.0 - eps) if v == t else 0.0))) for v in range(V)]


def matmul_nt(X, W):
    """Z[r][v] = sum_h X[r][h] W[v][h]."""
    return [[sum(a * b for a, b in zip(xr, wr)) for wr in W] for xr in X]
