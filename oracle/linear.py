"""FP64 oracle for fused linear cross-entropy (logits = X W^T never formed on GPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes follows the cut-cross-entropy package description (the
loss of ``linear_cross_entropy(embeddings, classifier, labels)``: the target
logit and the log-sum-exp over the whole vocabulary of X W^T) and the
Liger-Kernel fused linear cross-entropy PR (Summary: classifier GEMM fused
with NLL/LSE; Backward and Performance methodology: dZ from recomputed
logits, then dX = dZ W and dW = dZ^T X):

    Z  = X W^T                    (FP64 product of the exact BF16 or FP32 values)
    loss, stats = logits cross-entropy of Z   (the C core of this package)
    dZ = g_r (softmax(Z_r) - q_r)             (the C core of this package)
         [+ gH_r dH/dZ_r when an entropy gradient is given]
    dX = dZ W,   dW = dZ^T X                  (FP64 matrix products)

The scaled form (``scale`` s, the reading of the Liger-Kernel PR title's
"scaled" linear cross-entropy as a logit scale) is the same with Z = s X W^T;
by the chain rule its gradients are dX = s dZ W and dW = s dZ^T X, with dZ
the gradient with respect to the scaled logits.

Rows (tokens) are independent, so large problems are processed in token
chunks purely to bound host memory; dW is then the sum over chunks of
dZ_c^T X_c, which is the same sum over tokens split into consecutive ranges.
"""
from __future__ import annotations

import numpy as np

from . import add_entropy_grad, bf16_to_f64, ce_backward, ce_forward, entropy as _entropy


def _rows(a: np.ndarray, rows):
    return a if rows is None else a[np.asarray(rows, dtype=np.int64)]


def _dec(a: np.ndarray) -> np.ndarray:
    """The exact value of every input: BF16 bit patterns (uint16) and FP32
    values are widened exactly to float64 (the cross-entropy API page,
    Description: BF16 or FP32 input); float64 passes through."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.float64:
        return a
    raise TypeError(f"X and W must be BF16 bits (uint16), float32 or float64, got {a.dtype}")


def logits(X_bits: np.ndarray, W_bits: np.ndarray, rows=None) -> np.ndarray:
    """Z = X W^T in FP64 for the selected token rows."""
    X = _dec(_rows(X_bits, rows))
    W = _dec(W_bits)
    return X @ W.T


def forward(X_bits, W_bits, targets, label_smoothing=0.0, ignore_idx=-100, rows=None,
            token_chunk: int | None = None, scale: float = 1.0):
    """Per-token loss, stats (max, denominator, z_target, mean z) and lse.

    Returns ``(loss, stats, lse)`` for the selected rows (all by default)."""
    t_all = np.asarray(targets, np.int64).reshape(-1)
    idx = np.arange(t_all.size) if rows is None else np.asarray(rows, np.int64)
    W = _dec(W_bits)
    chunk = token_chunk or max(1, idx.size)
    loss = np.empty(idx.size)
    stats = np.empty((idx.size, 4))
    for s in range(0, idx.size, chunk):
        sel = idx[s:s + chunk]
        Z = scale * (_dec(X_bits[sel]) @ W.T)
        l, st, _ = ce_forward(Z, t_all[sel], label_smoothing, ignore_idx)
        loss[s:s + chunk] = l
        stats[s:s + chunk] = st
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = stats[:, 0] + np.log(stats[:, 1])
    return loss, stats, lse


def entropy(X_bits, W_bits, targets, ignore_idx=-100, token_chunk: int | None = None,
            scale: float = 1.0):
    """Per-token entropy of softmax(scale X W^T) in FP64 (0 for ignored tokens)."""
    t_all = np.asarray(targets, np.int64).reshape(-1)
    W = _dec(W_bits)
    M = t_all.size
    chunk = token_chunk or max(1, M)
    out = np.empty(M)
    for s in range(0, M, chunk):
        Z = scale * (_dec(X_bits[s:s + chunk]) @ W.T)
        out[s:s + chunk] = _entropy(Z, t_all[s:s + chunk], ignore_idx)
    return out


def backward(X_bits, W_bits, targets, g, label_smoothing=0.0, ignore_idx=-100,
             token_chunk: int | None = None, grad_entropy=None, scale: float = 1.0):
    """Full dX (M, H) and dW (V, H) in FP64.  ``g`` is g_r for every token;
    ``grad_entropy`` (per token, optional) adds the entropy's gradient;
    ``scale``: the logits are scale X W^T."""
    t_all = np.asarray(targets, np.int64).reshape(-1)
    g_all = np.asarray(g, np.float64).reshape(-1)
    M = t_all.size
    W = _dec(W_bits)
    dX = np.empty((M, W.shape[1]))
    dW = np.zeros(W.shape)
    chunk = token_chunk or M
    for s in range(0, M, chunk):
        Xc = _dec(X_bits[s:s + chunk])
        Z = scale * (Xc @ W.T)
        dZ = ce_backward(Z, t_all[s:s + chunk], g_all[s:s + chunk], label_smoothing, ignore_idx)
        if grad_entropy is not None:
            gh = np.asarray(grad_entropy, np.float64).reshape(-1)[s:s + chunk]
            add_entropy_grad(dZ, Z, t_all[s:s + chunk], gh, ignore_idx)
        dZ = scale * dZ  # the gradient with respect to X W^T
        dX[s:s + chunk] = dZ @ W
        dW += dZ.T @ Xc
    return dX, dW


def dx_rows(X_bits, W_bits, targets, g, rows, label_smoothing=0.0, ignore_idx=-100):
    """dX for selected token rows only: dZ_r W, with dZ_r from the full row of Z."""
    rows = np.asarray(rows, np.int64)
    t_all = np.asarray(targets, np.int64).reshape(-1)
    g_all = np.asarray(g, np.float64).reshape(-1)
    W = _dec(W_bits)
    Z = _dec(X_bits[rows]) @ W.T
    dZ = ce_backward(Z, t_all[rows], g_all[rows], label_smoothing, ignore_idx)
    return dZ @ W


def dw_rows(X_bits, W_bits, targets, g, lse, vrows, label_smoothing=0.0, ignore_idx=-100):
    """dW for selected vocabulary rows: sum over tokens r of dZ[r, v] X[r].

    ``lse`` is the FP64 log-sum-exp of every token (from ``forward``).  The
    gradient entry is written out from its definition,
    dZ[r, v] = g_r (exp(Z[r, v] - lse_r) - q_rv), q_rv = (1-eps)[v = t_r] + eps/V,
    and is zero for ignored tokens."""
    vrows = np.asarray(vrows, np.int64)
    t = np.asarray(targets, np.int64).reshape(-1)
    gg = np.asarray(g, np.float64).reshape(-1)
    X = _dec(X_bits)
    Wsel = _dec(W_bits[vrows])
    V = W_bits.shape[0]
    Zc = X @ Wsel.T                                       # (M, |vrows|)
    p = np.exp(Zc - np.asarray(lse, np.float64)[:, None])
    q = label_smoothing / V + (1.0 - label_smoothing) * (t[:, None] == vrows[None, :])
    dZ = gg[:, None] * (p - q)
    dZ[t == ignore_idx] = 0.0
    return dZ.T @ X
