"""FP64 oracle for vocabulary-sharded logits cross-entropy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The tensor-parallel flow of the TransformerEngine PR "Minimize the memory
usage of the fused cross entropy kernel" (Changes: a multi-GPU path with two
kernels; Sequence Diagram: the forward gathers local statistics across the
tensor-parallel group and continues from the global ones).  Each shard holds
a contiguous range of vocabulary columns; the pages name the steps but not
the statistics, so this follows the plainest reading:

  local   (per shard k, per row):  m_k = max z,  d_k = sum exp(z - m_k),
          s_k = sum z,  t_k = z_t if the shard holds the target column else 0
  global  m = max_k m_k,  d = sum_k d_k exp(m_k - m),  s = sum_k s_k,
          z_t = sum_k t_k (exactly one shard holds it)
  loss    (1 - eps)(m + ln d - z_t) + eps (m + ln d - s / V), V the FULL
          vocabulary, as for the unsharded logits (the cross-entropy API page,
          I/O Contract; label smoothing spreads eps over all V classes)
  grad    on shard k's columns: g_r (exp(z - m - ln d) - q), q as unsharded.

The optional entropy H = -sum_v p_v ln p_v (the Liger-Kernel PR's tensor-
parallel forward offers it; Summary: "optional entropy") needs one more local
statistic, the un-normalised mean log-ratio in bits,
  w_k = sum_v exp(z_v - m_k) (z_v - m_k) / ln 2,
moved to the global max like d:  W = sum_k exp(m_k - m) (ln 2 w_k + d_k (m_k - m)),
  H = ln d - W / d,
since -sum p ln p = ln d - sum_v exp(z_v - m) (z_v - m) / d.  Its gradient on a
shard is the unsharded one, g_H p_v (H + ln p_v) with the global statistics.

Plain NumPy in float64, one row at a time where that reads clearest.
"""
from __future__ import annotations

import numpy as np

from . import bf16_to_f64


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def shard_partials(logits_shard: np.ndarray, targets: np.ndarray, vocab_start: int,
                   ignore_idx: int = -100) -> np.ndarray:
    """Local statistics (N, 4) = (m_k, d_k, s_k, t_k) of one shard.

    ``logits_shard`` (N, V_local) (float32, float64 or BF16 bits) holds columns
    vocab_start .. vocab_start + V_local - 1; ``targets`` (N) index the full
    vocabulary.  Ignored rows are all zeros."""
    z = _f64(logits_shard).reshape(-1, np.asarray(logits_shard).shape[-1])
    t = np.asarray(targets, np.int64).reshape(-1)
    n, vl = z.shape
    out = np.zeros((n, 4))
    for r in range(n):
        if t[r] == ignore_idx:
            continue
        row = z[r]
        m = row.max()
        out[r, 0] = m
        out[r, 1] = np.exp(row - m).sum() if np.isfinite(m) else 0.0
        out[r, 2] = row.sum()
        c = t[r] - vocab_start
        out[r, 3] = row[c] if 0 <= c < vl else 0.0
    return out


def shard_partials_w(logits_shard: np.ndarray, targets: np.ndarray,
                     ignore_idx: int = -100) -> np.ndarray:
    """Local entropy statistic (N,) w_k = sum_v exp(z - m_k)(z - m_k) / ln 2 of
    one shard (see the module docstring); 0 for ignored rows."""
    z = _f64(logits_shard).reshape(-1, np.asarray(logits_shard).shape[-1])
    t = np.asarray(targets, np.int64).reshape(-1)
    out = np.zeros(z.shape[0])
    for r in range(z.shape[0]):
        if t[r] == ignore_idx:
            continue
        row = z[r]
        m = row.max()
        if not np.isfinite(m):
            continue
        e = np.exp(row - m)
        fin = np.isfinite(row)          # exp(-inf) (-inf) contributes 0
        out[r] = float(np.sum(e[fin] * (row[fin] - m))) / np.log(2.0)
    return out


def merge_entropy(partials, partials_w, targets: np.ndarray, ignore_idx: int = -100):
    """Per-row entropy (N,) from every shard's (m_k, d_k) and w_k; 0 for
    ignored rows."""
    P = np.stack([np.asarray(p, np.float64) for p in partials])          # (K, N, 4)
    Wk = np.stack([np.asarray(w, np.float64) for w in partials_w])       # (K, N)
    t = np.asarray(targets, np.int64).reshape(-1)
    out = np.zeros(t.size)
    ln2 = np.log(2.0)
    for r in range(t.size):
        if t[r] == ignore_idx:
            continue
        mk, dk, wk = P[:, r, 0], P[:, r, 1], Wk[:, r]
        m = mk.max()
        live = dk > 0
        f = np.exp(mk[live] - m)
        d = float(np.sum(dk[live] * f))
        W = float(np.sum(f * (ln2 * wk[live] + dk[live] * (mk[live] - m))))
        out[r] = np.log(d) - W / d
    return out


def merge_shards(partials, targets: np.ndarray, V: int, label_smoothing: float = 0.0,
                 ignore_idx: int = -100):
    """Global statistics and loss from the shards' local statistics.

    ``partials``: sequence of (N, 4) arrays, one per shard (any order).
    Returns ``(loss, stats)`` with stats (N, 4) = (m, d, z_t, mean z) over the
    full vocabulary of V columns, zeros for ignored rows; NaN loss (and z_t)
    for a target neither ignored nor in [0, V)."""
    P = np.stack([np.asarray(p, np.float64) for p in partials])      # (K, N, 4)
    t = np.asarray(targets, np.int64).reshape(-1)
    eps = float(label_smoothing)
    n = t.size
    loss = np.zeros(n)
    stats = np.zeros((n, 4))
    for r in range(n):
        if t[r] == ignore_idx:
            continue
        mk, dk, sk, tk = P[:, r, 0], P[:, r, 1], P[:, r, 2], P[:, r, 3]
        m = mk.max()
        if np.isfinite(m):
            d = float(np.sum(dk * np.exp(mk - m)))
        else:
            d = 0.0
        s = float(sk.sum())
        zt = float(tk.sum()) if 0 <= t[r] < V else np.nan
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = m + np.log(d)
            loss[r] = (1.0 - eps) * (lse - zt)
            if eps != 0.0:  # classes with q = 0 add no term (a -inf logit would give 0 * inf)
                loss[r] += eps * (lse - s / V)
        stats[r] = (m, d, zt, s / V)
    return loss, stats


def shard_backward(logits_shard: np.ndarray, targets: np.ndarray, vocab_start: int, V: int,
                   stats: np.ndarray, g: np.ndarray, label_smoothing: float = 0.0,
                   ignore_idx: int = -100) -> np.ndarray:
    """Gradient (N, V_local) of shard k's columns from the global statistics:
    g_r (exp(z - m - ln d) - q), q = (1 - eps)[v = t] + eps / V over the full
    vocabulary; ignored rows 0, out-of-range targets NaN."""
    z = _f64(logits_shard).reshape(-1, np.asarray(logits_shard).shape[-1])
    t = np.asarray(targets, np.int64).reshape(-1)
    gg = np.asarray(g, np.float64).reshape(-1)
    st = np.asarray(stats, np.float64).reshape(-1, 4)
    eps = float(label_smoothing)
    n, vl = z.shape
    cols = vocab_start + np.arange(vl)
    out = np.zeros((n, vl))
    for r in range(n):
        if t[r] == ignore_idx:
            continue
        if not (0 <= t[r] < V):
            out[r] = np.nan
            continue
        lse = st[r, 0] + np.log(st[r, 1])
        q = eps / V + (1.0 - eps) * (cols == t[r])
        out[r] = gg[r] * (np.exp(z[r] - lse) - q)
    return out


# --- vocabulary-sharded linear cross-entropy ----------------------------------
#
# The tensor-parallel form of the Liger-Kernel fused linear cross-entropy PR
# (Summary): the classifier W is split by vocabulary rows, shard k holding
# W_k = W[a_k:b_k].  Its logits are Z_k = X W_k^T, the columns a_k..b_k of
# Z = X W^T, so the forward is the logits flow above on Z_k; the backward
# gives dW_k = dZ_k^T X (rows a_k..b_k of dW) and dX_k = dZ_k W_k, whose sum
# over the shards is dX = dZ W.

def _dec_bf16(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def linear_shard_partials(X_bits: np.ndarray, W_shard_bits: np.ndarray, targets: np.ndarray,
                          vocab_start: int, ignore_idx: int = -100,
                          scale: float = 1.0) -> np.ndarray:
    """Local statistics (M, 4) of Z_k = s X W_k^T (see ``shard_partials``;
    s = ``scale``, the logit scale of the scaled form, 1 for the plain one)."""
    Zk = scale * (_dec_bf16(X_bits) @ _dec_bf16(W_shard_bits).T)
    return shard_partials(Zk, targets, vocab_start, ignore_idx)


def linear_shard_backward(X_bits: np.ndarray, W_shard_bits: np.ndarray, targets: np.ndarray,
                          vocab_start: int, V: int, stats: np.ndarray, g: np.ndarray,
                          label_smoothing: float = 0.0, ignore_idx: int = -100,
                          scale: float = 1.0):
    """(dX_k, dW_k) of one shard from the global statistics: dZ_k from
    ``shard_backward`` on Z_k = s X W_k^T, the gradient with respect to X W_k^T
    s dZ_k, then dX_k = s dZ_k W_k and dW_k = s dZ_k^T X."""
    X = _dec_bf16(X_bits)
    Wk = _dec_bf16(W_shard_bits)
    dZk = shard_backward(scale * (X @ Wk.T), targets, vocab_start, V, stats, g,
                         label_smoothing, ignore_idx)
    dZk = scale * dZk
    return dZk @ Wk, dZk.T @ X
