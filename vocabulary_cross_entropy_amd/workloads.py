"""Seeded synthetic inputs for the fused cross-entropy workloads.

This module only draws random numbers and packs them into the storage formats
the kernels read (FP32, or BF16 bit patterns rounded to nearest-even).  It holds
none of the loss arithmetic, so both the HIP path and the FP64 oracle can take
their inputs from it without sharing any of the method.

Recipe (same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64); draws are made in this order:
    logits (or X), then W, then targets, then the ignored-row mask.
  * Normal values are drawn in FP32 and, for BF16 storage, rounded to the
    nearest BF16 with ties to even.
  * "p% ignored" means exactly ``round(p * N)`` rows, chosen without
    replacement, whose target is set to ``IGNORE_INDEX``.
  * Zipf targets follow the finite law P(k) proportional to k**-s over
    k = 1..V (token id k-1), sampled by inverse CDF.

The five named workloads reproduce the shapes and value distributions of the
fused cross-entropy problem: the TransformerEngine cross-entropy API page
(I/O Contract: logits (B,SQ,V) or (SQ,B,V), targets, label smoothing, mean
reduction, ignore index -100), the TransformerEngine PR that saves statistics
instead of the derivative (validation comment: 4096 x 128256 BF16 logits), and
the Liger-Kernel fused linear cross-entropy PR (Performance methodology:
M=4096, H=4096, V=131072, BF16 inputs).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

IGNORE_INDEX = -100

DTYPE_FP32 = "fp32"
DTYPE_BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (nearest, ties to even); return uint16 bit patterns.

    Large arrays go through torch's multithreaded CPU cast (also nearest-even;
    the two agree bit for bit, which the CPU tests check)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size >= (1 << 22):
        try:
            import torch
            return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        except ImportError:
            pass
    return f32_to_bf16_bits_np(x)


def f32_to_bf16_bits_np(x: np.ndarray) -> np.ndarray:
    """NumPy statement of FP32 -> BF16 round to nearest even (bit patterns)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to FP32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _ignore_rows(rng: np.random.Generator, n: int, frac: float | None, count: int | None) -> np.ndarray:
    k = count if count is not None else int(round((frac or 0.0) * n))
    k = max(0, min(n, k))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(n, size=k, replace=False).astype(np.int64))


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Token ids in [0, V) with P(id = k-1) proportional to k**-s, by inverse CDF."""
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, V - 1).astype(np.int64)


@dataclass
class LogitsCase:
    """A logits cross-entropy problem as stored in memory.

    ``logits`` has shape (d0, d1, V): FP32 values, or BF16 bit patterns
    (uint16).  ``targets`` has shape (d0, d1) int64.  ``layout`` names what
    (d0, d1) are: "B,SQ" or "SQ,B".
    """

    name: str
    layout: str
    dtype: str
    logits: np.ndarray
    targets: np.ndarray
    label_smoothing: float
    reduce_loss: bool
    grad_output: np.ndarray  # FP32: shape (1,) when reduce_loss, else (d0, d1)
    ignore_idx: int = IGNORE_INDEX
    meta: dict = field(default_factory=dict)

    @property
    def d0(self) -> int:
        return self.logits.shape[0]

    @property
    def d1(self) -> int:
        return self.logits.shape[1]

    @property
    def V(self) -> int:
        return self.logits.shape[2]

    @property
    def N(self) -> int:
        return self.d0 * self.d1

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DTYPE_FP32 else 2


def make_logits(seed: int, d0: int, d1: int, V: int, *, dtype: str, sigma: float,
                ignore_frac: float | None = None, ignore_count: int | None = None,
                target_boost: float = 0.0, label_smoothing: float = 0.0,
                reduce_loss: bool = False, layout: str = "B,SQ",
                grad_output: str = "ones", name: str = "custom") -> LogitsCase:
    """Draw a logits problem.  ``target_boost`` is added (in FP32, before BF16
    rounding) to the target logit of every non-ignored row."""
    rng = np.random.default_rng(seed)
    z = _normal_f32(rng, (d0, d1, V), sigma)
    N = d0 * d1
    t = rng.integers(0, V, size=N, dtype=np.int64)
    ign = _ignore_rows(rng, N, ignore_frac, ignore_count)
    t[ign] = IGNORE_INDEX
    if target_boost != 0.0:
        zf = z.reshape(N, V)
        valid = np.nonzero(t != IGNORE_INDEX)[0]
        zf[valid, t[valid]] += np.float32(target_boost)
    if reduce_loss:
        go = np.ones(1, dtype=np.float32)
    elif grad_output == "ones":
        go = np.ones((d0, d1), dtype=np.float32)
    else:  # "random": per-token upstream gradients in [0.5, 1.5)
        go = (0.5 + rng.random((d0, d1))).astype(np.float32)
    logits = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z
    return LogitsCase(name=name, layout=layout, dtype=dtype, logits=logits,
                      targets=t.reshape(d0, d1), label_smoothing=label_smoothing,
                      reduce_loss=reduce_loss, grad_output=go,
                      meta=dict(seed=seed, sigma=sigma, n_ignored=int(ign.size),
                                target_boost=target_boost))


@dataclass
class LinearCase:
    """A fused linear cross-entropy problem: X (M,H) and W (V,H) as BF16 bits."""

    name: str
    X: np.ndarray
    W: np.ndarray
    targets: np.ndarray
    label_smoothing: float
    reduce_loss: bool
    grad_output: np.ndarray
    ignore_idx: int = IGNORE_INDEX
    meta: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.X.shape[0]

    @property
    def H(self) -> int:
        return self.X.shape[1]

    @property
    def V(self) -> int:
        return self.W.shape[0]


def make_linear(seed: int, M: int, H: int, V: int, *, ignore_frac: float | None = None,
                ignore_count: int | None = None, targets: str = "uniform", zipf_s: float = 1.1,
                label_smoothing: float = 0.0, reduce_loss: bool = True,
                grad_output: str = "ones", w_sigma: float | None = None,
                name: str = "custom", fp32: bool = False) -> LinearCase:
    """Draw X ~ N(0,1) and W ~ N(0, 1/H) (unless ``w_sigma``), both BF16
    (RNE from the FP32 draw), or with ``fp32`` the FP32 draws themselves."""
    rng = np.random.default_rng(seed)
    cast = (lambda a: a) if fp32 else f32_to_bf16_bits
    X = cast(_normal_f32(rng, (M, H), 1.0))
    ws = (1.0 / np.sqrt(H)) if w_sigma is None else w_sigma
    W = cast(_normal_f32(rng, (V, H), ws))
    if targets == "zipf":
        t = zipf_targets(rng, M, V, zipf_s)
    else:
        t = rng.integers(0, V, size=M, dtype=np.int64)
    ign = _ignore_rows(rng, M, ignore_frac, ignore_count)
    t[ign] = IGNORE_INDEX
    if reduce_loss:
        go = np.ones(1, dtype=np.float32)
    elif grad_output == "ones":
        go = np.ones(M, dtype=np.float32)
    else:
        go = (0.5 + rng.random(M)).astype(np.float32)
    return LinearCase(name=name, X=X, W=W, targets=t, label_smoothing=label_smoothing,
                      reduce_loss=reduce_loss, grad_output=go,
                      meta=dict(seed=seed, n_ignored=int(ign.size), w_sigma=ws))


# ---------------------------------------------------------------------------
# The named workloads.
# ---------------------------------------------------------------------------

def tiny_logits(label_smoothing: float = 0.0, reduce_loss: bool = False) -> LogitsCase:
    """B=2, SQ=4, V=1000, FP32 logits ~ N(0, 2^2), one ignored token."""
    return make_logits(1001, 2, 4, 1000, dtype=DTYPE_FP32, sigma=2.0, ignore_count=1,
                       label_smoothing=label_smoothing, reduce_loss=reduce_loss,
                       layout="B,SQ", name=f"tiny_fp32_ls{label_smoothing}_red{int(reduce_loss)}")


def medium_logits() -> LogitsCase:
    """(B,SQ,V) = (4, 1024, 32000) BF16 ~ N(0, 3^2), 5% ignored, eps 0.1, mean."""
    return make_logits(1002, 4, 1024, 32000, dtype=DTYPE_BF16, sigma=3.0, ignore_frac=0.05,
                       label_smoothing=0.1, reduce_loss=True, layout="B,SQ",
                       name="bsqv_4x1024_v32000_bf16")


def headline_logits() -> LogitsCase:
    """(SQ,B,V) = (2048, 2, 128256) BF16 ~ N(0, 4^2), target logit +8, 2%
    ignored, no smoothing, per-token loss."""
    return make_logits(1003, 2048, 2, 128256, dtype=DTYPE_BF16, sigma=4.0, ignore_frac=0.02,
                       target_boost=8.0, label_smoothing=0.0, reduce_loss=False,
                       layout="SQ,B", name="sqbv_2048x2_v128256_bf16")


def linear_4k() -> LinearCase:
    """X 4096 x 4096, W 131072 x 4096, 3% ignored, eps 0, mean."""
    return make_linear(1004, 4096, 4096, 131072, ignore_frac=0.03, label_smoothing=0.0,
                       reduce_loss=True, name="linear_m4096_h4096_v131072")


def linear_4k_f32() -> LinearCase:
    """linear_4k's shapes and recipe with FP32 X and W (the FP32 draws)."""
    return make_linear(1004, 4096, 4096, 131072, ignore_frac=0.03, label_smoothing=0.0,
                       reduce_loss=True, name="linear_f32_m4096_h4096_v131072", fp32=True)


def linear_16k() -> LinearCase:
    """X 16384 x 2304, W 256003 x 2304, Zipf(1.1) targets, 10% ignored, eps 0.1, mean."""
    return make_linear(1005, 16384, 2304, 256003, ignore_frac=0.10, targets="zipf",
                       zipf_s=1.1, label_smoothing=0.1, reduce_loss=True,
                       name="linear_m16384_h2304_v256003")
