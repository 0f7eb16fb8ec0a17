"""Comparison helpers for the parity tests (HIP path vs the FP64 oracle).

Tolerances (the floating-point bar the GPU path must meet):
  * per-token loss: |gpu - oracle| <= 1e-4 + 1e-5 |oracle|
  * FP32 gradient: |gpu - oracle| <= 1e-6
  * BF16 gradient: at most 1 BF16 ulp from the oracle rounded to nearest even
    (distance in the ordered integer encoding; +0 and -0 are equal), for
    every element outside the cancellation band.  The band is where
    G = g (p_v - q_v) nearly cancels, |G| < 2^-15 T with T = |g| (p_v + q_v),
    the size of the terms.  There even an ideal FP32 evaluation, which forms
    p_v and q_v each to one or two FP32 roundings (error up to 2 * 2^-24 T),
    can move G across a BF16 rounding boundary and land 2 ulps from the
    rounded oracle value: that takes an error of a whole BF16 ulp of G, at
    least 2^-8 |G|.  Inside the band the bar is |gpu - G| <= 2^-20 T + ulp(G):
    the kernel forms e^(z - m) from the exact difference z - m with a
    Cody-Waite reduction (the exponential unit's error plus about one
    rounding), d = sum e^(z - m) to a few roundings, g / d, g eps / V and the
    final fused multiply-add to one rounding each, about 10 * 2^-24 T in
    all, bounded here by 16 * 2^-24 T.  The band is counted and reported.
  * linear form: loss relative error <= 1e-3, dX and dW relative Frobenius
    error <= 5e-3
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

LOSS_ATOL, LOSS_RTOL = 1e-4, 1e-5
GRAD_FP32_ATOL = 1e-6
LINEAR_LOSS_RTOL = 1e-3
LINEAR_FROB_RTOL = 5e-3


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """FP32 values or BF16 bit patterns -> a device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device BF16 tensor -> uint16 bit patterns; FP32 -> float32."""
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().contiguous().cpu().numpy()


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def assert_loss_close(gpu: np.ndarray, ref: np.ndarray, what="loss"):
    gpu = np.asarray(gpu, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    finite = np.isfinite(ref)
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), f"{what}: NaN pattern differs"
    err = np.abs(gpu[finite] - ref[finite])
    bound = LOSS_ATOL + LOSS_RTOL * np.abs(ref[finite])
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, worst abs err "
                           f"{err.max():.3e} at {np.argmax(err)}")
    return float(err.max()) if err.size else 0.0


BAND_REL = 2.0 ** -15      # cancellation band: |G| < BAND_REL * T
BAND_ABS_REL = 2.0 ** -20  # bar inside the band: |gpu - G| <= BAND_ABS_REL * T + ulp(G)
# An extra term of the gradient formed less accurately than an ideal FP32
# evaluation (the entropy term, whose factor E_p[z] - z comes from FP32 values
# of magnitude |E_p[z]| + |z| and the forward's entropy) widens the band by
# 2^8 times its error bound 2^-18 T_H and the in-band bar by that bound.
EXTRA_ERR_REL = 2.0 ** -18


def grad_terms(ref64: np.ndarray, g_rows: np.ndarray, targets_rows: np.ndarray, eps: float,
               ignore_idx: int) -> np.ndarray:
    """T = |g| (p + q) per element, recovered from G = g (p - q)."""
    V = ref64.shape[1]
    q = np.full(ref64.shape, eps / V)
    valid = (targets_rows != ignore_idx) & (targets_rows >= 0) & (targets_rows < V)
    r = np.nonzero(valid)[0]
    q[r, targets_rows[r]] += 1.0 - eps
    g = np.asarray(g_rows, np.float64)[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(g != 0, ref64 / g + q, 0.0)
    T = np.abs(g) * (np.abs(p) + q)
    T[~valid] = 0.0
    return T


def assert_grad_bf16(gpu_bits: np.ndarray, ref64: np.ndarray, terms: np.ndarray, what="grad",
                     stats: dict | None = None, extra_terms: np.ndarray | None = None):
    """BF16 gradient bar (module docstring).  ``terms`` is T per element;
    ``extra_terms`` (optional) the size T_H of a term formed to the looser
    EXTRA_ERR_REL bound."""
    ref_bits = oracle.round_bf16(ref64)
    nan_ref = np.isnan(ref64)
    gpu_nan = (gpu_bits & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, gpu_nan), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err_bound = BAND_ABS_REL * terms
    band_edge = BAND_REL * terms
    if extra_terms is not None:
        err_bound = err_bound + EXTRA_ERR_REL * extra_terms
        band_edge = band_edge + 2.0 ** 8 * EXTRA_ERR_REL * extra_terms
    band = ok & (np.abs(ref64) < band_edge)
    out = ok & ~band
    d = bf16_ulp_distance(gpu_bits[out], ref_bits[out])
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, f"{what}: {int((d > 1).sum())} elements beyond 1 BF16 ulp (worst {worst})"
    nb = int(band.sum())
    worst_band = 0.0
    if nb:
        G = ref64[band]
        gv = oracle.bf16_to_f64(gpu_bits[band])
        _, e = np.frexp(np.maximum(np.abs(G), 2.0 ** -126))
        ulp = np.ldexp(1.0, e - 8)  # BF16 spacing at |G|
        err = np.abs(gv - G)
        bound = err_bound[band] + ulp
        assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} band elements out of bound"
        worst_band = float(np.max(err / (terms[band] + 1e-300)))
    if stats is not None:
        stats["elements"] = stats.get("elements", 0) + int(ok.sum())
        stats["band"] = stats.get("band", 0) + nb
        beyond = int((bf16_ulp_distance(gpu_bits[band], ref_bits[band]) > 1).sum()) if nb else 0
        stats["band_beyond_1ulp"] = stats.get("band_beyond_1ulp", 0) + beyond
        stats["worst_ulp"] = max(stats.get("worst_ulp", 0), worst)
        stats["worst_band_err_over_T"] = max(stats.get("worst_band_err_over_T", 0.0), worst_band)
    return worst


def assert_grad_fp32(gpu: np.ndarray, ref64: np.ndarray, what="grad"):
    nan_ref = np.isnan(ref64)
    assert np.array_equal(nan_ref, np.isnan(gpu)), f"{what}: NaN pattern differs"
    err = np.abs(gpu[~nan_ref].astype(np.float64) - ref64[~nan_ref])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= GRAD_FP32_ATOL, f"{what}: worst abs err {worst:.3e}"
    return worst


def rel_frobenius(gpu: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(np.asarray(gpu, np.float64) - ref)
    den = np.linalg.norm(ref)
    return float(num / den) if den > 0 else float(num)
