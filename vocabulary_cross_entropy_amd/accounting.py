"""Work models for the roofline: algorithmic bytes and flops per call.

Logits cross-entropy is bound by HBM traffic.  The forward must read every
logit of a non-ignored row once; the backward must read the same logits once
more and write the full gradient (ignored rows are written as zeros, never
read).  The nominal model counts every row (one read forward, one read plus
one write backward), the convention of the statistics-saving design in the
TransformerEngine PR (Changes: the backward reads fewer bytes than before).

Fused linear cross-entropy is bound by the matrix cores.  The Liger-Kernel
PR (Performance methodology) counts 2*M*H*V flops per classifier GEMM, one
GEMM forward and four for forward+backward (forward logits, recomputed
logits for dZ, dX and dW).
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense BF16 matrix peak (256 CU x 2.4 GHz)
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix peak


def ce_bytes(N: int, V: int, elem_bytes: int, n_ignored: int = 0, phase: str = "fb") -> int:
    """Algorithmic HBM bytes of logits cross-entropy (rows that are ignored
    are not read)."""
    read = (N - n_ignored) * V * elem_bytes
    write = N * V * elem_bytes
    if phase == "fwd":
        return read
    if phase == "bwd":
        return read + write
    if phase == "fb":
        return 2 * read + write
    raise ValueError(phase)


def ce_bytes_nominal(N: int, V: int, elem_bytes: int, phase: str = "fb") -> int:
    """Nominal bytes: 1 read forward, 1 read + 1 write backward, all rows."""
    return {"fwd": 1, "bwd": 2, "fb": 3}[phase] * N * V * elem_bytes


def linear_flops(M: int, H: int, V: int, phase: str = "fb") -> float:
    """Classifier GEMM flops: 2*M*H*V per GEMM; fwd = 1 GEMM, fb = 4 GEMMs,
    bwd = 3 GEMMs (recomputed logits, dX, dW)."""
    per = 2.0 * M * H * V
    return per * {"fwd": 1, "bwd": 3, "fb": 4}[phase]
