"""FP64 CPU oracle for fused cross-entropy over a large vocabulary.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``vocabulary_cross_entropy_amd``) never imports, links or calls it, and it
shares no code with the HIP kernels: the C core (``ce_ref.c``) decodes BF16
itself and works in double precision from the plain definitions.

Contents
  * ``ce_forward`` / ``ce_backward``: logits cross-entropy (C core, OpenMP
    over rows), following the TransformerEngine cross-entropy API page (I/O
    Contract) and the TransformerEngine PR that rebuilds the gradient from
    saved statistics (Changes; Sequence Diagram).
  * ``mean_loss`` / ``row_scale``: the averaged scalar loss over non-ignored
    rows and the per-row upstream factor g_r.
  * ``round_bf16``: FP64 -> BF16 round-to-nearest-even (C core).
  * ``linear``: fused linear cross-entropy in NumPy FP64 (``linear.py``).
  * ``shard``: vocabulary-sharded local statistics, their merge and the
    per-shard gradient in NumPy FP64 (``shard.py``).
  * ``shift``: the causal label shift (``shift.py``).
  * ``tiny``: a pure-Python ``math`` version for tiny cases (``tiny.py``).

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ce_ref.c")
_LIB = os.path.join(_HERE, "libce_ref.so")

DT_FP32, DT_BF16, DT_FP64 = 0, 1, 2

_lib = None


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile the C core with gcc (IEEE math, OpenMP).  With ``sanitize`` the
    build carries AddressSanitizer and UndefinedBehaviorSanitizer (any finding
    aborts); a process loads such a build only with the sanitizer runtime
    preloaded, through the VCE_ORACLE_LIB environment variable."""
    lib = out or _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        extra = SANITIZE_FLAGS if sanitize else []
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", *extra, _SRC, "-o",
                               tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("VCE_ORACLE_LIB")
        if alt:
            lib = ctypes.CDLL(alt)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.vce_oracle_forward.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, i64, i64,
                                           dbl, i64, vp, i64, vp, vp, vp]
        lib.vce_oracle_forward.restype = ctypes.c_int
        lib.vce_oracle_backward.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, i64, i64,
                                            dbl, i64, vp, vp, i64, vp]
        lib.vce_oracle_backward.restype = ctypes.c_int
        lib.vce_oracle_entropy.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, i64, i64,
                                           i64, vp, i64, vp]
        lib.vce_oracle_entropy.restype = ctypes.c_int
        lib.vce_oracle_entropy_grad.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, i64,
                                                i64, i64, vp, vp, i64, vp]
        lib.vce_oracle_entropy_grad.restype = ctypes.c_int
        lib.vce_oracle_round_bf16.argtypes = [vp, i64, vp]
        lib.vce_oracle_round_bf16.restype = None
        lib.vce_oracle_threads.argtypes = []
        lib.vce_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C core runs with."""
    return int(_load().vce_oracle_threads())


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_FP32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float64:
        return DT_FP64
    raise TypeError(f"unsupported logits storage {a.dtype}")


def _as_3d(logits: np.ndarray, targets: np.ndarray):
    """Accept (N, V) or (d0, d1, V) logits with matching targets; keep strides."""
    if logits.ndim == 2:
        logits = logits[None]
        targets = np.asarray(targets)[None]
    if logits.ndim != 3 or targets.shape != logits.shape[:2]:
        raise ValueError("logits must be (d0, d1, V) with targets (d0, d1)")
    if logits.strides[2] != logits.itemsize:
        logits = np.ascontiguousarray(logits)
    targets = np.asarray(targets, dtype=np.int64)
    return logits, targets


def ce_forward(logits: np.ndarray, targets: np.ndarray, label_smoothing: float = 0.0,
               ignore_idx: int = -100, rows: np.ndarray | None = None):
    """Per-row loss, saved statistics and the closed-form loss, in FP64.

    ``logits``: (d0, d1, V) or (N, V) array of float32, BF16 bits (uint16) or
    float64; leading strides may be arbitrary (views).  ``rows`` selects
    flattened row indices (row r = i0 * d1 + i1); default all rows.

    Returns ``(loss, stats, loss_closed)``: loss (n,), stats (n, 4) = (max,
    sum exp(z - max), z_target, mean z), and the closed form
    (1-eps)(lse - z_t) + eps (lse - mean z) (n,).
    """
    lg, tg = _as_3d(logits, targets)
    d0, d1, V = lg.shape
    it = lg.itemsize
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = d0 * d1 if rr is None else rr.size
    loss = np.empty(n, np.float64)
    stats = np.empty((n, 4), np.float64)
    closed = np.empty(n, np.float64)
    rc = _load().vce_oracle_forward(
        _ptr(lg), _dtype_code(lg), d0, d1, V, lg.strides[0] // it, lg.strides[1] // it,
        _ptr(tg), tg.strides[0] // 8, tg.strides[1] // 8, float(label_smoothing), int(ignore_idx),
        _ptr(rr), n, _ptr(loss), _ptr(stats), _ptr(closed))
    if rc != 0:
        raise ValueError("oracle forward rejected its arguments")
    return loss, stats, closed


def n_valid(targets: np.ndarray, ignore_idx: int = -100) -> int:
    return int(np.count_nonzero(np.asarray(targets) != ignore_idx))


def mean_loss(loss: np.ndarray, targets: np.ndarray, ignore_idx: int = -100) -> float:
    """Averaged scalar loss: sum over non-ignored rows / their count.  With no
    valid row the denominator is taken as 1, giving 0 (the pages are silent)."""
    t = np.asarray(targets).reshape(-1)
    valid = t != ignore_idx
    return float(np.sum(np.asarray(loss, np.float64).reshape(-1)[valid])) / max(int(valid.sum()), 1)


def row_scale(grad_output: np.ndarray, targets: np.ndarray, reduce_loss: bool,
              ignore_idx: int = -100) -> np.ndarray:
    """Per-row upstream factor g_r: grad_output[r], or grad_output / n_valid
    for the averaged loss.  Returned for every flattened row."""
    t = np.asarray(targets).reshape(-1)
    if reduce_loss:
        g = float(np.asarray(grad_output, np.float64).reshape(-1)[0]) / max(n_valid(t, ignore_idx), 1)
        return np.full(t.size, g, np.float64)
    return np.asarray(grad_output, np.float64).reshape(-1).copy()


def ce_backward(logits: np.ndarray, targets: np.ndarray, g: np.ndarray,
                label_smoothing: float = 0.0, ignore_idx: int = -100,
                rows: np.ndarray | None = None) -> np.ndarray:
    """Gradient rows g_r (softmax(z_r) - q_r) in FP64, shape (n, V).

    ``g`` holds g_r for every flattened row (see ``row_scale``); ``rows``
    selects which rows to return."""
    lg, tg = _as_3d(logits, targets)
    d0, d1, V = lg.shape
    it = lg.itemsize
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = d0 * d1 if rr is None else rr.size
    gsel = np.ascontiguousarray(np.asarray(g, np.float64).reshape(-1)[rr] if rr is not None
                                else np.asarray(g, np.float64).reshape(-1))
    grad = np.empty((n, V), np.float64)
    rc = _load().vce_oracle_backward(
        _ptr(lg), _dtype_code(lg), d0, d1, V, lg.strides[0] // it, lg.strides[1] // it,
        _ptr(tg), tg.strides[0] // 8, tg.strides[1] // 8, float(label_smoothing), int(ignore_idx),
        _ptr(gsel), _ptr(rr), n, _ptr(grad))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return grad


def entropy(logits: np.ndarray, targets: np.ndarray, ignore_idx: int = -100,
            rows: np.ndarray | None = None) -> np.ndarray:
    """Per-row entropy -sum_v p_v ln p_v of softmax(z) in FP64 (0 for ignored
    rows), the optional entropy output of the Liger-Kernel PR (Summary)."""
    lg, tg = _as_3d(logits, targets)
    d0, d1, V = lg.shape
    it = lg.itemsize
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = d0 * d1 if rr is None else rr.size
    ent = np.empty(n, np.float64)
    rc = _load().vce_oracle_entropy(
        _ptr(lg), _dtype_code(lg), d0, d1, V, lg.strides[0] // it, lg.strides[1] // it,
        _ptr(tg), tg.strides[0] // 8, tg.strides[1] // 8, int(ignore_idx), _ptr(rr), n, _ptr(ent))
    if rc != 0:
        raise ValueError("oracle entropy rejected its arguments")
    return ent


def add_entropy_grad(grad: np.ndarray, logits: np.ndarray, targets: np.ndarray,
                     grad_entropy: np.ndarray, ignore_idx: int = -100,
                     rows: np.ndarray | None = None) -> np.ndarray:
    """grad[i] += gH_r dH/dz for the selected rows, dH/dz_v = -p_v (ln p_v + H),
    in place (FP64, shape (n, V)); ``grad_entropy`` holds gH for every row."""
    lg, tg = _as_3d(logits, targets)
    d0, d1, V = lg.shape
    it = lg.itemsize
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = d0 * d1 if rr is None else rr.size
    gh = np.asarray(grad_entropy, np.float64).reshape(-1)
    gsel = np.ascontiguousarray(gh[rr] if rr is not None else gh)
    if grad.shape != (n, V) or grad.dtype != np.float64 or not grad.flags.c_contiguous:
        raise ValueError("grad must be a C-contiguous float64 (n, V) array")
    rc = _load().vce_oracle_entropy_grad(
        _ptr(lg), _dtype_code(lg), d0, d1, V, lg.strides[0] // it, lg.strides[1] // it,
        _ptr(tg), tg.strides[0] // 8, tg.strides[1] // 8, int(ignore_idx), _ptr(gsel), _ptr(rr), n,
        _ptr(grad))
    if rc != 0:
        raise ValueError("oracle entropy gradient rejected its arguments")
    return grad


def round_bf16(x: np.ndarray) -> np.ndarray:
    """FP64 -> BF16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().vce_oracle_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns as float64 (bits << 16 read as FP32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
