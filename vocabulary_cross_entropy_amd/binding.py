"""Thin Python binding of libvce (include/vce.h) over ctypes.

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if ``libvce.so`` is missing or the device is not a GPU,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvce.so")

DTYPE_FP32 = 0
DTYPE_BF16 = 1

STATUS = {0: "VCE_OK", 1: "VCE_EINVAL", 2: "VCE_EDTYPE", 3: "VCE_EALIGN", 4: "VCE_EALIAS",
          5: "VCE_EWORKSPACE", 6: "VCE_EHIP", 7: "VCE_EUNSUPPORTED", 8: "VCE_ESCRATCH"}

# (name, restype, argtypes) for every symbol include/vce.h declares.
_I64, _I32, _F32, _VP, _SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "vce_strerror": (ctypes.c_char_p, [_I32]),
    "ce_forward": (_I32, [_VP, _I32, _I64, _I64, _I64, _I64, _I64, _VP, _I64, _I64, _F32, _I32, _I64,
                          _VP, _VP, _VP, _VP, _VP, _VP]),
    "ce_backward": (_I32, [_VP, _VP, _I32, _I64, _I64, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _VP,
                           _VP, _VP, _VP, _F32, _I32, _I64, _I32, _VP]),
    "ce_forward_backward": (_I32, [_VP, _VP, _I32, _I64, _I64, _I64, _I64, _I64, _VP, _I64, _I64,
                                   _VP, _F32, _I32, _I64, _I32, _VP, _VP, _VP, _VP, _VP]),
    "ce_forward_shard": (_I32, [_VP, _I32, _I64, _I64, _I64, _I64, _I64, _VP, _I64, _I64, _I64,
                                _I64, _VP, _VP, _VP]),
    "ce_merge_shards": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _I64, _I64, _I64, _F32, _I32,
                               _I64, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ce_backward_shard": (_I32, [_VP, _VP, _I32, _I64, _I64, _I64, _I64, _I64, _VP, _I64, _I64,
                                 _I64, _I64, _VP, _VP, _VP, _VP, _VP, _F32, _I32, _I64, _I32,
                                 _VP]),
    "vce_shift_targets": (_I32, [_VP, _I64, _I64, _I64, _I64, _I32, _I64, _VP, _VP]),
    "lce_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "lce_forward": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _F32, _I32, _I64, _VP, _VP, _VP, _VP,
                           _VP, _VP, _SZ, _VP]),
    "lce_forward_noalloc": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _F32, _I32, _I64, _VP, _VP,
                                   _VP, _VP, _VP, _VP]),
    "lce_backward": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _F32, _I32,
                            _I64, _VP, _VP, _VP, _SZ, _VP]),
    "lce_forward_scaled": (_I32, [_VP, _VP, _I64, _I64, _I64, _F32, _VP, _F32, _I32, _I64, _VP,
                                  _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lce_backward_scaled": (_I32, [_VP, _VP, _I64, _I64, _I64, _F32, _VP, _VP, _VP, _VP, _VP,
                                   _VP, _F32, _I32, _I64, _VP, _VP, _VP, _SZ, _VP]),
    "lce_workspace_size_f32": (_SZ, [_I64, _I64, _I64]),
    "lce_forward_f32": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _F32, _I32, _I64, _VP, _VP, _VP,
                               _VP, _VP, _VP, _SZ, _VP]),
    "lce_backward_f32": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _F32,
                                _I32, _I64, _VP, _VP, _VP, _SZ, _VP]),
    "lce_forward_shard": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _VP, _VP,
                                 _SZ, _VP]),
    "lce_backward_shard": (_I32, [_VP, _VP, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _VP, _VP,
                                  _VP, _VP, _F32, _I32, _I64, _VP, _VP, _VP, _SZ, _VP]),
    "lce_forward_shard_scaled": (_I32, [_VP, _VP, _I64, _I64, _I64, _F32, _VP, _I64, _I64, _VP,
                                        _VP, _VP, _SZ, _VP]),
    "lce_backward_shard_scaled": (_I32, [_VP, _VP, _I64, _I64, _I64, _F32, _VP, _I64, _I64, _VP,
                                         _VP, _VP, _VP, _VP, _F32, _I32, _I64, _VP, _VP, _VP,
                                         _SZ, _VP]),
    "vce_gemm_bf16": (_I32, [_VP, _I64, _I32, _VP, _I64, _I32, _I64, _I64, _I64, _VP, _I64, _VP]),
}

_lib = None


class VceError(RuntimeError):
    def __init__(self, name: str, code: int, text: str):
        super().__init__(f"{name} failed: {STATUS.get(code, code)} ({text})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libvce.so (built in-tree by ``python -m vocabulary_cross_entropy_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m vocabulary_cross_entropy_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().vce_strerror(code).decode()


def _check(name: str, code: int):
    if code != 0:
        raise VceError(name, code, strerror(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_FP32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise RuntimeError("libvce runs on the GPU only: tensors must be on a HIP device")


def _check_buf(t, name: str, numel: int, dtype=torch.float32, *, one_ok: bool = False,
               like: torch.Tensor | None = None):
    """A tensor handed to the library as a flat buffer: its dtype, element
    count (``numel``, or 1 with ``one_ok``), contiguity (the library reads it
    in flattened row order) and device (that of ``like``).  None passes."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel and not (one_ok and t.numel() == 1):
        want = f"{numel}" + (" or 1" if one_ok else "")
        raise ValueError(f"{name} must hold {want} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")


def _check_rows(N: int, like: torch.Tensor, *, stats=None, n_valid=None, grad_output=None,
                reduce_loss=False, loss_tok=None, loss_mean=None, entropy=None,
                grad_entropy=None):
    """The per-row buffers of a logits or linear call with N rows."""
    _check_buf(stats, "stats", 4 * N, like=like)
    _check_buf(n_valid, "n_valid", 1, torch.int32, like=like)
    if grad_output is not None:
        _check_buf(grad_output, "grad_output", 1 if reduce_loss else N, like=like)
    _check_buf(loss_tok, "loss_tok", N, like=like)
    _check_buf(loss_mean, "loss_mean", 1, like=like)
    _check_buf(entropy, "entropy", N, like=like)
    _check_buf(grad_entropy, "grad_entropy", N, like=like)


def _logits3d(logits: torch.Tensor, targets: torch.Tensor):
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
        targets = targets.unsqueeze(0)
    if logits.dim() != 3 or tuple(targets.shape) != tuple(logits.shape[:2]):
        raise ValueError("logits must be (d0, d1, V) with targets (d0, d1)")
    if logits.stride(2) != 1:
        raise ValueError("the vocabulary dimension of logits must be contiguous")
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    return logits, targets


def _check_grad(grad: torch.Tensor, logits: torch.Tensor):
    if tuple(grad.shape) != tuple(logits.shape) or tuple(grad.stride()) != tuple(logits.stride()) \
            or grad.dtype != logits.dtype:
        raise ValueError("grad must have the shape, dtype and strides of logits")
    if grad.device != logits.device:
        raise ValueError(f"grad must be on {logits.device}, got {grad.device}")


def _grad_like(logits: torch.Tensor) -> torch.Tensor:
    """An uninitialised tensor with the dtype and strides of ``logits`` whose
    rows start at the same offset within 16 bytes (the backward splits the
    logits row and the gradient row at the same element)."""
    es = logits.element_size()
    pad = (logits.data_ptr() % 16) // es
    span = 1 + sum((n - 1) * st for n, st in zip(logits.shape, logits.stride()))
    buf = torch.empty(pad + span, dtype=logits.dtype, device=logits.device)
    return buf.as_strided(logits.shape, logits.stride(), pad)


def ce_forward(logits: torch.Tensor, targets: torch.Tensor, label_smoothing: float = 0.0,
               reduce_loss: bool = False, ignore_idx: int = -100, *, stream=None, out=None,
               with_entropy: bool = False):
    """Forward of logits cross-entropy.  Returns (loss_tok, loss_mean, stats, n_valid),
    plus the per-row entropy with ``with_entropy``; loss_mean and n_valid are None
    unless reduce_loss.  ``out`` gives the output tensors in the same order."""
    logits, targets = _logits3d(logits, targets)
    d0, d1, V = logits.shape
    dev = logits.device
    if out is None:
        loss_tok = torch.empty((d0, d1), dtype=torch.float32, device=dev)
        stats = torch.empty((d0, d1, 4), dtype=torch.float32, device=dev)
        loss_mean = torch.empty((), dtype=torch.float32, device=dev) if reduce_loss else None
        n_valid = torch.empty((), dtype=torch.int32, device=dev) if reduce_loss else None
        ent = torch.empty((d0, d1), dtype=torch.float32, device=dev) if with_entropy else None
    else:
        loss_tok, loss_mean, stats, n_valid = out[:4]
        ent = out[4] if with_entropy else None
    _check_rows(d0 * d1, logits, stats=stats, n_valid=n_valid, loss_tok=loss_tok,
                loss_mean=loss_mean, entropy=ent)
    _need_cuda(logits, targets)
    rc = lib().ce_forward(_ptr(logits), _dtype_code(logits), d0, d1, V, logits.stride(0),
                          logits.stride(1), _ptr(targets), targets.stride(0), targets.stride(1),
                          float(label_smoothing), int(bool(reduce_loss)), int(ignore_idx),
                          _ptr(loss_tok), _ptr(loss_mean), _ptr(stats), _ptr(n_valid), _ptr(ent),
                          _stream(stream))
    _check("ce_forward", rc)
    if with_entropy:
        return loss_tok, loss_mean, stats, n_valid, ent
    return loss_tok, loss_mean, stats, n_valid


def ce_backward(logits: torch.Tensor, targets: torch.Tensor, stats: torch.Tensor,
                n_valid: torch.Tensor | None, grad_output: torch.Tensor,
                label_smoothing: float = 0.0, reduce_loss: bool = False, ignore_idx: int = -100,
                overwrite_input: bool = False, *, grad: torch.Tensor | None = None, stream=None,
                entropy: torch.Tensor | None = None, grad_entropy: torch.Tensor | None = None):
    """Gradient of logits cross-entropy rebuilt from ``stats``.  With
    ``overwrite_input`` the logits tensor itself receives the gradient.  With
    ``grad_entropy`` (per row) the entropy's gradient is added; ``entropy`` is
    then the forward's entropy output."""
    logits, targets = _logits3d(logits, targets)
    d0, d1, V = logits.shape
    _check_rows(d0 * d1, logits, stats=stats, n_valid=n_valid if reduce_loss else None,
                grad_output=grad_output, reduce_loss=reduce_loss, entropy=entropy,
                grad_entropy=grad_entropy)
    if overwrite_input:
        grad = logits
    elif grad is None:
        grad = _grad_like(logits)
    elif grad.dim() == 2:
        grad = grad.unsqueeze(0)
    _check_grad(grad, logits)
    _need_cuda(logits, targets, stats, grad_output)
    rc = lib().ce_backward(_ptr(logits), _ptr(grad), _dtype_code(logits), d0, d1, V,
                           logits.stride(0), logits.stride(1), _ptr(targets), targets.stride(0),
                           targets.stride(1), _ptr(stats), _ptr(n_valid), _ptr(grad_output),
                           _ptr(entropy), _ptr(grad_entropy), float(label_smoothing),
                           int(bool(reduce_loss)), int(ignore_idx), int(bool(overwrite_input)),
                           _stream(stream))
    _check("ce_backward", rc)
    return grad


def ce_forward_backward(logits: torch.Tensor, targets: torch.Tensor, grad_output: torch.Tensor,
                        label_smoothing: float = 0.0, reduce_loss: bool = False,
                        ignore_idx: int = -100, overwrite_input: bool = False, *,
                        grad: torch.Tensor | None = None, stream=None, out=None):
    """``ce_forward`` then ``ce_backward`` with the same arguments, in one pass
    over the logits.  Returns (loss_tok, loss_mean, stats, n_valid, grad)."""
    logits, targets = _logits3d(logits, targets)
    d0, d1, V = logits.shape
    dev = logits.device
    if out is None:
        loss_tok = torch.empty((d0, d1), dtype=torch.float32, device=dev)
        stats = torch.empty((d0, d1, 4), dtype=torch.float32, device=dev)
        loss_mean = torch.empty((), dtype=torch.float32, device=dev) if reduce_loss else None
        n_valid = torch.empty((), dtype=torch.int32, device=dev) if reduce_loss else None
    else:
        loss_tok, loss_mean, stats, n_valid = out
    _check_rows(d0 * d1, logits, stats=stats, n_valid=n_valid, grad_output=grad_output,
                reduce_loss=reduce_loss, loss_tok=loss_tok, loss_mean=loss_mean)
    if overwrite_input:
        grad = logits
    elif grad is None:
        grad = _grad_like(logits)
    elif grad.dim() == 2:
        grad = grad.unsqueeze(0)
    _check_grad(grad, logits)
    _need_cuda(logits, targets, grad_output)
    rc = lib().ce_forward_backward(_ptr(logits), _ptr(grad), _dtype_code(logits), d0, d1, V,
                                   logits.stride(0), logits.stride(1), _ptr(targets),
                                   targets.stride(0), targets.stride(1), _ptr(grad_output),
                                   float(label_smoothing), int(bool(reduce_loss)),
                                   int(ignore_idx), int(bool(overwrite_input)), _ptr(loss_tok),
                                   _ptr(loss_mean), _ptr(stats), _ptr(n_valid), _stream(stream))
    _check("ce_forward_backward", rc)
    return loss_tok, loss_mean, stats, n_valid, grad


def ce_forward_shard(logits: torch.Tensor, targets: torch.Tensor, vocab_start: int,
                     ignore_idx: int = -100, *, stream=None, out=None, with_entropy: bool = False,
                     out_w=None):
    """Partial statistics (d0, d1, 4) of one vocabulary shard: ``logits`` holds
    columns vocab_start .. vocab_start + V_local - 1 of the full vocabulary.
    With ``with_entropy`` also the shard's entropy statistic (d0, d1), returned
    second."""
    logits, targets = _logits3d(logits, targets)
    d0, d1, V = logits.shape
    part = torch.empty((d0, d1, 4), dtype=torch.float32, device=logits.device) if out is None \
        else out
    pw = None
    if with_entropy:
        pw = torch.empty((d0, d1), dtype=torch.float32, device=logits.device) if out_w is None \
            else out_w
    _check_buf(part, "partial", 4 * d0 * d1, like=logits)
    _check_buf(pw, "partial_w", d0 * d1, like=logits)
    _need_cuda(logits, targets)
    rc = lib().ce_forward_shard(_ptr(logits), _dtype_code(logits), d0, d1, V, logits.stride(0),
                                logits.stride(1), _ptr(targets), targets.stride(0),
                                targets.stride(1), int(vocab_start), int(ignore_idx), _ptr(part),
                                _ptr(pw), _stream(stream))
    _check("ce_forward_shard", rc)
    return (part, pw) if with_entropy else part


def ce_merge_shards(partials: torch.Tensor, targets: torch.Tensor, V: int,
                    label_smoothing: float = 0.0, reduce_loss: bool = False,
                    ignore_idx: int = -100, *, stream=None, out=None,
                    partials_w: torch.Tensor | None = None, out_entropy=None):
    """Merge stacked shard partials (n_shards, d0, d1, 4) (or (n_shards, N, 4)
    with targets (N)) into (loss_tok, loss_mean, stats, n_valid) over the full
    vocabulary of V columns, as ce_forward returns them.  With ``partials_w``
    (the shards' entropy statistics stacked the same way) the per-row entropy
    is appended."""
    if targets.dim() == 1:
        targets = targets.unsqueeze(0)
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    d0, d1 = targets.shape
    if not partials.is_contiguous() or partials.dtype != torch.float32 or \
            partials.numel() != partials.shape[0] * d0 * d1 * 4:
        raise ValueError("partials must be contiguous float32 (n_shards, d0, d1, 4)")
    dev = partials.device
    if out is None:
        loss_tok = torch.empty((d0, d1), dtype=torch.float32, device=dev)
        stats = torch.empty((d0, d1, 4), dtype=torch.float32, device=dev)
        loss_mean = torch.empty((), dtype=torch.float32, device=dev) if reduce_loss else None
        n_valid = torch.empty((), dtype=torch.int32, device=dev) if reduce_loss else None
    else:
        loss_tok, loss_mean, stats, n_valid = out
    _check_rows(d0 * d1, partials, stats=stats, n_valid=n_valid, loss_tok=loss_tok,
                loss_mean=loss_mean, entropy=out_entropy)
    _need_cuda(partials, targets)
    ent = None
    if partials_w is not None:
        if not partials_w.is_contiguous() or partials_w.dtype != torch.float32 or \
                partials_w.numel() != partials.shape[0] * d0 * d1:
            raise ValueError("partials_w must be contiguous float32 (n_shards, d0, d1)")
        ent = torch.empty((d0, d1), dtype=torch.float32, device=dev) if out_entropy is None \
            else out_entropy
    rc = lib().ce_merge_shards(_ptr(partials), _ptr(partials_w), partials.shape[0], d0, d1,
                               _ptr(targets), targets.stride(0), targets.stride(1), int(V),
                               float(label_smoothing), int(bool(reduce_loss)), int(ignore_idx),
                               _ptr(loss_tok), _ptr(loss_mean), _ptr(stats), _ptr(n_valid),
                               _ptr(ent), _stream(stream))
    _check("ce_merge_shards", rc)
    if ent is not None:
        return loss_tok, loss_mean, stats, n_valid, ent
    return loss_tok, loss_mean, stats, n_valid


def ce_backward_shard(logits: torch.Tensor, targets: torch.Tensor, vocab_start: int, V: int,
                      stats: torch.Tensor, n_valid: torch.Tensor | None,
                      grad_output: torch.Tensor, label_smoothing: float = 0.0,
                      reduce_loss: bool = False, ignore_idx: int = -100,
                      overwrite_input: bool = False, *, grad: torch.Tensor | None = None,
                      stream=None, entropy: torch.Tensor | None = None,
                      grad_entropy: torch.Tensor | None = None):
    """Gradient of one vocabulary shard's logits from the merged ``stats``
    (with ``grad_entropy``, plus the entropy's, ``entropy`` the merged one)."""
    logits, targets = _logits3d(logits, targets)
    d0, d1, VL = logits.shape
    _check_rows(d0 * d1, logits, stats=stats, n_valid=n_valid if reduce_loss else None,
                grad_output=grad_output, reduce_loss=reduce_loss, entropy=entropy,
                grad_entropy=grad_entropy)
    if overwrite_input:
        grad = logits
    elif grad is None:
        grad = _grad_like(logits)
    elif grad.dim() == 2:
        grad = grad.unsqueeze(0)
    _check_grad(grad, logits)
    _need_cuda(logits, targets, stats, grad_output)
    rc = lib().ce_backward_shard(_ptr(logits), _ptr(grad), _dtype_code(logits), d0, d1, VL,
                                 logits.stride(0), logits.stride(1), _ptr(targets),
                                 targets.stride(0), targets.stride(1), int(vocab_start), int(V),
                                 _ptr(stats), _ptr(n_valid), _ptr(grad_output), _ptr(entropy),
                                 _ptr(grad_entropy), float(label_smoothing),
                                 int(bool(reduce_loss)), int(ignore_idx),
                                 int(bool(overwrite_input)), _stream(stream))
    _check("ce_backward_shard", rc)
    return grad


def shift_targets(targets: torch.Tensor, seq_axis: int, ignore_idx: int = -100, *,
                  stream=None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal label shift of (d0, d1) (or (M,) as one sequence) int64 targets
    along ``seq_axis``: each position takes the next position's label, the
    last one ``ignore_idx``.  Returns a contiguous tensor of the same shape."""
    _need_cuda(targets)
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    t2 = targets.unsqueeze(0) if targets.dim() == 1 else targets
    if t2.dim() != 2:
        raise ValueError("targets must be (d0, d1) or (M,)")
    if targets.dim() == 1 and seq_axis == 0:
        raise ValueError("a 1-D target vector is one sequence: use seq_axis 1 (or -1)")
    seq_axis = 1 if seq_axis == -1 else seq_axis
    d0, d1 = t2.shape
    res = torch.empty(targets.shape, dtype=torch.int64, device=targets.device) if out is None \
        else out
    rc = lib().vce_shift_targets(_ptr(t2), d0, d1, t2.stride(0), t2.stride(1), int(seq_axis),
                                 int(ignore_idx), _ptr(res), _stream(stream))
    _check("vce_shift_targets", rc)
    return res


def lce_workspace_size(M: int, H: int, V: int) -> int:
    return int(lib().lce_workspace_size(M, H, V))


def lce_workspace_size_f32(M: int, H: int, V: int) -> int:
    return int(lib().lce_workspace_size_f32(M, H, V))


def lce_workspace(M: int, H: int, V: int, device="cuda", f32: bool = False) -> torch.Tensor:
    """Workspace for the BF16 linear form, or with ``f32`` for the FP32 one."""
    n = lce_workspace_size_f32(M, H, V) if f32 else lce_workspace_size(M, H, V)
    if n == 0:
        raise ValueError(f"no workspace plan for M={M}, H={H}, V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_linear(X, W, targets, dtype=torch.bfloat16):
    if X.dtype != dtype or W.dtype != dtype:
        raise TypeError(f"X and W must be {dtype}")
    if not (X.is_contiguous() and W.is_contiguous() and targets.is_contiguous()):
        raise ValueError("X, W and targets must be contiguous")
    if X.dim() != 2 or W.dim() != 2 or X.shape[1] != W.shape[1] or targets.numel() != X.shape[0]:
        raise ValueError("X (M,H), W (V,H), targets (M)")
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    if W.device != X.device or targets.device != X.device:
        raise ValueError("X, W and targets must be on one device")


def _check_like(t, name: str, ref: torch.Tensor):
    """An output with the shape and dtype of ``ref`` (dX like X, dW like W)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype:
        raise ValueError(f"{name} must be {ref.dtype} of shape {tuple(ref.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def lce_forward(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                label_smoothing: float = 0.0, reduce_loss: bool = True, ignore_idx: int = -100,
                *, workspace: torch.Tensor | None = None, stream=None, out=None,
                with_entropy: bool = False, logit_scale: float = 1.0):
    """Fused linear cross-entropy forward, BF16 X and W.  Returns (loss_tok,
    loss_mean, stats, n_valid), plus the per-token entropy with ``with_entropy``.
    ``logit_scale`` (finite, > 0): the loss of logit_scale * X W^T
    (``lce_forward_scaled``); the backward must get the same value."""
    return _lce_forward(False, X, W, targets, label_smoothing, reduce_loss, ignore_idx,
                        workspace, stream, out, with_entropy, logit_scale)


def lce_forward_noalloc(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                        label_smoothing: float = 0.0, reduce_loss: bool = True,
                        ignore_idx: int = -100, *, stream=None, out=None,
                        with_entropy: bool = False):
    """``lce_forward`` with the library's static scratch instead of a workspace
    (no device allocation by the library; ``out`` lets the caller supply the
    outputs too).  Problems beyond the scratch raise (VCE_ESCRATCH)."""
    _check_linear(X, W, targets)
    M, H = X.shape
    V = W.shape[0]
    dev = X.device
    if out is None:
        loss_tok = torch.empty(M, dtype=torch.float32, device=dev)
        stats = torch.empty((M, 4), dtype=torch.float32, device=dev)
        loss_mean = torch.empty((), dtype=torch.float32, device=dev) if reduce_loss else None
        n_valid = torch.empty((), dtype=torch.int32, device=dev) if reduce_loss else None
        ent = torch.empty(M, dtype=torch.float32, device=dev) if with_entropy else None
    else:
        loss_tok, loss_mean, stats, n_valid = out[:4]
        ent = out[4] if with_entropy else None
    _check_rows(M, X, stats=stats, n_valid=n_valid, loss_tok=loss_tok, loss_mean=loss_mean,
                entropy=ent)
    _need_cuda(X, W, targets)
    rc = lib().lce_forward_noalloc(_ptr(X), _ptr(W), M, H, V, _ptr(targets),
                                   float(label_smoothing), int(bool(reduce_loss)),
                                   int(ignore_idx), _ptr(loss_tok), _ptr(loss_mean), _ptr(stats),
                                   _ptr(n_valid), _ptr(ent), _stream(stream))
    _check("lce_forward_noalloc", rc)
    if with_entropy:
        return loss_tok, loss_mean, stats, n_valid, ent
    return loss_tok, loss_mean, stats, n_valid


def lce_forward_f32(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                    label_smoothing: float = 0.0, reduce_loss: bool = True,
                    ignore_idx: int = -100, *, workspace: torch.Tensor | None = None,
                    stream=None, out=None, with_entropy: bool = False):
    """As ``lce_forward`` for FP32 X and W (workspace from ``lce_workspace(..., f32=True)``)."""
    return _lce_forward(True, X, W, targets, label_smoothing, reduce_loss, ignore_idx,
                        workspace, stream, out, with_entropy)


def _lce_forward(f32, X, W, targets, label_smoothing, reduce_loss, ignore_idx, workspace,
                 stream, out, with_entropy, logit_scale=1.0):
    _check_linear(X, W, targets, torch.float32 if f32 else torch.bfloat16)
    M, H = X.shape
    V = W.shape[0]
    dev = X.device
    if workspace is None:
        workspace = lce_workspace(M, H, V, dev, f32)
    if out is None:
        loss_tok = torch.empty(M, dtype=torch.float32, device=dev)
        stats = torch.empty((M, 4), dtype=torch.float32, device=dev)
        loss_mean = torch.empty((), dtype=torch.float32, device=dev) if reduce_loss else None
        n_valid = torch.empty((), dtype=torch.int32, device=dev) if reduce_loss else None
        ent = torch.empty(M, dtype=torch.float32, device=dev) if with_entropy else None
    else:
        loss_tok, loss_mean, stats, n_valid = out[:4]
        ent = out[4] if with_entropy else None
    _check_rows(M, X, stats=stats, n_valid=n_valid, loss_tok=loss_tok, loss_mean=loss_mean,
                entropy=ent)
    _check_buf(workspace, "workspace", workspace.numel(), torch.uint8, like=X)
    _need_cuda(X, W, targets)
    if logit_scale != 1.0:
        name = "lce_forward_scaled"
        rc = lib().lce_forward_scaled(_ptr(X), _ptr(W), M, H, V, float(logit_scale),
                                      _ptr(targets), float(label_smoothing),
                                      int(bool(reduce_loss)), int(ignore_idx), _ptr(loss_tok),
                                      _ptr(loss_mean), _ptr(stats), _ptr(n_valid), _ptr(ent),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    else:
        name = "lce_forward_f32" if f32 else "lce_forward"
        rc = getattr(lib(), name)(_ptr(X), _ptr(W), M, H, V, _ptr(targets),
                                  float(label_smoothing), int(bool(reduce_loss)),
                                  int(ignore_idx), _ptr(loss_tok), _ptr(loss_mean), _ptr(stats),
                                  _ptr(n_valid), _ptr(ent), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    _check(name, rc)
    if with_entropy:
        return loss_tok, loss_mean, stats, n_valid, ent
    return loss_tok, loss_mean, stats, n_valid


def lce_backward(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, stats: torch.Tensor,
                 n_valid: torch.Tensor | None, grad_output: torch.Tensor,
                 label_smoothing: float = 0.0, reduce_loss: bool = True, ignore_idx: int = -100,
                 *, workspace: torch.Tensor | None = None, dX: torch.Tensor | None = None,
                 dW: torch.Tensor | None = None, stream=None, entropy: torch.Tensor | None = None,
                 grad_entropy: torch.Tensor | None = None, logit_scale: float = 1.0):
    """Fused linear cross-entropy backward.  Returns (dX, dW), BF16.  With
    ``grad_entropy`` the entropy's gradient is added (``entropy``: the
    forward's entropy output).  ``logit_scale``: as given to the forward."""
    return _lce_backward(False, X, W, targets, stats, n_valid, grad_output, label_smoothing,
                         reduce_loss, ignore_idx, workspace, dX, dW, stream, entropy,
                         grad_entropy, logit_scale)


def lce_backward_f32(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                     stats: torch.Tensor, n_valid: torch.Tensor | None,
                     grad_output: torch.Tensor, label_smoothing: float = 0.0,
                     reduce_loss: bool = True, ignore_idx: int = -100, *,
                     workspace: torch.Tensor | None = None, dX: torch.Tensor | None = None,
                     dW: torch.Tensor | None = None, stream=None,
                     entropy: torch.Tensor | None = None,
                     grad_entropy: torch.Tensor | None = None):
    """As ``lce_backward`` for FP32 X and W; (dX, dW) FP32."""
    return _lce_backward(True, X, W, targets, stats, n_valid, grad_output, label_smoothing,
                         reduce_loss, ignore_idx, workspace, dX, dW, stream, entropy,
                         grad_entropy)


def _lce_backward(f32, X, W, targets, stats, n_valid, grad_output, label_smoothing,
                  reduce_loss, ignore_idx, workspace, dX, dW, stream, entropy, grad_entropy,
                  logit_scale=1.0):
    _check_linear(X, W, targets, torch.float32 if f32 else torch.bfloat16)
    M, H = X.shape
    V = W.shape[0]
    if workspace is None:
        workspace = lce_workspace(M, H, V, X.device, f32)
    dX = torch.empty_like(X) if dX is None else dX
    dW = torch.empty_like(W) if dW is None else dW
    _check_rows(M, X, stats=stats, n_valid=n_valid if reduce_loss else None,
                grad_output=grad_output, reduce_loss=reduce_loss, entropy=entropy,
                grad_entropy=grad_entropy)
    _check_like(dX, "dX", X)
    _check_like(dW, "dW", W)
    _check_buf(workspace, "workspace", workspace.numel(), torch.uint8, like=X)
    _need_cuda(X, W, targets, stats, grad_output)
    if logit_scale != 1.0:
        name = "lce_backward_scaled"
        rc = lib().lce_backward_scaled(_ptr(X), _ptr(W), M, H, V, float(logit_scale),
                                       _ptr(targets), _ptr(stats), _ptr(n_valid),
                                       _ptr(grad_output), _ptr(entropy), _ptr(grad_entropy),
                                       float(label_smoothing), int(bool(reduce_loss)),
                                       int(ignore_idx), _ptr(dX), _ptr(dW), _ptr(workspace),
                                       workspace.numel(), _stream(stream))
    else:
        name = "lce_backward_f32" if f32 else "lce_backward"
        rc = getattr(lib(), name)(_ptr(X), _ptr(W), M, H, V, _ptr(targets), _ptr(stats),
                                  _ptr(n_valid), _ptr(grad_output), _ptr(entropy),
                                  _ptr(grad_entropy), float(label_smoothing),
                                  int(bool(reduce_loss)), int(ignore_idx), _ptr(dX), _ptr(dW),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check(name, rc)
    return dX, dW


def lce_forward_shard(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, vocab_start: int,
                      ignore_idx: int = -100, *, workspace: torch.Tensor | None = None,
                      stream=None, out=None, with_entropy: bool = False, out_w=None,
                      logit_scale: float = 1.0):
    """Partial statistics (M, 4) of the vocabulary shard W (V_local, H) holding
    rows vocab_start .. vocab_start + V_local - 1 of the full classifier; with
    ``with_entropy`` also its entropy statistic (M), returned second.  With
    ``logit_scale`` s the shard's logits are s X W^T
    (``lce_forward_shard_scaled``); every shard and the backward take the
    same s."""
    _check_linear(X, W, targets)
    M, H = X.shape
    V = W.shape[0]
    if workspace is None:
        workspace = lce_workspace(M, H, V, X.device)
    part = torch.empty((M, 4), dtype=torch.float32, device=X.device) if out is None else out
    pw = None
    if with_entropy:
        pw = torch.empty(M, dtype=torch.float32, device=X.device) if out_w is None else out_w
    _check_buf(part, "partial", 4 * M, like=X)
    _check_buf(pw, "partial_w", M, like=X)
    _need_cuda(X, W, targets)
    if logit_scale != 1.0:
        name = "lce_forward_shard_scaled"
        rc = lib().lce_forward_shard_scaled(_ptr(X), _ptr(W), M, H, V, float(logit_scale),
                                            _ptr(targets), int(vocab_start), int(ignore_idx),
                                            _ptr(part), _ptr(pw), _ptr(workspace),
                                            workspace.numel(), _stream(stream))
    else:
        name = "lce_forward_shard"
        rc = lib().lce_forward_shard(_ptr(X), _ptr(W), M, H, V, _ptr(targets), int(vocab_start),
                                     int(ignore_idx), _ptr(part), _ptr(pw), _ptr(workspace),
                                     workspace.numel(), _stream(stream))
    _check(name, rc)
    return (part, pw) if with_entropy else part


def lce_backward_shard(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, vocab_start: int,
                       V: int, stats: torch.Tensor, n_valid: torch.Tensor | None,
                       grad_output: torch.Tensor, label_smoothing: float = 0.0,
                       reduce_loss: bool = True, ignore_idx: int = -100, *,
                       workspace: torch.Tensor | None = None, dX: torch.Tensor | None = None,
                       dW: torch.Tensor | None = None, stream=None,
                       entropy: torch.Tensor | None = None,
                       grad_entropy: torch.Tensor | None = None,
                       logit_scale: float = 1.0):
    """(dX share, dW) of one vocabulary shard from the merged ``stats``; the
    shards' dX shares sum to the full dX.  ``entropy``, ``grad_entropy`` as in
    ``ce_backward_shard``; ``logit_scale`` as given to ``lce_forward_shard``
    (``lce_backward_shard_scaled``)."""
    _check_linear(X, W, targets)
    M, H = X.shape
    VL = W.shape[0]
    if workspace is None:
        workspace = lce_workspace(M, H, VL, X.device)
    dX = torch.empty_like(X) if dX is None else dX
    dW = torch.empty_like(W) if dW is None else dW
    _check_rows(M, X, stats=stats, n_valid=n_valid if reduce_loss else None,
                grad_output=grad_output, reduce_loss=reduce_loss, entropy=entropy,
                grad_entropy=grad_entropy)
    _check_like(dX, "dX", X)
    _check_like(dW, "dW", W)
    _need_cuda(X, W, targets, stats, grad_output)
    if logit_scale != 1.0:
        name = "lce_backward_shard_scaled"
        rc = lib().lce_backward_shard_scaled(_ptr(X), _ptr(W), M, H, VL, float(logit_scale),
                                             _ptr(targets), int(vocab_start), int(V),
                                             _ptr(stats), _ptr(n_valid), _ptr(grad_output),
                                             _ptr(entropy), _ptr(grad_entropy),
                                             float(label_smoothing), int(bool(reduce_loss)),
                                             int(ignore_idx), _ptr(dX), _ptr(dW),
                                             _ptr(workspace), workspace.numel(), _stream(stream))
    else:
        name = "lce_backward_shard"
        rc = lib().lce_backward_shard(_ptr(X), _ptr(W), M, H, VL, _ptr(targets),
                                      int(vocab_start), int(V), _ptr(stats), _ptr(n_valid),
                                      _ptr(grad_output), _ptr(entropy), _ptr(grad_entropy),
                                      float(label_smoothing), int(bool(reduce_loss)),
                                      int(ignore_idx), _ptr(dX), _ptr(dW), _ptr(workspace),
                                      workspace.numel(), _stream(stream))
    _check(name, rc)
    return dX, dW


def gemm_bf16(P: torch.Tensor, Q: torch.Tensor, K: int | None = None, *, p_dim: bool = False,
              q_dim: bool = False, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """C[i, j] = sum_k P(i, k) Q(j, k) with the library's matrix-core GEMM.

    P is (rows, K) K-contiguous, or with ``p_dim`` (K, rows) holding P(i, k) at
    [k, i]; likewise Q with ``q_dim``.  BF16, row-major, unit inner stride."""
    _need_cuda(P, Q)
    rows = P.shape[1] if p_dim else P.shape[0]
    cols = Q.shape[1] if q_dim else Q.shape[0]
    if K is None:
        K = P.shape[0] if p_dim else P.shape[1]
    C = torch.empty((rows, cols), dtype=torch.float32, device=P.device) if out is None else out
    rc = lib().vce_gemm_bf16(_ptr(P), P.stride(0), int(p_dim), _ptr(Q), Q.stride(0), int(q_dim),
                             rows, cols, K, _ptr(C), C.stride(0), _stream(stream))
    _check("vce_gemm_bf16", rc)
    return C
