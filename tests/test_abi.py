"""Host-side checks of the C-ABI (no GPU needed, no kernel is launched).

Every call below is rejected by argument validation before any HIP call, so
it runs on a machine without a GPU.  Fake device addresses are never
dereferenced.
"""
import ctypes
import os
import re

import pytest

from vocabulary_cross_entropy_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vce.h")

A = 0x7F0000000000  # a fake, 256-byte aligned device address (never touched)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from vocabulary_cross_entropy_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ce_forward", "ce_backward", "lce_forward", "lce_backward", "lce_workspace_size",
              "vce_strerror", "vce_gemm_bf16", "vce_transpose_bf16"):
        assert n in names
    assert set(names) == set(binding.SIGNATURES), "binding and header disagree"


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_strerror(L):
    for code, name in binding.STATUS.items():
        assert L.vce_strerror(code)
    assert L.vce_strerror(0) == b"success"
    assert L.vce_strerror(99) == b"unknown status"


def fwd(L, logits=A, dtype=1, d0=2, d1=3, V=1000, ls0=3000, ls1=1000, targets=A, ts0=3, ts1=1,
        eps=0.0, reduce_loss=0, ignore=-100, loss_tok=A, loss_mean=A, stats=A, n_valid=A):
    return L.ce_forward(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, eps, reduce_loss,
                        ignore, loss_tok, loss_mean, stats, n_valid, None)


def bwd(L, logits=A, grad=A + (1 << 30), dtype=1, d0=2, d1=3, V=1000, ls0=3000, ls1=1000, targets=A,
        ts0=3, ts1=1, stats=A, n_valid=A, go=A, eps=0.0, reduce_loss=0, ignore=-100, overwrite=0):
    return L.ce_backward(logits, grad, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, stats, n_valid,
                         go, eps, reduce_loss, ignore, overwrite, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(V=0), 1), (dict(d0=-1), 1), (dict(ls1=-5), 1), (dict(ts0=-1), 1),
    (dict(eps=1.5), 1), (dict(eps=-0.1), 1), (dict(eps=float("nan")), 1),
    (dict(reduce_loss=2), 1),
    (dict(logits=None), 1), (dict(targets=None), 1), (dict(loss_tok=None), 1), (dict(stats=None), 1),
    (dict(reduce_loss=1, loss_mean=None), 1), (dict(reduce_loss=1, n_valid=None), 1),
    (dict(logits=A + 1), 3), (dict(dtype=0, logits=A + 2), 3), (dict(targets=A + 4), 3),
    (dict(stats=A + 4), 3),
    (dict(d0=1 << 32, d1=1 << 32), 1),
    (dict(d0=1 << 20, d1=1 << 12), 1),  # N above INT32_MAX rows
])
def test_ce_forward_rejects(L, kw, code):
    assert fwd(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 2), (dict(V=-3), 1), (dict(eps=2.0), 1), (dict(overwrite=2), 1),
    (dict(grad=None), 1), (dict(stats=None), 1), (dict(go=None), 1),
    (dict(reduce_loss=1, n_valid=None), 1),
    (dict(overwrite=1), 4),                     # in place but grad != logits
    (dict(grad=A + 4096), 4),                   # separate buffers that overlap
    (dict(grad=A + (1 << 30) + 2), 3),          # rows would split at different 16-byte boundaries
    (dict(stats=A + 8), 3),
])
def test_ce_backward_rejects(L, kw, code):
    assert bwd(L, **kw) == code


def test_lce_workspace_size(L):
    assert L.lce_workspace_size(0, 8, 8) >= 0
    assert L.lce_workspace_size(-1, 8, 8) == 0
    assert L.lce_workspace_size(4, 0, 8) == 0
    assert L.lce_workspace_size(4, 8, 0) == 0
    small = L.lce_workspace_size(4096, 4096, 131072)
    big = L.lce_workspace_size(16384, 2304, 256003)
    assert 0 < small < big
    # the workspace holds no logit matrix: a third of one BF16 (M, V) matrix at most
    assert big < 16384 * 256003 * 2 // 3


def lfwd(L, X=A, W=A, M=64, H=64, V=1000, targets=A, eps=0.0, reduce_loss=1, ignore=-100,
         loss_tok=A, loss_mean=A, stats=A, n_valid=A, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_size(max(M, 0), H, V)
    return L.lce_forward(X, W, M, H, V, targets, eps, reduce_loss, ignore, loss_tok, loss_mean,
                         stats, n_valid, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(H=0), 1), (dict(V=0), 1), (dict(eps=3.0), 1),
    (dict(H=12), 7),
    (dict(X=None), 1), (dict(W=None), 1), (dict(targets=None), 1), (dict(ws=None), 1),
    (dict(X=A + 8), 3), (dict(W=A + 2), 3), (dict(ws=A + 16), 3),
    (dict(ws_bytes=1), 5),
    (dict(reduce_loss=1, loss_mean=None), 1), (dict(stats=A + 4), 3),
])
def test_lce_forward_rejects(L, kw, code):
    assert lfwd(L, **kw) == code


def test_lce_backward_rejects(L):
    ws = L.lce_workspace_size(64, 64, 1000)

    def call(**kw):
        a = dict(X=A, W=A, M=64, H=64, V=1000, targets=A, stats=A, n_valid=A, go=A, eps=0.0,
                 reduce_loss=1, ignore=-100, dX=A, dW=A, ws=A, ws_bytes=ws)
        a.update(kw)
        return L.lce_backward(a["X"], a["W"], a["M"], a["H"], a["V"], a["targets"], a["stats"],
                              a["n_valid"], a["go"], a["eps"], a["reduce_loss"], a["ignore"],
                              a["dX"], a["dW"], a["ws"], a["ws_bytes"], None)

    assert call(dW=None) == 1
    assert call(dX=None) == 1
    assert call(dX=A + 2) == 3
    assert call(ws_bytes=ws - 1) == 5
    assert call(reduce_loss=1, n_valid=None) == 1
    assert call(H=20) == 7


def test_gemm_rejects(L):
    g = L.vce_gemm_bf16
    assert g(A, 64, A, 64, 10, 10, 12, A, 10, None) == 7      # K not a multiple of 8
    assert g(A, 64, A, 64, 10, 10, 64, A, 5, None) == 1       # ldc < cols
    assert g(A, 32, A, 64, 10, 10, 64, A, 10, None) == 1      # ldp < K
    assert g(A + 2, 64, A, 64, 10, 10, 64, A, 10, None) == 3
    assert g(A, 64, A, 1 << 23, 10, 10, 64, A, 10, None) == 7  # leading dim too large
    assert g(A, 64, A, 64, 0, 10, 64, A, 10, None) == 0       # empty: nothing to do


def test_transpose_rejects(L):
    t = L.vce_transpose_bf16
    assert t(A, 10, 20, 16, A + (1 << 20), 16, None) == 1     # ld_src < cols
    assert t(A, 10, 20, 24, A + (1 << 20), 8, None) == 1      # ld_dst < rows
    assert t(A, 10, 20, 20, A + (1 << 20), 16, None) == 3     # ld_src not a multiple of 8
    assert t(A + 2, 10, 20, 24, A + (1 << 20), 16, None) == 3
    assert t(A, 10, 20, 24, A + 64, 16, None) == 4            # overlapping buffers
    assert t(A, 0, 20, 24, A + (1 << 20), 16, None) == 0
