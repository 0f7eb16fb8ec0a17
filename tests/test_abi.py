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
              "vce_strerror", "vce_gemm_bf16"):
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
        eps=0.0, reduce_loss=0, ignore=-100, loss_tok=A, loss_mean=A, stats=A, n_valid=A,
        entropy=None):
    return L.ce_forward(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, eps, reduce_loss,
                        ignore, loss_tok, loss_mean, stats, n_valid, entropy, None)


def bwd(L, logits=A, grad=A + (1 << 30), dtype=1, d0=2, d1=3, V=1000, ls0=3000, ls1=1000, targets=A,
        ts0=3, ts1=1, stats=A, n_valid=A, go=A, eps=0.0, reduce_loss=0, ignore=-100, overwrite=0,
        entropy=None, grad_entropy=None):
    return L.ce_backward(logits, grad, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, stats, n_valid,
                         go, entropy, grad_entropy, eps, reduce_loss, ignore, overwrite, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(V=0), 1), (dict(d0=-1), 1), (dict(ls1=-5), 1), (dict(ts0=-1), 1),
    (dict(eps=1.5), 1), (dict(eps=-0.1), 1), (dict(eps=float("nan")), 1),
    (dict(reduce_loss=2), 1),
    (dict(logits=None), 1), (dict(targets=None), 1), (dict(loss_tok=None), 1), (dict(stats=None), 1),
    (dict(reduce_loss=1, loss_mean=None), 1), (dict(reduce_loss=1, n_valid=None), 1),
    (dict(logits=A + 1), 3), (dict(dtype=0, logits=A + 2), 3), (dict(targets=A + 4), 3),
    (dict(stats=A + 4), 3), (dict(entropy=A + 2), 3),
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
    (dict(grad_entropy=A), 1),                  # entropy gradient without the entropy
    (dict(entropy=A, grad_entropy=A + 2), 3),
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
         loss_tok=A, loss_mean=A, stats=A, n_valid=A, entropy=None, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_size(max(M, 0), H, V)
    return L.lce_forward(X, W, M, H, V, targets, eps, reduce_loss, ignore, loss_tok, loss_mean,
                         stats, n_valid, entropy, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(H=0), 1), (dict(V=0), 1), (dict(eps=3.0), 1),
    (dict(H=12), 7),
    (dict(X=None), 1), (dict(W=None), 1), (dict(targets=None), 1), (dict(ws=None), 1),
    (dict(X=A + 8), 3), (dict(W=A + 2), 3), (dict(ws=A + 16), 3),
    (dict(ws_bytes=1), 5),
    (dict(reduce_loss=1, loss_mean=None), 1), (dict(stats=A + 4), 3), (dict(entropy=A + 1), 3),
])
def test_lce_forward_rejects(L, kw, code):
    assert lfwd(L, **kw) == code


def test_lce_backward_rejects(L):
    ws = L.lce_workspace_size(64, 64, 1000)

    def call(**kw):
        a = dict(X=A, W=A, M=64, H=64, V=1000, targets=A, stats=A, n_valid=A, go=A, ent=None,
                 gent=None, eps=0.0, reduce_loss=1, ignore=-100, dX=A, dW=A, ws=A, ws_bytes=ws)
        a.update(kw)
        return L.lce_backward(a["X"], a["W"], a["M"], a["H"], a["V"], a["targets"], a["stats"],
                              a["n_valid"], a["go"], a["ent"], a["gent"], a["eps"],
                              a["reduce_loss"], a["ignore"], a["dX"], a["dW"], a["ws"],
                              a["ws_bytes"], None)

    assert call(dW=None) == 1
    assert call(dX=None) == 1
    assert call(dX=A + 2) == 3
    assert call(ws_bytes=ws - 1) == 5
    assert call(reduce_loss=1, n_valid=None) == 1
    assert call(H=20) == 7
    assert call(gent=A) == 1            # entropy gradient without the entropy
    assert call(ent=A, gent=A + 2) == 3


def test_lce_workspace_size_f32(L):
    assert L.lce_workspace_size_f32(-1, 8, 8) == 0
    assert L.lce_workspace_size_f32(4, 12, 8) == 0
    M, H, V = 4096, 4096, 131072
    f32 = L.lce_workspace_size_f32(M, H, V)
    # BF16 hi and lo planes of X and W (4 (M + V) H bytes) come on top of the
    # BF16 form's partials, and dZ takes two planes instead of one
    assert f32 >= 4 * (M + V) * H + L.lce_workspace_size(M, H, V) - M * H * 4


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(eps=-0.5), 1), (dict(H=12), 7),
    (dict(X=None), 1), (dict(W=A + 4), 3), (dict(ws=A + 128), 3), (dict(ws_bytes=1), 5),
    (dict(reduce_loss=2), 1), (dict(stats=A + 8), 3),
])
def test_lce_forward_f32_rejects(L, kw, code):
    a = dict(X=A, W=A, M=64, H=64, V=1000, targets=A, eps=0.0, reduce_loss=1, ignore=-100,
             loss_tok=A, loss_mean=A, stats=A, n_valid=A, entropy=None, ws=A, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = L.lce_workspace_size_f32(max(a["M"], 0), a["H"], a["V"])
    assert L.lce_forward_f32(a["X"], a["W"], a["M"], a["H"], a["V"], a["targets"], a["eps"],
                             a["reduce_loss"], a["ignore"], a["loss_tok"], a["loss_mean"],
                             a["stats"], a["n_valid"], a["entropy"], a["ws"], a["ws_bytes"],
                             None) == code


def test_lce_backward_f32_rejects(L):
    ws = L.lce_workspace_size_f32(64, 64, 1000)
    assert ws > L.lce_workspace_size(64, 64, 1000)

    def call(**kw):
        a = dict(X=A, W=A, M=64, H=64, V=1000, targets=A, stats=A, n_valid=A, go=A, ent=None,
                 gent=None, eps=0.0, reduce_loss=1, ignore=-100, dX=A, dW=A, ws=A, ws_bytes=ws)
        a.update(kw)
        return L.lce_backward_f32(a["X"], a["W"], a["M"], a["H"], a["V"], a["targets"],
                                  a["stats"], a["n_valid"], a["go"], a["ent"], a["gent"],
                                  a["eps"], a["reduce_loss"], a["ignore"], a["dX"], a["dW"],
                                  a["ws"], a["ws_bytes"], None)

    assert call(dW=None) == 1
    assert call(dX=A + 4) == 3
    assert call(dW=A + 8) == 3
    # the BF16 form's workspace is too small for the FP32 form
    assert call(ws_bytes=L.lce_workspace_size(64, 64, 1000)) == 5
    assert call(gent=A) == 1
    assert call(H=20) == 7


def test_gemm_rejects(L):
    g = L.vce_gemm_bf16

    def call(P=A, ldp=64, p_dim=0, Q=A, ldq=64, q_dim=0, rows=10, cols=10, K=64, C=A, ldc=10):
        return g(P, ldp, p_dim, Q, ldq, q_dim, rows, cols, K, C, ldc, None)

    assert call(K=12) == 7                          # K-contiguous operand, K not a multiple of 8
    # K need not be a multiple of 8 when both operands are dim-contiguous: the
    # call gets as far as the (last) alignment check
    assert call(P=A + 2, p_dim=1, q_dim=1, K=12, rows=16, cols=16, ldc=16) == 3
    assert call(p_dim=1) == 7                       # dim-contiguous P needs rows % 8 == 0
    assert call(q_dim=1, rows=16, ldc=16) == 7      # dim-contiguous Q needs cols % 8 == 0
    assert call(p_dim=2) == 1
    assert call(ldc=5) == 1                         # ldc < cols
    assert call(ldp=32) == 1                        # ldp < K
    assert call(p_dim=1, rows=16, ldp=8) == 1       # ldp < rows for a dim-contiguous P
    assert call(P=A + 2) == 3
    assert call(ldq=1 << 23) == 7                   # leading dimension too large
    assert call(rows=0) == 0                        # empty: nothing to do


def fshard(L, logits=A, dtype=1, d0=2, d1=3, V=1000, ls0=3000, ls1=1000, targets=A, ts0=3, ts1=1,
           v0=0, ignore=-100, partial=A, partial_w=None):
    return L.ce_forward_shard(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, v0, ignore,
                              partial, partial_w, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), 2), (dict(V=0), 1), (dict(v0=-1), 1), (dict(v0=(1 << 63) - 10), 1),
    (dict(partial=None), 1), (dict(logits=None), 1), (dict(partial=A + 8), 3),
    (dict(logits=A + 1), 3), (dict(d0=1 << 20, d1=1 << 12), 1), (dict(partial_w=A + 2), 3),
])
def test_ce_forward_shard_rejects(L, kw, code):
    assert fshard(L, **kw) == code


def test_ce_forward_shard_empty_is_a_no_op(L):
    assert fshard(L, d0=0, partial=None) == 0


def merge(L, partials=A, k=4, d0=2, d1=3, targets=A, ts0=3, ts1=1, V=1000, eps=0.0,
          reduce_loss=0, ignore=-100, loss_tok=A, loss_mean=A, stats=A, n_valid=A,
          partials_w=None, entropy=None):
    return L.ce_merge_shards(partials, partials_w, k, d0, d1, targets, ts0, ts1, V, eps,
                             reduce_loss, ignore, loss_tok, loss_mean, stats, n_valid, entropy,
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1), (dict(V=0), 1), (dict(d1=-1), 1), (dict(ts1=-1), 1), (dict(eps=1.01), 1),
    (dict(reduce_loss=3), 1), (dict(reduce_loss=1, loss_mean=None), 1),
    (dict(reduce_loss=1, n_valid=None), 1), (dict(partials=None), 1), (dict(stats=None), 1),
    (dict(loss_tok=None), 1), (dict(targets=None), 1),
    (dict(partials=A + 4), 3), (dict(stats=A + 8), 3), (dict(targets=A + 4), 3),
    (dict(k=1 << 40, d0=1 << 15, d1=1 << 15), 1),
    (dict(entropy=A), 1),                         # entropy without the shards' statistics
    (dict(entropy=A + 2, partials_w=A), 3), (dict(entropy=A, partials_w=A + 1), 3),
])
def test_ce_merge_shards_rejects(L, kw, code):
    assert merge(L, **kw) == code


def bshard(L, logits=A, grad=A + (1 << 30), dtype=1, d0=2, d1=3, VL=1000, ls0=3000, ls1=1000,
           targets=A, ts0=3, ts1=1, v0=0, V=8000, stats=A, n_valid=A, go=A, ent=None, gent=None,
           eps=0.0, reduce_loss=0, ignore=-100, overwrite=0):
    return L.ce_backward_shard(logits, grad, dtype, d0, d1, VL, ls0, ls1, targets, ts0, ts1, v0, V,
                               stats, n_valid, go, ent, gent, eps, reduce_loss, ignore, overwrite,
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2), (dict(VL=0), 1), (dict(v0=-1), 1), (dict(V=999), 1),
    (dict(v0=7001), 1),                          # the shard would end past the vocabulary
    (dict(eps=-1.0), 1), (dict(overwrite=3), 1), (dict(grad=None), 1), (dict(stats=None), 1),
    (dict(go=None), 1), (dict(reduce_loss=1, n_valid=None), 1),
    (dict(overwrite=1), 4), (dict(grad=A + 4096), 4), (dict(grad=A + (1 << 30) + 2), 3),
    (dict(stats=A + 4), 3), (dict(gent=A), 1), (dict(ent=A, gent=A + 2), 3),
])
def test_ce_backward_shard_rejects(L, kw, code):
    assert bshard(L, **kw) == code


def test_lce_shard_rejects(L):
    ws = L.lce_workspace_size(64, 64, 1000)

    def fwd_(**kw):
        a = dict(X=A, W=A, M=64, H=64, VL=1000, targets=A, v0=0, ignore=-100, part=A, pw=None,
                 ws=A, ws_bytes=ws)
        a.update(kw)
        return L.lce_forward_shard(a["X"], a["W"], a["M"], a["H"], a["VL"], a["targets"], a["v0"],
                                   a["ignore"], a["part"], a["pw"], a["ws"], a["ws_bytes"], None)

    assert fwd_(v0=-1) == 1
    assert fwd_(part=None) == 1
    assert fwd_(part=A + 4) == 3
    assert fwd_(H=12) == 7
    assert fwd_(ws_bytes=ws - 1) == 5
    assert fwd_(X=A + 2) == 3
    assert fwd_(M=0, part=None) == 0
    assert fwd_(pw=A + 1) == 3

    def bwd_(**kw):
        a = dict(X=A, W=A, M=64, H=64, VL=1000, targets=A, v0=0, V=4000, stats=A, n_valid=A,
                 go=A, ent=None, gent=None, eps=0.0, reduce_loss=1, ignore=-100, dX=A, dW=A,
                 ws=A, ws_bytes=ws)
        a.update(kw)
        return L.lce_backward_shard(a["X"], a["W"], a["M"], a["H"], a["VL"], a["targets"],
                                    a["v0"], a["V"], a["stats"], a["n_valid"], a["go"], a["ent"],
                                    a["gent"], a["eps"], a["reduce_loss"], a["ignore"], a["dX"],
                                    a["dW"], a["ws"], a["ws_bytes"], None)

    assert bwd_(V=999) == 1
    assert bwd_(v0=3001) == 1
    assert bwd_(v0=-2) == 1
    assert bwd_(dW=None) == 1
    assert bwd_(dX=None) == 1
    assert bwd_(stats=A + 4) == 3
    assert bwd_(n_valid=A + 2) == 3
    assert bwd_(ws_bytes=ws - 1) == 5
    assert bwd_(eps=2.0) == 1
    assert bwd_(gent=A) == 1
    assert bwd_(ent=A + 2, gent=A) == 3


def test_shift_targets_rejects(L):
    s = L.vce_shift_targets

    def call(targets=A, d0=2, d1=8, ts0=8, ts1=1, axis=1, ignore=-100, out=A + (1 << 20)):
        return s(targets, d0, d1, ts0, ts1, axis, ignore, out, None)

    assert call(axis=2) == 1
    assert call(d0=-1) == 1
    assert call(ts1=-1) == 1
    assert call(targets=None) == 1
    assert call(out=None) == 1
    assert call(targets=A + 4) == 3
    assert call(out=A + 8) == 4           # overlaps the targets it reads
    assert call(d0=0, targets=None, out=None) == 0


def test_ce_forward_backward_rejects(L):
    def call(**kw):
        a = dict(logits=A, grad=A + (1 << 30), dtype=1, d0=2, d1=3, V=1000, ls0=3000, ls1=1000,
                 targets=A, ts0=3, ts1=1, go=A, eps=0.0, reduce_loss=1, ignore=-100,
                 overwrite=0, loss_tok=A, loss_mean=A, stats=A, n_valid=A)
        a.update(kw)
        return L.ce_forward_backward(a["logits"], a["grad"], a["dtype"], a["d0"], a["d1"],
                                     a["V"], a["ls0"], a["ls1"], a["targets"], a["ts0"],
                                     a["ts1"], a["go"], a["eps"], a["reduce_loss"], a["ignore"],
                                     a["overwrite"], a["loss_tok"], a["loss_mean"], a["stats"],
                                     a["n_valid"], None)

    assert call(dtype=4) == 2
    assert call(V=0) == 1
    assert call(eps=1.5) == 1
    assert call(overwrite=2) == 1
    assert call(reduce_loss=1, loss_mean=None) == 1
    assert call(go=None) == 1
    assert call(grad=None) == 1
    assert call(stats=None) == 1
    assert call(stats=A + 4) == 3
    assert call(go=A + 2) == 3
    assert call(overwrite=1) == 4                   # overwrite needs grad == logits
    assert call(grad=A + 4096) == 4                 # overlapping buffers
    assert call(grad=A + (1 << 30) + 2) == 3        # rows split at different 16 B phases


def noalloc(L, X=A, W=A, M=64, H=64, V=1000, targets=A, eps=0.0, reduce_loss=0, ignore=-100,
            loss_tok=A, loss_mean=A, stats=A, n_valid=A, entropy=None):
    return L.lce_forward_noalloc(X, W, M, H, V, targets, eps, reduce_loss, ignore, loss_tok,
                                 loss_mean, stats, n_valid, entropy, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(V=0), 1), (dict(eps=2.0), 1), (dict(H=12), 7),
    (dict(X=None), 1), (dict(targets=None), 1), (dict(stats=None), 1),
    (dict(X=A + 8), 3), (dict(stats=A + 4), 3),
    # the forward's partials beyond the 64 MiB static scratch: 16 * 1001 tiles * 16384
    (dict(M=16384, H=2304, V=256003), 8),
    # just past the limit: 16 * 1025 * 4096 + 4 * 4096 bytes > 64 MiB
    (dict(M=4096, H=64, V=262145), 8),
])
def test_lce_forward_noalloc_rejects(L, kw, code):
    # every rejection comes from the host checks: nothing is launched and the
    # static scratch is not looked up
    assert noalloc(L, **kw) == code
    assert L.vce_strerror(code)


@pytest.mark.parametrize("scale,code", [
    (0.0, 1), (-1.0, 1), (float("nan"), 1), (float("inf"), 1),
])
def test_lce_scaled_reject_a_bad_scale(L, scale, code):
    # logit_scale must be finite and > 0; checked before anything else
    ws = L.lce_workspace_size(64, 64, 1000)
    assert L.lce_forward_scaled(A, A, 64, 64, 1000, scale, A, 0.0, 1, -100, A, A, A, A, None, A,
                                ws, None) == code
    assert L.lce_backward_scaled(A, A, 64, 64, 1000, scale, A, A, A, A, None, None, 0.0, 1, -100,
                                 A, A, A, ws, None) == code


def test_lce_scaled_share_the_other_checks(L):
    ws = L.lce_workspace_size(64, 64, 1000)
    assert L.lce_forward_scaled(A, A, 64, 12, 1000, 0.5, A, 0.0, 1, -100, A, A, A, A, None, A,
                                ws, None) == 7
    assert L.lce_forward_scaled(A, A, 64, 64, 1000, 0.5, A, 0.0, 1, -100, A, A, A, A, None, A,
                                1, None) == 5
    assert L.lce_backward_scaled(A, A, 64, 64, 1000, 2.0, A, A, A, A, None, None, 0.0, 1, -100,
                                 None, A, A, ws, None) == 1


@pytest.mark.parametrize("scale", [0.0, -2.0, float("nan"), float("inf")])
def test_lce_shard_scaled_reject_a_bad_scale(L, scale):
    ws = L.lce_workspace_size(64, 64, 1000)
    assert L.lce_forward_shard_scaled(A, A, 64, 64, 1000, scale, A, 0, -100, A, None, A, ws,
                                      None) == 1
    assert L.lce_backward_shard_scaled(A, A, 64, 64, 1000, scale, A, 0, 4000, A, A, A, None,
                                       None, 0.0, 1, -100, A, A, A, ws, None) == 1


def test_lce_shard_scaled_share_the_other_checks(L):
    ws = L.lce_workspace_size(64, 64, 1000)
    # H not a multiple of 8
    assert L.lce_forward_shard_scaled(A, A, 64, 12, 1000, 0.5, A, 0, -100, A, None, A, ws,
                                      None) == 7
    # negative vocab_start; shard beyond the full vocabulary
    assert L.lce_forward_shard_scaled(A, A, 64, 64, 1000, 0.5, A, -1, -100, A, None, A, ws,
                                      None) == 1
    assert L.lce_backward_shard_scaled(A, A, 64, 64, 1000, 0.5, A, 3500, 4000, A, A, A, None,
                                       None, 0.0, 1, -100, A, A, A, ws, None) == 1
    # workspace too small; no dW
    assert L.lce_forward_shard_scaled(A, A, 64, 64, 1000, 0.5, A, 0, -100, A, None, A, 1,
                                      None) == 5
    assert L.lce_backward_shard_scaled(A, A, 64, 64, 1000, 2.0, A, 0, 4000, A, A, A, None, None,
                                       0.0, 1, -100, A, None, A, ws, None) == 1
