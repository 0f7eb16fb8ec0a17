"""Pins for the FP64 fused linear cross-entropy oracle (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import linear, tiny
from vocabulary_cross_entropy_amd import workloads as wl

IGN = -100


def _case(seed, M, H, V, n_ign=0, f64=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, H))
    W = rng.standard_normal((V, H)) / np.sqrt(H) * 2.0
    t = rng.integers(0, V, size=M).astype(np.int64)
    if n_ign:
        t[rng.choice(M, n_ign, replace=False)] = IGN
    if not f64:
        X = wl.f32_to_bf16_bits(X.astype(np.float32))
        W = wl.f32_to_bf16_bits(W.astype(np.float32))
    return X, W, t


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("reduce_loss", [False, True])
def test_against_torch_autograd_float64(eps, reduce_loss):
    # The linear CE is cross_entropy(X W^T): torch float64 autograd gives loss, dX, dW.
    X, W, t = _case(1, 12, 16, 37, n_ign=2, f64=False)
    Xt = torch.tensor(oracle.bf16_to_f64(X), requires_grad=True)
    Wt = torch.tensor(oracle.bf16_to_f64(W), requires_grad=True)
    red = "mean" if reduce_loss else "none"
    ref = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(t), ignore_index=IGN,
                                            label_smoothing=eps, reduction=red)
    go = np.array([1.5]) if reduce_loss else np.random.default_rng(1).uniform(0.5, 1.5, 12)
    ref.backward(torch.tensor(go[0] if reduce_loss else go, dtype=torch.float64))
    loss, stats, lse = linear.forward(X, W, t, eps)
    if reduce_loss:
        assert oracle.mean_loss(loss, t) == pytest.approx(ref.item(), rel=1e-12)
    else:
        np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    g = oracle.row_scale(go, t, reduce_loss)
    dX, dW = linear.backward(X, W, t, g, eps)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_finite_differences_tiny():
    # M=3, H=4, V=7: central differences of the summed loss wrt every X and W entry.
    X, W, t = _case(2, 3, 4, 7)
    eps = 0.15
    g = np.ones(3)
    dX, dW = linear.backward(X, W, t, g, eps)
    h = 1e-6

    def total(Xa, Wa):
        loss, _, _ = linear.forward(Xa, Wa, t, eps)
        return loss.sum()

    for i in range(3):
        for j in range(4):
            Xp = X.copy(); Xp[i, j] += h
            Xm = X.copy(); Xm[i, j] -= h
            assert abs((total(Xp, W) - total(Xm, W)) / (2 * h) - dX[i, j]) < 1e-7
    for v in range(7):
        for j in range(4):
            Wp = W.copy(); Wp[v, j] += h
            Wm = W.copy(); Wm[v, j] -= h
            assert abs((total(X, Wp) - total(X, Wm)) / (2 * h) - dW[v, j]) < 1e-7


def test_finite_differences_with_entropy_tiny():
    # J = sum_r g_r loss_r + gH_r H_r: its gradient is dX, dW from backward()
    # with grad_entropy (M=3, H=4, V=7, central differences)
    X, W, t = _case(4, 3, 4, 7)
    eps = 0.1
    g = np.array([1.0, 0.5, -0.25])
    gH = np.array([0.8, -1.2, 0.3])
    dX, dW = linear.backward(X, W, t, g, eps, grad_entropy=gH)
    h = 1e-6

    def total(Xa, Wa):
        loss, _, _ = linear.forward(Xa, Wa, t, eps)
        return float(np.dot(g, loss) + np.dot(gH, linear.entropy(Xa, Wa, t)))

    for i in range(3):
        for j in range(4):
            Xp = X.copy(); Xp[i, j] += h
            Xm = X.copy(); Xm[i, j] -= h
            assert abs((total(Xp, W) - total(Xm, W)) / (2 * h) - dX[i, j]) < 1e-7
    for v in range(7):
        for j in range(4):
            Wp = W.copy(); Wp[v, j] += h
            Wm = W.copy(); Wm[v, j] -= h
            assert abs((total(X, Wp) - total(X, Wm)) / (2 * h) - dW[v, j]) < 1e-7


def test_pure_python_tiny():
    X, W, t = _case(3, 2, 3, 5)
    Z = tiny.matmul_nt(X.tolist(), W.tolist())
    loss, _, _ = linear.forward(X, W, t, 0.2)
    for r in range(2):
        assert loss[r] == pytest.approx(tiny.loss_row(Z[r], int(t[r]), 0.2), rel=1e-13)


def test_invariants():
    X, W, t = _case(4, 20, 8, 31, n_ign=3)
    g = np.random.default_rng(4).uniform(0.5, 2.0, 20)
    for eps in (0.0, 0.3):
        dX, dW = linear.backward(X, W, t, g, eps)
        # every dZ row sums to zero, so the columns of dW sum to zero
        np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-12)
        # ignored tokens get no gradient
        np.testing.assert_array_equal(dX[t == IGN], 0.0)
    # all vocabulary rows equal: every logit in a row is equal, dX = sum_v dZ w = 0
    Weq = np.tile(W[:1], (31, 1))
    dX, _ = linear.backward(X, Weq, t, g, 0.1)
    np.testing.assert_allclose(dX, 0.0, atol=1e-13)
    loss, _, _ = linear.forward(X, Weq, t, 0.1)
    np.testing.assert_allclose(loss[t != IGN], np.log(31), rtol=1e-12)


def test_sampled_rows_match_full():
    X, W, t = _case(5, 40, 16, 53, n_ign=4, f64=False)
    g = oracle.row_scale(np.array([1.0]), t, True)
    eps = 0.1
    loss, stats, lse = linear.forward(X, W, t, eps)
    dX, dW = linear.backward(X, W, t, g, eps)
    rows = np.array([0, 7, 39, 3])
    l2, _, lse2 = linear.forward(X, W, t, eps, rows=rows)
    np.testing.assert_allclose(l2, loss[rows], rtol=1e-14)
    np.testing.assert_allclose(linear.dx_rows(X, W, t, g, rows, eps), dX[rows], rtol=1e-12, atol=1e-16)
    vrows = np.array([0, 52, 11])
    np.testing.assert_allclose(linear.dw_rows(X, W, t, g, lse, vrows, eps), dW[vrows],
                               rtol=1e-11, atol=1e-15)
    # token chunking only splits independent rows
    loss_c, _, _ = linear.forward(X, W, t, eps, token_chunk=7)
    np.testing.assert_array_equal(loss_c, loss)
    dXc, dWc = linear.backward(X, W, t, g, eps, token_chunk=9)
    np.testing.assert_allclose(dXc, dX, rtol=1e-14, atol=1e-18)
    np.testing.assert_allclose(dWc, dW, rtol=1e-12, atol=1e-15)


# --- FP32 inputs ------------------------------------------------------------------

def _case_f32(seed, M, H, V, n_ign=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, H)).astype(np.float32)
    W = (rng.standard_normal((V, H)) / np.sqrt(H) * 2.0).astype(np.float32)
    t = rng.integers(0, V, size=M).astype(np.int64)
    if n_ign:
        t[rng.choice(M, n_ign, replace=False)] = IGN
    return X, W, t


@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_f32_inputs_against_torch_autograd_float64(eps):
    # FP32 X and W are taken at their exact values: torch float64 autograd on
    # the widened values gives the same loss, dX and dW (a path that rounded
    # them to BF16 would be off by ~1e-3 here).
    X, W, t = _case_f32(31, 10, 24, 53, n_ign=2)
    Xt = torch.tensor(X.astype(np.float64), requires_grad=True)
    Wt = torch.tensor(W.astype(np.float64), requires_grad=True)
    ref = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(t), ignore_index=IGN,
                                            label_smoothing=eps, reduction="sum")
    ref.backward()
    loss, _, _ = linear.forward(X, W, t, eps)
    assert loss.sum() == pytest.approx(ref.item(), rel=1e-12)
    g = np.where(t == IGN, 0.0, 1.0)
    dX, dW = linear.backward(X, W, t, g, eps)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_f32_inputs_that_are_bf16_values_match_the_bf16_path():
    # FP32 arrays holding BF16-representable values give bit-identical results
    # to the BF16 bit patterns of the same values.
    Xb, Wb, t = _case(32, 9, 16, 41, n_ign=1, f64=False)
    Xf = oracle.bf16_to_f64(Xb).astype(np.float32)
    Wf = oracle.bf16_to_f64(Wb).astype(np.float32)
    lb, sb, _ = linear.forward(Xb, Wb, t, 0.1)
    lf, sf, _ = linear.forward(Xf, Wf, t, 0.1)
    np.testing.assert_array_equal(lf, lb)
    np.testing.assert_array_equal(sf[t != IGN], sb[t != IGN])
    g = np.linspace(0.5, 1.5, 9)
    for a, b in zip(linear.backward(Xf, Wf, t, g, 0.1), linear.backward(Xb, Wb, t, g, 0.1)):
        np.testing.assert_array_equal(a, b)


def test_f32_inputs_pure_python_tiny():
    X, W, t = _case_f32(33, 3, 5, 6)
    Z = tiny.matmul_nt(X.astype(np.float64).tolist(), W.astype(np.float64).tolist())
    loss, _, _ = linear.forward(X, W, t)
    for r in range(3):
        assert loss[r] == pytest.approx(tiny.loss_row(Z[r], int(t[r]), 0.0), rel=1e-13)


# --- the scaled form: logits = s X W^T --------------------------------------------

@pytest.mark.parametrize("scale", [0.7, 3.0])
@pytest.mark.parametrize("eps,reduce_loss", [(0.0, False), (0.1, True)])
def test_scaled_against_torch_autograd_float64(scale, eps, reduce_loss):
    # cross_entropy(s X W^T) by torch float64 autograd: loss, dX, dW
    X, W, t = _case(21, 12, 16, 37, n_ign=2, f64=False)
    Xt = torch.tensor(oracle.bf16_to_f64(X), requires_grad=True)
    Wt = torch.tensor(oracle.bf16_to_f64(W), requires_grad=True)
    red = "mean" if reduce_loss else "none"
    ref = torch.nn.functional.cross_entropy(scale * (Xt @ Wt.T), torch.tensor(t),
                                            ignore_index=IGN, label_smoothing=eps, reduction=red)
    go = np.array([1.5]) if reduce_loss else np.random.default_rng(2).uniform(0.5, 1.5, 12)
    ref.backward(torch.tensor(go[0] if reduce_loss else go, dtype=torch.float64))
    loss, _, _ = linear.forward(X, W, t, eps, scale=scale)
    if reduce_loss:
        assert oracle.mean_loss(loss, t) == pytest.approx(ref.item(), rel=1e-12)
    else:
        np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    g = oracle.row_scale(go, t, reduce_loss)
    dX, dW = linear.backward(X, W, t, g, eps, scale=scale)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_scaled_finite_differences_with_entropy_tiny():
    # J = sum_r g_r loss_r + gH_r H_r at logits s X W^T, central differences
    X, W, t = _case(22, 3, 4, 7)
    eps, s = 0.1, 1.7
    g = np.array([1.0, 0.5, -0.25])
    gH = np.array([0.8, -1.2, 0.3])
    dX, dW = linear.backward(X, W, t, g, eps, grad_entropy=gH, scale=s)
    h = 1e-6

    def total(Xa, Wa):
        loss, _, _ = linear.forward(Xa, Wa, t, eps, scale=s)
        return float(np.dot(g, loss) + np.dot(gH, linear.entropy(Xa, Wa, t, scale=s)))

    for i in range(3):
        for j in range(4):
            Xp = X.copy(); Xp[i, j] += h
            Xm = X.copy(); Xm[i, j] -= h
            assert abs((total(Xp, W) - total(Xm, W)) / (2 * h) - dX[i, j]) < 1e-7
    for v in range(7):
        for j in range(4):
            Wp = W.copy(); Wp[v, j] += h
            Wm = W.copy(); Wm[v, j] -= h
            assert abs((total(X, Wp) - total(X, Wm)) / (2 * h) - dW[v, j]) < 1e-7


def test_scaled_equals_unscaled_with_scaled_classifier():
    # s X W^T = X (s W)^T: the same loss and dX; dW_scaled = s dW of the unscaled
    # problem at W' = s W (chain rule), for any s > 0
    X, W, t = _case(23, 9, 8, 21, n_ign=1)
    s, eps = 2.5, 0.05
    g = np.random.default_rng(3).uniform(0.5, 1.5, 9)
    l1, st1, _ = linear.forward(X, W, t, eps, scale=s)
    l2, st2, _ = linear.forward(X, s * W, t, eps)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    np.testing.assert_allclose(st1, st2, rtol=1e-13)
    dX1, dW1 = linear.backward(X, W, t, g, eps, scale=s)
    dX2, dW2 = linear.backward(X, s * W, t, g, eps)
    np.testing.assert_allclose(dX1, dX2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dW1, s * dW2, rtol=1e-12, atol=1e-13)
