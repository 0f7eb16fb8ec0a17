"""Parity of the causal label shift (vce_shift_targets) with the oracle, and of
the loss and gradients computed from shifted targets, through the C-ABI."""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from oracle.shift import shift_targets as oshift
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, assert_grad_bf16, assert_loss_close,
                          grad_terms, rel_frobenius, to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


@pytest.mark.parametrize("d0,d1", [(1, 1), (3, 1), (1, 7), (4, 1000), (1000, 3)])
@pytest.mark.parametrize("axis", [0, 1])
def test_shift_is_exact(d0, d1, axis):
    rng = np.random.default_rng(d0 * 31 + d1 + axis)
    t = rng.integers(-1, 50000, size=(d0, d1)).astype(np.int64)
    t[rng.random((d0, d1)) < 0.1] = IGN
    got = vce.shift_targets(torch.from_numpy(t).cuda(), axis).cpu().numpy()
    np.testing.assert_array_equal(got, oshift(t, axis, IGN))
    # a transposed (strided) view of the targets gives the transposed result
    tt = torch.from_numpy(np.ascontiguousarray(t.T)).cuda().t()
    np.testing.assert_array_equal(vce.shift_targets(tt, axis).cpu().numpy(), oshift(t, axis, IGN))


@pytest.mark.parametrize("layout,axis", [("B,SQ", 1), ("SQ,B", 0)])
def test_logits_with_shifted_targets(layout, axis):
    d0, d1 = (3, 300) if layout == "B,SQ" else (300, 3)
    case = wl.make_logits(41, d0, d1, 32000, dtype=wl.DTYPE_BF16, sigma=3.0, ignore_frac=0.05,
                          label_smoothing=0.1, reduce_loss=True, layout=layout)
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    ts = vce.shift_targets(t, axis)
    loss, mean, stats, nv = vce.ce_forward(z, ts, 0.1, True)
    grad = vce.ce_backward(z, ts, stats, nv, torch.ones(1, device="cuda"), 0.1, True)
    torch.cuda.synchronize()
    tsh = oshift(case.targets, axis, IGN)
    ref_loss, _, _ = oracle.ce_forward(case.logits, tsh, 0.1, IGN)
    assert_loss_close(loss.cpu().numpy(), ref_loss)
    rm = oracle.mean_loss(ref_loss, tsh, IGN)
    assert abs(mean.item() - rm) <= 1e-4 + 1e-5 * abs(rm)
    assert nv.item() == oracle.n_valid(tsh, IGN)
    g = oracle.row_scale(np.ones(1), tsh, True, IGN)
    rows = np.arange(0, case.N, 7)
    ref = oracle.ce_backward(case.logits, tsh, g, 0.1, IGN, rows=rows)
    gb = to_host_bits(grad).reshape(case.N, -1)[rows]
    assert_grad_bf16(gb, ref, grad_terms(ref, g[rows], tsh.reshape(-1)[rows], 0.1, IGN))
    last = (tsh.reshape(-1) == IGN)
    assert np.all(to_host_bits(grad).reshape(case.N, -1)[last] == 0)


def test_linear_with_shifted_targets():
    B, T = 3, 200
    case = wl.make_linear(42, B * T, 256, 5000, ignore_count=10, label_smoothing=0.0,
                          reduce_loss=True)
    X, W = to_device(case.X, "bf16"), to_device(case.W, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    ts = vce.shift_targets(t.view(B, T), 1).reshape(-1)
    loss, mean, stats, nv = vce.lce_forward(X, W, ts)
    dX, dW = vce.lce_backward(X, W, ts, stats, nv, torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    tsh = oshift(case.targets.reshape(B, T), 1, IGN).reshape(-1)
    rl, _, _ = linear.forward(case.X, case.W, tsh, 0.0, IGN)
    valid = tsh != IGN
    got = loss.cpu().numpy().astype(np.float64)
    assert np.all(got[~valid] == 0.0)
    assert np.max(np.abs(got[valid] - rl[valid]) / np.abs(rl[valid])) <= LINEAR_LOSS_RTOL
    g = oracle.row_scale(np.ones(1), tsh, True, IGN)
    rdX, rdW = linear.backward(case.X, case.W, tsh, g, 0.0, IGN)
    assert rel_frobenius(oracle.bf16_to_f64(to_host_bits(dX)), rdX) <= LINEAR_FROB_RTOL
    assert rel_frobenius(oracle.bf16_to_f64(to_host_bits(dW)), rdW) <= LINEAR_FROB_RTOL
