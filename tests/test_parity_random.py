"""A seeded random sweep of shapes and options through the C-ABI, every case
against the FP64 oracle.

Logits form: random (d0, d1, V), dtype, label smoothing, reduction, ignored
rows and spread of the logits, half of the cases passed as the transposed view
of the other layout's storage; forward, backward into a separate buffer and in place,
and the one-pass call (bitwise the two calls).  Linear form: random (M, H, V),
smoothing, reduction, ignored rows, with and without a logit scale; loss, dX
and dW.  The draws are fixed by the seeds, so a failure names a case that
runs again the same way."""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, assert_grad_bf16, assert_grad_fp32,
                          assert_loss_close, grad_terms, rel_frobenius, to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-random] {msg}", flush=True)


def _logits_draws(n, seed):
    rng = np.random.default_rng(seed)
    draws = []
    for i in range(n):
        V = int(np.exp(rng.uniform(0.0, np.log(70000.0))))
        d0, d1 = int(rng.integers(1, 5)), int(rng.integers(1, 17))
        N = d0 * d1
        draws.append(dict(
            i=i, V=max(V, 1), d0=d0, d1=d1,
            dtype="bf16" if rng.random() < 0.6 else "fp32",
            eps=float(rng.choice([0.0, 0.05, 0.3, 1.0])),
            red=bool(rng.random() < 0.5),
            n_ign=int(rng.integers(0, N + 1)) if rng.random() < 0.2 else int(rng.integers(0, N // 4 + 1)),
            sigma=float(rng.choice([0.5, 3.0, 12.0])),
            view=bool(rng.random() < 0.5)))
    return draws


LOGITS_DRAWS = _logits_draws(40, 9001)


@pytest.mark.parametrize("d", LOGITS_DRAWS, ids=[f"c{d['i']}-{d['dtype']}-V{d['V']}"
                                                for d in LOGITS_DRAWS])
def test_random_logits(d):
    case = wl.make_logits(9100 + d["i"], d["d0"], d["d1"], d["V"], dtype=d["dtype"],
                          sigma=d["sigma"], ignore_count=d["n_ign"], label_smoothing=d["eps"],
                          reduce_loss=d["red"], grad_output="random")
    _say(f"case {d}")
    eps, red, V = d["eps"], d["red"], d["V"]
    # the call sees (d0, d1, V); with `view` it is the transposed view of a
    # (d1, d0, V) tensor, so its leading strides are not row-major
    if d["view"]:
        z = to_device(np.ascontiguousarray(case.logits.transpose(1, 0, 2)), d["dtype"]).transpose(0, 1)
        t = torch.from_numpy(np.ascontiguousarray(case.targets.T)).cuda().transpose(0, 1)
    else:
        z = to_device(case.logits, d["dtype"])
        t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    go = go.reshape(-1) if red else go
    loss, mean, stats, nv = vce.ce_forward(z, t, eps, red, IGN)
    grad = vce.ce_backward(z, t, stats, nv, go, eps, red, IGN)
    zc = z.clone()
    grad_ip = vce.ce_backward(zc, t, stats, nv, go, eps, red, IGN, overwrite_input=True)
    fb = vce.ce_forward_backward(z, t, go, eps, red, IGN)
    torch.cuda.synchronize()

    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, eps, IGN)
    assert_loss_close(loss.cpu().numpy(), ref_loss)
    valid = (case.targets.reshape(-1) != IGN) & np.isfinite(ref_loss.reshape(-1))
    st = stats.cpu().numpy().reshape(-1, 4)[valid]
    np.testing.assert_array_equal(st[:, 0], ref_stats[valid, 0].astype(np.float32))
    np.testing.assert_array_equal(st[:, 2], ref_stats[valid, 2].astype(np.float32))
    np.testing.assert_allclose(st[:, 1], ref_stats[valid, 1], rtol=2e-5)
    if red:
        rm = oracle.mean_loss(ref_loss, case.targets, IGN)
        assert abs(mean.item() - rm) <= 1e-4 + 1e-5 * abs(rm)
        assert nv.item() == oracle.n_valid(case.targets, IGN)

    g = oracle.row_scale(case.grad_output, case.targets, red, IGN)
    ref = oracle.ce_backward(case.logits, case.targets, g, eps, IGN)
    N = d["d0"] * d["d1"]
    gpu = to_host_bits(grad).reshape(N, V)
    if d["dtype"] == "bf16":
        T = grad_terms(ref, g, case.targets.reshape(-1), eps, IGN)
        assert_grad_bf16(gpu, ref, T, "grad")
    else:
        assert_grad_fp32(gpu, ref, "grad")
    # in place: the same bits as the separate buffer; one pass: the two calls' bits
    assert torch.equal(grad_ip, grad)
    assert torch.equal(fb[4], grad)
    assert torch.equal(torch.nan_to_num(fb[0]), torch.nan_to_num(loss))
    assert torch.equal(torch.nan_to_num(fb[2]), torch.nan_to_num(stats))


def _linear_draws(n, seed):
    rng = np.random.default_rng(seed)
    draws = []
    for i in range(n):
        M = int(rng.integers(1, 700))
        draws.append(dict(
            i=i, M=M, H=8 * int(rng.integers(1, 41)),
            V=int(np.exp(rng.uniform(0.0, np.log(40000.0)))),
            eps=float(rng.choice([0.0, 0.1, 0.5])),
            red=bool(rng.random() < 0.5),
            n_ign=int(rng.integers(0, M // 3 + 1)),
            scale=float(rng.choice([1.0, 1.0, 0.3, 2.5]))))
    return draws


LINEAR_DRAWS = _linear_draws(16, 9002)


@pytest.mark.parametrize("d", LINEAR_DRAWS, ids=[f"c{d['i']}-M{d['M']}-H{d['H']}-V{d['V']}"
                                                for d in LINEAR_DRAWS])
def test_random_linear(d):
    M, H, V, eps, red, s = d["M"], d["H"], max(d["V"], 1), d["eps"], d["red"], d["scale"]
    case = wl.make_linear(9200 + d["i"], M, H, V, ignore_count=d["n_ign"], label_smoothing=eps,
                          reduce_loss=red, grad_output="random")
    _say(f"case {d}")
    X, W = to_device(case.X, "bf16"), to_device(case.W, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    loss, mean, stats, nv = vce.lce_forward(X, W, t, eps, red, IGN, logit_scale=s)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, eps, red, IGN, logit_scale=s)
    torch.cuda.synchronize()
    ref_loss, _, _ = linear.forward(case.X, case.W, case.targets, eps, IGN, scale=s)
    valid = case.targets != IGN
    lg = loss.cpu().numpy().astype(np.float64)
    assert np.all(lg[~valid] == 0.0)
    # V = 1: every loss is 0 (p = 1 = q); elsewhere relative to the loss
    err = np.abs(lg[valid] - ref_loss[valid])
    assert np.all(err <= LINEAR_LOSS_RTOL * np.abs(ref_loss[valid]) + 1e-6), float(err.max(initial=0))
    if red:
        rm = oracle.mean_loss(ref_loss, case.targets, IGN)
        assert abs(mean.item() - rm) <= LINEAR_LOSS_RTOL * abs(rm) + 1e-6
        assert nv.item() == oracle.n_valid(case.targets, IGN)
    g = oracle.row_scale(case.grad_output, case.targets, red, IGN)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, eps, IGN, scale=s)
    gx = oracle.bf16_to_f64(to_host_bits(dX))
    gw = oracle.bf16_to_f64(to_host_bits(dW))
    if np.linalg.norm(rdX) == 0.0:
        # V = 1 (p = 1 = q) or every row ignored: the exact gradients are 0; the
        # kernel's p is 1 to within a few FP32 roundings, so each dZ entry is at
        # most s g_r 2^-20 (16 roundings) and dX, dW at most that through W, X
        u = s * 2.0 ** -20 * np.abs(g)
        xa, wa = np.abs(oracle.bf16_to_f64(case.X)), np.abs(oracle.bf16_to_f64(case.W))
        assert np.all(np.abs(gx) <= u[:, None] * wa.sum(axis=0)[None, :])
        assert np.all(np.abs(gw) <= (u @ xa)[None, :])
        return
    fx, fw = rel_frobenius(gx, rdX), rel_frobenius(gw, rdW)
    _say(f"dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL
