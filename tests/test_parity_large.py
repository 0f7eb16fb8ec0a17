"""Parity at the largest sizes: tensors whose byte offsets pass 2^31 and 2^32
and whose element counts pass 2^31, so that any 32-bit index or offset in
the kernels, the workspace layout or the host arithmetic would show.

  * logits, (B, SQ, V) = (2, 8256, 131072) BF16: 4.33e9 bytes, 2.16e9
    elements; rows from 16384 on start past 2^32 bytes.  Every row's loss and
    the mean against the FP64 oracle, gradient rows sampled on both sides of
    the boundaries, and the one-pass form bit for bit against the two calls.
  * linear, M = 300, H = 4096, V = 262147 BF16: W and dW are 2.15e9 bytes;
    vocabulary rows from 262144 on lie past 2^31 bytes.
  * linear with FP32 inputs, M = 64, H = 4096, V = 262147: W and dW are
    4.29e9 bytes (rows from 262144 on past 2^32) and so is the workspace's
    block of BF16 planes.

Each case is checked against the FP64 oracle to the bars of the smaller
tests (every token's loss; sampled rows of the gradients, dX and dW)."""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, assert_grad_bf16,
                          assert_loss_close, grad_terms, rel_frobenius, to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-large] {msg}", flush=True)


def _bf16_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def test_logits_bf16_past_4gib():
    B, SQ, V = 2, 8256, 131072
    N = B * SQ
    assert N * V * 2 > 2 ** 32 and N * V > 2 ** 31
    _say(f"generating (B,SQ,V) = ({B},{SQ},{V}) BF16")
    case = wl.make_logits(6001, B, SQ, V, dtype="bf16", sigma=4.0, ignore_count=33,
                          label_smoothing=0.1, reduce_loss=True, name="logits_past_4gib")
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    _say("forward and backward")
    loss, mean, stats, nv = vce.ce_forward(z, t, 0.1, True, IGN)
    grad = vce.ce_backward(z, t, stats, nv, go, 0.1, True, IGN)
    torch.cuda.synchronize()

    _say("oracle forward over every row")
    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, 0.1, IGN)
    gl = loss.cpu().numpy().reshape(-1)
    err = assert_loss_close(gl, ref_loss)
    ref_mean = oracle.mean_loss(ref_loss, case.targets, IGN)
    assert abs(float(mean.item()) - ref_mean) <= 1e-4 + 1e-5 * abs(ref_mean)
    assert int(nv.item()) == oracle.n_valid(case.targets, IGN)
    st = stats.cpu().numpy().reshape(-1, 4)
    valid = case.targets.reshape(-1) != IGN
    np.testing.assert_array_equal(st[valid, 0], ref_stats[valid, 0].astype(np.float32))
    np.testing.assert_allclose(st[valid, 1], ref_stats[valid, 1], rtol=2e-5)

    # gradient rows around 2^31 elements (row 16384 starts at 2^32 bytes) and at the ends
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 16383, 16384, 16385, N - 2, N - 1],
                                     rng.choice(N, 12, replace=False)]))
    g = oracle.row_scale(case.grad_output, case.targets, True, IGN)
    ref = oracle.ce_backward(case.logits, case.targets, g, 0.1, IGN, rows=rows)
    gsel = to_host_bits(grad.view(N, V)[torch.from_numpy(rows).cuda()])
    T = grad_terms(ref, g[rows], case.targets.reshape(-1)[rows], 0.1, IGN)
    worst = assert_grad_bf16(gsel, ref, T, "grad rows past 4 GiB")
    _say(f"max loss err {err:.2e}, worst grad ulp {worst} over {rows.size} rows")

    _say("one pass against the two calls")
    res = vce.ce_forward_backward(z, t, go, 0.1, True, IGN)
    torch.cuda.synchronize()
    assert torch.equal(res[0], loss) and torch.equal(res[1], mean)
    assert torch.equal(res[2], stats) and torch.equal(res[3], nv)
    assert torch.equal(res[4], grad)
    del res
    res = vce.ce_forward_backward(z, t, go, 0.1, True, IGN, overwrite_input=True)
    torch.cuda.synchronize()
    assert torch.equal(res[4], grad) and res[4].data_ptr() == z.data_ptr()


def _linear_sampled(case, dX_dev, dW_dev, decode, ref_lse, frob_tol, rows_extra=()):
    """Relative Frobenius errors of sampled dX and dW rows against the oracle."""
    M, V = case.M, case.V
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rng = np.random.default_rng(12)
    valid = np.nonzero(case.targets != case.ignore_idx)[0]
    rows = np.unique(np.concatenate([rng.choice(valid, min(10, valid.size), replace=False),
                                     [0, M - 1]]))
    rdx = linear.dx_rows(case.X, case.W, case.targets, g, rows, case.label_smoothing,
                         case.ignore_idx)
    fx = rel_frobenius(decode(dX_dev[torch.from_numpy(rows).cuda()]), rdx)
    vrows = np.unique(np.concatenate([rng.choice(V, 16, replace=False), list(rows_extra),
                                      case.targets[valid][:4]]))
    vrows = vrows[(vrows >= 0) & (vrows < V)]
    rdw = linear.dw_rows(case.X, case.W, case.targets, g, ref_lse, vrows,
                         case.label_smoothing, case.ignore_idx)
    fw = rel_frobenius(decode(dW_dev[torch.from_numpy(vrows).cuda()]), rdw)
    assert fx <= frob_tol and fw <= frob_tol, (fx, fw)
    return fx, fw


def test_linear_bf16_w_past_2gib():
    M, H, V = 300, 4096, 262147
    assert V * H * 2 > 2 ** 31
    _say(f"generating linear M={M} H={H} V={V} BF16")
    case = wl.make_linear(6002, M, H, V, ignore_count=7, label_smoothing=0.1, reduce_loss=True,
                          name="linear_w_past_2gib")
    X, W = _bf16_dev(case.X), _bf16_dev(case.W)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    loss, mean, stats, nv = vce.lce_forward(X, W, t, 0.1, True, IGN)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, IGN)
    torch.cuda.synchronize()
    _say("oracle forward")
    rl, rs, lse = linear.forward(case.X, case.W, case.targets, 0.1, IGN)
    valid = case.targets != IGN
    gl = loss.cpu().numpy().astype(np.float64)
    assert np.all(gl[~valid] == 0.0)
    lw = float((np.abs(gl[valid] - rl[valid]) / np.abs(rl[valid])).max())
    assert lw <= LINEAR_LOSS_RTOL, lw
    rm = oracle.mean_loss(rl, case.targets, IGN)
    assert abs(float(mean.item()) - rm) <= LINEAR_LOSS_RTOL * abs(rm)
    assert int(nv.item()) == oracle.n_valid(case.targets, IGN)
    _say("oracle dX and dW rows")
    dec = lambda x: oracle.bf16_to_f64(to_host_bits(x))
    fx, fw = _linear_sampled(case, dX, dW, dec, lse, LINEAR_FROB_RTOL,
                             rows_extra=(262143, 262144, 262145, V - 1))
    _say(f"loss rel {lw:.2e}, dX rows frob {fx:.2e}, dW rows frob {fw:.2e}")


def test_linear_f32_w_past_4gib():
    M, H, V = 64, 4096, 262147
    assert V * H * 4 > 2 ** 32 and 4 * (M + V) * H > 2 ** 32
    _say(f"generating linear M={M} H={H} V={V} FP32")
    case = wl.make_linear(6003, M, H, V, ignore_count=2, label_smoothing=0.0, reduce_loss=True,
                          fp32=True, name="linear_f32_w_past_4gib")
    X = torch.from_numpy(case.X).cuda()
    W = torch.from_numpy(case.W).cuda()
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    loss, mean, stats, nv = vce.lce_forward_f32(X, W, t, 0.0, True, IGN)
    dX, dW = vce.lce_backward_f32(X, W, t, stats, nv, go, 0.0, True, IGN)
    torch.cuda.synchronize()
    _say("oracle forward")
    rl, rs, lse = linear.forward(case.X, case.W, case.targets, 0.0, IGN)
    valid = case.targets != IGN
    tol = 2e-4 * max(1.0, float(case.meta["w_sigma"]) * np.sqrt(H))
    gl = loss.cpu().numpy().astype(np.float64)
    assert np.all(gl[~valid] == 0.0)
    lw = float(np.abs(gl[valid] - rl[valid]).max())
    assert lw <= tol, lw
    _say("oracle dX and dW rows")
    dec = lambda x: x.cpu().numpy().astype(np.float64)
    fx, fw = _linear_sampled(case, dX, dW, dec, lse, 5e-5,
                             rows_extra=(262143, 262144, 262145, V - 1))
    _say(f"loss abs {lw:.2e}, dX rows frob {fx:.2e}, dW rows frob {fw:.2e}")
