"""The library keeps no state between calls: calls issued on two streams at
once, each with its own buffers (and, for the linear form, its own
workspace), give exactly the results of the same calls made one after the
other."""
import pytest
import torch

import vocabulary_cross_entropy_amd as vce
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import to_device

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-streams] {msg}", flush=True)


def _logits_inputs(seed, V, eps, red):
    case = wl.make_logits(seed, 4, 300, V, dtype="bf16", sigma=3.0, ignore_count=9,
                          label_smoothing=eps, reduce_loss=red, grad_output="random")
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    return z, t, go.reshape(-1) if red else go


def _logits_step(z, t, go, eps, red, stream=None):
    out = vce.ce_forward(z, t, eps, red, IGN, stream=stream)
    grad = vce.ce_backward(z, t, out[2], out[3], go, eps, red, IGN, stream=stream)
    fb = vce.ce_forward_backward(z, t, go, eps, red, IGN, stream=stream)
    return [x for x in out if x is not None] + [grad] + [x for x in fb if x is not None]


def test_logits_calls_on_two_streams():
    a = _logits_inputs(7001, 30000, 0.1, True)
    b = _logits_inputs(7002, 12000, 0.0, False)
    ref_a = _logits_step(*a, 0.1, True)
    ref_b = _logits_step(*b, 0.0, False)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(sa):
            got_a = _logits_step(*a, 0.1, True, stream=sa)
        with torch.cuda.stream(sb):
            got_b = _logits_step(*b, 0.0, False, stream=sb)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(got_a, ref_a)):
            assert torch.equal(x, y), f"stream a, rep {rep}, output {i}"
        for i, (x, y) in enumerate(zip(got_b, ref_b)):
            assert torch.equal(x, y), f"stream b, rep {rep}, output {i}"
    _say("logits: 3 concurrent repetitions equal the serial results")


def _linear_inputs(seed, M, H, V):
    case = wl.make_linear(seed, M, H, V, ignore_count=5, label_smoothing=0.1, reduce_loss=True)
    X = torch.from_numpy(case.X.view("int16")).cuda().view(torch.bfloat16)
    W = torch.from_numpy(case.W.view("int16")).cuda().view(torch.bfloat16)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    ws = vce.lce_workspace(M, H, V)
    return X, W, t, go, ws


def _linear_step(X, W, t, go, ws, stream=None):
    loss, mean, stats, nv = vce.lce_forward(X, W, t, 0.1, True, IGN, workspace=ws,
                                            stream=stream)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, IGN, workspace=ws,
                              stream=stream)
    return [loss, mean, stats, nv, dX, dW]


def test_linear_calls_on_two_streams():
    a = _linear_inputs(7003, 700, 512, 40000)
    b = _linear_inputs(7004, 300, 264, 70001)
    ref_a = _linear_step(*a)
    ref_b = _linear_step(*b)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(sa):
            got_a = _linear_step(*a, stream=sa)
        with torch.cuda.stream(sb):
            got_b = _linear_step(*b, stream=sb)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(got_a, ref_a)):
            assert torch.equal(x, y), f"stream a, rep {rep}, output {i}"
        for i, (x, y) in enumerate(zip(got_b, ref_b)):
            assert torch.equal(x, y), f"stream b, rep {rep}, output {i}"
    _say("linear: 3 concurrent repetitions equal the serial results")
