"""The Python binding rejects malformed tensors before they reach the C ABI,
which reads every buffer as raw memory in flattened row order (no GPU needed:
the checks run before the device check, which CPU tensors then fail)."""
import pytest
import torch

import vocabulary_cross_entropy_amd as vce

N_D0, N_D1, V = 2, 3, 16


def _logits():
    z = torch.zeros((N_D0, N_D1, V), dtype=torch.float32)
    t = torch.zeros((N_D0, N_D1), dtype=torch.int64)
    return z, t


def _bwd(**kw):
    z, t = _logits()
    args = dict(stats=torch.zeros((N_D0, N_D1, 4)), n_valid=None,
                grad_output=torch.ones((N_D0, N_D1)), reduce_loss=False)
    args.update(kw)
    return vce.ce_backward(z, t, args["stats"], args["n_valid"], args["grad_output"], 0.0,
                           args["reduce_loss"])


def test_valid_cpu_tensors_reach_the_device_check():
    with pytest.raises(RuntimeError, match="GPU only"):
        _bwd()


@pytest.mark.parametrize("kw,exc", [
    (dict(grad_output=torch.ones((N_D0, N_D1), dtype=torch.float64)), TypeError),
    (dict(grad_output=torch.ones((N_D0, N_D1), dtype=torch.bfloat16)), TypeError),
    # an (SQ,B) view of (B,SQ) storage: the library would read it in the wrong order
    (dict(grad_output=torch.ones((N_D1, N_D0)).t()), ValueError),
    (dict(grad_output=torch.ones(N_D0 * N_D1 + 1)), ValueError),
    (dict(grad_output=torch.ones(1)), ValueError),            # per-token loss needs N values
    (dict(stats=torch.zeros((N_D0, N_D1, 3))), ValueError),
    (dict(stats=torch.zeros((N_D0, N_D1, 4), dtype=torch.float16)), TypeError),
    (dict(reduce_loss=True, grad_output=torch.ones(1), n_valid=torch.zeros((), dtype=torch.float32)),
     TypeError),
    (dict(reduce_loss=True, grad_output=torch.ones(1), n_valid=torch.zeros(2, dtype=torch.int32)),
     ValueError),
])
def test_ce_backward_rejects_malformed_buffers(kw, exc):
    with pytest.raises(exc):
        _bwd(**kw)


def test_reduced_backward_takes_one_grad_output():
    with pytest.raises(RuntimeError, match="GPU only"):
        _bwd(reduce_loss=True, grad_output=torch.ones(1), n_valid=torch.zeros((), dtype=torch.int32))


def test_ce_forward_rejects_malformed_outputs():
    z, t = _logits()
    good = (torch.empty((N_D0, N_D1)), None, torch.empty((N_D0, N_D1, 4)), None)
    with pytest.raises(RuntimeError, match="GPU only"):
        vce.ce_forward(z, t, out=good)
    bad_stats = (good[0], None, torch.empty((N_D0, N_D1, 4), dtype=torch.float64), None)
    with pytest.raises(TypeError):
        vce.ce_forward(z, t, out=bad_stats)
    bad_loss = (torch.empty((N_D1, N_D0)).t(), None, good[2], None)
    with pytest.raises(ValueError):
        vce.ce_forward(z, t, out=bad_loss)


def test_ce_forward_backward_rejects_malformed_grad_output():
    z, t = _logits()
    with pytest.raises(TypeError):
        vce.ce_forward_backward(z, t, torch.ones((N_D0, N_D1), dtype=torch.float64))
    with pytest.raises(ValueError):
        vce.ce_forward_backward(z, t, torch.ones((N_D1, N_D0)).t())


def test_grad_buffer_must_match_logits():
    z, t = _logits()
    with pytest.raises(ValueError):
        vce.ce_backward(z, t, torch.zeros((N_D0, N_D1, 4)), None, torch.ones((N_D0, N_D1)),
                        grad=torch.zeros((N_D0, N_D1, V), dtype=torch.float64))


def _linear():
    X = torch.zeros((4, 8), dtype=torch.bfloat16)
    W = torch.zeros((16, 8), dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int64)
    return X, W, t


def test_lce_backward_rejects_malformed_buffers():
    X, W, t = _linear()
    stats, go = torch.zeros((4, 4)), torch.ones(1)
    nv = torch.zeros((), dtype=torch.int32)
    ws = torch.zeros(1, dtype=torch.uint8)
    with pytest.raises(RuntimeError, match="GPU only"):
        vce.lce_backward(X, W, t, stats, nv, go, workspace=ws)
    with pytest.raises(TypeError):
        vce.lce_backward(X, W, t, stats, nv, go.double(), workspace=ws)
    with pytest.raises(ValueError):
        vce.lce_backward(X, W, t, torch.zeros((4, 3)), nv, go, workspace=ws)
    with pytest.raises(ValueError):
        vce.lce_backward(X, W, t, stats, nv, go, workspace=ws,
                         dX=torch.zeros((4, 8), dtype=torch.float32))
    with pytest.raises(ValueError):
        vce.lce_backward(X, W, t, stats, nv, go, workspace=ws,
                         dW=torch.zeros((8, 16), dtype=torch.bfloat16).t())
    with pytest.raises(ValueError):
        vce.lce_backward(X, W, t, stats, None, torch.ones(4), reduce_loss=False, workspace=ws,
                         dX=torch.zeros((4, 9), dtype=torch.bfloat16))


def test_lce_forward_rejects_malformed_outputs():
    X, W, t = _linear()
    ws = torch.zeros(1, dtype=torch.uint8)
    out = (torch.empty(4), torch.empty(()), torch.empty((4, 4)), torch.empty((), dtype=torch.int32))
    with pytest.raises(RuntimeError, match="GPU only"):
        vce.lce_forward(X, W, t, workspace=ws, out=out)
    with pytest.raises(TypeError):
        vce.lce_forward(X, W, t, workspace=ws, out=(out[0], out[1], out[2], torch.empty(())))
    with pytest.raises(ValueError):
        vce.lce_forward(X, W, t, workspace=ws, out=(torch.empty(5),) + out[1:])
