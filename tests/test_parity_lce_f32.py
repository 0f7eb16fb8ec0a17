"""Parity of the FP32-input linear cross-entropy (lce_forward_f32 /
lce_backward_f32) with the FP64 oracle on the exact FP32 values.

Tolerances, from the arithmetic (the kernels' products are hi*hi + hi*lo +
lo*hi of BF16 planes with hi + lo within 2^-16 of each FP32 value, FP32
accumulation, dZ split the same way before the dX and dW products):
  * each product is off by at most ~3 * 2^-16 of its size, with random signs,
    so a logit of unit scale is off by ~5e-6 (rms) and a per-token loss by
    a few 1e-5 at most; FP32 accumulation adds less.  The loss tolerance is
    2e-4 per unit of logit scale: a product missing one cross term is off
    by ~5e-3 and rounding the inputs to BF16 by ~7e-3.
  * dX and dW: relative Frobenius error ~3e-6 from the split (measured up to
    9e-6 with FP32 accumulation); the tolerance is 5e-5, below the 1.5e-4 to
    4e-4 of a dZ kept in one BF16 plane and the ~2e-3 of BF16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import rel_frobenius

pytestmark = pytest.mark.gpu

F32_LOSS_ATOL = 2e-4      # per unit of logit scale
F32_FROB_RTOL = 5e-5


def _say(msg):
    print(f"[parity-lce-f32] {msg}", flush=True)


def run_f32(case, ws=None, with_entropy=False, grad_entropy=None):
    X = torch.from_numpy(case.X).cuda()
    W = torch.from_numpy(case.W).cuda()
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    fw = vce.lce_forward_f32(X, W, t, case.label_smoothing, case.reduce_loss, case.ignore_idx,
                             workspace=ws, with_entropy=with_entropy)
    loss, mean, stats, nv = fw[:4]
    ent = fw[4] if with_entropy else None
    ge = None if grad_entropy is None else torch.from_numpy(grad_entropy).cuda()
    dX, dW = vce.lce_backward_f32(X, W, t, stats, nv, go, case.label_smoothing,
                                  case.reduce_loss, case.ignore_idx, workspace=ws,
                                  entropy=ent if ge is not None else None, grad_entropy=ge)
    torch.cuda.synchronize()
    assert dX.dtype == torch.float32 and dW.dtype == torch.float32
    out = dict(loss=loss.cpu().numpy().astype(np.float64), stats=stats.cpu().numpy(),
               dX=dX.cpu().numpy().astype(np.float64), dW=dW.cpu().numpy().astype(np.float64))
    if with_entropy:
        out["entropy"] = ent.cpu().numpy().astype(np.float64)
    if case.reduce_loss:
        out["mean"] = float(mean.item())
        out["n_valid"] = int(nv.item())
    return out


def logit_scale(case):
    return max(1.0, float(case.meta["w_sigma"]) * np.sqrt(case.X.shape[1]))


def check(case, out, grad_entropy=None):
    valid = case.targets != case.ignore_idx
    tol = F32_LOSS_ATOL * logit_scale(case)
    rl, rs, _ = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                               case.ignore_idx)
    assert np.all(out["loss"][~valid] == 0.0)
    err = np.abs(out["loss"][valid] - rl[valid])
    lw = float(err.max()) if err.size else 0.0
    assert lw <= tol, lw
    if case.reduce_loss:
        rm = oracle.mean_loss(rl, case.targets, case.ignore_idx)
        assert abs(out["mean"] - rm) <= tol
        assert out["n_valid"] == oracle.n_valid(case.targets, case.ignore_idx)
    st, r = out["stats"][valid], rs[valid]
    np.testing.assert_allclose(st[:, 0], r[:, 0], atol=tol)          # row max
    np.testing.assert_allclose(st[:, 1], r[:, 1], rtol=2 * tol)      # denominator
    np.testing.assert_allclose(st[:, 2], r[:, 2], atol=tol)          # target logit
    np.testing.assert_allclose(st[:, 3], r[:, 3], atol=tol)          # logit mean
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, case.label_smoothing,
                               case.ignore_idx, grad_entropy=grad_entropy)
    fx, fw = rel_frobenius(out["dX"], rdX), rel_frobenius(out["dW"], rdW)
    _say(f"{case.name}: loss abs {lw:.2e} (tol {tol:.1e}), dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= F32_FROB_RTOL and fw <= F32_FROB_RTOL, (fx, fw)
    # ignored tokens get exactly zero dX rows
    assert np.all(out["dX"][~valid] == 0.0)
    return lw, fx, fw


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("reduce_loss", [True, False])
def test_f32_small(eps, reduce_loss):
    case = wl.make_linear(3101, 300, 264, 1000, ignore_count=7, label_smoothing=eps,
                          reduce_loss=reduce_loss, grad_output="random", fp32=True,
                          name=f"f32_small_eps{eps}_red{int(reduce_loss)}")
    check(case, run_f32(case))


@pytest.mark.parametrize("M,H,V", [
    (1, 64, 777),          # one token, masked K (64 < 128)
    (520, 136, 9000),      # ragged tokens, K not a multiple of 128, ragged vocabulary
    (257, 2304, 4000),     # the second workload's hidden size
    (700, 264, 70001),     # three vocabulary chunks, the last ragged
    (300, 128, 65536),     # exactly two full vocabulary chunks
])
def test_f32_shapes(M, H, V):
    case = wl.make_linear(3200 + M, M, H, V, ignore_count=min(5, M - 1), label_smoothing=0.1,
                          reduce_loss=True, fp32=True, name=f"f32_m{M}_h{H}_v{V}")
    check(case, run_f32(case))


def test_f32_large_logits():
    # logit scale 4: the tolerance scales with it
    case = wl.make_linear(3301, 200, 64, 5000, ignore_count=3, w_sigma=0.5, fp32=True,
                          reduce_loss=False, grad_output="random", name="f32_scale4")
    check(case, run_f32(case))


def test_f32_beats_bf16_rounding():
    # The FP32 form is not a rounding of its inputs to BF16: its errors are far
    # below those of the BF16 form run on the rounded inputs.
    case = wl.make_linear(3401, 256, 256, 3000, ignore_count=4, fp32=True, name="f32_vs_bf16")
    lw, fx, fw = check(case, run_f32(case))
    Xb = wl.f32_to_bf16_bits(case.X)
    Wb = wl.f32_to_bf16_bits(case.W)
    rl, _, _ = linear.forward(case.X, case.W, case.targets, 0.0, case.ignore_idx)
    bl, _, _ = linear.forward(Xb, Wb, case.targets, 0.0, case.ignore_idx)
    valid = case.targets != case.ignore_idx
    bf16_err = float(np.abs(bl - rl)[valid].max())
    _say(f"loss error of BF16-rounded inputs {bf16_err:.2e} vs FP32 form {lw:.2e}")
    assert lw * 20 < bf16_err


def test_f32_with_entropy():
    case = wl.make_linear(3501, 300, 128, 2500, ignore_count=6, label_smoothing=0.1,
                          reduce_loss=True, fp32=True, name="f32_entropy")
    ge = np.random.default_rng(7).uniform(-1.0, 1.0, 300).astype(np.float32)
    out = run_f32(case, with_entropy=True, grad_entropy=ge)
    valid = case.targets != case.ignore_idx
    rh = linear.entropy(case.X, case.W, case.targets, case.ignore_idx)
    np.testing.assert_allclose(out["entropy"][valid], rh[valid], atol=F32_LOSS_ATOL)
    check(case, out, grad_entropy=ge.astype(np.float64))


def test_f32_workspace_reuse_and_empty_batch():
    case = wl.make_linear(3601, 96, 64, 1500, ignore_count=2, fp32=True, name="f32_reuse")
    ws = vce.lce_workspace(96, 64, 1500, "cuda", f32=True)
    a = run_f32(case, ws=ws)
    b = run_f32(case, ws=ws)
    for k in ("loss", "stats", "dX", "dW"):
        np.testing.assert_array_equal(a[k], b[k])     # deterministic
    # M = 0: the mean is 0 and dW is zeroed
    X = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    W = torch.from_numpy(case.W).cuda()
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    loss, mean, stats, nv = vce.lce_forward_f32(X, W, t, 0.0, True)
    dW = torch.full_like(W, 7.0)
    dX, dW = vce.lce_backward_f32(X, W, t, stats, nv, torch.ones(1, device="cuda"), 0.0, True,
                                  dW=dW)
    torch.cuda.synchronize()
    assert float(mean.item()) == 0.0 and int(nv.item()) == 0
    assert torch.count_nonzero(dW).item() == 0


def test_f32_all_ignored():
    case = wl.make_linear(3701, 64, 64, 800, ignore_count=64, fp32=True, name="f32_all_ignored")
    out = run_f32(case)
    assert np.all(out["loss"] == 0.0) and out["mean"] == 0.0 and out["n_valid"] == 0
    assert np.all(out["dX"] == 0.0) and np.all(out["dW"] == 0.0)


def test_f32_m4096_h4096_v131072():
    """The benchmarked FP32 shape: every token's loss and statistics against the
    oracle's stored values (tests/golden, written by make_linear_golden.py),
    sampled rows of dX and dW computed by the oracle."""
    import hashlib
    import os
    case = wl.linear_4k_f32()
    _say(case.name)
    gold = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                case.name + ".npz"))
    h = hashlib.sha256()
    for a in (case.X, case.W, case.targets):
        h.update(np.ascontiguousarray(a).tobytes())
    assert str(gold["digest"]) == h.hexdigest(), "regenerated inputs differ from the golden's"
    out = run_f32(case)
    valid = case.targets != case.ignore_idx
    tol = F32_LOSS_ATOL * logit_scale(case)
    err = np.abs(out["loss"] - gold["loss"])[valid]
    assert float(err.max()) <= tol, float(err.max())
    assert np.all(out["loss"][~valid] == 0.0)
    rm = oracle.mean_loss(gold["loss"], case.targets, case.ignore_idx)
    assert abs(out["mean"] - rm) <= tol
    st, r = out["stats"][valid], gold["stats"][valid]
    np.testing.assert_allclose(st[:, 0], r[:, 0], atol=tol)
    np.testing.assert_allclose(st[:, 1], r[:, 1], rtol=2 * tol)
    np.testing.assert_allclose(st[:, 2], r[:, 2], atol=tol)
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rng = np.random.default_rng(11)
    vidx = np.nonzero(valid)[0]
    rows = np.unique(np.concatenate([rng.choice(vidx, 24, replace=False), [0, case.M - 1]]))
    rdx = linear.dx_rows(case.X, case.W, case.targets, g, rows, case.label_smoothing,
                         case.ignore_idx)
    fx = rel_frobenius(out["dX"][rows], rdx)
    V = case.V
    vrows = np.unique(np.concatenate([rng.choice(V, 24, replace=False),
                                      [0, 1, V - 1, 32767, 32768, 65536],
                                      np.unique(case.targets[vidx])[:4]]))
    rdw = linear.dw_rows(case.X, case.W, case.targets, g, gold["lse"], vrows,
                         case.label_smoothing, case.ignore_idx)
    fw = rel_frobenius(out["dW"][vrows], rdw)
    _say(f"{case.name}: loss abs {float(err.max()):.2e}, dX rows frob {fx:.2e}, "
         f"dW rows frob {fw:.2e}")
    assert fx <= F32_FROB_RTOL and fw <= F32_FROB_RTOL, (fx, fw)


def test_f32_graph_capture_replay():
    # the FP32 calls (split, GEMMs, merge, mean) captured on a side stream and
    # replayed three times with eager work in between: bit-identical to eager
    case = wl.make_linear(3801, 200, 128, 3000, ignore_count=3, label_smoothing=0.1,
                          fp32=True, name="f32_graph")
    X = torch.from_numpy(case.X).cuda()
    W = torch.from_numpy(case.W).cuda()
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    ws = vce.lce_workspace(200, 128, 3000, "cuda", f32=True)
    loss, mean, stats = (torch.empty(200, device="cuda"), torch.empty((), device="cuda"),
                         torch.empty((200, 4), device="cuda"))
    nv = torch.empty((), dtype=torch.int32, device="cuda")
    dX, dW = torch.empty_like(X), torch.empty_like(W)
    out = (loss, mean, stats, nv)
    vce.lce_forward_f32(X, W, t, 0.1, True, workspace=ws, out=out)
    vce.lce_backward_f32(X, W, t, stats, nv, go, 0.1, True, workspace=ws, dX=dX, dW=dW)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (loss, mean, stats, dX, dW)]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            vce.lce_forward_f32(X, W, t, 0.1, True, workspace=ws, out=out, stream=s)
            vce.lce_backward_f32(X, W, t, stats, nv, go, 0.1, True, workspace=ws, dX=dX, dW=dW,
                                 stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (loss, mean, stats, dX, dW):
            x.zero_()
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "mean", "stats", "dX", "dW"), (loss, mean, stats, dX, dW),
                              ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
    _say("graph capture + 3 replays of lce_forward_f32 + lce_backward_f32: bit-identical")
