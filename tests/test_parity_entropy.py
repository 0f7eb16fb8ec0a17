"""Parity of the optional entropy output and its gradient (the "optional
entropy" of the Liger-Kernel PR, Summary) with the FP64 oracle, for both the
logits and the linear form, through the C-ABI.

Entropy values are held to the loss bar (1e-4 abs + 1e-5 rel; the linear form
to its loss bar, 1e-3 rel).  The gradient with an entropy term: BF16 to 1 ulp
of the rounded oracle value outside the cancellation band, which the entropy
term's size T_H = |gH| p (|E_p[z]| + |z|) widens by 2^-10 T_H (2^8 times its
error bound 2^-18 T_H, see below); FP32 to
1e-6 + 2^-18 T_H (the term multiplies E_p[z] - z, formed in FP32 from values
of magnitude |E_p[z]| + |z|, so a few of their ulps carry through; the plain
bar 1e-6 is kept where gH = 0); dX and dW of the linear form to 5e-3 relative
Frobenius."""
import numpy as np
import pytest
import torch

import oracle
from oracle import linear as olin
import vocabulary_cross_entropy_amd as vce
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, assert_grad_bf16, assert_loss_close,
                          rel_frobenius, to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-entropy] {msg}", flush=True)


def _grad_entropy(seed, shape):
    return (np.random.default_rng(seed).standard_normal(shape) * 0.7).astype(np.float32)


def _terms(z_rows, ref_stats, H, g, gH, targets, eps, ignore_idx):
    """Per-element magnitudes of the summands of g (p - q) + gH p (E_p[z] - z):
    T = |g| (p + q) and T_H = |gH| p (|E_p[z]| + |z|)."""
    V = z_rows.shape[1]
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        lse = ref_stats[:, 0] + np.log(ref_stats[:, 1])
        p = np.exp(z_rows - lse[:, None])
    q = np.full(z_rows.shape, eps / V)
    valid = (targets != ignore_idx) & (targets >= 0) & (targets < V)
    r = np.nonzero(valid)[0]
    q[r, targets[r]] += 1.0 - eps
    E = (lse - H)[:, None]
    zf = np.where(np.isfinite(z_rows), np.abs(z_rows), 0.0)
    T = np.abs(g)[:, None] * (p + q)
    T_H = np.abs(gH)[:, None] * p * (np.abs(E) + zf)
    T[~valid] = 0.0
    T_H[~valid] = 0.0
    return np.nan_to_num(T), np.nan_to_num(T_H)


def _assert_grad_fp32_entropy(gpu, ref, T_H, what):
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(gpu)), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(gpu[ok].astype(np.float64) - ref[ok])
    bound = 1e-6 + 2.0 ** -18 * T_H[ok]
    assert np.all(err <= bound), (f"{what}: {int((err > bound).sum())} elements out of bound, "
                                  f"worst err {err.max():.3e}")
    return float(err.max()) if err.size else 0.0


def _entropy_term_size(z_rows, ref_stats, H, gH, targets, ignore_idx):
    """T_H = |gH| p (|E_p[z]| + |z|) per element (0 for ignored rows)."""
    V = z_rows.shape[1]
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        lse = ref_stats[:, 0] + np.log(ref_stats[:, 1])
        p = np.exp(z_rows - lse[:, None])
    zf = np.where(np.isfinite(z_rows), np.abs(z_rows), 0.0)
    T = np.abs(gH)[:, None] * p * (np.abs(lse - H)[:, None] + zf)
    T[targets == ignore_idx] = 0.0
    return np.nan_to_num(T)


def _run_logits(case, gH):
    z = to_device(case.logits, case.dtype)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    go = go.reshape(-1) if case.reduce_loss else go
    plain = vce.ce_forward(z, t, case.label_smoothing, case.reduce_loss, case.ignore_idx)
    loss, mean, stats, nv, ent = vce.ce_forward(z, t, case.label_smoothing, case.reduce_loss,
                                                case.ignore_idx, with_entropy=True)
    gHd = torch.from_numpy(gH).cuda()
    grad = vce.ce_backward(z, t, stats, nv, go, case.label_smoothing, case.reduce_loss,
                           case.ignore_idx, entropy=ent, grad_entropy=gHd)
    grad_plain = vce.ce_backward(z, t, stats, nv, go, case.label_smoothing, case.reduce_loss,
                                 case.ignore_idx, entropy=ent)  # no grad_entropy: plain path
    grad_ref_plain = vce.ce_backward(z, t, stats, nv, go, case.label_smoothing, case.reduce_loss,
                                     case.ignore_idx)
    torch.cuda.synchronize()
    # computing the entropy changes nothing else, bit for bit
    assert torch.equal(plain[0], loss) and torch.equal(plain[2], stats)
    assert torch.equal(grad_plain, grad_ref_plain)
    return dict(loss=loss.cpu().numpy(), ent=ent.cpu().numpy().reshape(-1), grad=to_host_bits(grad))


@pytest.mark.parametrize("dtype,V,eps,reduce_loss", [
    ("fp32", 1000, 0.0, False), ("fp32", 4099, 0.1, True), ("bf16", 32000, 0.1, True),
    ("bf16", 128256, 0.0, False), ("bf16", 1001, 0.05, False)])
def test_entropy_logits(dtype, V, eps, reduce_loss):
    case = wl.make_logits(4000 + V, 3, 37, V, dtype=dtype, sigma=3.0, ignore_count=4,
                          label_smoothing=eps, reduce_loss=reduce_loss, grad_output="random")
    gH = _grad_entropy(4100 + V, case.N)
    _say(f"logits {dtype} V={V} eps={eps} reduce={reduce_loss}")
    out = _run_logits(case, gH)
    ref_H = oracle.entropy(case.logits, case.targets, case.ignore_idx)
    err = assert_loss_close(out["ent"], ref_H, "entropy")
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    ref = oracle.ce_backward(case.logits, case.targets, g, eps, case.ignore_idx)
    oracle.add_entropy_grad(ref, case.logits, case.targets, gH, case.ignore_idx)
    gpu = out["grad"].reshape(case.N, V)
    _, st, _ = oracle.ce_forward(case.logits, case.targets, eps, case.ignore_idx)
    if dtype == "fp32":
        z = case.logits.reshape(case.N, V).astype(np.float64)
        T_H = _entropy_term_size(z, st, ref_H, gH.astype(np.float64), case.targets.reshape(-1),
                                 case.ignore_idx)
        worst = _assert_grad_fp32_entropy(gpu, ref, T_H, "grad with entropy")
    else:
        z = oracle.bf16_to_f64(case.logits.reshape(case.N, V))
        T, T_H = _terms(z, st, ref_H, g, gH.astype(np.float64), case.targets.reshape(-1), eps,
                        case.ignore_idx)
        worst = assert_grad_bf16(gpu, ref, T, "grad with entropy", extra_terms=T_H)
    _say(f"entropy max abs err {err:.2e}; gradient worst {worst}")


def test_entropy_negative_infinity_columns():
    # padded vocabulary: p = 0 there, and neither the entropy nor its gradient
    # may turn 0 * inf into NaN
    case = wl.make_logits(4200, 2, 9, 2000, dtype="fp32", sigma=2.0, ignore_count=2,
                          label_smoothing=0.1, reduce_loss=False, grad_output="random")
    case.logits[:, :, 1900:] = -np.inf
    gH = _grad_entropy(4201, case.N)
    out = _run_logits(case, gH)
    ref_H = oracle.entropy(case.logits, case.targets, case.ignore_idx)
    assert np.all(np.isfinite(out["ent"]))
    assert_loss_close(out["ent"], ref_H, "entropy")
    g = oracle.row_scale(case.grad_output, case.targets, False, case.ignore_idx)
    ref = oracle.ce_backward(case.logits, case.targets, g, 0.1, case.ignore_idx)
    oracle.add_entropy_grad(ref, case.logits, case.targets, gH, case.ignore_idx)
    gpu = out["grad"].reshape(case.N, 2000)  # FP32 logits: FP32 gradient
    # p = 0 there: only -g eps/V remains (smoothing puts eps/V on every class)
    valid = case.targets.reshape(-1) != case.ignore_idx
    assert np.all(np.isfinite(gpu[valid]))
    _, st, _ = oracle.ce_forward(case.logits, case.targets, 0.1, case.ignore_idx)
    T_H = _entropy_term_size(case.logits.reshape(case.N, 2000).astype(np.float64), st, ref_H,
                             gH.astype(np.float64), case.targets.reshape(-1), case.ignore_idx)
    _assert_grad_fp32_entropy(gpu, ref, T_H, "grad with entropy, -inf columns")


@pytest.mark.parametrize("M,V", [(700, 9000), (520, 70001)])
def test_entropy_linear(M, V):
    case = wl.make_linear(4300 + M, M, 256, V, ignore_frac=0.05, label_smoothing=0.1,
                          reduce_loss=True)
    _say(f"linear M={M} H=256 V={V}")
    X, W = to_device(case.X, "bf16"), to_device(case.W, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda().reshape(-1)
    gH = _grad_entropy(4400 + M, M)
    plain = vce.lce_forward(X, W, t, 0.1, True)
    loss, mean, stats, nv, ent = vce.lce_forward(X, W, t, 0.1, True, with_entropy=True)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, entropy=ent,
                              grad_entropy=torch.from_numpy(gH).cuda())
    torch.cuda.synchronize()
    assert torch.equal(plain[0], loss) and torch.equal(plain[2], stats)
    ref_H = olin.entropy(case.X, case.W, case.targets, case.ignore_idx)
    e = np.abs(ent.cpu().numpy() - ref_H)
    rel = float(np.max(e / np.maximum(np.abs(ref_H), 1e-3)))
    assert rel <= LINEAR_LOSS_RTOL, f"entropy rel err {rel:.2e}"
    g = oracle.row_scale(case.grad_output, case.targets, True, case.ignore_idx)
    rdX, rdW = olin.backward(case.X, case.W, case.targets, g, 0.1, case.ignore_idx,
                             grad_entropy=gH)
    fx = rel_frobenius(oracle.bf16_to_f64(to_host_bits(dX)), rdX)
    fw = rel_frobenius(oracle.bf16_to_f64(to_host_bits(dW)), rdW)
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL, (fx, fw)
    _say(f"entropy rel err {rel:.2e}; dX frob {fx:.2e}, dW frob {fw:.2e}")
