"""Parity of the scaled linear form (loss of logit_scale * X W^T) with the
FP64 oracle, through the C-ABI (lce_forward_scaled / lce_backward_scaled).

"Scaled" is read as a positive factor on the logits before the softmax (the
Liger-Kernel PR names a "fused scaled linear cross-entropy" without saying
what is scaled)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import binding
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, rel_frobenius, to_device, to_host_bits

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[parity-lce-scaled] {msg}", flush=True)


def _run(case, scale, *, W=None, with_entropy=False, gH=None):
    X = to_device(case.X, "bf16")
    Wd = to_device(case.W if W is None else W, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    ws = vce.lce_workspace(case.M, case.H, case.V)
    f = vce.lce_forward(X, Wd, t, case.label_smoothing, case.reduce_loss, case.ignore_idx,
                        workspace=ws, with_entropy=with_entropy, logit_scale=scale)
    loss, mean, stats, nv = f[:4]
    ent = f[4] if with_entropy else None
    dX, dW = vce.lce_backward(X, Wd, t, stats, nv, go, case.label_smoothing, case.reduce_loss,
                              case.ignore_idx, workspace=ws, logit_scale=scale, entropy=ent,
                              grad_entropy=None if gH is None else torch.from_numpy(gH).cuda())
    torch.cuda.synchronize()
    return dict(loss=loss, mean=mean, stats=stats, n_valid=nv, entropy=ent, dX=dX, dW=dW)


@pytest.mark.parametrize("log2_scale", [3, -2])
def test_power_of_two_scale_is_bitwise_the_scaled_classifier(log2_scale):
    # s X W^T with s = 2^k equals X (2^k W)^T exactly in BF16 and FP32, so the
    # loss, statistics and dX are bitwise those of the unscaled call with
    # W 2^k, and dW is 2^k times its dW (three vocabulary chunks, the last
    # ragged, so the grouped backward launches are covered)
    case = wl.make_linear(5100 + log2_scale, 520, 136, 70001, ignore_frac=0.05,
                          label_smoothing=0.1, reduce_loss=False, grad_output="random")
    s = 2.0 ** log2_scale
    w2 = wl.bf16_bits_to_f32(case.W) * np.float32(s)
    W2 = wl.f32_to_bf16_bits(w2)
    assert np.array_equal(wl.bf16_bits_to_f32(W2), w2)
    a = _run(case, s)
    b = _run(case, 1.0, W=W2)
    for k in ("loss", "stats", "dX"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["dW"].float(), s * b["dW"].float())
    _say(f"scale 2^{log2_scale}: bitwise the unscaled call with W * 2^{log2_scale}")


def test_scale_one_through_the_scaled_entry_points_is_bitwise_the_plain_ones():
    case = wl.make_linear(5110, 300, 264, 3000, ignore_count=7, label_smoothing=0.1,
                          reduce_loss=True)
    X, W = to_device(case.X, "bf16"), to_device(case.W, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    ws = vce.lce_workspace(case.M, case.H, case.V)
    loss, mean, stats, nv = vce.lce_forward(X, W, t, 0.1, True, workspace=ws)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, workspace=ws)
    L = binding.lib()
    loss1, stats1 = torch.empty_like(loss), torch.empty_like(stats)
    mean1, nv1 = torch.empty_like(mean), torch.empty_like(nv)
    dX1, dW1 = torch.empty_like(dX), torch.empty_like(dW)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.lce_forward_scaled(p(X), p(W), case.M, case.H, case.V, 1.0, p(t), 0.1, 1, -100,
                                p(loss1), p(mean1), p(stats1), p(nv1), None, p(ws), ws.numel(),
                                s) == 0
    assert L.lce_backward_scaled(p(X), p(W), case.M, case.H, case.V, 1.0, p(t), p(stats1),
                                 p(nv1), p(go), None, None, 0.1, 1, -100, p(dX1), p(dW1), p(ws),
                                 ws.numel(), s) == 0
    torch.cuda.synchronize()
    for x, y in ((loss, loss1), (mean, mean1), (stats, stats1), (nv, nv1), (dX, dX1), (dW, dW1)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("scale,eps,reduce_loss", [(0.7, 0.1, True), (1.9, 0.0, False)])
def test_scaled_against_the_oracle(scale, eps, reduce_loss):
    case = wl.make_linear(5120, 520, 136, 70001, ignore_frac=0.05, label_smoothing=eps,
                          reduce_loss=reduce_loss, grad_output="random")
    out = _run(case, scale)
    ref_loss, ref_stats, _ = linear.forward(case.X, case.W, case.targets, eps, case.ignore_idx,
                                            scale=scale)
    valid = case.targets != case.ignore_idx
    loss = out["loss"].cpu().numpy().astype(np.float64)
    assert np.all(loss[~valid] == 0.0)
    rel = float(np.max(np.abs(loss[valid] - ref_loss[valid]) / np.abs(ref_loss[valid])))
    assert rel <= LINEAR_LOSS_RTOL, rel
    st = out["stats"].cpu().numpy()[valid]
    rs = ref_stats[valid]
    np.testing.assert_allclose(st[:, 0], rs[:, 0], atol=1e-3 * scale)   # row max (scaled)
    np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-3)           # denominator
    np.testing.assert_allclose(st[:, 2], rs[:, 2], atol=1e-3 * scale)   # target logit (scaled)
    np.testing.assert_allclose(st[:, 3], rs[:, 3], atol=1e-4 * scale)   # logit mean (scaled)
    if reduce_loss:
        rm = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
        assert abs(out["mean"].item() - rm) <= LINEAR_LOSS_RTOL * abs(rm)
    g = oracle.row_scale(case.grad_output, case.targets, reduce_loss, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, eps, case.ignore_idx,
                               scale=scale)
    fx = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dX"])), rdX)
    fw = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dW"])), rdW)
    _say(f"scale {scale}: loss rel {rel:.2e}, dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL


def test_scaled_with_entropy_against_the_oracle():
    case = wl.make_linear(5130, 700, 256, 9000, ignore_frac=0.05, label_smoothing=0.1,
                          reduce_loss=True)
    scale = 1.6
    gH = np.random.default_rng(5131).uniform(-1.0, 1.0, case.M).astype(np.float32)
    out = _run(case, scale, with_entropy=True, gH=gH)
    ref_H = linear.entropy(case.X, case.W, case.targets, case.ignore_idx, scale=scale)
    e = np.abs(out["entropy"].cpu().numpy() - ref_H)
    rel = float(np.max(e / np.maximum(np.abs(ref_H), 1e-3)))
    assert rel <= LINEAR_LOSS_RTOL, f"entropy rel err {rel:.2e}"
    g = oracle.row_scale(case.grad_output, case.targets, True, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, 0.1, case.ignore_idx,
                               grad_entropy=gH.astype(np.float64), scale=scale)
    fx = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dX"])), rdX)
    fw = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dW"])), rdW)
    _say(f"entropy rel err {rel:.2e}; dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL


# --- vocabulary shards of the scaled form (tensor-parallel scaled linear CE) ---

from oracle import shard as oshard  # noqa: E402


def _run_shards(case, bounds, scale, *, Ws_bits=None, with_entropy=False, gH=None):
    """Shard forwards, merge, shard backwards through the binding."""
    X = to_device(case.X, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    if Ws_bits is None:
        Ws_bits = [np.ascontiguousarray(case.W[a:b]) for a, b in bounds]
    Ws = [to_device(w, "bf16") for w in Ws_bits]
    parts = torch.empty((len(bounds), case.M, 4), dtype=torch.float32, device="cuda")
    pws = torch.empty((len(bounds), case.M), dtype=torch.float32, device="cuda")
    for k, ((a, b), Wk) in enumerate(zip(bounds, Ws)):
        vce.lce_forward_shard(X, Wk, t, a, case.ignore_idx, out=parts[k],
                              with_entropy=with_entropy, out_w=pws[k], logit_scale=scale)
    m = vce.ce_merge_shards(parts, t, case.V, case.label_smoothing, case.reduce_loss,
                            case.ignore_idx, partials_w=pws if with_entropy else None)
    loss, mean, stats, nv = m[:4]
    ent = m[4] if with_entropy else None
    gHd = None if gH is None else torch.from_numpy(gH).cuda()
    outs = [vce.lce_backward_shard(X, Wk, t, a, case.V, stats, nv, go, case.label_smoothing,
                                   case.reduce_loss, case.ignore_idx, entropy=ent,
                                   grad_entropy=gHd, logit_scale=scale)
            for (a, b), Wk in zip(bounds, Ws)]
    torch.cuda.synchronize()
    return dict(parts=parts, pws=pws, loss=loss, mean=mean, stats=stats, n_valid=nv,
                entropy=ent, dX=[o[0] for o in outs], dW=[o[1] for o in outs])


SHARD_BOUNDS = [(0, 2000), (2000, 6500), (6500, 9000)]


def test_scaled_shards_against_the_oracle():
    case = wl.make_linear(5140, 700, 264, 9000, ignore_count=20, label_smoothing=0.1,
                          reduce_loss=True)
    scale = 0.7
    out = _run_shards(case, SHARD_BOUNDS, scale)
    valid = case.targets != case.ignore_idx
    for k, (a, b) in enumerate(SHARD_BOUNDS):
        ref = oshard.linear_shard_partials(case.X, case.W[a:b], case.targets, a,
                                           case.ignore_idx, scale=scale)
        got = out["parts"][k].cpu().numpy()
        assert np.all(got[~valid] == 0.0)
        np.testing.assert_allclose(got[valid, 0], ref[valid, 0], atol=1e-3)
        np.testing.assert_allclose(got[valid, 1], ref[valid, 1], rtol=2e-3)
        np.testing.assert_allclose(got[valid, 2], ref[valid, 2], rtol=1e-3, atol=0.05)
        np.testing.assert_allclose(got[valid, 3], ref[valid, 3], atol=1e-3)
    ref_loss, ref_stats, _ = linear.forward(case.X, case.W, case.targets, 0.1, case.ignore_idx,
                                            scale=scale)
    loss = out["loss"].cpu().numpy().reshape(-1).astype(np.float64)
    assert np.all(loss[~valid] == 0.0)
    rel = float(np.max(np.abs(loss[valid] - ref_loss[valid]) / np.abs(ref_loss[valid])))
    assert rel <= LINEAR_LOSS_RTOL, rel
    rm = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
    assert abs(out["mean"].item() - rm) <= LINEAR_LOSS_RTOL * abs(rm)
    g = oracle.row_scale(case.grad_output, case.targets, True, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, 0.1, case.ignore_idx,
                               scale=scale)
    for k, (a, b) in enumerate(SHARD_BOUNDS):
        rdXk, _ = oshard.linear_shard_backward(case.X, case.W[a:b], case.targets, a, case.V,
                                               ref_stats, g, 0.1, case.ignore_idx, scale=scale)
        fx = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dX"][k])), rdXk)
        fw = rel_frobenius(oracle.bf16_to_f64(to_host_bits(out["dW"][k])), rdW[a:b])
        assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL, (k, fx, fw)
    fsum = rel_frobenius(sum(oracle.bf16_to_f64(to_host_bits(d)) for d in out["dX"]), rdX)
    _say(f"shards, scale {scale}: loss rel {rel:.2e}, summed dX frob {fsum:.2e}")
    assert fsum <= LINEAR_FROB_RTOL


def test_scaled_shards_with_entropy_against_the_oracle():
    case = wl.make_linear(5150, 300, 192, 6000, ignore_count=9, label_smoothing=0.1,
                          reduce_loss=True)
    bounds = [(0, 2500), (2500, 6000)]
    scale = 1.6
    gH = (np.random.default_rng(5151).standard_normal(case.M) * 0.7).astype(np.float32)
    out = _run_shards(case, bounds, scale, with_entropy=True, gH=gH)
    valid = case.targets != case.ignore_idx
    H = out["entropy"].cpu().numpy().reshape(-1).astype(np.float64)
    ref_H = linear.entropy(case.X, case.W, case.targets, case.ignore_idx, scale=scale)
    assert np.all(H[~valid] == 0.0)
    rel = float(np.max(np.abs(H[valid] - ref_H[valid]) / np.abs(ref_H[valid])))
    assert rel <= LINEAR_LOSS_RTOL, rel
    g = oracle.row_scale(case.grad_output, case.targets, True, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, 0.1, case.ignore_idx,
                               grad_entropy=gH.astype(np.float64), scale=scale)
    dX = sum(oracle.bf16_to_f64(to_host_bits(d)) for d in out["dX"])
    dW = np.concatenate([oracle.bf16_to_f64(to_host_bits(d)) for d in out["dW"]])
    fx, fw = rel_frobenius(dX, rdX), rel_frobenius(dW, rdW)
    _say(f"shards with entropy, scale {scale}: H rel {rel:.2e}, dX frob {fx:.2e}, "
         f"dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL


def test_power_of_two_scale_shards_are_bitwise_the_scaled_classifier():
    # as for the unsharded form: s = 2^k on every shard equals the unscaled
    # shards of W 2^k exactly (partials, merged results and dX shares; dW
    # shares 2^k times theirs); the second shard spans two backward chunks
    case = wl.make_linear(5160, 520, 256, 70001, ignore_count=5, label_smoothing=0.1,
                          reduce_loss=False, grad_output="random")
    bounds = [(0, 33000), (33000, 70001)]
    s = 2.0 ** -3
    w2 = wl.bf16_bits_to_f32(case.W) * np.float32(s)
    W2 = wl.f32_to_bf16_bits(w2)
    assert np.array_equal(wl.bf16_bits_to_f32(W2), w2)
    a = _run_shards(case, bounds, s)
    b = _run_shards(case, bounds, 1.0, Ws_bits=[np.ascontiguousarray(W2[x:y]) for x, y in bounds])
    for k in ("parts", "loss", "stats"):
        assert torch.equal(a[k], b[k]), k
    for k in range(len(bounds)):
        assert torch.equal(a["dX"][k], b["dX"][k])
        assert torch.equal(a["dW"][k].float(), s * b["dW"][k].float())
    _say("shards, scale 2^-3: bitwise the unscaled shards of W * 2^-3")


def test_scale_one_through_the_scaled_shard_entry_points_is_bitwise_the_plain_ones():
    case = wl.make_linear(5170, 300, 264, 3000, ignore_count=7, label_smoothing=0.1,
                          reduce_loss=True)
    a0, a1 = 1000, 3000
    X = to_device(case.X, "bf16")
    Wk = to_device(np.ascontiguousarray(case.W[a0:a1]), "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    ws = vce.lce_workspace(case.M, case.H, a1 - a0)
    part, pw = vce.lce_forward_shard(X, Wk, t, a0, -100, workspace=ws, with_entropy=True)
    stats = torch.rand((case.M, 4), device="cuda") + 1.0  # any merged statistics will do
    nv = torch.full((), case.M - 7, dtype=torch.int32, device="cuda")
    dX, dW = vce.lce_backward_shard(X, Wk, t, a0, case.V, stats, nv, go, 0.1, True,
                                    workspace=ws)
    L = binding.lib()
    part1, pw1 = torch.empty_like(part), torch.empty_like(pw)
    dX1, dW1 = torch.empty_like(dX), torch.empty_like(dW)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.lce_forward_shard_scaled(p(X), p(Wk), case.M, case.H, a1 - a0, 1.0, p(t), a0,
                                      -100, p(part1), p(pw1), p(ws), ws.numel(), s) == 0
    assert L.lce_backward_shard_scaled(p(X), p(Wk), case.M, case.H, a1 - a0, 1.0, p(t), a0,
                                       case.V, p(stats), p(nv), p(go), None, None, 0.1, 1,
                                       -100, p(dX1), p(dW1), p(ws), ws.numel(), s) == 0
    torch.cuda.synchronize()
    for x, y in ((part, part1), (pw, pw1), (dX, dX1), (dW, dW1)):
        assert torch.equal(x, y)
