"""Parity of the vocabulary-sharded logits cross-entropy (ce_forward_shard,
ce_merge_shards, ce_backward_shard) with the FP64 oracle, through the C-ABI.

Each case draws the full logits, cuts the vocabulary into contiguous shards
(uneven, at unaligned column offsets), runs the per-shard forward on each,
stacks the partials in shard order as a gather would, merges, and runs the
per-shard backward.  Merged loss and statistics are held to the bar of the
unsharded forward against the unsharded oracle; every shard's gradient to the
bar of the unsharded gradient (the columns of the oracle's full-row
gradient).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import shard as oshard
import vocabulary_cross_entropy_amd as vce
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (assert_grad_bf16, assert_grad_fp32, assert_loss_close, grad_terms,
                          to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-shard] {msg}", flush=True)


def _bounds(V, k, seed):
    if k == 1:
        return [(0, V)]
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, V), k - 1, replace=False))
    b = [0, *[int(c) for c in cuts], V]
    return list(zip(b[:-1], b[1:]))


def _even_bounds(V, k):
    s = V // k
    return [(i * s, V if i == k - 1 else (i + 1) * s) for i in range(k)]


def run_sharded(case, bounds, *, separate=False, overwrite=False):
    """Sharded forward + merge + backward on the GPU.  ``separate``: each shard
    is its own contiguous tensor (as one process per shard would hold it);
    otherwise the shards are column views of one full tensor."""
    z = to_device(case.logits, case.dtype)
    t = torch.from_numpy(case.targets).cuda()
    N, V = case.N, case.V
    if separate:
        shards = [z[:, :, a:b].contiguous() for a, b in bounds]
    else:
        shards = [z[:, :, a:b] for a, b in bounds]
    parts = torch.empty((len(bounds), case.d0, case.d1, 4), dtype=torch.float32, device="cuda")
    for k, ((a, b), zk) in enumerate(zip(bounds, shards)):
        vce.ce_forward_shard(zk, t, a, case.ignore_idx, out=parts[k])
    loss, loss_mean, stats, n_valid = vce.ce_merge_shards(
        parts, t, V, case.label_smoothing, case.reduce_loss, case.ignore_idx)
    go = torch.from_numpy(case.grad_output).cuda()
    go = go.reshape(-1) if case.reduce_loss else go
    grads = []
    for (a, b), zk in zip(bounds, shards):
        gk = vce.ce_backward_shard(zk, t, a, V, stats, n_valid, go, case.label_smoothing,
                                   case.reduce_loss, case.ignore_idx, overwrite_input=overwrite)
        grads.append(gk)
    torch.cuda.synchronize()
    out = dict(parts=parts.cpu().numpy().reshape(len(bounds), N, 4),
               loss=loss.cpu().numpy().reshape(-1), stats=stats.cpu().numpy().reshape(-1, 4),
               grads=[to_host_bits(g).reshape(N, -1) for g in grads])
    if case.reduce_loss:
        out["loss_mean"] = float(loss_mean.item())
        out["n_valid"] = int(n_valid.item())
    return out


def check_partials(case, bounds, out, rows=None):
    N, V = case.N, case.V
    lg = case.logits.reshape(N, V)
    t = case.targets.reshape(-1)
    sel = np.arange(N) if rows is None else rows
    for k, (a, b) in enumerate(bounds):
        ref = oshard.shard_partials(lg[sel, a:b], t[sel], a, case.ignore_idx)
        got = out["parts"][k][sel]
        np.testing.assert_array_equal(got[:, 0], ref[:, 0].astype(np.float32))   # exact max
        np.testing.assert_array_equal(got[:, 3], ref[:, 3].astype(np.float32))   # exact z_t
        np.testing.assert_allclose(got[:, 1], ref[:, 1], rtol=2e-5)
        # sum z over V_local terms: FP32 accumulation, error below ~ V_local 2^-24 sum |z|
        zk = (oracle.bf16_to_f64(lg[sel, a:b]) if case.dtype == wl.DTYPE_BF16
              else lg[sel, a:b].astype(np.float64))
        fin = np.isfinite(ref[:, 2])
        np.testing.assert_array_equal(got[~fin, 2], ref[~fin, 2])
        with np.errstate(invalid="ignore"):
            bound = 1e-5 + (b - a) * 2.0 ** -22 * np.abs(zk[fin]).sum(1)
        assert np.all(np.abs(got[fin, 2] - ref[fin, 2]) <= bound), f"shard {k}: sum z"


def check_merged(case, out, rows=None):
    N = case.N
    sel = np.arange(N) if rows is None else rows
    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, case.label_smoothing,
                                               case.ignore_idx, rows=sel)
    err = assert_loss_close(out["loss"][sel], ref_loss, "merged loss")
    tsel = case.targets.reshape(-1)[sel]
    valid = (tsel != case.ignore_idx) & np.isfinite(ref_loss)
    st = out["stats"][sel][valid]
    rs = ref_stats[valid]
    np.testing.assert_array_equal(st[:, 0], rs[:, 0].astype(np.float32))
    np.testing.assert_array_equal(st[:, 2], rs[:, 2].astype(np.float32))
    np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-5)
    np.testing.assert_allclose(st[:, 3], rs[:, 3], rtol=0, atol=1e-5)
    assert np.all(out["stats"][sel][tsel == case.ignore_idx] == 0.0)
    if case.reduce_loss and rows is None:
        ref_mean = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
        assert abs(out["loss_mean"] - ref_mean) <= 1e-4 + 1e-5 * abs(ref_mean)
        assert out["n_valid"] == oracle.n_valid(case.targets, case.ignore_idx)
    return err


def check_grads(case, bounds, out, rows=None, chunk=256):
    N = case.N
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    tflat = case.targets.reshape(-1)
    sel = np.arange(N) if rows is None else np.asarray(rows)
    band = {}
    worst = 0
    for s in range(0, sel.size, chunk):
        rr = sel[s:s + chunk]
        ref = oracle.ce_backward(case.logits, case.targets, g, case.label_smoothing,
                                 case.ignore_idx, rows=rr)
        if case.dtype == wl.DTYPE_BF16:
            T = grad_terms(ref, g[rr], tflat[rr], case.label_smoothing, case.ignore_idx)
        for k, (a, b) in enumerate(bounds):
            gk = out["grads"][k][rr]
            if case.dtype == wl.DTYPE_BF16:
                worst = max(worst, assert_grad_bf16(gk, ref[:, a:b], T[:, a:b],
                                                    f"shard {k} rows {s}..", band))
            else:
                worst = max(worst, assert_grad_fp32(gk, ref[:, a:b], f"shard {k} rows {s}.."))
    if band:
        _say(f"grad: {band['elements']} elements, worst {band['worst_ulp']} ulp outside the "
             f"cancellation band; band {band['band']} elements")
    return worst


CASES = [
    # (name, case factory, number of shards, split seed)
    ("tiny_fp32_3", lambda: wl.make_logits(11, 2, 4, 1000, dtype=wl.DTYPE_FP32, sigma=2.0,
                                           ignore_count=1, label_smoothing=0.1), 3, 1),
    ("fp32_mean_5", lambda: wl.make_logits(12, 3, 77, 5003, dtype=wl.DTYPE_FP32, sigma=3.0,
                                           ignore_frac=0.1, reduce_loss=True,
                                           label_smoothing=0.2), 5, 2),
    ("bf16_v32000_8", lambda: wl.make_logits(13, 4, 256, 32000, dtype=wl.DTYPE_BF16, sigma=3.0,
                                             ignore_frac=0.05, label_smoothing=0.1,
                                             reduce_loss=True), 8, 3),
    ("bf16_sqb_v50257_7", lambda: wl.make_logits(14, 300, 2, 50257, dtype=wl.DTYPE_BF16,
                                                 sigma=4.0, ignore_frac=0.02, target_boost=8.0,
                                                 layout="SQ,B", grad_output="random"), 7, 4),
]


@pytest.mark.parametrize("separate", [False, True], ids=["views", "separate"])
@pytest.mark.parametrize("name,make,k,seed", CASES, ids=[c[0] for c in CASES])
def test_sharded_matches_oracle(name, make, k, seed, separate):
    case = make()
    bounds = _bounds(case.V, k, seed)
    _say(f"{name} N={case.N} V={case.V} shards={bounds} separate={separate}")
    out = run_sharded(case, bounds, separate=separate)
    check_partials(case, bounds, out)
    err = check_merged(case, out)
    worst = check_grads(case, bounds, out)
    _say(f"{name}: worst loss err {err:.2e}, worst grad {worst}")


def test_one_shard_is_bitwise_the_unsharded_forward():
    case = wl.make_logits(15, 8, 128, 32000, dtype=wl.DTYPE_BF16, sigma=3.0, ignore_frac=0.05,
                          label_smoothing=0.1, reduce_loss=True)
    z = to_device(case.logits, case.dtype)
    t = torch.from_numpy(case.targets).cuda()
    loss, mean, stats, nv = vce.ce_forward(z, t, 0.1, True, IGN)
    part = vce.ce_forward_shard(z, t, 0, IGN)
    l2, m2, s2, n2 = vce.ce_merge_shards(part.unsqueeze(0), t, case.V, 0.1, True, IGN)
    go = torch.ones(1, device="cuda")
    g1 = vce.ce_backward(z, t, stats, nv, go, 0.1, True, IGN)
    g2 = vce.ce_backward_shard(z, t, 0, case.V, s2, n2, go, 0.1, True, IGN)
    torch.cuda.synchronize()
    for name, a, b in (("loss", loss, l2), ("stats", stats, s2), ("mean", mean, m2)):
        a, b = a.cpu().numpy().reshape(-1), b.cpu().numpy().reshape(-1)
        diff = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0]
        assert diff.size == 0, (f"{name}: {diff.size} differ, first at {diff[:4]}: "
                                f"{a[diff[:4]]} vs {b[diff[:4]]}")
    assert torch.equal(nv, n2)
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))


def test_headline_shape_eight_shards_sampled():
    """(SQ, B, V) = (2048, 2, 128256) BF16 over 8 shards of 16032 columns, each
    its own contiguous tensor; loss and statistics on every row, partials and
    gradients on sampled rows (the oracle recomputes those rows in full)."""
    case = wl.headline_logits()
    bounds = _even_bounds(case.V, 8)
    _say(f"headline shard shape N={case.N} V={case.V} V_local={bounds[0][1] - bounds[0][0]}")
    out = run_sharded(case, bounds, separate=True)
    rows = np.random.default_rng(5).choice(case.N, 192, replace=False)
    check_partials(case, bounds, out, rows=rows)
    check_merged(case, out)
    check_grads(case, bounds, out, rows=rows)


def test_in_place_shard_backward():
    case = wl.make_logits(16, 2, 64, 9001, dtype=wl.DTYPE_BF16, sigma=3.0, ignore_count=3,
                          label_smoothing=0.05)
    bounds = _bounds(case.V, 4, 6)
    out = run_sharded(case, bounds, separate=True, overwrite=True)
    check_merged(case, out)
    check_grads(case, bounds, out)


def test_edge_targets_and_padded_shard():
    # targets: ignored, = V (outside), negative, in the last real column, in the
    # first column of a shard; the last shard is padded vocabulary (-inf)
    case = wl.make_logits(17, 1, 12, 4099, dtype=wl.DTYPE_FP32, sigma=2.0, label_smoothing=0.0)
    V = case.V
    z = case.logits.reshape(12, V)
    z[:, 4000:] = -np.inf
    bounds = [(0, 1500), (1500, 2901), (2901, 4000), (4000, V)]
    t = case.targets.reshape(-1)
    t[:] = np.minimum(t, 3999)
    t[0], t[1], t[2], t[3], t[4] = IGN, V, -7, 3999, 1500
    out = run_sharded(case, bounds)
    assert out["loss"][0] == 0.0 and np.isnan(out["loss"][1]) and np.isnan(out["loss"][2])
    check_partials(case, bounds, out)
    check_merged(case, out)
    check_grads(case, bounds, out)
    # padded columns: p = 0, so the gradient there is -g eps / V = 0 here
    assert np.all(out["grads"][3][3:] == 0.0)


# --- linear form ---------------------------------------------------------------

from oracle import linear  # noqa: E402
from vce_testutil import LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, rel_frobenius  # noqa: E402


def run_linear_sharded(case, bounds):
    X = to_device(case.X, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    Ws = [to_device(np.ascontiguousarray(case.W[a:b]), "bf16") for a, b in bounds]
    parts = torch.empty((len(bounds), case.M, 4), dtype=torch.float32, device="cuda")
    for k, ((a, b), Wk) in enumerate(zip(bounds, Ws)):
        vce.lce_forward_shard(X, Wk, t, a, case.ignore_idx, out=parts[k])
    loss, mean, stats, nv = vce.ce_merge_shards(parts, t, case.V, case.label_smoothing,
                                                case.reduce_loss, case.ignore_idx)
    outs = [vce.lce_backward_shard(X, Wk, t, a, case.V, stats, nv, go, case.label_smoothing,
                                   case.reduce_loss, case.ignore_idx)
            for (a, b), Wk in zip(bounds, Ws)]
    torch.cuda.synchronize()
    out = dict(parts=parts.cpu().numpy(), loss=loss.cpu().numpy().reshape(-1).astype(np.float64),
               stats=stats.cpu().numpy().reshape(-1, 4),
               dX=[oracle.bf16_to_f64(to_host_bits(o[0])) for o in outs],
               dW=[oracle.bf16_to_f64(to_host_bits(o[1])) for o in outs])
    if case.reduce_loss:
        out["mean"] = float(mean.item())
        out["n_valid"] = int(nv.item())
    return out


LINEAR_CASES = [
    ("m700_h264_v9000_3", lambda: wl.make_linear(21, 700, 264, 9000, ignore_count=20,
                                                 label_smoothing=0.1, reduce_loss=True),
     [(0, 2000), (2000, 6500), (6500, 9000)]),
    # the second shard spans two backward chunks of the vocabulary
    ("m520_h256_v70001_2", lambda: wl.make_linear(22, 520, 256, 70001, ignore_count=5,
                                                  reduce_loss=False, grad_output="random"),
     [(0, 33000), (33000, 70001)]),
]


@pytest.mark.parametrize("name,make,bounds", LINEAR_CASES, ids=[c[0] for c in LINEAR_CASES])
def test_linear_sharded_matches_oracle(name, make, bounds):
    case = make()
    _say(f"linear {name} M={case.M} H={case.H} V={case.V} shards={bounds}")
    out = run_linear_sharded(case, bounds)
    valid = case.targets != case.ignore_idx
    # local statistics of each shard
    for k, (a, b) in enumerate(bounds):
        ref = oshard.linear_shard_partials(case.X, case.W[a:b], case.targets, a, case.ignore_idx)
        got = out["parts"][k]
        assert np.all(got[~valid] == 0.0)
        np.testing.assert_allclose(got[valid, 0], ref[valid, 0], atol=1e-3)
        np.testing.assert_allclose(got[valid, 1], ref[valid, 1], rtol=2e-3)
        np.testing.assert_allclose(got[valid, 2], ref[valid, 2], rtol=1e-3, atol=0.05)
        np.testing.assert_allclose(got[valid, 3], ref[valid, 3], atol=1e-3)
        outside = valid & ~((case.targets >= a) & (case.targets < b))
        assert np.all(got[outside, 3] == 0.0)
    # merged loss and statistics against the unsharded oracle
    ref_loss, ref_stats, _ = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                                            case.ignore_idx)
    assert np.all(out["loss"][~valid] == 0.0)
    rel = np.abs(out["loss"][valid] - ref_loss[valid]) / np.abs(ref_loss[valid])
    assert rel.max() <= LINEAR_LOSS_RTOL, rel.max()
    np.testing.assert_allclose(out["stats"][valid, 1], ref_stats[valid, 1], rtol=2e-3)
    np.testing.assert_allclose(out["stats"][valid, 2], ref_stats[valid, 2], atol=1e-3)
    if case.reduce_loss:
        rm = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
        assert abs(out["mean"] - rm) <= LINEAR_LOSS_RTOL * abs(rm)
        assert out["n_valid"] == oracle.n_valid(case.targets, case.ignore_idx)
    # gradients: dW rows per shard, dX shares per shard and their sum
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, case.label_smoothing,
                               case.ignore_idx)
    for k, (a, b) in enumerate(bounds):
        rdXk, _ = oshard.linear_shard_backward(case.X, case.W[a:b], case.targets, a, case.V,
                                               ref_stats, g, case.label_smoothing,
                                               case.ignore_idx)
        fw = rel_frobenius(out["dW"][k], rdW[a:b])
        fx = rel_frobenius(out["dX"][k], rdXk)
        _say(f"shard {k}: dW frob {fw:.2e}, dX share frob {fx:.2e}")
        assert fw <= LINEAR_FROB_RTOL and fx <= LINEAR_FROB_RTOL
    fsum = rel_frobenius(sum(out["dX"]), rdX)
    _say(f"{name}: loss rel {rel.max():.2e}, summed dX frob {fsum:.2e}")
    assert fsum <= LINEAR_FROB_RTOL


def test_linear_empty_batch_zeroes_dW():
    H, V = 64, 1000
    X = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    W = torch.randn((V, H), device="cuda").to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    st = torch.empty((0, 4), device="cuda")
    go = torch.ones(1, device="cuda")
    nv = torch.zeros((), dtype=torch.int32, device="cuda")
    ws = vce.lce_workspace(0, H, V)
    dW = torch.full_like(W, 3.0)
    vce.lce_backward(X, W, t, st, nv, go, workspace=ws, dW=dW)
    dW2 = torch.full_like(W, 3.0)
    vce.lce_backward_shard(X, W, t, 0, 2 * V, st, nv, go, workspace=ws, dW=dW2)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW).item() == 0 and torch.count_nonzero(dW2).item() == 0


# --- entropy over shards (the optional entropy of the tensor-parallel forward) ---------

def _stack_entropy_logits(case, bounds, zd, t):
    parts = torch.empty((len(bounds), case.d0, case.d1, 4), dtype=torch.float32, device="cuda")
    pws = torch.empty((len(bounds), case.d0, case.d1), dtype=torch.float32, device="cuda")
    shards = [zd[:, :, a:b].contiguous() for a, b in bounds]
    for k, ((a, b), zk) in enumerate(zip(bounds, shards)):
        vce.ce_forward_shard(zk, t, a, case.ignore_idx, out=parts[k], with_entropy=True,
                             out_w=pws[k])
    return shards, parts, pws


@pytest.mark.parametrize("dtype,V,k", [("bf16", 9000, 3), ("fp32", 4099, 4), ("bf16", 128256, 8)])
def test_sharded_entropy_logits(dtype, V, k):
    case = wl.make_logits(4100 + k, 4, 64, V, dtype=dtype, sigma=3.0, ignore_count=9,
                          label_smoothing=0.1, reduce_loss=True)
    bounds = _bounds(V, k, 17)
    _say(f"sharded entropy {dtype} V={V} shards={len(bounds)}")
    zd = to_device(case.logits, dtype)
    t = torch.from_numpy(case.targets).cuda()
    shards, parts, pws = _stack_entropy_logits(case, bounds, zd, t)
    loss, mean, stats, nv, ent = vce.ce_merge_shards(parts, t, V, 0.1, True, case.ignore_idx,
                                                     partials_w=pws)
    # the shards' w against the oracle's local statistic
    N = case.N
    lg = case.logits.reshape(N, V)
    valid = case.targets.reshape(-1) != case.ignore_idx
    for kk, (a, b) in enumerate(bounds):
        ref_w = oshard.shard_partials_w(lg[:, a:b], case.targets, case.ignore_idx)
        got_w = pws[kk].cpu().numpy().reshape(-1).astype(np.float64)
        assert np.all(got_w[~valid] == 0.0)
        np.testing.assert_allclose(got_w[valid], ref_w[valid], rtol=2e-5, atol=2e-3)
    # merged entropy against the unsharded oracle, at the loss bar
    H = ent.cpu().numpy().reshape(-1).astype(np.float64)
    ref_H = oracle.entropy(case.logits, case.targets, case.ignore_idx)
    assert_loss_close(H, ref_H)
    # the gradient with an entropy term: every shard's columns are bitwise the
    # unsharded backward's from the same merged statistics and entropy
    gH = (np.random.default_rng(5).standard_normal((case.d0, case.d1)) * 0.7).astype(np.float32)
    gHd = torch.from_numpy(gH).cuda()
    go = torch.ones(1, device="cuda")
    full = vce.ce_backward(zd, t, stats, nv, go, 0.1, True, case.ignore_idx, entropy=ent,
                           grad_entropy=gHd)
    for (a, b), zk in zip(bounds, shards):
        gk = vce.ce_backward_shard(zk, t, a, V, stats, nv, go, 0.1, True, case.ignore_idx,
                                   entropy=ent, grad_entropy=gHd)
        assert torch.equal(gk, full[:, :, a:b].contiguous()), (a, b)
    torch.cuda.synchronize()


def test_one_shard_entropy_is_bitwise_the_unsharded_one():
    case = wl.make_logits(4200, 8, 32, 5003, dtype="bf16", sigma=3.0, ignore_count=7,
                          label_smoothing=0.0, reduce_loss=False)
    zd = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    part, pw = vce.ce_forward_shard(zd, t, 0, IGN, with_entropy=True)
    l2, _, s2, _, e2 = vce.ce_merge_shards(part.unsqueeze(0), t, case.V, 0.0, False, IGN,
                                           partials_w=pw.unsqueeze(0))
    l1, _, s1, _, e1 = vce.ce_forward(zd, t, 0.0, False, IGN, with_entropy=True)
    torch.cuda.synchronize()
    assert torch.equal(e1, e2) and torch.equal(l1, l2) and torch.equal(s1, s2)


def test_linear_sharded_entropy():
    case = wl.make_linear(4300, 300, 192, 6000, ignore_count=9, label_smoothing=0.1,
                          reduce_loss=True)
    bounds = [(0, 2500), (2500, 6000)]
    X = to_device(case.X, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    Ws = [to_device(np.ascontiguousarray(case.W[a:b]), "bf16") for a, b in bounds]
    parts = torch.empty((2, case.M, 4), dtype=torch.float32, device="cuda")
    pws = torch.empty((2, case.M), dtype=torch.float32, device="cuda")
    for k, ((a, b), Wk) in enumerate(zip(bounds, Ws)):
        vce.lce_forward_shard(X, Wk, t, a, IGN, out=parts[k], with_entropy=True, out_w=pws[k])
    loss, mean, stats, nv, ent = vce.ce_merge_shards(parts, t, case.V, 0.1, True, IGN,
                                                     partials_w=pws)
    gH = (np.random.default_rng(6).standard_normal(case.M) * 0.7).astype(np.float32)
    gHd = torch.from_numpy(gH).cuda()
    go = torch.ones(1, device="cuda")
    outs = [vce.lce_backward_shard(X, Wk, t, a, case.V, stats, nv, go, 0.1, True, IGN,
                                   entropy=ent, grad_entropy=gHd)
            for (a, b), Wk in zip(bounds, Ws)]
    torch.cuda.synchronize()
    valid = case.targets != IGN
    H = ent.cpu().numpy().reshape(-1).astype(np.float64)
    ref_H = linear.entropy(case.X, case.W, case.targets, IGN)
    assert np.all(H[~valid] == 0.0)
    rel = np.abs(H[valid] - ref_H[valid]) / np.abs(ref_H[valid])
    assert rel.max() <= LINEAR_LOSS_RTOL, rel.max()
    g = oracle.row_scale(case.grad_output, case.targets, True, IGN)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, 0.1, IGN,
                               grad_entropy=gH.astype(np.float64))
    dX = sum(oracle.bf16_to_f64(to_host_bits(o[0])) for o in outs)
    dW = np.concatenate([oracle.bf16_to_f64(to_host_bits(o[1])) for o in outs])
    fx, fw = rel_frobenius(dX, rdX), rel_frobenius(dW, rdW)
    _say(f"linear sharded entropy: H rel {rel.max():.2e}, dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL
