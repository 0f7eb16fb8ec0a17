"""Parity of the HIP fused linear cross-entropy (lce_forward / lce_backward)
and of its matrix-core GEMM building block with the FP64 oracle."""
import hashlib
import os
import time

import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import LINEAR_FROB_RTOL, LINEAR_LOSS_RTOL, rel_frobenius, to_device, to_host_bits

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _say(msg):
    print(f"[parity-lce] {msg}", flush=True)


def _bf16(a):
    return to_device(a, "bf16")


# --- the GEMM building block -----------------------------------------------------

@pytest.mark.parametrize("p_dim,q_dim", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("rows,cols,K", [(300, 520, 200), (512, 768, 4096), (40, 8, 8),
                                         (776, 1000, 4104), (4096, 256, 64), (264, 256, 333),
                                         (264, 520, 128), (520, 256, 256), (256, 264, 192)])
def test_gemm(rows, cols, K, p_dim, q_dim):
    """The GEMM core in each operand layout against an FP64 product of the same
    BF16 values.  Ragged rows, columns and K cover the masked loads; a
    dim-contiguous operand needs its dim to be a multiple of 8 and a
    K-contiguous one its K."""
    if (not p_dim or not q_dim) and K % 8:
        pytest.skip("a K-contiguous operand needs K % 8 == 0")
    if (p_dim and rows % 8) or (q_dim and cols % 8):
        pytest.skip("a dim-contiguous operand needs its dim % 8 == 0")
    rng = np.random.default_rng(rows * 7 + cols + K)
    Pm = wl.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    Qm = wl.f32_to_bf16_bits(rng.standard_normal((cols, K)).astype(np.float32))
    Pd = _bf16(np.ascontiguousarray(Pm.T) if p_dim else Pm)
    Qd = _bf16(np.ascontiguousarray(Qm.T) if q_dim else Qm)
    C = vce.gemm_bf16(Pd, Qd, K, p_dim=p_dim, q_dim=q_dim)
    torch.cuda.synchronize()
    Pf, Qf = oracle.bf16_to_f64(Pm), oracle.bf16_to_f64(Qm)
    ref = Pf @ Qf.T
    scale = np.abs(Pf) @ np.abs(Qf).T
    err = np.abs(C.cpu().numpy().astype(np.float64) - ref)
    # FP32 accumulation of exact BF16 products: error far below 2^-14 of the
    # sum of |terms|; an indexing mistake gives errors of the order of the terms
    assert np.all(err <= 2.0 ** -14 * scale + 1e-30), float((err / (scale + 1e-30)).max())


@pytest.mark.parametrize("p_dim,q_dim", [(False, False), (True, True)])
def test_gemm_empty_k(p_dim, q_dim):
    """K = 0: the empty sum writes zeros over whatever C held (the tile's first
    k-step normally writes the accumulators; with no k-step they are cleared)."""
    rows, cols = 264, 520
    P = _bf16(wl.f32_to_bf16_bits(np.ones((8, rows) if p_dim else (rows, 8), np.float32)))
    Q = _bf16(wl.f32_to_bf16_bits(np.ones((8, cols) if q_dim else (cols, 8), np.float32)))
    C = torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    vce.gemm_bf16(P, Q, 0, p_dim=p_dim, q_dim=q_dim, out=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0


# --- helpers -----------------------------------------------------------------------

def run_lce(case, ws=None):
    X, W = _bf16(case.X), _bf16(case.W)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    loss, mean, stats, nv = vce.lce_forward(X, W, t, case.label_smoothing, case.reduce_loss,
                                            case.ignore_idx, workspace=ws)
    dX, dW = vce.lce_backward(X, W, t, stats, nv, go, case.label_smoothing, case.reduce_loss,
                              case.ignore_idx, workspace=ws)
    torch.cuda.synchronize()
    out = dict(loss=loss.cpu().numpy().astype(np.float64), stats=stats.cpu().numpy(),
               dX=oracle.bf16_to_f64(to_host_bits(dX)), dW_dev=dW)
    if case.reduce_loss:
        out["mean"] = float(mean.item())
        out["n_valid"] = int(nv.item())
    return out


def check_loss(case, out, ref_loss, ref_stats=None):
    valid = case.targets != case.ignore_idx
    assert np.all(out["loss"][~valid] == 0.0)
    rel = np.abs(out["loss"][valid] - ref_loss[valid]) / np.abs(ref_loss[valid])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= LINEAR_LOSS_RTOL, worst
    if case.reduce_loss:
        rm = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
        assert abs(out["mean"] - rm) <= LINEAR_LOSS_RTOL * abs(rm)
        assert out["n_valid"] == oracle.n_valid(case.targets, case.ignore_idx)
    if ref_stats is not None:
        st, rs = out["stats"][valid], ref_stats[valid]
        np.testing.assert_allclose(st[:, 0], rs[:, 0], atol=1e-3)       # row max of FP32 logits
        np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-3)       # denominator
        np.testing.assert_allclose(st[:, 2], rs[:, 2], atol=1e-3)       # target logit
        np.testing.assert_allclose(st[:, 3], rs[:, 3], atol=1e-4)       # logit mean
    return worst


def full_check(case):
    out = run_lce(case)
    ref_loss, ref_stats, _ = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                                            case.ignore_idx)
    lw = check_loss(case, out, ref_loss, ref_stats)
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, case.label_smoothing,
                               case.ignore_idx)
    dW = oracle.bf16_to_f64(to_host_bits(out["dW_dev"]))
    fx, fw = rel_frobenius(out["dX"], rdX), rel_frobenius(dW, rdW)
    _say(f"{case.name}: loss rel {lw:.2e}, dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL
    return out


@pytest.mark.parametrize("eps", [0.0, 0.1, 1.0])
@pytest.mark.parametrize("reduce_loss", [True, False])
def test_linear_small(eps, reduce_loss):
    case = wl.make_linear(3001, 300, 264, 1000, ignore_count=7, label_smoothing=eps,
                          reduce_loss=reduce_loss, grad_output="random",
                          name=f"small_eps{eps}_red{int(reduce_loss)}")
    full_check(case)


@pytest.mark.parametrize("log2_scale", [14, 22])
def test_linear_large_logits(log2_scale):
    # W scaled by 2^k (exact in BF16) puts the logits near 2^k: the exponent
    # offsets m log2(e) and lse log2(e) then round by up to 2^(k-24), which the
    # epilogues take back out per token.
    case = wl.make_linear(3010 + log2_scale, 300, 264, 3000, ignore_count=7,
                          label_smoothing=0.1, reduce_loss=True,
                          name=f"large_logits_2^{log2_scale}")
    w = wl.bf16_bits_to_f32(case.W) * np.float32(2.0 ** log2_scale)
    case.W = wl.f32_to_bf16_bits(w)
    assert np.array_equal(wl.bf16_bits_to_f32(case.W), w)
    out = run_lce(case)
    ref_loss, ref_stats, _ = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                                            case.ignore_idx)
    lw = check_loss(case, out, ref_loss)
    # The logits themselves carry the FP32 GEMM's rounding, relative to their
    # size (here up to about 2^(k+2)), so the row max and the target logit are
    # compared relative to that size; d = sum exp(z - m) inherits absolute
    # logit errors of that order and is not compared.
    valid = case.targets != case.ignore_idx
    st, rs = out["stats"][valid], ref_stats[valid]
    size = 2.0 ** (log2_scale + 3)
    np.testing.assert_allclose(st[:, 0], rs[:, 0], rtol=0, atol=2e-5 * size)
    np.testing.assert_allclose(st[:, 2], rs[:, 2], rtol=0, atol=2e-5 * size)
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rdX, rdW = linear.backward(case.X, case.W, case.targets, g, case.label_smoothing,
                               case.ignore_idx)
    dW = oracle.bf16_to_f64(to_host_bits(out["dW_dev"]))
    fx, fw = rel_frobenius(out["dX"], rdX), rel_frobenius(dW, rdW)
    _say(f"{case.name}: loss rel {lw:.2e}, dX frob {fx:.2e}, dW frob {fw:.2e}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL


def test_linear_multichunk_ragged_vocab():
    # three backward chunks, the last ragged; V not a multiple of any tile
    case = wl.make_linear(3002, 520, 136, 70001, ignore_frac=0.05, label_smoothing=0.1,
                          reduce_loss=False, grad_output="random", name="m520_h136_v70001")
    full_check(case)


@pytest.mark.parametrize("M", [4097, 5000])
def test_linear_token_wave_boundaries(M):
    case = wl.make_linear(3003 + M, M, 128, 3001, ignore_frac=0.03, targets="zipf",
                          label_smoothing=0.1, reduce_loss=True, name=f"m{M}_h128_v3001")
    full_check(case)


@pytest.mark.parametrize("M,H,V", [(1, 8, 7), (3, 16, 300), (257, 8, 2), (17, 72, 257),
                                   (40, 8, 65)])
def test_linear_degenerate_shapes(M, H, V):
    # one token, the narrowest hidden size (one 8-element chunk of a K slice),
    # two classes, one row past a token tile, one column past a vocabulary tile
    case = wl.make_linear(3020 + M + V, M, H, V, ignore_count=0, label_smoothing=0.1,
                          reduce_loss=M > 2, grad_output="random", name=f"m{M}_h{H}_v{V}")
    full_check(case)


def test_linear_single_class():
    # V = 1: p = 1 = q for every row, so the loss and both gradients are 0 (to
    # within the rounding of exp(0) and of the statistics)
    case = wl.make_linear(3030, 40, 24, 1, ignore_count=3, label_smoothing=0.1,
                          reduce_loss=False, grad_output="random")
    out = run_lce(case)
    ref_loss, _, _ = linear.forward(case.X, case.W, case.targets, 0.1, case.ignore_idx)
    assert np.all(ref_loss == 0.0)
    assert np.max(np.abs(out["loss"])) <= 1e-6
    # each dZ entry is g_r (p - 1) with p = 1 to within a few FP32 roundings:
    # at most g_r 2^-20 (16 roundings), and dX, dW at most that through W, X
    g = oracle.row_scale(case.grad_output, case.targets, False, case.ignore_idx)
    u = 2.0 ** -20 * np.abs(g)
    xa, wa = np.abs(oracle.bf16_to_f64(case.X)), np.abs(oracle.bf16_to_f64(case.W))
    dW = oracle.bf16_to_f64(to_host_bits(out["dW_dev"]))
    assert np.all(np.abs(out["dX"]) <= u[:, None] * wa.sum(axis=0)[None, :])
    assert np.all(np.abs(dW) <= (u @ xa)[None, :])


def test_linear_all_ignored():
    case = wl.make_linear(3004, 64, 64, 500, ignore_count=64, reduce_loss=True)
    out = run_lce(case)
    assert out["mean"] == 0.0 and out["n_valid"] == 0
    assert np.all(out["dX"] == 0.0)
    assert torch.count_nonzero(out["dW_dev"].float()).item() == 0


def test_linear_matches_logits_form():
    # lce_forward(X, W) against ce_forward on Z = X W^T formed by the same GEMM core
    case = wl.make_linear(3005, 256, 512, 4096, ignore_count=5, label_smoothing=0.1,
                          reduce_loss=True)
    X, W = _bf16(case.X), _bf16(case.W)
    t = torch.from_numpy(case.targets).cuda()
    loss, mean, stats, nv = vce.lce_forward(X, W, t, 0.1, True)
    Z = vce.gemm_bf16(X, W)
    loss2, mean2, stats2, nv2 = vce.ce_forward(Z, t, 0.1, True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(loss.cpu().numpy(), loss2.cpu().numpy().reshape(-1), rtol=1e-5,
                               atol=1e-5)
    assert nv.item() == nv2.item()


def test_linear_graph_capture_replay():
    # lce_forward and lce_backward only enqueue kernels on the given stream
    # (no allocation, no memset, no synchronisation), so both can be captured
    # into one graph and replayed; every replay must equal the eager result
    # bit for bit (the kernels are deterministic).  Two vocabulary chunks make
    # the dX accumulator path part of the graph.
    case = wl.make_linear(3007, 600, 256, 40000, ignore_frac=0.05, label_smoothing=0.1,
                          reduce_loss=True)
    X, W = _bf16(case.X), _bf16(case.W)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    M, H, V = case.X.shape[0], case.X.shape[1], case.W.shape[0]
    ws = vce.lce_workspace(M, H, V)
    loss = torch.empty(M, device="cuda")
    mean = torch.empty((), device="cuda")
    stats = torch.empty((M, 4), device="cuda")
    nv = torch.empty((), dtype=torch.int32, device="cuda")
    dX, dW = torch.empty_like(X), torch.empty_like(W)
    out = (loss, mean, stats, nv)
    vce.lce_forward(X, W, t, 0.1, True, workspace=ws, out=out)
    vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, workspace=ws, dX=dX, dW=dW)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (loss, mean, stats, dX, dW)]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            vce.lce_forward(X, W, t, 0.1, True, workspace=ws, out=out, stream=s)
            vce.lce_backward(X, W, t, stats, nv, go, 0.1, True, workspace=ws, dX=dX, dW=dW,
                             stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (loss, mean, stats, dX, dW):
            x.zero_()
        ws.fill_(0xAB)  # eager work between replays; the graph must not depend on it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "mean", "stats", "dX", "dW"), (loss, mean, stats, dX, dW),
                              ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
    _say("graph capture + 3 replays of lce_forward + lce_backward: bit-identical")


def test_linear_deterministic():
    case = wl.make_linear(3006, 700, 192, 9000, ignore_frac=0.1, label_smoothing=0.1)
    a, b = run_lce(case), run_lce(case)
    np.testing.assert_array_equal(a["loss"], b["loss"])
    np.testing.assert_array_equal(a["dX"], b["dX"])
    assert torch.equal(a["dW_dev"], b["dW_dev"])


# --- the full-size workloads: every token's loss against stored oracle values,
# --- sampled rows of dX and dW, invariants, then the whole dX and dW --------------

def _digest(case):
    h = hashlib.sha256()
    for a in (case.X, case.W, case.targets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def full_size(case):
    gold = np.load(os.path.join(GOLDEN, case.name + ".npz"))
    assert str(gold["digest"]) == _digest(case), "regenerated inputs differ from the golden's"
    out = run_lce(case)
    lw = check_loss(case, out, gold["loss"], gold["stats"])
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    rng = np.random.default_rng(7)
    valid = np.nonzero(case.targets != case.ignore_idx)[0]
    rows = np.unique(np.concatenate([rng.choice(valid, 24, replace=False), [0, case.M - 1]]))
    rdx = linear.dx_rows(case.X, case.W, case.targets, g, rows, case.label_smoothing,
                         case.ignore_idx)
    fx = rel_frobenius(out["dX"][rows], rdx)
    V = case.V
    vrows = np.unique(np.concatenate([rng.choice(V, 24, replace=False),
                                      [0, 1, 2, V - 1, V - 2, 32767, 32768],
                                      np.unique(case.targets[valid])[:4]]))
    vrows = vrows[vrows < V]
    rdw = linear.dw_rows(case.X, case.W, case.targets, g, gold["lse"], vrows,
                         case.label_smoothing, case.ignore_idx)
    dW = out["dW_dev"]
    dws = oracle.bf16_to_f64(to_host_bits(dW[torch.from_numpy(vrows).cuda()]))
    fw = rel_frobenius(dws, rdw)
    # Invariant at full size: every row of dZ sums to zero, so every column of
    # dW sums to zero up to BF16 rounding.  Rounding model: dZ entries and dW
    # entries carry relative errors below 2^-9; the dominant dZ entry of a row,
    # g_r (p_t - 1), is close to the same value -g for most rows, so its
    # rounding error is systematic (bounded by 2^-8 |sum_r g_r X_rh|); the rest
    # are independent (at most 6 standard deviations of their sum).
    colsum = dW.double().sum(dim=0).cpu().numpy()
    D = (dW.double() ** 2).sum(dim=0).cpu().numpy()
    Xf = oracle.bf16_to_f64(case.X)
    gx = g[:, None] * Xf
    S, Q = gx.sum(axis=0), (gx ** 2).sum(axis=0)
    bound = 2.0 ** -8 * np.abs(S) + 6 * 2.0 ** -9 * np.sqrt((Q + D) / 3)
    ratio = float(np.max(np.abs(colsum) / bound))
    _say(f"{case.name}: loss rel {lw:.2e}, dX rows frob {fx:.2e}, dW rows frob {fw:.2e}, "
         f"max |colsum dW| / bound {ratio:.2f}")
    assert fx <= LINEAR_FROB_RTOL and fw <= LINEAR_FROB_RTOL
    assert ratio <= 1.0
    # The whole dX and dW against the FP64 oracle (the Liger-Kernel PR reports
    # its error over whole tensors, Correctness).  The oracle runs over token
    # ranges to bound host memory: each range gives its dX rows and its share
    # of dW = sum over tokens of dZ_r^T X_r, summed here.
    dWg = oracle.bf16_to_f64(to_host_bits(dW))
    del dW, out["dW_dev"]
    t0 = time.perf_counter()
    ref_dW = np.zeros(dWg.shape)
    num_x = den_x = 0.0
    step = 2048
    for s in range(0, case.M, step):
        e = min(case.M, s + step)
        rdx_s, rdw_s = linear.backward(case.X[s:e], case.W, case.targets[s:e], g[s:e],
                                       case.label_smoothing, case.ignore_idx)
        num_x += float(np.sum((out["dX"][s:e] - rdx_s) ** 2))
        den_x += float(np.sum(rdx_s ** 2))
        ref_dW += rdw_s
        del rdx_s, rdw_s
        _say(f"  oracle dX/dW over tokens {s}..{e - 1}: {time.perf_counter() - t0:.0f} s")
    fxw = (num_x / den_x) ** 0.5
    fww = rel_frobenius(dWg, ref_dW)
    _say(f"{case.name}: whole-matrix relative Frobenius error dX {fxw:.2e}, dW {fww:.2e} "
         f"(oracle {time.perf_counter() - t0:.0f} s)")
    assert fxw <= LINEAR_FROB_RTOL and fww <= LINEAR_FROB_RTOL


def test_linear_m4096_h4096_v131072():
    case = wl.linear_4k()
    _say(case.name)
    full_size(case)


def test_linear_m16384_h2304_v256003():
    case = wl.linear_16k()
    _say(case.name)
    full_size(case)
