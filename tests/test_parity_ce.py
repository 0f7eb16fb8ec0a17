"""Parity of the HIP logits cross-entropy (ce_forward / ce_backward) with the
FP64 oracle, element by element, through the C-ABI."""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import (assert_grad_bf16, assert_grad_fp32, assert_loss_close, grad_terms,
                          to_device, to_host_bits)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-ce] {msg}", flush=True)


def run_case(case: wl.LogitsCase, overwrite: bool = False, logits_dev=None):
    """Forward and backward on the GPU; returns host copies of everything."""
    z = to_device(case.logits, case.dtype) if logits_dev is None else logits_dev
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    loss, loss_mean, stats, n_valid = vce.ce_forward(z, t, case.label_smoothing, case.reduce_loss,
                                                     case.ignore_idx)
    grad = vce.ce_backward(z, t, stats, n_valid, go.reshape(-1) if case.reduce_loss else go,
                           case.label_smoothing, case.reduce_loss, case.ignore_idx,
                           overwrite_input=overwrite)
    torch.cuda.synchronize()
    out = dict(loss=loss.cpu().numpy(), stats=stats.cpu().numpy().reshape(-1, 4),
               grad=to_host_bits(grad))
    if case.reduce_loss:
        out["loss_mean"] = float(loss_mean.item())
        out["n_valid"] = int(n_valid.item())
    return out


def check_forward(case, out):
    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, case.label_smoothing,
                                               case.ignore_idx)
    err = assert_loss_close(out["loss"], ref_loss)
    valid = (case.targets.reshape(-1) != case.ignore_idx) & np.isfinite(ref_loss)
    st = out["stats"][valid]
    rs = ref_stats[valid]
    # row max and target logit are exact input values: bitwise equal
    np.testing.assert_array_equal(st[:, 0], rs[:, 0].astype(np.float32))
    np.testing.assert_array_equal(st[:, 2], rs[:, 2].astype(np.float32))
    np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-5)
    np.testing.assert_allclose(st[:, 3], rs[:, 3], rtol=0, atol=1e-5)
    if case.reduce_loss:
        ref_mean = oracle.mean_loss(ref_loss, case.targets, case.ignore_idx)
        assert abs(out["loss_mean"] - ref_mean) <= 1e-4 + 1e-5 * abs(ref_mean)
        assert out["n_valid"] == oracle.n_valid(case.targets, case.ignore_idx)
    return err


def check_backward(case, out, chunk=256):
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    N, V = case.N, case.V
    gpu = out["grad"].reshape(N, V)
    tflat = case.targets.reshape(-1)
    worst = 0
    band = {}
    for s in range(0, N, chunk):
        rows = np.arange(s, min(N, s + chunk))
        ref = oracle.ce_backward(case.logits, case.targets, g, case.label_smoothing,
                                 case.ignore_idx, rows=rows)
        if case.dtype == wl.DTYPE_BF16:
            T = grad_terms(ref, g[rows], tflat[rows], case.label_smoothing, case.ignore_idx)
            worst = max(worst, assert_grad_bf16(gpu[rows], ref, T, f"grad rows {s}..", band))
        else:
            worst = max(worst, assert_grad_fp32(gpu[rows], ref, f"grad rows {s}.."))
    if band:
        _say(f"grad: {band['elements']} elements, worst {band['worst_ulp']} ulp outside the "
             f"cancellation band; band {band['band']} elements ({band['band_beyond_1ulp']} beyond "
             f"1 ulp, worst err/T {band['worst_band_err_over_T']:.2e})")
    return worst


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("reduce_loss", [False, True])
def test_tiny_fp32(eps, reduce_loss):
    case = wl.tiny_logits(eps, reduce_loss)
    _say(case.name)
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out)


def test_bsqv_v32000_bf16_full():
    case = wl.medium_logits()
    _say(case.name)
    out = run_case(case)
    err = check_forward(case, out)
    worst = check_backward(case, out, chunk=512)
    _say(f"max loss err {err:.2e}, worst grad ulp {worst}")


@pytest.fixture(scope="module")
def headline():
    _say("generating the (SQ,B,V) = (2048, 2, 128256) workload")
    return wl.headline_logits()


def test_sqbv_v128256_bf16_separate(headline):
    _say(headline.name + " separate gradient buffer")
    out = run_case(headline)
    err = check_forward(headline, out)
    worst = check_backward(headline, out, chunk=512)
    _say(f"max loss err {err:.2e}, worst grad ulp {worst}")


def test_sqbv_v128256_bf16_in_place_equals_separate(headline):
    _say(headline.name + " in place vs separate")
    sep = run_case(headline)
    inp = run_case(headline, overwrite=True)
    np.testing.assert_array_equal(inp["grad"], sep["grad"])
    np.testing.assert_array_equal(inp["loss"], sep["loss"])


def test_in_place_takes_no_device_memory(headline):
    """The memory claim of the statistics-saving design, measured at the
    (2048, 2, 128256) BF16 shape (TransformerEngine PR "Minimize the memory
    usage of the fused cross entropy kernel", downstream validation: the
    in-place backward needs no additional allocation): the saved state is 20
    bytes per token (the loss and four row statistics), and a forward plus an
    in-place backward take no device memory beyond their arguments -- the
    device's free bytes (which see allocations made outside torch too) and
    torch's allocator are unchanged across the two calls, after one warm call."""
    c = headline
    z = to_device(c.logits, c.dtype)
    t = torch.from_numpy(c.targets).cuda()
    go = torch.from_numpy(c.grad_output).cuda()
    assert not c.reduce_loss
    loss = torch.empty((c.d0, c.d1), device="cuda")
    stats = torch.empty((c.d0, c.d1, 4), device="cuda")
    out = (loss, None, stats, None)

    def call():
        vce.ce_forward(z, t, c.label_smoothing, False, c.ignore_idx, out=out)
        g = vce.ce_backward(z, t, stats, None, go, c.label_smoothing, False, c.ignore_idx,
                            overwrite_input=True)
        assert g.data_ptr() == z.data_ptr()

    call()
    torch.cuda.synchronize()
    free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    call()
    torch.cuda.synchronize()
    free1, peak = torch.cuda.mem_get_info()[0], torch.cuda.max_memory_allocated()
    saved = loss.numel() * loss.element_size() + stats.numel() * stats.element_size()
    _say(f"logits {z.numel() * z.element_size()} B, saved state {saved} B "
         f"({saved / c.N:.0f} B/token); device bytes taken {free0 - free1}, torch peak extra "
         f"{peak - alloc0}")
    assert saved == 20 * c.N
    assert free1 == free0
    assert peak == alloc0


@pytest.mark.parametrize("V,dtype", [(1, "fp32"), (7, "bf16"), (9, "fp32"), (1001, "bf16"),
                                     (1003, "fp32"), (4099, "bf16"), (33333, "bf16"),
                                     (16383, "bf16"), (16385, "bf16"), (32767, "bf16"),
                                     (32769, "bf16"), (8191, "fp32"), (8193, "fp32"),
                                     (16385, "fp32"), (16384, "bf16"), (24576, "bf16"),
                                     (24577, "bf16"), (8192, "fp32"), (12288, "fp32"),
                                     (12289, "fp32")])
def test_ragged_vocab(V, dtype):
    # V not a multiple of the vector width: rows start at every 16-byte phase.
    # Widths around one pass of the forward's 512 threads (4 loads of 16 B
    # each: 16384 BF16 or 8192 FP32 elements) and of the backward's 1024
    # (32768 BF16, 16384 FP32) leave 0, 1 or all-but-one vectors in the last
    # partial chunk.  Rows of at most 32 KB (16384 BF16, 8192 FP32) take the
    # backward's smaller workgroup and rows of at most 48 KB (24576 BF16,
    # 12288 FP32) the forward's: both sides of each limit are here.
    case = wl.make_logits(2000 + V, 3, 5, V, dtype=dtype, sigma=3.0, ignore_count=2,
                          label_smoothing=0.05, reduce_loss=False, grad_output="random")
    _say(f"ragged V={V} {dtype}")
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out)


@pytest.mark.parametrize("V,dtype,reduce_loss", [(32000, "bf16", True), (128256, "bf16", False),
                                               (4099, "fp32", False), (1000, "fp32", True)])
def test_full_smoothing(V, dtype, reduce_loss):
    # eps = 1: every class gets 1/V, the target none, so the loss is lse - mean z
    # whatever the target and the gradient is g (p - 1/V) (the target's (1 - eps)
    # term vanishes); the oracle states q = (1 - eps) onehot + eps / V directly.
    case = wl.make_logits(2110 + V, 2, 16, V, dtype=dtype, sigma=3.0, ignore_count=3,
                          label_smoothing=1.0, reduce_loss=reduce_loss, grad_output="random")
    _say(f"full smoothing V={V} {dtype} reduce={reduce_loss}")
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out)


@pytest.mark.parametrize("kind", ["offset_fp32", "wide_bf16"])
def test_large_logits(kind):
    # Logits far from 0: an offset of 1e4 (z - m still exact in FP32) and a
    # spread of sigma = 100 in BF16 (most exponentials underflow to 0).
    if kind == "offset_fp32":
        case = wl.make_logits(2120, 2, 8, 3000, dtype="fp32", sigma=2.0, ignore_count=2,
                              grad_output="random")
        case.logits += np.float32(1e4)
    else:
        case = wl.make_logits(2121, 2, 8, 32000, dtype="bf16", sigma=100.0, ignore_count=2,
                              label_smoothing=0.1, reduce_loss=True)
    _say(f"large logits: {kind}")
    out = run_case(case)
    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, case.label_smoothing,
                                               case.ignore_idx)
    assert_loss_close(out["loss"], ref_loss)
    valid = case.targets.reshape(-1) != case.ignore_idx
    st, rs = out["stats"][valid], ref_stats[valid]
    np.testing.assert_array_equal(st[:, 0], rs[:, 0].astype(np.float32))
    np.testing.assert_array_equal(st[:, 2], rs[:, 2].astype(np.float32))
    np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-5)
    # the mean logit is an FP32 sum over the row: its error scales with the
    # size of the logits (1e4 here), not with the mean
    size = np.abs(oracle.bf16_to_f64(case.logits) if case.dtype == "bf16" else
                  case.logits.astype(np.float64)).reshape(case.N, -1).max(axis=1)[valid]
    assert np.all(np.abs(st[:, 3] - rs[:, 3]) <= 1e-5 + 2e-7 * size)
    check_backward(case, out)


@pytest.mark.parametrize("V,dtype", [(32000, "bf16"), (128256, "bf16"), (4099, "fp32")])
def test_rows_masked_with_the_most_negative_finite_value(V, dtype):
    # All but a few logits of each row set to the most negative finite value
    # (a finite mask instead of -inf): most threads' first chunks then hold
    # nothing else, and their running maximum lies far below the row's.  Their
    # terms must vanish in the merge (e^(m_old - m) = 0), not poison d.  The
    # mean logit overflows FP32 here, so eps = 0 and the saved mean is not
    # compared.
    case = wl.make_logits(2130 + V, 2, 8, V, dtype=dtype, sigma=3.0, ignore_count=2,
                          grad_output="random")
    rng = np.random.default_rng(V)
    keep = np.zeros((case.N, V), bool)
    for r in range(case.N):
        keep[r, rng.choice(V, 5, replace=False)] = True
    tf = case.targets.reshape(-1)
    keep[np.arange(case.N)[tf >= 0], tf[tf >= 0]] = True
    flat = case.logits.reshape(case.N, V)
    flat[~keep] = np.uint16(0xFF7F) if dtype == "bf16" else np.float32(-3.4028235e38)
    _say(f"masked rows V={V} {dtype}")
    out = run_case(case)
    ref_loss, ref_stats, _ = oracle.ce_forward(case.logits, case.targets, 0.0, case.ignore_idx)
    assert_loss_close(out["loss"], ref_loss)
    valid = tf != case.ignore_idx
    st, rs = out["stats"][valid], ref_stats[valid]
    np.testing.assert_array_equal(st[:, 0], rs[:, 0].astype(np.float32))
    np.testing.assert_array_equal(st[:, 2], rs[:, 2].astype(np.float32))
    np.testing.assert_allclose(st[:, 1], rs[:, 1], rtol=2e-5)
    check_backward(case, out)
    # the one-pass form reduces the same way
    z = to_device(case.logits, case.dtype)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    l1, _, s1, _, g1 = vce.ce_forward_backward(z, t, go)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(l1.cpu().numpy(), out["loss"])
    np.testing.assert_array_equal(s1.cpu().numpy().reshape(-1, 4), out["stats"])
    np.testing.assert_array_equal(to_host_bits(g1), out["grad"])


def test_fp32_large_vocab():
    case = wl.make_logits(2101, 8, 8, 128256, dtype="fp32", sigma=4.0, ignore_count=3,
                          target_boost=8.0, label_smoothing=0.1, reduce_loss=True)
    _say("fp32 V=128256")
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out)


def test_many_short_rows():
    case = wl.make_logits(2102, 70, 1000, 64, dtype="bf16", sigma=2.0, ignore_frac=0.1,
                          label_smoothing=0.2, reduce_loss=True)
    _say("70000 rows of V=64")
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out, chunk=8192)


def test_strided_layout_view():
    # (SQ,B,V) storage passed as a (B,SQ,V) view: the strides carry the layout.
    case = wl.make_logits(2103, 64, 4, 5000, dtype="bf16", sigma=3.0, ignore_count=5,
                          label_smoothing=0.1, reduce_loss=True, layout="SQ,B")
    _say("transposed (B,SQ,V) view of (SQ,B,V) storage")
    z_sb = to_device(case.logits, "bf16")
    t_sb = torch.from_numpy(case.targets).cuda()
    zv, tv = z_sb.transpose(0, 1), t_sb.transpose(0, 1)
    go = torch.ones(1, device="cuda")
    loss, mean, stats, nv = vce.ce_forward(zv, tv, 0.1, True)
    grad = vce.ce_backward(zv, tv, stats, nv, go, 0.1, True)
    torch.cuda.synchronize()
    ref_loss, _, _ = oracle.ce_forward(case.logits.transpose(1, 0, 2), case.targets.T, 0.1)
    assert_loss_close(loss.cpu().numpy(), ref_loss)
    g = oracle.row_scale(np.ones(1), case.targets, True)
    ref_grad = oracle.ce_backward(case.logits.transpose(1, 0, 2), case.targets.T, g, 0.1)
    gb = to_host_bits(grad.contiguous()).reshape(-1, 5000)
    T = grad_terms(ref_grad, g.reshape(64, 4).T.reshape(-1), case.targets.T.reshape(-1), 0.1, IGN)
    assert_grad_bf16(gb, ref_grad, T)
    assert grad.stride() == zv.stride()


def test_all_rows_ignored():
    case = wl.make_logits(2104, 2, 16, 300, dtype="bf16", sigma=1.0, ignore_count=32,
                          reduce_loss=True)
    out = run_case(case)
    assert out["loss_mean"] == 0.0 and out["n_valid"] == 0
    assert np.all(out["loss"] == 0.0)
    assert np.all((out["grad"] & 0x7FFF) == 0)


def test_target_out_of_range_and_ignore_inside_vocab():
    case = wl.make_logits(2105, 1, 6, 500, dtype="fp32", sigma=2.0, reduce_loss=False)
    case.targets[0, :] = [3, 500, -1, 7, 42, 7]
    case.ignore_idx = 7
    out = run_case(case)
    ref_loss, _, _ = oracle.ce_forward(case.logits, case.targets, 0.0, ignore_idx=7)
    assert_loss_close(out["loss"], ref_loss)
    flat = out["loss"].reshape(-1)
    assert np.isnan(flat[1]) and np.isnan(flat[2])
    assert flat[3] == 0.0 and flat[5] == 0.0
    check_backward(case, out)


def test_negative_infinity_columns():
    case = wl.make_logits(2106, 2, 4, 2000, dtype="fp32", sigma=2.0, reduce_loss=False)
    case.logits[:, :, 1990:] = -np.inf
    case.targets[case.targets >= 1990] = 5
    out = run_case(case)
    check_forward(case, out)
    check_backward(case, out)


def test_deterministic():
    case = wl.make_logits(2107, 8, 64, 32000, dtype="bf16", sigma=3.0, ignore_frac=0.05,
                          label_smoothing=0.1, reduce_loss=True)
    a = run_case(case)
    b = run_case(case)
    for k in ("loss", "stats", "grad"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["loss_mean"] == b["loss_mean"]


def test_empty_batch():
    z = torch.empty((0, 4, 100), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    loss, mean, stats, nv = vce.ce_forward(z, t, 0.0, True)
    torch.cuda.synchronize()
    assert mean.item() == 0.0 and nv.item() == 0 and loss.numel() == 0


def test_graph_capture_replay():
    # Every call only enqueues kernels on the given stream, so forward and
    # backward can be captured and replayed.
    case = wl.make_logits(2108, 4, 256, 8000, dtype="bf16", sigma=3.0, ignore_frac=0.05,
                          label_smoothing=0.1, reduce_loss=True)
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    loss = torch.empty((4, 256), device="cuda")
    mean = torch.empty((), device="cuda")
    stats = torch.empty((4, 256, 4), device="cuda")
    nv = torch.empty((), dtype=torch.int32, device="cuda")
    grad = torch.empty_like(z)
    out = (loss, mean, stats, nv)
    vce.ce_forward(z, t, 0.1, True, out=out)
    vce.ce_backward(z, t, stats, nv, go, 0.1, True, grad=grad)
    torch.cuda.synchronize()
    ref = (loss.clone(), mean.clone(), grad.clone())
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        loss.zero_(); grad.zero_()
        with torch.cuda.graph(graph, stream=s):
            vce.ce_forward(z, t, 0.1, True, out=out, stream=s)
            vce.ce_backward(z, t, stats, nv, go, 0.1, True, grad=grad, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        loss.zero_(); mean.zero_(); grad.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref[0]) and torch.equal(mean, ref[1]) and torch.equal(grad, ref[2])

