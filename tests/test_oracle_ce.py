"""Pins for the FP64 logits cross-entropy oracle (CPU only).

Each test ties the oracle to something other than itself: a closed form, an
invariant, finite differences, a special case, torch's float64 library
routine (the API page presents the op as a drop-in for
torch.nn.functional.cross_entropy), or an independent pure-Python statement.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import tiny
from vocabulary_cross_entropy_amd import workloads as wl

IGN = -100


def _rand_logits(seed, N, V, sigma=2.0, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, V)) * sigma).astype(dtype)


def _rand_targets(seed, N, V, n_ign=0):
    rng = np.random.default_rng(seed + 7)
    t = rng.integers(0, V, size=N).astype(np.int64)
    if n_ign:
        t[rng.choice(N, n_ign, replace=False)] = IGN
    return t


# --- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("V", [1, 7, 1000, 128256])
@pytest.mark.parametrize("eps", [0.0, 0.1, 0.5, 1.0])
@pytest.mark.parametrize("storage", ["fp32", "bf16", "fp64"])
def test_uniform_logits_loss_is_ln_V(V, eps, storage):
    # Equal logits give p = 1/V, so -sum q ln p = ln V whatever eps is.
    N = 3
    val = 2.5  # exactly representable in BF16 and FP32
    if storage == "fp32":
        z = np.full((N, V), val, np.float32)
    elif storage == "bf16":
        z = np.full((N, V), wl.f32_to_bf16_bits(np.array([val], np.float32))[0], np.uint16)
    else:
        z = np.full((N, V), val, np.float64)
    t = np.array([0, V - 1, (V // 2)], np.int64)
    loss, stats, closed = oracle.ce_forward(z, t, eps)
    # A sequential FP64 sum of V terms carries up to ~V * 2^-53 relative error.
    rtol = 1e-12 + V * 2.0 ** -52
    np.testing.assert_allclose(loss, math.log(V), rtol=rtol, atol=1e-12)
    np.testing.assert_allclose(closed, math.log(V), rtol=rtol, atol=1e-12)
    np.testing.assert_array_equal(stats[:, 0], val)
    np.testing.assert_allclose(stats[:, 1], V, rtol=1e-14)
    np.testing.assert_array_equal(stats[:, 2], val)
    np.testing.assert_allclose(stats[:, 3], val, rtol=1e-14)
    if V <= 1000:
        g = np.array([1.0, 0.5, 2.0])
        grad = oracle.ce_backward(z, t, g, eps)
        for i in range(N):
            want = np.full(V, g[i] * (1.0 / V - eps / V))
            want[t[i]] -= g[i] * (1.0 - eps)
            np.testing.assert_allclose(grad[i], want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("eps", [0.1, 0.37, 1.0])
def test_smoothed_loss_closed_form(eps):
    # Definition -sum q ln p equals (1-eps)(lse - z_t) + eps (lse - mean z).
    z = _rand_logits(1, 32, 513, sigma=3.0)
    t = _rand_targets(1, 32, 513, n_ign=3)
    loss, stats, closed = oracle.ce_forward(z, t, eps)
    np.testing.assert_allclose(loss, closed, rtol=1e-12, atol=1e-12)
    # and it is not the unsmoothed loss
    loss0, _, _ = oracle.ce_forward(z, t, 0.0)
    valid = t != IGN
    assert np.all(np.abs(loss0[valid] - loss[valid]) > 1e-3)


def test_lse_against_direct_sum():
    # lse = m + ln d must equal ln sum exp z computed without the shift
    # (safe here: |z| is small).
    z = _rand_logits(2, 8, 300, sigma=1.0)
    t = _rand_targets(2, 8, 300)
    _, stats, _ = oracle.ce_forward(z, t, 0.0)
    lse = stats[:, 0] + np.log(stats[:, 1])
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-13)
    np.testing.assert_array_equal(stats[:, 0], z.max(axis=1))
    np.testing.assert_array_equal(stats[:, 2], z[np.arange(8), t])
    np.testing.assert_allclose(stats[:, 3], z.mean(axis=1), rtol=1e-12, atol=1e-15)


# --- invariants ---------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 0.1, 0.9])
def test_gradient_rows_sum_to_zero(eps):
    z = _rand_logits(3, 16, 777, sigma=4.0)
    t = _rand_targets(3, 16, 777, n_ign=2)
    g = np.random.default_rng(3).uniform(0.5, 2.0, 16)
    grad = oracle.ce_backward(z, t, g, eps)
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-12)
    # target column is the only negative entry when eps = 0
    if eps == 0.0:
        for i in np.nonzero(t != IGN)[0]:
            assert grad[i, t[i]] < 0
            assert np.all(np.delete(grad[i], t[i]) >= 0)


def test_ignored_rows_are_zero_and_excluded_from_mean():
    z = _rand_logits(4, 10, 50)
    t = _rand_targets(4, 10, 50)
    t[[2, 7]] = IGN
    loss, _, _ = oracle.ce_forward(z, t, 0.1)
    assert loss[2] == 0.0 and loss[7] == 0.0
    grad = oracle.ce_backward(z, t, np.ones(10), 0.1)
    assert np.all(grad[2] == 0.0) and np.all(grad[7] == 0.0)
    valid = t != IGN
    assert oracle.mean_loss(loss, t) == pytest.approx(loss[valid].sum() / 8, rel=1e-15)
    g = oracle.row_scale(np.array([3.0]), t, reduce_loss=True)
    np.testing.assert_allclose(g, 3.0 / 8)
    # changing the logits of an ignored row changes nothing
    z2 = z.copy()
    z2[2] += 100.0
    loss2, _, _ = oracle.ce_forward(z2, t, 0.1)
    np.testing.assert_array_equal(loss, loss2)


def test_all_rows_ignored_mean_is_zero():
    z = _rand_logits(5, 4, 9)
    t = np.full(4, IGN, np.int64)
    loss, _, _ = oracle.ce_forward(z, t, 0.1)
    assert oracle.mean_loss(loss, t) == 0.0
    np.testing.assert_array_equal(oracle.row_scale(np.array([1.0]), t, True), 1.0)


def test_vocab_of_one():
    z = np.array([[3.0], [-1.0]])
    t = np.array([0, 0], np.int64)
    for eps in (0.0, 0.4):
        loss, _, _ = oracle.ce_forward(z, t, eps)
        np.testing.assert_array_equal(loss, 0.0)
        np.testing.assert_array_equal(oracle.ce_backward(z, t, np.ones(2), eps), 0.0)


def test_target_out_of_range_is_nan():
    z = _rand_logits(6, 3, 11)
    t = np.array([11, -1, 4], np.int64)
    loss, _, _ = oracle.ce_forward(z, t, 0.0)
    assert np.isnan(loss[0]) and np.isnan(loss[1]) and np.isfinite(loss[2])
    grad = oracle.ce_backward(z, t, np.ones(3), 0.0)
    assert np.all(np.isnan(grad[:2])) and np.all(np.isfinite(grad[2]))


def test_ignore_index_inside_vocab_range():
    z = _rand_logits(7, 4, 20)
    t = np.array([5, 3, 5, 0], np.int64)
    loss, _, _ = oracle.ce_forward(z, t, 0.0, ignore_idx=5)
    assert loss[0] == 0.0 and loss[2] == 0.0 and loss[1] > 0 and loss[3] > 0


def test_negative_infinity_column():
    # A -inf logit (padded vocabulary) has p = 0 and must not disturb the rest.
    z = _rand_logits(8, 4, 30)
    t = _rand_targets(8, 4, 29)
    zi = np.concatenate([z[:, :29], np.full((4, 1), -np.inf)], axis=1)
    loss_ref, _, _ = oracle.ce_forward(z[:, :29], t, 0.0)
    loss, _, _ = oracle.ce_forward(zi, t, 0.0)
    np.testing.assert_allclose(loss, loss_ref, rtol=1e-14)
    grad = oracle.ce_backward(zi, t, np.ones(4), 0.0)
    np.testing.assert_array_equal(grad[:, 29], 0.0)
    # with smoothing, the -inf class receives eps/V of the target mass: loss is +inf
    loss_s, _, _ = oracle.ce_forward(zi, t, 0.1)
    assert np.all(np.isinf(loss_s))


def test_finite_mask_columns():
    # Columns masked with the most negative finite FP32 value behave like
    # absent classes when eps = 0: loss and kept gradients equal those of the
    # row without them (e^(-FLT_MAX - m) is 0 in FP64 too), masked gradients
    # are 0.  The same with the BF16 pattern 0xFF7F.
    z = _rand_logits(11, 3, 12, dtype=np.float32)
    keep = np.array([0, 2, 3, 7, 11])
    t = np.array([2, 7, 11], np.int64)
    zm = np.full((3, 12), np.float32(-3.4028235e38), np.float32)
    zm[:, keep] = z[:, keep]
    remap = {v: i for i, v in enumerate(keep)}
    tk = np.array([remap[int(x)] for x in t], np.int64)
    loss_ref, _, _ = oracle.ce_forward(z[:, keep], tk, 0.0)
    loss, stats, _ = oracle.ce_forward(zm, t, 0.0)
    np.testing.assert_allclose(loss, loss_ref, rtol=1e-14)
    g = np.array([1.0, 0.5, 2.0])
    grad = oracle.ce_backward(zm, t, g, 0.0)
    np.testing.assert_allclose(grad[:, keep], oracle.ce_backward(z[:, keep], tk, g, 0.0),
                               rtol=1e-13, atol=1e-16)
    mask = np.ones(12, bool)
    mask[keep] = False
    assert np.all(grad[:, mask] == 0.0)
    zb = np.full((3, 12), 0xFF7F, np.uint16)
    zb[:, keep] = (zm[:, keep].view(np.uint32) >> 16).astype(np.uint16)
    lb, _, _ = oracle.ce_forward(zb, t, 0.0)
    lbr, _, _ = oracle.ce_forward(zb[:, keep], tk, 0.0)
    np.testing.assert_allclose(lb, lbr, rtol=1e-14)


# --- finite differences ----------------------------------------------------------

@pytest.mark.parametrize("V", [2, 3, 5, 17])
@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_gradient_matches_central_differences(V, eps):
    rng = np.random.default_rng(V)
    z = rng.standard_normal((2, V)) * 2.0
    t = np.array([0, V - 1], np.int64)
    g = np.array([1.0, 0.7])
    grad = oracle.ce_backward(z, t, g, eps)
    h = 1e-6
    for i in range(2):
        for v in range(V):
            zp = z.copy(); zp[i, v] += h
            zm = z.copy(); zm[i, v] -= h
            lp, _, _ = oracle.ce_forward(zp, t, eps)
            lm, _, _ = oracle.ce_forward(zm, t, eps)
            fd = g[i] * (lp[i] - lm[i]) / (2 * h)
            assert abs(fd - grad[i, v]) <= 1e-7, (i, v, fd, grad[i, v])


# --- library cross-check: torch float64 ------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 0.1, 0.3])
def test_against_torch_float64(eps):
    N, V = 24, 97
    z = _rand_logits(9, N, V, sigma=3.0)
    t = _rand_targets(9, N, V, n_ign=4)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    tt = torch.tensor(t)
    ref = torch.nn.functional.cross_entropy(zt, tt, ignore_index=IGN, label_smoothing=eps,
                                            reduction="none")
    loss, _, _ = oracle.ce_forward(z, t, eps)
    np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    go = np.random.default_rng(9).uniform(0.5, 1.5, N)
    ref.backward(torch.tensor(go))
    grad = oracle.ce_backward(z, t, oracle.row_scale(go, t, False), eps)
    np.testing.assert_allclose(grad, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    # mean over non-ignored rows
    zt.grad = None
    refm = torch.nn.functional.cross_entropy(zt, tt, ignore_index=IGN, label_smoothing=eps,
                                             reduction="mean")
    assert oracle.mean_loss(loss, t) == pytest.approx(refm.item(), rel=1e-12)
    refm.backward(torch.tensor(2.0, dtype=torch.float64))
    gradm = oracle.ce_backward(z, t, oracle.row_scale(np.array([2.0]), t, True), eps)
    np.testing.assert_allclose(gradm, zt.grad.numpy(), rtol=1e-12, atol=1e-14)


# --- independent pure-Python statement ------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 0.25])
def test_against_pure_python(eps):
    z = _rand_logits(10, 5, 13, sigma=2.0)
    t = np.array([0, 12, IGN, 6, 3], np.int64)
    g = [1.0, 0.5, 1.0, 2.0, 1.5]
    loss, _, _ = oracle.ce_forward(z, t, eps)
    grad = oracle.ce_backward(z, t, np.array(g), eps)
    for i in range(5):
        assert loss[i] == pytest.approx(tiny.loss_row(list(z[i]), int(t[i]), eps), rel=1e-13, abs=1e-15)
        np.testing.assert_allclose(grad[i], tiny.grad_row(list(z[i]), int(t[i]), g[i], eps),
                                   rtol=1e-12, atol=1e-16)


# --- storage and layout ------------------------------------------------------------

def test_bf16_decoding():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x8000, 0x7F7F], np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 3.140625
    assert v[3] == 2.0 ** -133
    assert v[4] == np.inf and v[5] == -np.inf
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == (2 - 2 ** -7) * 2.0 ** 127
    # the C core widens BF16 the same way: its max statistic is the exact value
    z = bits[[0, 1, 2]].reshape(1, 3)
    _, st, _ = oracle.ce_forward(z, np.array([0]), 0.0)
    assert st[0, 0] == 3.140625 and st[0, 2] == 1.0


def test_round_bf16_cases():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -0.0, 2.0 ** -133,
                  2.0 ** -134, 3 * 2.0 ** -134, 3.4e38, -3.0e38, np.inf, np.nan, 1e-50])
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x8000, 0x0001, 0x0000, 0x0002, 0x7F80, 0xFF62,
            0x7F80, 0x7FC0, 0x0000]
    got = oracle.round_bf16(x)
    assert [int(b) for b in got] == want


def test_round_bf16_against_torch():
    # torch rounds FP32 -> BF16 to nearest even; on FP32-representable inputs the
    # FP64 rounding must agree bit for bit.
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-40, 40, 200000))).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # and the input generator's FP32 -> BF16 rounding agrees with torch too
    np.testing.assert_array_equal(wl.f32_to_bf16_bits_np(x), ref)
    big = np.tile(x, 25)  # large enough for the torch path
    np.testing.assert_array_equal(wl.f32_to_bf16_bits(big), wl.f32_to_bf16_bits_np(big))


def test_layouts_and_strides():
    # (SQ,B,V) storage addressed as a (B,SQ,V) strided view gives the same rows.
    rng = np.random.default_rng(12)
    SQ, B, V = 5, 3, 40
    z = rng.standard_normal((SQ, B, V)).astype(np.float32)
    t = rng.integers(0, V, size=(SQ, B)).astype(np.int64)
    t[1, 2] = IGN
    loss_sb, st_sb, _ = oracle.ce_forward(z, t, 0.1)
    zv = z.transpose(1, 0, 2)  # (B, SQ, V) view, no copy
    tv = t.T
    loss_bs, st_bs, _ = oracle.ce_forward(zv, tv, 0.1)
    # row (b, s) of the view is row (s, b) of the storage
    for s in range(SQ):
        for b in range(B):
            assert loss_bs[b * SQ + s] == loss_sb[s * B + b]
    g = np.ones(SQ * B)
    gr_sb = oracle.ce_backward(z, t, g, 0.1)
    gr_bs = oracle.ce_backward(zv, tv, g, 0.1)
    np.testing.assert_array_equal(gr_bs[1 * SQ + 4], gr_sb[4 * B + 1])
    # row subsets return exactly the selected rows
    rows = np.array([7, 0, 14])
    l_sub, _, _ = oracle.ce_forward(z, t, 0.1, rows=rows)
    np.testing.assert_array_equal(l_sub, loss_sb[rows])
    np.testing.assert_array_equal(oracle.ce_backward(z, t, g, 0.1, rows=rows), gr_sb[rows])


# --- entropy (the optional output of the Liger-Kernel PR, Summary) -------------

@pytest.mark.parametrize("V", [1, 2, 7, 1000, 128256])
def test_entropy_uniform_is_ln_V(V):
    # p = 1/V: -sum p ln p = ln V
    z = np.full((1, 2, V), 0.75)
    t = np.zeros((1, 2), np.int64)
    h = oracle.entropy(z, t)
    # a V-term FP64 sum: rounding grows with V
    np.testing.assert_allclose(h, math.log(V), rtol=1e-13 + V * 2.0 ** -52, atol=1e-15)


@pytest.mark.parametrize("a,b", [(0.0, 0.0), (1.5, -0.5), (-3.0, 7.0), (30.0, 0.0)])
def test_entropy_two_classes_is_binary_entropy(a, b):
    # textbook binary entropy of p = sigmoid(a - b), q = 1 - p = sigmoid(b - a),
    # with ln p and ln q in their cancellation-free forms
    x = a - b
    lp = -math.log1p(math.exp(-x)) if x >= 0 else x - math.log1p(math.exp(x))
    lq = -math.log1p(math.exp(x)) if x <= 0 else -x - math.log1p(math.exp(-x))
    ref = -(math.exp(lp) * lp + math.exp(lq) * lq)
    h = oracle.entropy(np.array([[[a, b]]]), np.zeros((1, 1), np.int64))
    # ln p = z - lse carries an absolute FP64 rounding of about ulp(lse)
    # (3.6e-15 at lse = 30), which dominates when H itself is ~1e-12
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-14)


def test_entropy_point_mass_is_zero_and_ignored_rows_are_zero():
    z = np.full((1, 3, 9), -np.inf)
    z[0, :, 4] = 2.0  # all mass on one class
    t = np.array([[1, IGN, 4]], np.int64)
    h = oracle.entropy(z, t)
    assert h[0] == 0.0 and h[1] == 0.0 and h[2] == 0.0


def test_entropy_shift_invariance_and_target_independence():
    z = _rand_logits(51, 6, 300, sigma=3.0)
    t1, t2 = _rand_targets(51, 6, 300), _rand_targets(52, 6, 300)
    h1 = oracle.entropy(z, t1)
    np.testing.assert_allclose(oracle.entropy(z + 11.0, t1), h1, rtol=1e-12)
    np.testing.assert_array_equal(oracle.entropy(z, t2), h1)


def test_entropy_against_torch_float64():
    z = _rand_logits(53, 40, 3001, sigma=2.5)
    t = _rand_targets(53, 40, 3001, n_ign=3)
    ref = torch.distributions.Categorical(logits=torch.from_numpy(z)).entropy().numpy()
    ref[t == IGN] = 0.0
    np.testing.assert_allclose(oracle.entropy(z, t), ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("V", [2, 3, 5, 17])
def test_entropy_gradient_matches_central_differences(V):
    rng = np.random.default_rng(60 + V)
    z = rng.standard_normal((3, V)) * 1.5
    t = np.zeros(3, np.int64)
    gH = np.array([1.0, -0.7, 2.5])
    grad = np.zeros((3, V))
    oracle.add_entropy_grad(grad, z, t, gH)
    h = 1e-6
    for r in range(3):
        for v in range(V):
            zp, zm = z.copy(), z.copy()
            zp[r, v] += h
            zm[r, v] -= h
            fd = (oracle.entropy(zp, t)[r] - oracle.entropy(zm, t)[r]) / (2 * h)
            assert abs(grad[r, v] - gH[r] * fd) <= 1e-7, (r, v)


def test_entropy_gradient_rows_sum_to_zero_and_ignored_rows_untouched():
    # sum_v dH/dz_v = -sum p (ln p + H) = H - H = 0
    z = _rand_logits(61, 8, 500, sigma=2.0)
    t = _rand_targets(61, 8, 500, n_ign=2)
    grad = np.full((8, 500), 0.25)
    oracle.add_entropy_grad(grad, z, t, np.linspace(-1, 1, 8))
    np.testing.assert_allclose((grad - 0.25).sum(axis=1), 0.0, atol=1e-12)
    assert np.all(grad[t == IGN] == 0.25)
