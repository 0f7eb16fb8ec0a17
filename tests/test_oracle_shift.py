"""Pins for the causal label shift of the oracle (CPU only): the shifted loss
equals torch's float64 cross-entropy of the usual causal-LM formulation,
logits[:, :-1] scored against labels[:, 1:], which shares no code with it."""
import numpy as np
import pytest
import torch

import oracle
from oracle.shift import shift_targets

IGN = -100


def test_tiny_by_hand():
    t = np.array([[1, 2, 3], [4, 5, 6]])
    np.testing.assert_array_equal(shift_targets(t, 1), [[2, 3, IGN], [5, 6, IGN]])
    np.testing.assert_array_equal(shift_targets(t, 0), [[4, 5, 6], [IGN, IGN, IGN]])


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_shifted_loss_equals_the_causal_formulation(eps):
    rng = np.random.default_rng(3)
    B, S, V = 3, 17, 50
    z = rng.standard_normal((B, S, V)) * 2
    lab = rng.integers(0, V, size=(B, S))
    lab[0, 5] = IGN
    sh = shift_targets(lab, 1)
    loss, _, _ = oracle.ce_forward(z, sh, eps, IGN)
    ref = torch.nn.functional.cross_entropy(
        torch.from_numpy(z[:, :-1].reshape(-1, V)), torch.from_numpy(lab[:, 1:].reshape(-1)),
        ignore_index=IGN, reduction="none", label_smoothing=eps).numpy().reshape(B, S - 1)
    loss = loss.reshape(B, S)
    np.testing.assert_allclose(loss[:, :-1], ref, rtol=1e-12, atol=1e-12)
    assert np.all(loss[:, -1] == 0.0)
    mean_ref = torch.nn.functional.cross_entropy(
        torch.from_numpy(z[:, :-1].reshape(-1, V)), torch.from_numpy(lab[:, 1:].reshape(-1)),
        ignore_index=IGN, label_smoothing=eps).item()
    assert oracle.mean_loss(loss, sh, IGN) == pytest.approx(mean_ref, rel=1e-12)


def test_sequence_along_axis_0():
    # (SQ, B) storage: shifting along axis 0 is the transpose of shifting (B, SQ) along axis 1
    rng = np.random.default_rng(4)
    lab = rng.integers(0, 100, size=(4, 9))
    np.testing.assert_array_equal(shift_targets(lab.T.copy(), 0), shift_targets(lab, 1).T)
