"""lce_forward_noalloc, the linear forward that runs in the library's static
scratch instead of a caller workspace (for callers that cannot allocate),
against lce_forward through the C-ABI: the same kernels on the same inputs,
so every output must be equal bit for bit, on consecutive calls that reuse
the scratch with a smaller problem second, at the scratch's size limit, and
with the entropy output; a problem beyond the scratch is refused before
anything is launched."""
import numpy as np
import pytest
import torch

import oracle
import vocabulary_cross_entropy_amd as vce
from oracle import linear
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import LINEAR_LOSS_RTOL, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)


def _case(seed, M, H, V, eps):
    c = wl.make_linear(seed, M, H, V, ignore_frac=0.05, label_smoothing=eps, reduce_loss=True)
    return c, to_device(c.X, "bf16"), to_device(c.W, "bf16"), torch.from_numpy(c.targets).cuda()


def _same(case, X, W, t, with_entropy=False):
    eps = case.label_smoothing
    ref = vce.lce_forward(X, W, t, eps, True, with_entropy=with_entropy)
    got = vce.lce_forward_noalloc(X, W, t, eps, True, with_entropy=with_entropy)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"output {i} differs (M={case.M}, V={case.V})"
    return got


def test_noalloc_equals_the_workspace_forward_twice_second_smaller():
    big = _case(9101, 4096, 512, 40000, 0.1)
    small = _case(9102, 300, 256, 9000, 0.0)
    _say("M=4096 H=512 V=40000, then M=300 H=256 V=9000, one shared scratch")
    _same(*big)
    out = _same(*small)
    # the second, smaller call also against the oracle (the scratch still
    # holds the first call's partials beyond the second one's)
    case = small[0]
    rl, _, _ = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                              case.ignore_idx)
    err = np.abs(out[0].cpu().numpy().astype(np.float64) - rl) / np.maximum(np.abs(rl), 1e-30)
    assert np.max(err[case.targets != case.ignore_idx]) <= LINEAR_LOSS_RTOL
    rmean = oracle.mean_loss(rl, case.targets, case.ignore_idx)
    assert abs(out[1].item() - rmean) <= LINEAR_LOSS_RTOL * abs(rmean)


def test_noalloc_with_entropy():
    _same(*_case(9103, 520, 256, 70001, 0.05), with_entropy=True)


def test_noalloc_at_the_scratch_limit():
    # 4 * 16 MiB less one tile plane + the target logits: just inside 64 MiB
    case, X, W, t = _case(9104, 4096, 64, 261888, 0.0)
    _say("M=4096 H=64 V=261888 (the largest V that fits at M=4096)")
    _same(case, X, W, t)


def test_noalloc_refuses_a_problem_beyond_the_scratch():
    case, X, W, t = _case(9105, 4096, 64, 262144, 0.0)
    loss = torch.full((4096,), 7.0, device="cuda")
    out = (loss, torch.full((), 7.0, device="cuda"), torch.full((4096, 4), 7.0, device="cuda"),
           torch.full((), 7, dtype=torch.int32, device="cuda"))
    with pytest.raises(vce.VceError) as e:
        vce.lce_forward_noalloc(X, W, t, 0.0, True, out=out)
    assert e.value.code == 8
    torch.cuda.synchronize()
    assert torch.all(loss == 7.0) and out[3].item() == 7  # nothing was launched
