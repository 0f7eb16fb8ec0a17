"""Parity of the one-pass forward + backward (ce_forward_backward): its
outputs are, bit for bit, those of ce_forward followed by ce_backward with the
same arguments (which the other logits tests hold to the FP64 oracle), and
one case is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

import vocabulary_cross_entropy_amd as vce
from vocabulary_cross_entropy_amd import workloads as wl
from vce_testutil import to_device, to_host_bits
from test_parity_ce import check_backward, check_forward

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


def _say(msg):
    print(f"[parity-fb] {msg}", flush=True)


def two_call(z, t, go, eps, red, overwrite):
    zc = z.clone() if overwrite else z
    loss, mean, stats, nv = vce.ce_forward(zc, t, eps, red, IGN)
    grad = vce.ce_backward(zc, t, stats, nv, go, eps, red, IGN, overwrite_input=overwrite)
    return loss, mean, stats, nv, grad


def one_pass(z, t, go, eps, red, overwrite):
    zc = z.clone() if overwrite else z
    return vce.ce_forward_backward(zc, t, go, eps, red, IGN, overwrite_input=overwrite)


def assert_same(a, b, red):
    names = ("loss", "mean", "stats", "n_valid", "grad")
    for name, x, y in zip(names, a, b):
        if x is None and y is None:
            continue
        if name in ("mean", "n_valid") and not red:
            continue
        assert torch.equal(x, y) or (torch.isnan(x).equal(torch.isnan(y)) and
                                     torch.equal(torch.nan_to_num(x), torch.nan_to_num(y))), name


def _case(seed, d0, d1, V, dtype, eps, red, layout="B,SQ", n_ign=3, sigma=3.0):
    return wl.make_logits(seed, d0, d1, V, dtype=dtype, sigma=sigma, ignore_count=n_ign,
                          label_smoothing=eps, reduce_loss=red, grad_output="random",
                          layout=layout)


@pytest.mark.parametrize("dtype,V", [("bf16", 1), ("fp32", 2), ("bf16", 9),
                                     ("fp32", 1000), ("bf16", 7), ("bf16", 1001),
                                     ("fp32", 4099), ("bf16", 32000), ("bf16", 65537),
                                     ("fp32", 65536), ("bf16", 131072),
                                     ("bf16", 131080), ("fp32", 70000),
                                     ("bf16", 24576), ("bf16", 24577), ("fp32", 12289),
                                     ("bf16", 40000), ("bf16", 90001), ("bf16", 100003),
                                     ("bf16", 128256),
                                     ("fp32", 45000)])
@pytest.mark.parametrize("eps,red", [(0.0, False), (0.1, True), (1.0, False)])
@pytest.mark.parametrize("overwrite", [False, True])
def test_one_pass_equals_two_calls(dtype, V, eps, red, overwrite):
    # 131080 BF16 and 70000 FP32 exceed the on-chip row and take the two sweeps;
    # 24576 / 24577 BF16 and 12289 FP32 sit at the forward's workgroup-size limit;
    # 65537 .. 131072 BF16 and 32769 .. 65536 FP32 keep part of the row in LDS
    # (90001: none of it, the registers hold the whole row; 100003 and 45000:
    # rows that start off a 16-byte boundary)
    case = _case(5000 + V, 3, 17, V, dtype, eps, red)
    z = to_device(case.logits, dtype)
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    go = go.reshape(-1) if red else go
    a = two_call(z, t, go, eps, red, overwrite)
    b = one_pass(z, t, go, eps, red, overwrite)
    torch.cuda.synchronize()
    assert_same(a, b, red)


@pytest.mark.parametrize("V", [3000, 100001])
def test_one_pass_edge_targets_and_infinite_columns(V):
    # 100001 takes the kernel that keeps part of the row in LDS (and rows that
    # start off a 16-byte boundary)
    live = V * 5 // 6
    case = _case(5101, 2, 40, V, "bf16", 0.1, False, n_ign=5)
    lg = case.logits.reshape(-1, V)
    lg[:, live:] = np.uint16(0xFF80)          # -inf padding columns (BF16 bits)
    tt = case.targets.reshape(-1)
    tt[:] = np.minimum(tt, live - 1)
    tt[0], tt[1], tt[2] = V, -3, live - 1     # out of range (twice) and the last live column
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    for overwrite in (False, True):
        a = two_call(z, t, go, 0.1, False, overwrite)
        b = one_pass(z, t, go, 0.1, False, overwrite)
        torch.cuda.synchronize()
        assert_same(a, b, False)
        assert torch.isnan(b[0].reshape(-1)[:2]).all()


@pytest.mark.parametrize("V", [5000, 70001])
def test_one_pass_strided_view(V):
    # (SQ,B,V) storage used as a (B,SQ,V) view
    case = _case(5102, 64, 4, V, "bf16", 0.1, True, layout="SQ,B")
    zs = to_device(case.logits, "bf16")
    ts = torch.from_numpy(case.targets).cuda()
    zv, tv = zs.transpose(0, 1), ts.transpose(0, 1)
    go = torch.ones(1, device="cuda")
    a = two_call(zv, tv, go, 0.1, True, False)
    b = one_pass(zv, tv, go, 0.1, True, False)
    torch.cuda.synchronize()
    assert_same(a, b, True)


def test_one_pass_headline_shape_against_oracle():
    """The (SQ,B,V) = (2048, 2, 128256) BF16 workload, in place, against the
    FP64 oracle (loss and statistics; gradient rows checked in full) and
    bitwise against the two calls."""
    case = wl.headline_logits()
    _say(case.name)
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.from_numpy(case.grad_output).cuda()
    a = two_call(z, t, go, 0.0, False, True)
    b = one_pass(z, t, go, 0.0, False, True)
    torch.cuda.synchronize()
    assert_same(a, b, False)
    out = dict(loss=b[0].cpu().numpy(), stats=b[2].cpu().numpy().reshape(-1, 4),
               grad=to_host_bits(b[4]))
    check_forward(case, out)
    check_backward(case, out, chunk=512)


def test_one_pass_all_ignored_and_empty():
    case = _case(5103, 2, 8, 900, "fp32", 0.0, True, n_ign=16)
    z = to_device(case.logits, "fp32")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    loss, mean, stats, nv, grad = one_pass(z, t, go, 0.0, True, False)
    torch.cuda.synchronize()
    assert float(mean.item()) == 0.0 and int(nv.item()) == 0
    assert torch.count_nonzero(grad).item() == 0 and torch.count_nonzero(loss).item() == 0
    ze = torch.empty((0, 4, 900), device="cuda")
    te = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    loss, mean, stats, nv, grad = vce.ce_forward_backward(ze, te, go, 0.0, True)
    torch.cuda.synchronize()
    assert float(mean.item()) == 0.0 and int(nv.item()) == 0


@pytest.mark.parametrize("V", [12000, 70001])
def test_one_pass_and_shards_graph_capture_replay(V):
    # The one-pass call and the three shard calls only enqueue kernels on the
    # given stream, so they are captured and replayed like the others; every
    # replay (with eager work and synchronisation between them) must give the
    # eager outputs bit for bit.  70001 takes the one-pass kernel with part of
    # the row in LDS (dynamic LDS, set at launch).
    d0, d1, S = 2, 384, 3
    case = _case(5104, d0, d1, V, "bf16", 0.1, True)
    z = to_device(case.logits, "bf16")
    t = torch.from_numpy(case.targets).cuda()
    go = torch.ones(1, device="cuda")
    loss = torch.empty((d0, d1), device="cuda")
    mean = torch.empty((), device="cuda")
    stats = torch.empty((d0, d1, 4), device="cuda")
    nv = torch.empty((), dtype=torch.int32, device="cuda")
    grad = torch.empty_like(z)
    out = (loss, mean, stats, nv)
    bounds = [0, 4000, 8000, V]
    parts = torch.empty((S, d0, d1, 4), device="cuda")
    sl = torch.empty((d0, d1), device="cuda")
    smean = torch.empty((), device="cuda")
    sst = torch.empty((d0, d1, 4), device="cuda")
    snv = torch.empty((), dtype=torch.int32, device="cuda")
    sgrad = [torch.empty((d0, d1, bounds[k + 1] - bounds[k]), dtype=torch.bfloat16,
                         device="cuda") for k in range(S)]
    zs = [z[:, :, bounds[k]:bounds[k + 1]].contiguous() for k in range(S)]

    def work(stream=None):
        vce.ce_forward_backward(z, t, go, 0.1, True, IGN, grad=grad, out=out, stream=stream)
        for k in range(S):
            vce.ce_forward_shard(zs[k], t, bounds[k], IGN, out=parts[k], stream=stream)
        vce.ce_merge_shards(parts, t, V, 0.1, True, IGN, out=(sl, smean, sst, snv), stream=stream)
        for k in range(S):
            vce.ce_backward_shard(zs[k], t, bounds[k], V, sst, snv, go, 0.1, True, IGN,
                                  grad=sgrad[k], stream=stream)

    work()
    torch.cuda.synchronize()
    outs = [loss, mean, stats, nv, grad, sl, smean, sst, snv] + sgrad
    ref = [x.clone() for x in outs]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            work(stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.zero_()
        work()                      # eager work between the replays
        torch.cuda.synchronize()
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"
