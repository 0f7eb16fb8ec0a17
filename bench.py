"""Benchmark of the fused vocabulary cross-entropy hot path on one MI355X.

One step = one pass of the logits cross-entropy hot path over one batch:
ce_forward (online-softmax row sweep + deterministic mean when reduced) then
ce_backward (gradient rebuilt from the saved statistics into a separate
buffer).  The headline workload is (SQ,B,V) = (2048, 2, 128256) BF16 logits,
4096 tokens, the shape of the TransformerEngine PR's validation comment.
Inputs are synthetic and resident in HBM before the timed region.

Each workload first runs untimed for at least 50 ms of GPU time (the clocks
come back up after the host has spent time building it), then W warmup steps;
the K timed steps run back to back with one pair of HIP events around all of
them (nothing recorded in between); each phase is then timed in a loop of its
own.  Printed: ONE JSON line with throughput (tokens/s), the roofline of the
dominant kernel (the backward sweep, HBM bound: its algorithmic bytes per
launch over its average launch duration, events on the stream it runs on), the
same for the whole forward + backward step, the FP64 CPU oracle timed on a
bounded sample of each workload, and the fused linear cross-entropy timed the
same way against the BF16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CE fwd+bwd tokens/s (N=4096,V=128256 bf16); % of HBM / MFMA roofline"


def _bf16_dev(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _event_pairs(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def _graph_step_ms(step, steps: int, warmup: int) -> float:
    """Average time of `step` replayed from a HIP graph captured on a side
    stream (every call of the library is stream-ordered and capture-safe)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # warm the side stream once outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e = _event_pairs(1)[0]
    e[0].record()
    for _ in range(steps):
        g.replay()
    e[1].record()
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) / steps


SETTLE_MS = 50.0


def _settle(step, min_ms: float = SETTLE_MS) -> None:
    """Untimed work before a workload's warmup steps: after an idle stretch
    (the host builds the next workload) the GPU's clocks take ~20 ms of work to
    come back up -- 4096 x 32000 BF16 steps measured ~155 us in the first 30
    and ~131 us after 150 -- so each workload first runs its step for at least
    `min_ms` of GPU time, then the W warmup steps, then the K timed steps."""
    import torch
    torch.cuda.synchronize()
    done = 0.0
    n = 1
    while done < min_ms:
        e = _event_pairs(1)[0]
        e[0].record()
        for _ in range(n):
            step()
        e[1].record()
        torch.cuda.synchronize()
        done += e[0].elapsed_time(e[1])
        n = min(2 * n, 64)


def _loop_ms(fn, steps: int) -> float:
    """Average time of ``fn`` over ``steps`` back-to-back calls, from one pair of
    HIP events on the current stream around the whole loop (nothing recorded
    between the calls)."""
    import torch
    torch.cuda.synchronize()
    e = _event_pairs(1)[0]
    e[0].record()
    for _ in range(steps):
        fn()
    e[1].record()
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) / steps


def _inplace_memory(vce, zin, z, t, eps, red, out, stats, go) -> dict:
    """Device memory of a forward + in-place backward, measured rather than
    assumed: what the saved state occupies (per-row loss and the four row
    statistics) against the logits, and how much device memory the two calls
    take beyond their arguments -- the device's free bytes (hipMemGetInfo,
    which also sees allocations made outside torch) and torch's allocator,
    before and after, one warm call first."""
    import torch

    def call():
        zin.copy_(z)
        vce.ce_forward(zin, t, eps, red, out=out)
        vce.ce_backward(zin, t, stats, out[3], go, eps, red, overwrite_input=True)

    call()
    torch.cuda.synchronize()
    free0, torch0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    call()
    torch.cuda.synchronize()
    free1, peak = torch.cuda.mem_get_info()[0], torch.cuda.max_memory_allocated()
    saved = out[0].numel() * out[0].element_size() + stats.numel() * stats.element_size()
    return dict(
        logits_bytes=z.numel() * z.element_size(),
        saved_state_bytes=saved,
        saved_state_bytes_per_token=saved / out[0].numel(),
        fp32_gradient_bytes=z.numel() * 4,
        inplace_fwd_bwd_device_bytes_taken=free0 - free1,
        inplace_fwd_bwd_torch_peak_extra_bytes=peak - torch0,
    )


def bench_logits(case, steps: int, warmup: int):
    """One step = ce_forward (statistics, loss; the averaged loss and the count
    by a one-workgroup kernel when the loss is reduced) then ce_backward into a
    separate gradient buffer."""
    import torch
    import vocabulary_cross_entropy_amd as vce
    from vocabulary_cross_entropy_amd import accounting

    from vocabulary_cross_entropy_amd import workloads as wl

    dev = torch.device("cuda:0")
    if case.dtype == wl.DTYPE_BF16:
        z = _bf16_dev(case.logits, dev)
    else:
        z = torch.from_numpy(np.ascontiguousarray(case.logits)).to(dev)
    t = torch.from_numpy(case.targets).to(dev)
    go = torch.from_numpy(case.grad_output).to(dev)
    if case.reduce_loss:
        go = go.reshape(-1)
    N, V = case.N, case.V
    loss = torch.empty((case.d0, case.d1), device=dev)
    mean = torch.empty((), device=dev)
    stats = torch.empty((case.d0, case.d1, 4), device=dev)
    nv = torch.empty((), dtype=torch.int32, device=dev)
    grad = torch.empty_like(z)
    out = (loss, mean if case.reduce_loss else None, stats, nv if case.reduce_loss else None)
    eps, red = case.label_smoothing, case.reduce_loss

    def fwd():
        vce.ce_forward(z, t, eps, red, out=out)

    def bwd():
        vce.ce_backward(z, t, stats, out[3], go, eps, red, grad=grad)

    def step():
        fwd()
        bwd()

    _settle(step)
    for _ in range(warmup):
        step()
    # timed region: K whole steps, bracketed by synchronisation, with one pair
    # of events around all of them and none in between
    whole = _event_pairs(1)[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    whole[0].record()
    for _ in range(steps):
        step()
    whole[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = whole[0].elapsed_time(whole[1])

    # each phase in a loop of its own, events around the loop only: the
    # forward's and the backward kernel's average launch durations
    fwd_ms = _loop_ms(fwd, steps)
    bwd_ms = _loop_ms(bwd, steps)

    # the same step captured once in a HIP graph and replayed: the GPU time of
    # the step without the host's per-call launch work between kernels
    graph_ms = _graph_step_ms(step, steps, warmup)

    # the one-pass forward + backward (grad_output known up front): the same
    # outputs, the logits read once
    def step_fb():
        vce.ce_forward_backward(z, t, go, eps, red, grad=grad, out=out)

    for _ in range(warmup):
        step_fb()
    fb_ms = _loop_ms(step_fb, steps)

    # in-place backward: logits restored before each launch, outside its events
    zin = torch.empty_like(z)
    mem = _inplace_memory(vce, zin, z, t, eps, red, out, stats, go)
    ip_ms = []
    for i in range(max(3, min(steps, 10))):
        zin.copy_(z)
        vce.ce_forward(zin, t, eps, red, out=out)
        e = _event_pairs(1)[0]
        e[0].record()
        vce.ce_backward(zin, t, stats, out[3], go, eps, red, overwrite_input=True)
        e[1].record()
        torch.cuda.synchronize()
        ip_ms.append(e[0].elapsed_time(e[1]))

    # context only: a plain device-to-device copy of the same tensor (torch's
    # copy kernel), read + write of the logits' bytes, as a practical ceiling
    # for a read-and-write sweep; never the roofline's denominator
    cp_ms = []
    for _ in range(max(3, min(steps, 10))):
        e = _event_pairs(1)[0]
        e[0].record()
        zin.copy_(z)
        e[1].record()
        torch.cuda.synchronize()
        cp_ms.append(e[0].elapsed_time(e[1]))
    copy_GBs = 2 * z.numel() * z.element_size() / (statistics.median(cp_ms) * 1e-3) / 1e9

    n_ign = int(case.meta["n_ignored"])
    es = case.elem_bytes
    b_fwd = accounting.ce_bytes(N, V, es, n_ign, "fwd")
    b_bwd = accounting.ce_bytes(N, V, es, n_ign, "bwd")
    ms_step = total_ms / steps
    return dict(
        ms_per_step=ms_step, wall_s=wall, tokens_per_s=N * steps / (total_ms * 1e-3),
        fwd_ms_avg=fwd_ms, bwd_ms_avg=bwd_ms, bwd_inplace_ms_median=statistics.median(ip_ms),
        fwd_GBs=b_fwd / (fwd_ms * 1e-3) / 1e9, bwd_GBs=b_bwd / (bwd_ms * 1e-3) / 1e9,
        fb_GBs=(b_fwd + b_bwd) / (ms_step * 1e-3) / 1e9,
        bytes_fwd=b_fwd, bytes_bwd=b_bwd, graph_ms_per_step=graph_ms, one_pass_ms=fb_ms,
        bytes_fb_nominal=accounting.ce_bytes_nominal(N, V, es, "fb"), copy_GBs=copy_GBs,
        memory=mem,
    )


def bench_linear(case, steps: int, warmup: int, f32: bool = False):
    """The linear form's forward + backward steps; with ``f32`` the FP32-input
    entry points (FP32 X, W, dX, dW)."""
    import torch
    import vocabulary_cross_entropy_amd as vce
    from vocabulary_cross_entropy_amd import accounting

    dev = torch.device("cuda:0")
    if f32:
        X, W = torch.from_numpy(case.X).to(dev), torch.from_numpy(case.W).to(dev)
    else:
        X, W = _bf16_dev(case.X, dev), _bf16_dev(case.W, dev)
    t = torch.from_numpy(case.targets).to(dev)
    go = torch.ones(1, device=dev)
    M, H, V = case.M, case.H, case.V
    ws = vce.lce_workspace(M, H, V, dev, f32)
    fwd = vce.lce_forward_f32 if f32 else vce.lce_forward
    bwd = vce.lce_backward_f32 if f32 else vce.lce_backward
    loss = torch.empty(M, device=dev)
    mean = torch.empty((), device=dev)
    stats = torch.empty((M, 4), device=dev)
    nv = torch.empty((), dtype=torch.int32, device=dev)
    dX, dW = torch.empty_like(X), torch.empty_like(W)
    out = (loss, mean, stats, nv)
    eps = case.label_smoothing

    def f_step():
        fwd(X, W, t, eps, True, workspace=ws, out=out)

    def b_step():
        bwd(X, W, t, stats, nv, go, eps, True, workspace=ws, dX=dX, dW=dW)

    def step():
        f_step()
        b_step()

    _settle(step)
    for _ in range(warmup):
        step()
    whole = _event_pairs(1)[0]
    torch.cuda.synchronize()
    whole[0].record()
    for _ in range(steps):
        step()
    whole[1].record()
    torch.cuda.synchronize()
    total_ms = whole[0].elapsed_time(whole[1])
    avg_f = _loop_ms(f_step, steps)
    avg_b = _loop_ms(b_step, steps)
    f_fwd = accounting.linear_flops(M, H, V, "fwd")
    f_fb = accounting.linear_flops(M, H, V, "fb")
    f_bwd = accounting.linear_flops(M, H, V, "bwd")
    ms_step = total_ms / steps
    peak = accounting.BF16_MFMA_PEAK_TFLOPS
    if f32:
        # FP32 products as three BF16 products: the matrix cores do three
        # times the nominal 8 M H V flops (plus the split of X and W per call)
        fb = f_fb / (ms_step * 1e-3) / 1e12
        return dict(
            workload=case.name, M=M, H=H, V=V, ms_per_step=ms_step,
            tokens_per_s=M * steps / (total_ms * 1e-3),
            fwd_ms=avg_f, bwd_ms=avg_b,
            fb_tflops_fp32_equivalent=fb,
            fb_frac_of_fp32_mfma_peak=fb / accounting.FP32_MFMA_PEAK_TFLOPS,
            fb_bf16_mfma_tflops=3 * fb, fb_frac_of_bf16_mfma_peak=3 * fb / peak,
            workspace_MiB=ws.numel() / 2 ** 20,
        )
    return dict(
        workload=case.name, M=M, H=H, V=V, ms_per_step=ms_step,
        tokens_per_s=M * steps / (total_ms * 1e-3),
        fwd_ms=avg_f, bwd_ms=avg_b,
        fb_tflops=f_fb / (ms_step * 1e-3) / 1e12,
        roofline={"bound": "mfma", "achieved": round(f_fwd / (avg_f * 1e-3) / 1e12, 2),
                  "peak": peak, "unit": "TFLOP/s",
                  "frac": round(f_fwd / (avg_f * 1e-3) / 1e12 / peak, 4),
                  "traffic": recorded_traffic("lce_forward"),
                  "kernel": "lce_forward (GEMM + online-LSE epilogue, merge)"},
        bwd_tflops=f_bwd / (avg_b * 1e-3) / 1e12,
        fb_frac_of_peak=f_fb / (ms_step * 1e-3) / 1e12 / peak,
        workspace_MiB=ws.numel() / 2 ** 20,
    )


def _time_steps(step, steps: int, warmup: int):
    import torch
    _settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    whole = _event_pairs(1)[0]
    whole[0].record()
    for _ in range(steps):
        step()
    whole[1].record()
    torch.cuda.synchronize()
    return whole[0].elapsed_time(whole[1]) / steps


def bench_sharded_logits(case, n_shards: int, steps: int, warmup: int):
    """One vocabulary shard of the logits workload, as one of n_shards
    processes would run it: local statistics of its V/n_shards columns, the
    merge of all shards' statistics (the other shards' partials computed
    beforehand, standing in for the gather), and its backward."""
    import torch
    import vocabulary_cross_entropy_amd as vce
    from vocabulary_cross_entropy_amd import accounting

    dev = torch.device("cuda:0")
    z = _bf16_dev(case.logits, dev)
    t = torch.from_numpy(case.targets).to(dev)
    go = torch.from_numpy(case.grad_output).to(dev)
    N, V = case.N, case.V
    vl = V // n_shards
    shards = [z[:, :, k * vl:(k + 1) * vl].contiguous() for k in range(n_shards)]
    del z
    parts = torch.empty((n_shards, case.d0, case.d1, 4), device=dev)
    for k in range(n_shards):
        vce.ce_forward_shard(shards[k], t, k * vl, out=parts[k])
    zk = shards[0]
    del shards
    loss = torch.empty((case.d0, case.d1), device=dev)
    stats = torch.empty((case.d0, case.d1, 4), device=dev)
    grad = torch.empty_like(zk)
    eps = case.label_smoothing

    def fwd():
        vce.ce_forward_shard(zk, t, 0, out=parts[0])
        vce.ce_merge_shards(parts, t, V, eps, False, out=(loss, None, stats, None))

    def bwd():
        vce.ce_backward_shard(zk, t, 0, V, stats, None, go, eps, False, grad=grad)

    def step():
        fwd()
        bwd()

    ms = _time_steps(step, steps, warmup)
    ms_b = _time_steps(bwd, steps, warmup)
    b_bwd = accounting.ce_bytes(N, vl, 2, int(case.meta["n_ignored"]), "bwd")
    return dict(workload=f"logits_ce_shard_sqbv_2048x2_v{vl}_of_{V}", n_shards=n_shards,
                V_local=vl, ms_per_step=round(ms, 4), tokens_per_s=round(N / (ms * 1e-3), 1),
                bwd_ms=round(ms_b, 4),
                bwd_hbm_frac=round(b_bwd / (ms_b * 1e-3) / 1e9 / accounting.HBM_PEAK_GBS, 4))


def bench_sharded_linear(case, n_shards: int, steps: int, warmup: int):
    """One vocabulary shard of the linear workload (W split by rows into
    n_shards), forward statistics + merge + backward (dW rows and the dX
    share), as one of n_shards processes would run it."""
    import torch
    import vocabulary_cross_entropy_amd as vce
    from vocabulary_cross_entropy_amd import accounting

    dev = torch.device("cuda:0")
    M, H, V = case.M, case.H, case.V
    vl = V // n_shards
    X = _bf16_dev(case.X, dev)
    t = torch.from_numpy(case.targets).to(dev)
    go = torch.ones(1, device=dev)
    ws = vce.lce_workspace(M, H, vl, dev)
    parts = torch.empty((n_shards, M, 4), device=dev)
    for k in range(n_shards):
        Wk = _bf16_dev(case.W[k * vl:(k + 1) * vl], dev)
        vce.lce_forward_shard(X, Wk, t, k * vl, workspace=ws, out=parts[k])
    Wk = _bf16_dev(case.W[:vl], dev)
    loss, mean = torch.empty(M, device=dev), torch.empty((), device=dev)
    stats, nv = torch.empty((M, 4), device=dev), torch.empty((), dtype=torch.int32, device=dev)
    dX, dW = torch.empty_like(X), torch.empty_like(Wk)
    eps = case.label_smoothing

    def step():
        vce.lce_forward_shard(X, Wk, t, 0, workspace=ws, out=parts[0])
        vce.ce_merge_shards(parts, t, V, eps, True, out=(loss, mean, stats, nv))
        vce.lce_backward_shard(X, Wk, t, 0, V, stats, nv, go, eps, True, workspace=ws, dX=dX,
                               dW=dW)

    ms = _time_steps(step, steps, warmup)
    f = accounting.linear_flops(M, H, vl, "fb")
    return dict(workload=f"linear_ce_shard_m{M}_h{H}_v{vl}_of_{V}", n_shards=n_shards,
                V_local=vl, ms_per_step=round(ms, 4), tflops=round(f / (ms * 1e-3) / 1e12, 1),
                frac_of_mfma_peak=round(f / (ms * 1e-3) / 1e12 / accounting.BF16_MFMA_PEAK_TFLOPS,
                                        4))


def recorded_traffic(key: str):
    """HBM bytes per launch of kernel `key`, from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary under profiles/ (copy-calibrated), or None when the kernel's
    sources have changed since the counters were taken (sha256 of the listed files)."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_hbm_bytes_*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-json:"):
                    continue
                rec = json.loads(line.split(":", 1)[1]).get(key)
                if rec is None:
                    continue
                h = hashlib.sha256()
                for src in rec["sources"]:
                    with open(os.path.join(ROOT, src), "rb") as g:
                        h.update(g.read())
                return rec["bytes_per_launch"] if h.hexdigest() == rec["sha256"] else None
    return None


def cpu_baseline(case, budget_s: float = 10.0):
    """The FP64 oracle (C core, OpenMP over rows) on a bounded sample of the
    workload: 64-row batches of randomly chosen rows, forward (loss and
    statistics) then backward (gradient rows), until the time budget is spent
    (passes over all rows repeat if the budget allows)."""
    import oracle
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    N = case.N
    rng = np.random.default_rng(0)
    order = rng.permutation(N)
    done, chunk = 0, 64
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s = done % N
        rows = np.sort(order[s:s + chunk])
        oracle.ce_forward(case.logits, case.targets, case.label_smoothing, case.ignore_idx, rows=rows)
        oracle.ce_backward(case.logits, case.targets, g, case.label_smoothing, case.ignore_idx,
                           rows=rows)
        done += rows.size
    el = time.perf_counter() - t0
    return {"value": round(done / el, 1), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{done} row passes over random rows of the {N}-row workload "
                      f"(forward + backward, FP64), {el:.1f} s"}


def cpu_baseline_linear(case, tokens: int = 512):
    """The FP64 oracle of the linear form (NumPy FP64 products, the C core for
    the loss and dZ) on a bounded sample: the first ``tokens`` tokens through
    the full vocabulary, forward (loss and statistics) and backward (their dX
    rows and their share of dW), one call each."""
    import oracle
    from oracle import linear
    g = oracle.row_scale(case.grad_output, case.targets, case.reduce_loss, case.ignore_idx)
    sel = slice(0, min(tokens, case.M))
    t0 = time.perf_counter()
    linear.forward(case.X[sel], case.W, case.targets[sel], case.label_smoothing, case.ignore_idx)
    linear.backward(case.X[sel], case.W, case.targets[sel], g[sel], case.label_smoothing,
                    case.ignore_idx)
    el = time.perf_counter() - t0
    n = sel.stop - sel.start
    return {"value": round(n / el, 2), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"tokens 0..{n - 1} of the {case.M}-token workload through all "
                      f"{case.V} classes (forward + backward, FP64), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-linear", action="store_true", help="skip the fused linear form")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the one-shard-of-eight vocabulary-sharded runs")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the (B,SQ,V) = (4,1024,32000) logits, the tiny logits and the "
                         "M=16384 H=2304 V=256003 linear workloads")
    ap.add_argument("--no-f32", action="store_true",
                    help="skip the FP32-input run of the linear form")
    ap.add_argument("--only", choices=["logits", "linear"], default=None,
                    help="run one form only (for profiling)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    from vocabulary_cross_entropy_amd import accounting
    from vocabulary_cross_entropy_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cpu_on = not args.no_cpu
    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        say("copy calibration: 5 copies of 1 GiB done")
    say("generating the (SQ,B,V) = (2048, 2, 128256) BF16 workload")
    case = wl.headline_logits()
    res = None
    if args.only in (None, "logits"):
        res = bench_logits(case, args.steps, args.warmup)
        say(f"logits CE: {res['ms_per_step']:.3f} ms/step")
    sharded = {}
    if res is not None and not args.no_shard:
        sharded["logits"] = bench_sharded_logits(case, 8, args.steps, min(args.warmup, 5))
        say(f"logits CE, one shard of 8: {sharded['logits']['ms_per_step']:.3f} ms/step")
    other = {}
    if res is not None and not args.no_other:
        mcase = wl.medium_logits()
        r = bench_logits(mcase, args.steps, args.warmup)
        b_fb = r["bytes_fwd"] + r["bytes_bwd"]
        other[mcase.name] = {
            "ms_per_step": round(r["ms_per_step"], 4),
            "tokens_per_s": round(r["tokens_per_s"], 1),
            "fwd_ms": round(r["fwd_ms_avg"], 4),
            "bwd_ms": round(r["bwd_ms_avg"], 4),
            "fb_GBs": round(r["fb_GBs"], 1),
            "fb_frac_of_hbm_peak": round(r["fb_GBs"] / accounting.HBM_PEAK_GBS, 4),
            "fb_nominal_frac_of_hbm_peak": round(
                r["bytes_fb_nominal"] / (r["ms_per_step"] * 1e-3) / 1e9
                / accounting.HBM_PEAK_GBS, 4),
            "fb_bytes": b_fb,
            "graph_replay_ms_per_step": round(r["graph_ms_per_step"], 4),
            "one_pass_ms_per_step": round(r["one_pass_ms"], 4),
            "one_pass_tokens_per_s": round(mcase.N / (r["one_pass_ms"] * 1e-3), 1),
            "cpu_baseline": cpu_baseline(mcase, 5.0) if cpu_on else None}
        say(f"logits CE {mcase.name}: {r['ms_per_step']:.4f} ms/step")
        del mcase
        # the tiny correctness workload (B=2, SQ=4, V=1000 FP32) in its four
        # label-smoothing x reduction settings: launch-bound, so only its step
        # time is reported (a roofline fraction would mean nothing here)
        for eps_, red_ in ((0.0, False), (0.0, True), (0.1, False), (0.1, True)):
            tcase = wl.tiny_logits(eps_, red_)
            r = bench_logits(tcase, args.steps, args.warmup)
            other[tcase.name] = {"ms_per_step": round(r["ms_per_step"], 4),
                                 "tokens_per_s": round(r["tokens_per_s"], 1),
                                 "one_pass_ms_per_step": round(r["one_pass_ms"], 4),
                                 "bound": "launch latency",
                                 "cpu_baseline": cpu_baseline(tcase, 1.0) if cpu_on else None}
        say("logits CE tiny workloads: " + ", ".join(
            str(v["ms_per_step"]) for k, v in other.items() if k.startswith("tiny")) + " ms/step")
    lin = None
    if not args.no_linear and args.only in (None, "linear"):
        say("generating the linear workload M=4096 H=4096 V=131072")
        lcase = wl.linear_4k()
        lin = bench_linear(lcase, max(3, min(args.steps, 10)), min(args.warmup, 3))
        say(f"linear CE: {lin['ms_per_step']:.3f} ms/step")
        if not args.no_shard:
            sharded["linear"] = bench_sharded_linear(lcase, 8, max(3, min(args.steps, 10)),
                                                     min(args.warmup, 3))
            say(f"linear CE, one shard of 8: {sharded['linear']['ms_per_step']:.3f} ms/step")
        if cpu_on:
            lin["cpu_baseline"] = cpu_baseline_linear(lcase)
            say(f"linear CE oracle: {lin['cpu_baseline']['sample']}")
        del lcase
        if not args.no_other:
            say("generating the linear workload M=16384 H=2304 V=256003")
            l5case = wl.linear_16k()
            l5 = bench_linear(l5case, max(3, min(args.steps, 5)), min(args.warmup, 2))
            other[l5["workload"]] = {k: (round(v, 4) if isinstance(v, float) else v)
                                     for k, v in l5.items()
                                     if k in ("ms_per_step", "tokens_per_s", "fwd_ms",
                                              "bwd_ms", "fb_tflops", "bwd_tflops",
                                              "fb_frac_of_peak", "workspace_MiB")}
            other[l5["workload"]]["fwd_tflops"] = l5["roofline"]["achieved"]
            if cpu_on:
                other[l5["workload"]]["cpu_baseline"] = cpu_baseline_linear(l5case)
            del l5case
            say(f"linear CE {l5['workload']}: {l5['ms_per_step']:.3f} ms/step")
        if not args.no_f32:
            say("generating the FP32 linear workload M=4096 H=4096 V=131072")
            lin["fp32_inputs"] = bench_linear(wl.linear_4k_f32(), max(3, min(args.steps, 5)),
                                              min(args.warmup, 2), f32=True)
            say(f"linear CE, FP32 inputs: {lin['fp32_inputs']['ms_per_step']:.3f} ms/step")
    if res is None:
        print(json.dumps({"linear_ce": lin}))
        return
    cpu = cpu_baseline(case) if cpu_on else None
    peak = accounting.HBM_PEAK_GBS
    b_fb = res["bytes_fwd"] + res["bytes_bwd"]
    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "logits_ce_fwd_bwd_sqbv_2048x2_v128256", "tokens": case.N,
                   "V": case.V, "layout": "SQ,B,V", "storage": "bf16",
                   "label_smoothing": case.label_smoothing, "reduce_loss": case.reduce_loss,
                   "ignored_rows": case.meta["n_ignored"], "grad": "separate buffer"},
        # the dominant kernel (the backward sweep): its algorithmic bytes per
        # launch over its average launch duration (events around a loop of its
        # launches on the stream it runs on)
        "roofline": {"bound": "hbm", "achieved": round(res["bwd_GBs"], 1), "peak": peak,
                     "unit": "GB/s", "frac": round(res["bwd_GBs"] / peak, 4),
                     "traffic": recorded_traffic("ce_bwd"),
                     "kernel": "ce_bwd (ce_backward row sweep)",
                     "bytes_per_launch": res["bytes_bwd"]},
        # the whole step the metric names: forward + backward algorithmic bytes
        # over ms_per_step
        "fb_roofline": {"bound": "hbm", "achieved": round(res["fb_GBs"], 1), "peak": peak,
                        "unit": "GB/s", "frac": round(res["fb_GBs"] / peak, 4),
                        "bytes_per_step": b_fb,
                        "nominal_frac": round(res["bytes_fb_nominal"] / (res["ms_per_step"] * 1e-3)
                                              / 1e9 / peak, 4)},
        "cpu_baseline": cpu,
        "phases": {"fwd_ms": round(res["fwd_ms_avg"], 4),
                   "bwd_ms": round(res["bwd_ms_avg"], 4),
                   "bwd_inplace_ms_median": round(res["bwd_inplace_ms_median"], 4),
                   "fwd_GBs": round(res["fwd_GBs"], 1), "bwd_GBs": round(res["bwd_GBs"], 1),
                   "fb_GBs": round(res["fb_GBs"], 1),
                   "graph_replay_ms_per_step": round(res["graph_ms_per_step"], 4),
                   "one_pass_ms_per_step": round(res["one_pass_ms"], 4),
                   "one_pass_tokens_per_s": round(case.N / (res["one_pass_ms"] * 1e-3), 1),
                   "one_pass_GBs": round(res["bytes_bwd"] / (res["one_pass_ms"] * 1e-3) / 1e9,
                                         1),
                   "copy_ceiling_GBs": round(res["copy_GBs"], 1),
                   "bwd_frac_of_copy_ceiling": round(res["bwd_GBs"] / res["copy_GBs"], 4)},
        "memory": res["memory"],
        "linear_ce": lin,
        "vocab_sharded_one_of_8": sharded or None,
        "other_configs": other or None,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
