"""Host-side checks of the benchmark's contract and work models (no GPU):
the one-GPU refusal, the algorithmic byte and flop counts that the roofline
figures divide by, and the committed HBM-traffic record."""
import os
import subprocess
import sys

import pytest

from vocabulary_cross_entropy_amd import accounting
from vocabulary_cross_entropy_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""        # no JSON line for a run that did not happen


def test_logits_bytes_at_the_headline():
    # (SQ, B, V) = (2048, 2, 128256) BF16 with 82 ignored rows: the forward
    # reads the 4014 other rows once; the backward reads them again and writes
    # all 4096 rows
    N, V = 4096, 128256
    assert accounting.ce_bytes(N, V, 2, 82, "fwd") == 4014 * V * 2 == 1_029_639_168
    assert accounting.ce_bytes(N, V, 2, 82, "bwd") == 2_080_312_320
    assert accounting.ce_bytes(N, V, 2, 82, "fb") == 3_109_951_488
    # the nominal count of the statistics-saving flow: three passes over every row
    assert accounting.ce_bytes_nominal(N, V, 2, "fb") == 3_152_019_456
    with pytest.raises(ValueError):
        accounting.ce_bytes(N, V, 2, 0, "both")


def test_generated_ignored_count_is_the_one_the_byte_model_gets():
    # the generator's ignored count is what the byte model is given
    case = wl.make_logits(7, 2, 8, 16, dtype="bf16", sigma=1.0, ignore_count=3)
    assert int((case.targets == wl.IGNORE_INDEX).sum()) == 3 == case.meta["n_ignored"]


def test_linear_flops():
    # the classifier GEMM of the M = H = 4096, V = 131072 workload
    assert accounting.linear_flops(4096, 4096, 131072, "fwd") == 2.0 * 4096 * 4096 * 131072
    assert accounting.linear_flops(4096, 4096, 131072, "fb") == 17_592_186_044_416.0
    assert accounting.linear_flops(16384, 2304, 256003, "fb") == 8.0 * 16384 * 2304 * 256003


def test_peaks():
    assert accounting.HBM_PEAK_GBS == 8000.0
    # 256 CUs x 2.4 GHz x 4096 BF16 flop per clock per CU
    assert abs(accounting.BF16_MFMA_PEAK_TFLOPS - 256 * 2.4e9 * 4096 / 1e12) < 0.1


def test_recorded_traffic_is_current_and_near_the_algorithmic_bytes():
    # The committed FETCH_SIZE / WRITE_SIZE record is reported only while the
    # kernel sources still hash to what was profiled; when it is reported it
    # must be close to the algorithmic bytes of the backward (no re-reads).
    sys.path.insert(0, ROOT)
    import bench
    t = bench.recorded_traffic("ce_bwd")
    if t is None:
        pytest.skip("kernel sources changed since the HBM counters were taken")
    assert 1.0 <= t / 2_080_312_320 <= 1.01
