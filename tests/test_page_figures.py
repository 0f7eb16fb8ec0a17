"""Pin the work accounting and the headline workload to figures the pages print."""
import json
import os

import pytest

from vocabulary_cross_entropy_amd import accounting

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_te_memory_figures_match_headline_shape():
    g = GOLD["te_memory"]
    N, V = g["logits_rows"], g["vocab"]
    # the FP32 derivative the old design saved, and the BF16 gradient buffer
    assert round(N * V * 4 / 2 ** 30, 2) == g["fp32_derivative_GiB"]
    assert round(N * V * 2 / 2 ** 20) == g["bf16_gradient_MiB"]
    # one BF16 gradient buffer is the backward's write; with no ignored rows the
    # algorithmic model equals the nominal one (1 read fwd, 1 read + 1 write bwd)
    assert accounting.ce_bytes(N, V, 2, 0, "bwd") == 2 * N * V * 2
    assert accounting.ce_bytes(N, V, 2, 0, "fb") == accounting.ce_bytes_nominal(N, V, 2, "fb")
    # ignored rows are written but never read
    assert accounting.ce_bytes(N, V, 2, 82, "fwd") == (N - 82) * V * 2


@pytest.mark.parametrize("row", GOLD["liger_tp1"]["rows"],
                         ids=lambda r: f"{r['M']}x{r['H']}x{r['V']}-{r['phase']}")
def test_linear_flop_convention(row):
    # TF/s printed = flops / time: it reproduces within the rounding of the
    # printed figures (+-0.0005 ms, +-0.05 TF/s; a median over 30 runs adds a
    # little more, so twice that is allowed) only with 2*M*H*V per GEMM and
    # four GEMMs for forward+backward.
    f = accounting.linear_flops(row["M"], row["H"], row["V"], row["phase"])
    tol = 2 * (row["tflops"] * 0.0005 / row["ms"] + 0.05)
    assert f / (row["ms"] * 1e-3) / 1e12 == pytest.approx(row["tflops"], abs=tol)
    if row["phase"] == "fb":
        f3 = accounting.linear_flops(row["M"], row["H"], row["V"], "bwd")
        assert abs(f3 / (row["ms"] * 1e-3) / 1e12 - row["tflops"]) > 100
