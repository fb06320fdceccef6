"""The benchmark's work model on the CPU: the algorithmic FLOPs of a prefill
for every workload (forward of every layer, head, backward of the fast
blocks, flash recomputation not counted), the SGD kernel's algorithmic bytes
and the read without updates.  Values are the closed forms evaluated
independently for each workload's shapes (3B at 128K: 1,645.6 TFLOP, of
which 1,214.9 forward)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("name,tflop", [("c2", 3.0440), ("c3", 90.762), ("c4", 1645.56), ("c5", 6624.30)])
def test_prefill_flops(name, tflop):
    cfg = synth.config(name)
    assert bench.prefill_flops(cfg, cfg["T"]) / 1e12 == pytest.approx(tflop, rel=2e-4)


def test_forward_flops_and_sgd_bytes_3b():
    cfg = synth.config("c4")
    assert bench.forward_flops(cfg, cfg["T"]) / 1e12 == pytest.approx(1214.9, rel=2e-4)
    # per fast weight 10 B (fp32 master read + write, bf16 copy), plus both
    # bf16 operands over the chunk's 1024 tokens: 408.9 MB per launch on
    # average; the design's 14 B per weight: 559.9 MB
    d, F = 3072, 8192
    up = 10 * 2 * F * d + 2 * (2 * F + d) * 1024
    dn = 10 * d * F + 2 * (d + F) * 1024
    assert bench.sgd_bytes_per_launch(cfg, cfg["T"]) == pytest.approx((up + dn) / 2, rel=1e-9)
    assert bench.sgd_bytes_per_launch(cfg, cfg["T"]) / 1e6 == pytest.approx(408.9, abs=0.05)
    assert bench.sgd_bytes_per_launch(cfg, cfg["T"], per_weight=14) / 1e6 == pytest.approx(559.9, abs=0.05)
    assert bench.sgd_flops_per_launch(cfg, cfg["T"]) == pytest.approx(2.0 * (d * F + 2 * F * d) * 1024 / 2,
                                                                      rel=1e-9)


def test_static_second_mlp_adds_its_products():
    cfg = synth.config("c4")
    cs = synth.config("c4", static_mlp=1)
    T, q, d, F = cfg["T"], cfg["n_fast"], cfg["d_model"], cfg["d_ff"]
    extra = 2 * (2 * T * q * 3 * d * F)      # its forward and its two input-gradient products
    assert bench.prefill_flops(cs, T) - bench.prefill_flops(cfg, T) == pytest.approx(extra, rel=1e-12)
