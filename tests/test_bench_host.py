"""Host logic of bench.py on the CPU: the layer-solve roofline arithmetic
(t_roof from the algorithmic work of each stage and the published peaks) and
the check of the per-step flags and losses that the stream-ordered steps leave
in device memory."""
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_layer_solve_roofline_arithmetic():
    rows = n = 4096
    tokens = 65536
    stage = {"hessian": 1.3, "prepare": 3.0, "quantize": 1.0}
    r = bench.layer_solve_roofline([(rows, n, 4, 128)], [(n, tokens)], stage)
    # Hessian: n(n+1) flop per token on the bf16 MFMA (2.5 PFLOP/s)
    t_h = n * (n + 1) * tokens / 2.5e15 * 1e3
    assert math.isclose(r["stages"]["hessian"]["t_roof_ms"], t_h, rel_tol=1e-12)
    assert math.isclose(r["stages"]["hessian"]["t_roof_ms"], 0.4399120252928, rel_tol=1e-9)
    # prepare: 2n^3/3 flop in fp64 (78.6 TFLOP/s)
    t_p = 2.0 * n ** 3 / 3 / 78.6e12 * 1e3
    assert math.isclose(r["stages"]["prepare"]["t_roof_ms"], t_p, rel_tol=1e-12)
    # quantize: sweep + split-bf16 updates + minimal I/O; each part positive
    parts = r["stages"]["quantize"]["parts_ms"]
    assert all(v > 0 for v in parts.values())
    assert math.isclose(sum(parts.values()), r["stages"]["quantize"]["t_roof_ms"], rel_tol=1e-12)
    assert math.isclose(parts["sweep_fp32_valu"], rows * n * 128 / 157.3e12 * 1e3, rel_tol=1e-12)
    assert math.isclose(parts["split_bf16_updates"], 3.0 * rows * n * (n - 128) / 2.5e15 * 1e3, rel_tol=1e-12)
    # fractions are t_roof / t_measured, for the stages, the solve and the step
    for k, st in r["stages"].items():
        assert math.isclose(st["frac"], st["t_roof_ms"] / stage[k], rel_tol=1e-12)
    solve = r["stages"]["prepare"]["t_roof_ms"] + r["stages"]["quantize"]["t_roof_ms"]
    assert math.isclose(r["solve"]["frac"], solve / (stage["prepare"] + stage["quantize"]), rel_tol=1e-12)
    assert math.isclose(r["step"]["t_roof_ms"], solve + t_h, rel_tol=1e-12)
    assert r["step"]["t_ms"] == pytest.approx(5.3)


def test_layer_solve_roofline_counts_a_shared_hessian_once():
    stage = {"hessian": 1.0, "prepare": 1.0, "quantize": 1.0}
    one = bench.layer_solve_roofline([(4096, 4096, 4, 128)], [(4096, 1024)], stage)
    three = bench.layer_solve_roofline([(4096, 4096, 4, 128)] * 3, [(4096, 1024)], stage)
    assert three["stages"]["hessian"]["t_roof_ms"] == one["stages"]["hessian"]["t_roof_ms"]
    assert three["stages"]["prepare"]["t_roof_ms"] == one["stages"]["prepare"]["t_roof_ms"]
    assert math.isclose(three["stages"]["quantize"]["t_roof_ms"], 3 * one["stages"]["quantize"]["t_roof_ms"],
                        rel_tol=1e-12)


def test_check_steps():
    torch = pytest.importorskip("torch")
    bench._check_steps(torch.zeros(4, dtype=torch.int32), torch.full((4,), 2.5, dtype=torch.float64))
    bench._check_steps(torch.zeros(2, dtype=torch.int32))
    with pytest.raises(RuntimeError, match="not positive definite"):
        bench._check_steps(torch.tensor([0, 1, 0], dtype=torch.int32))
    with pytest.raises(RuntimeError, match="differ or are not finite"):
        bench._check_steps(torch.zeros(2, dtype=torch.int32), torch.tensor([1.0, 1.5], dtype=torch.float64))
    with pytest.raises(RuntimeError, match="differ or are not finite"):
        bench._check_steps(torch.zeros(2, dtype=torch.int32), torch.tensor([math.nan, math.nan], dtype=torch.float64))
    with pytest.raises(RuntimeError, match="differ or are not finite"):   # a step that never wrote its loss
        bench._check_steps(torch.zeros(2, dtype=torch.int32), torch.tensor([-1.0, -1.0], dtype=torch.float64))
