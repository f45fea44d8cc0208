"""Pins for the oracle's pre-norm sum over several input buffers (Mojo
allreduce_residual_rmsnorm_fp8, Args: input_buffers, residual,
residual_output): s = round_to_in_dtype(residual + sum of the inputs), the
exact sum rounded once, then the FP8 path on s.

Hand rows (tests/golden/hand_rows.json, "allreduce_rows") fix the one
rounding of the exact sum, where rounding after each addition would differ.
Invariants: one input is the residual path itself; the order of the inputs
does not matter (the sums are exact); a zero input changes nothing; the
quantized outputs are the FP8 path's on the stored sum."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
KW = dict(eps=1e-6, weight_offset=0.0, scale_ub=1200.0, out_fmt="e4m3fn", scales_dtype="f32")


def bits(vals, dt):
    return workloads.bits(torch.tensor(vals, dtype=torch.float64).to(TD[dt]))


@pytest.mark.parametrize("row", GOLDEN["allreduce_rows"], ids=lambda r: r["id"])
def test_hand_rows(row):
    dt = row["in_dtype"]
    s = oracle.sum_round([bits([v], dt) for v in row["inputs"]], bits([row["residual"]], dt), in_dtype=dt)
    width = 8 if dt == "f32" else 4
    assert [f"0x{int(b):0{width}X}" for b in np.ravel(s).view(np.uint32 if dt == "f32" else np.uint16)] == \
        row["expect_residual_out_bits"]


def _rand(rows, hidden, dt, n, seed):
    rng = np.random.default_rng(seed)
    mk = lambda: bits(rng.standard_normal((rows, hidden)), dt)  # noqa: E731
    return [mk() for _ in range(n)], mk(), bits(rng.uniform(0.5, 1.5, hidden), dt)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_one_input_is_the_residual_path(dt):
    ins, r, g = _rand(37, 96, dt, 1, 1)
    a = oracle.allreduce_residual_rmsnorm_fp8(ins, r, g, in_dtype=dt, **KW)
    b = oracle.rmsnorm_fp8(ins[0], g, in_dtype=dt, residual=r, **KW)
    assert np.array_equal(a["residual_out"], b["residual_out"])
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_input_order_and_zero_inputs(dt):
    ins, r, g = _rand(29, 64, dt, 5, 2)
    a = oracle.sum_round(ins, r, in_dtype=dt)
    assert np.array_equal(a, oracle.sum_round(ins[::-1], r, in_dtype=dt))
    assert np.array_equal(a, oracle.sum_round([ins[2], ins[0], ins[4], ins[1], ins[3]], r, in_dtype=dt))
    zero = np.zeros_like(ins[0])
    assert np.array_equal(a, oracle.sum_round(ins + [zero, zero], r, in_dtype=dt))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_sum_matches_the_exact_sum_rounded_once(dt):
    # 16-bit inputs: the float64 sum of a few of them is exact here, so the
    # stored value is torch's single rounding of that sum
    ins, r, _ = _rand(16, 128, dt, 8, 3)
    vals = [torch.from_numpy(t.view(np.int16)).view(TD[dt]).double().numpy() for t in ins + [r]]
    exact = np.sum(np.stack(vals), axis=0)
    want = workloads.bits(torch.from_numpy(exact).to(TD[dt]))
    assert np.array_equal(oracle.sum_round(ins, r, in_dtype=dt), want)


def test_quantized_outputs_are_the_fp8_path_on_the_sum():
    ins, r, g = _rand(21, 256, "bf16", 3, 4)
    a = oracle.allreduce_residual_rmsnorm_fp8(ins, r, g, in_dtype="bf16", **KW)
    b = oracle.rmsnorm_fp8(a["residual_out"], g, in_dtype="bf16", **KW)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
