"""Pins of the SiLU-and-mul oracle (oracle/glu.py) against things other than itself."""

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits, make_inputs


def test_silu_matches_torch_in_float64():
    """A library routine: torch's SiLU (x * sigmoid(x)) in float64."""
    x = np.concatenate([np.linspace(-60, 60, 24001), [-1e3, -745.0, -0.0, 0.0, 1e-300, 710.0, 1e3]])
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    got = oracle.silu(x)
    assert np.allclose(got, ref, rtol=1e-15, atol=1e-300)
    assert np.all(np.signbit(got[x == -1e3]) | (got[x == -1e3] == 0))


def test_silu_odd_part_identity():
    """silu(x) - silu(-x) = x: the logistic function satisfies s(x) + s(-x) = 1."""
    x = np.linspace(-40, 40, 8001)
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-13)


def test_silu_closed_forms_and_slope_bound():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(np.log(3.0)) == pytest.approx(0.75 * np.log(3.0), rel=1e-15)   # s(ln 3) = 3/4
    x = np.linspace(-30, 30, 600001)
    slope = np.abs(np.diff(oracle.silu(x)) / np.diff(x))
    assert slope.max() <= oracle.SILU_SLOPE_MAX and slope.max() > 1.09


def test_gate_is_the_first_half_and_up_the_second():
    g = np.array([[2.0, -1.0, 0.0]])
    u = np.array([[3.0, 5.0, 7.0]])
    h = oracle.glu_values(np.concatenate([g, u], axis=1))
    assert np.allclose(h, [[2.0 / (1 + np.exp(-2.0)) * 3.0, -1.0 / (1 + np.e) * 5.0, 0.0]], rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.glu_values(np.ones((1, 3)))


@pytest.mark.parametrize("fmt", [oracle.FMT_FP8_DYNAMIC, oracle.FMT_W8A8_INT8, oracle.FMT_BLOCK_FP8])
def test_glu_bound_accepts_binary32_evaluation_and_rejects_a_swapped_half(fmt):
    """A binary32 evaluation of the fused epilogue (the way a kernel computes
    it, from binary32 epilogue values) passes; using the up half as the gate
    fails on most elements."""
    M, I, K = 6, 256, 512
    x, w = make_inputs(K, 2 * I, M, 0.02, seed=9)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    h_ref, h_true, bound = oracle.glu_reference(fmt, r)
    if fmt == oracle.FMT_W8A8_INT8:
        t = (oracle.f32(r["S"]) * np.asarray(r["s_a"], np.float32)[:, None]) * np.asarray(r["s_w"], np.float32)[None, :]
    else:
        t = oracle.f32(r["y_true"])                     # one binary32 rounding of the exact value
    t = t.astype(np.float32)
    g, u = t[:, :I], t[:, I:]
    h32 = (g / (np.float32(1) + np.exp(-g))) * u       # binary32 throughout
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(h32), h_ref, h_true, bound)
    assert st["ok"], st
    bad = (u / (np.float32(1) + np.exp(-u))) * u
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(bad.astype(np.float32)), h_ref, h_true, bound)
    assert not st["ok"] and st["n_fail"] > 0.5 * M * I
