"""GPU parity of the SiLU-and-mul epilogue (merged gate/up weight, output
silu(gate) * up) against the oracle's glu_reference: within one bf16 ulp of
the reference or inside the bound that carries the linear's accumulation
bound through SiLU and the product (INT8: binary32 evaluation error only)."""

import itertools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import dev_bf16, host_bf16_bits, MIN_FRAC_WITHIN_ULP, pack_ref, requires_gpu
from tests.instantiations import cases
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]
# swap x (waves_n, waves_k) x batch x activation mode (2 packed A_q, 4 fused quantization)
GVARIANTS = list(itertools.product([0, 1], [(1, 4), (2, 2), (4, 1), (1, 8), (2, 4)], [1, 2], [2, 4]))
SPLITS = [1, 2, 4]


def _codes_u8(fmt, q):
    q = np.asarray(q)
    return q.astype(np.int8).view(np.uint8) if fmt == ql.W8A8_INT8 else q.astype(np.uint8)


def _dev_codes(fmt, q_u8):
    t = torch.from_numpy(np.ascontiguousarray(q_u8)).cuda()
    return t.view(torch.int8) if fmt == ql.W8A8_INT8 else t.view(torch.float8_e4m3fn)


def _run_glu(plan, fmt, r, xb):
    """Run a SiLU-and-mul plan on the oracle's codes (a_mode 2) or on X (a_mode 4)."""
    M, N, K = plan.M, plan.N, plan.K
    w_p = ql.pack_weight(_dev_codes(fmt, _codes_u8(fmt, r["w_q"])))
    w_s = torch.from_numpy(np.asarray(r["s_w"], np.float32)).cuda()
    y = torch.full((M, N // 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = plan.new_workspace()
    if plan.config["a_mode"] == 4:
        a_p = ql.act_buffer(plan)
        a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
        ql.qlinear_forward(plan, dev_bf16(xb), a_p, a_s, w_p, w_s, y, ws)
    else:
        a_p = _dev_codes(fmt, pack_ref(_codes_u8(fmt, r["a_q"])))
        a_s = torch.from_numpy(np.asarray(r["s_a"], np.float32)).cuda()
        ql.qlinear_run(plan, a_p, a_s, w_p, w_s, y, ws)
    torch.cuda.synchronize()
    return host_bf16_bits(y), ws


def _check(fmt, r, h, plan, waves_k):
    h_ref, h_true, bound = oracle.glu_reference(fmt, r, split=plan.facts["chunks"], waves_k=waves_k)
    st = oracle.check_fp8_parity(h, h_ref, h_true, bound)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


def _glu_args(fmt, vi):
    swap, (wn, wk), pf, amode = GVARIANTS[vi]
    M = [1, 3, 13][vi % 3] if amode == 4 else [5, 20, 29][vi % 3]
    I = [304, 528][vi % 2]                            # several tiles + a ragged last one
    K = 1024 if amode == 4 or fmt == ql.BLOCK_FP8 else 1040
    split = SPLITS[(vi // 2) % len(SPLITS)]
    cfg = dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=32, prefetch=pf, a_mode=amode,
               w_layout=1)
    return fmt, M, 2 * I, K, cfg


GLU_CASES = cases("glu", [(f, vi) for f in FMTS for vi in range(len(GVARIANTS))], _glu_args,
                  ql.qlinear_plan_glu_with_config)


@pytest.mark.parametrize("fmt,vi", GLU_CASES)
def test_every_glu_instantiation_matches_oracle(fmt, vi):
    _, M, N2, K, cfg = _glu_args(fmt, vi)
    wk = cfg["waves_k"]
    x, w = make_inputs(K, N2, M, 0.02, seed=6000 + vi * 3 + fmt)
    xb = bf16_bits(x)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    plan = ql.qlinear_plan_glu_with_config(fmt, M, N2, K, cfg)
    assert plan.facts["epilogue"] == 1
    h, ws = _run_glu(plan, fmt, r, xb)
    _check(fmt, r, h, plan, wk)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 4, 16, 32])
def test_glu_plan_on_the_gate_up_shape(fmt, M):
    """The planner's SiLU-and-mul plan for the 8B gate_up weight (24576 x 4096
    = gate 12288 + up 12288), checked on 64 sampled output columns."""
    I, K = 12288, 4096
    ql.load_default_table()
    x, w = make_inputs(K, 2 * I, M, 0.02, seed=31 + M)
    xb = bf16_bits(x)
    plan = ql.qlinear_plan_glu(fmt, M, 2 * I, K, 2)
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    y = torch.empty(M, I, dtype=torch.bfloat16, device="cuda")
    a_p = ql.act_buffer(plan)
    a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_p, a_s, ql.pack_weight(w_q), w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    h = host_bf16_bits(y)
    rng = np.random.default_rng(M)
    if fmt == ql.BLOCK_FP8:             # whole 128-row scale blocks on both halves
        nb = int(rng.integers(0, I // 128))
        cols = np.arange(nb * 128, nb * 128 + 128)
    else:
        cols = np.sort(rng.choice(I, 64, replace=False))
    rows = np.concatenate([cols, I + cols])
    r = oracle.reference(fmt, xb, bf16_bits(w[torch.from_numpy(rows)]))
    h_ref, h_true, bound = oracle.glu_reference(fmt, r, split=plan.facts["chunks"])
    st = oracle.check_fp8_parity(h[:, cols], h_ref, h_true, bound)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


@pytest.mark.parametrize("fmt", FMTS)
def test_glu_plan_with_k_zero_writes_only_its_output(fmt):
    """K = 0: the SiLU-and-mul output [M, N/2] becomes silu(0) * 0 = 0 and the
    run writes nothing past it (the sentinel after Y keeps its value)."""
    M, N = 4, 64
    plan = ql.qlinear_plan_glu(fmt, M, N, 0, 1)
    buf = torch.full((2 * M * (N // 2),), 3.0, dtype=torch.bfloat16, device="cuda")
    y = buf[:M * (N // 2)].view(M, N // 2)
    e = torch.empty(16, dtype=torch.uint8, device="cuda")
    f = torch.empty(16, dtype=torch.float32, device="cuda")
    ql.qlinear_run(plan, e, f, e, f, y)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0
    assert bool(torch.all(buf[M * (N // 2):] == 3.0))


def _glu_case(i):
    import random
    rng = random.Random(700 + i)
    fmt = FMTS[i % 3]
    M = rng.choice([1, 2, 3, 5, 9, 16, 17, 24, 32])
    I = 16 * rng.randint(1, 64)
    K = 128 * rng.randint(1, 24) if fmt == ql.BLOCK_FP8 else 16 * rng.randint(8, 200)
    return fmt, M, I, K, rng.choice([1, 2])


GLU_CASES = [_glu_case(i) for i in range(24)]


@pytest.mark.parametrize("fmt,M,I,K,a_packed", GLU_CASES,
                         ids=["f%d_M%d_I%d_K%d_a%d" % c for c in GLU_CASES])
def test_glu_table_free_plans_match_oracle(fmt, M, I, K, a_packed):
    """SiLU-and-mul plans for shapes the table lacks (the heuristic's plan,
    reshaped to the SiLU-and-mul kernels): gate/up weights [2I, K] against the
    oracle, with quantized activations in (a_packed 1) or X in (2)."""
    ql.qlinear_table_clear()
    try:
        plan = ql.qlinear_plan_glu(fmt, M, 2 * I, K, a_packed)
    finally:
        ql.load_default_table()
    x, w = make_inputs(K, 2 * I, M, 0.02, seed=M * 7 + I + K)
    xb = bf16_bits(x)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    h, ws = _run_glu(plan, fmt, r, xb)
    _check(fmt, r, h, plan, plan.config["waves_k"])
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0
