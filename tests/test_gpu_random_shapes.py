"""GPU parity on seeded random shapes that no sweep-table entry covers.

Each case draws a format, a token count (mostly decode, M <= 64, some
tiled, up to 200), ragged N and K and one of the four operand layouts,
lets the planner's heuristic choose the algorithm and its configuration,
and runs the whole forward (quantizer, or the quantizer fused into the
GEMM, then the GEMM) through the C ABI.  The activation codes are compared
byte for byte with the oracle's where the plan writes them, and the bf16
output is bit-exact for INT8 and within the oracle's acceptance rule for
FP8_Dynamic and Block_FP8.
"""

import random

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import fp8_check, fp8_ok, host_bf16_bits, host_codes, pack_ref, requires_gpu
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]

FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]
LAYOUTS = [(0, 0), (1, 0), (1, 1), (1, 2)]   # (w_layout, a_packed) of qlinear_plan_layouts


def _case(i):
    rng = random.Random(1000 + i)
    fmt = FMTS[i % 3]
    M = rng.randint(1, 64) if rng.random() < 0.75 else rng.randint(65, 200)
    N = rng.randint(1, 1500)
    K = 128 * rng.randint(1, 20) if fmt == ql.BLOCK_FP8 else 16 * rng.randint(1, 160)
    return fmt, M, N, K, LAYOUTS[rng.randrange(4)]


CASES = [_case(i) for i in range(96)]


@pytest.mark.parametrize("fmt,M,N,K,layout", CASES,
                         ids=["f%d_M%d_N%d_K%d_w%da%d" % (c[0], c[1], c[2], c[3], c[4][0], c[4][1]) for c in CASES])
def test_random_shape_forward_matches_oracle(fmt, M, N, K, layout):
    x, w = make_inputs(K, N, M, 0.02, seed=M * 131 + N * 7 + K)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, *layout)
    cfg = plan.config
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    if cfg["w_layout"] == 1:
        w_q = ql.pack_weight(w_q)
    a_q = ql.act_buffer(plan)
    a_s = ql.act_scale_buffer(plan)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_q, a_s, w_q, w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    label = (fmt, M, N, K, layout, cfg)
    codes = np.asarray(r["a_q"])
    if cfg["a_mode"] in (2, 3):
        raw = codes.astype(np.int8).view(np.uint8) if fmt == ql.W8A8_INT8 else codes
        n = ql.qlinear_packed_act_bytes(M, K)
        assert np.array_equal(a_q[:n].view(torch.uint8).cpu().numpy(), pack_ref(raw)), label
    elif cfg["a_mode"] in (0, 1):
        assert np.array_equal(host_codes(fmt, a_q[:M * K].view(M, K)), codes), label
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(host_bf16_bits(y), r["y_ref"]), label
    else:
        st = fp8_check(fmt, r, host_bf16_bits(y), plan.facts["chunks"])
        assert fp8_ok(st), (label, st)


# ---------------------------------------------------------------- MXFP8 / MXFP4

def _mx_case(i):
    rng = random.Random(5000 + i)
    fmt = ql.MXFP8 if i % 2 == 0 else ql.MXFP4
    M = rng.randint(65, 200) if fmt == ql.MXFP8 and rng.random() < 0.25 else rng.randint(1, 64)
    return fmt, M, rng.randint(1, 1500), 128 * rng.randint(1, 24), (1, rng.choice((1, 2)))


MX_CASES = [_mx_case(i) for i in range(32)]


@pytest.mark.parametrize("fmt,M,N,K,layout", MX_CASES,
                         ids=["f%d_M%d_N%d_K%d_a%d" % (c[0], c[1], c[2], c[3], c[4][1]) for c in MX_CASES])
def test_random_shape_mx_forward_matches_oracle(fmt, M, N, K, layout):
    """MX forwards: the E4M3 codes and E8M0 bytes the forward writes equal the
    oracle's (packed layout, scales in lane order) and the output passes the
    oracle's MX acceptance rule."""
    from oracle import mx
    from tests.gpu_util import pack_mx_scales_ref
    x, w = make_inputs(K, N, M, 0.02, seed=M * 131 + N * 7 + K + 1)
    xb, wb = bf16_bits(x), bf16_bits(w)
    r = (mx.mx_reference if fmt == ql.MXFP8 else mx.mx4_reference)(xb, wb)
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, *layout)
    cfg = plan.config
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    w_p = ql.pack_weight(w_q) if fmt == ql.MXFP8 else ql.pack_weight_fp4(w_q)
    a_q = ql.act_buffer(plan)
    a_s = ql.act_scale_buffer(plan)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_q, a_s, w_p, ql.pack_mx_scales(w_s), y, plan.new_workspace())
    torch.cuda.synchronize()
    label = (fmt, M, N, K, layout, cfg)
    n = ql.qlinear_packed_act_bytes(M, K)
    ns = ql.qlinear_packed_mx_scale_bytes(M, K)
    assert np.array_equal(a_q[:n].view(torch.uint8).cpu().numpy(), pack_ref(np.asarray(r["a_q"]))), label
    assert np.array_equal(a_s.view(torch.uint8).flatten()[:ns].cpu().numpy(),
                          pack_mx_scales_ref(r["s_a"], K)), label
    waves_k = cfg["waves_k"] if cfg["algo"] == ql.ALGO_DECODE else 1
    d = oracle.summation_depth(K, split=plan.facts["chunks"], waves_k=waves_k)
    bound = mx.MxBound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], d, fp4=fmt == ql.MXFP4)
    st = oracle.check_fp8_parity(host_bf16_bits(y), r["y_ref"], r["y_true"], bound)
    assert fp8_ok(st), (label, st)
