"""GPU parity of the decode GEMM with fused activation quantization (a_mode 4):
per-token amax for FP8_Dynamic and INT8, per 1 x 128 group for Block_FP8.

One launch reads bf16 X, quantizes it inside every workgroup and runs the
GEMM.  What it writes out must be exactly what the two-launch path writes:
the packed codes and the scales bit-exact against the oracle, INT8 outputs
bit-exact, FP8 outputs inside the oracle's acceptance rule.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import dev_bf16, fp8_check, fp8_ok, host_bf16_bits, MIN_FRAC_WITHIN_ULP, pack_ref, requires_gpu
from tests.instantiations import cases
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]

# waves per workgroup x waves sharing K x rows per wave x batch x swap
FVARIANTS = [v for v in itertools.product([4, 8, 16], [1, 2, 4, 8, 16], [16, 32, 64], [1, 2, 4], [0, 1])
             if v[1] <= v[0] and not (v[0] > 4 and v[3] == 4)]
# token count x K (M*K <= 16384, K % 512 == 0)
SHAPES = [(1, 4096), (3, 4096), (16, 1024), (2, 8192), (1, 512), (5, 2048)]
SPLITS = [1, 2, 4, 8]


def _codes_u8(fmt, q):
    q = np.asarray(q)
    return q.astype(np.int8).view(np.uint8) if fmt == ql.W8A8_INT8 else q.astype(np.uint8)


def _forward(plan, fmt, xb, w_q, w_s, y_fill=float("nan")):
    """qlinear_forward with fresh output buffers (filled with garbage first)."""
    M, N, K = plan.M, plan.N, plan.K
    a_p = ql.act_buffer(plan)
    a_p.view(torch.uint8).fill_(0xA5)
    a_s = torch.full(ql.act_scale_shape(fmt, M, K), -7.0, dtype=torch.float32, device="cuda")
    y = torch.full((M, N), y_fill, dtype=torch.bfloat16, device="cuda")
    ws = plan.new_workspace()
    ql.qlinear_forward(plan, dev_bf16(xb), a_p, a_s, w_q, w_s, y, ws)
    torch.cuda.synchronize()
    return a_p, a_s, host_bf16_bits(y), ws


def _check(fmt, r, plan, a_p, a_s, y, label, waves_k=16):
    M, K = plan.M, plan.K
    n = ql.qlinear_packed_act_bytes(M, K)
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(_codes_u8(fmt, r["a_q"]))), label
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), np.asarray(r["s_a"], np.float32).view(np.uint32)), label
    if fmt == ql.W8A8_INT8:
        bad = np.argwhere(y != r["y_ref"])
        assert bad.size == 0, (label, bad[:5])
    else:
        st = fp8_check(fmt, r, y, plan.facts["chunks"], waves_k)
        assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (label, st)


def _weights(fmt, r):
    w_q = torch.from_numpy(_codes_u8(fmt, r["w_q"])).cuda()
    w_q = w_q.view(torch.int8) if fmt == ql.W8A8_INT8 else w_q.view(torch.float8_e4m3fn)
    return ql.pack_weight(w_q), torch.from_numpy(np.asarray(r["s_w"], np.float32)).cuda()


def _fused_args(fmt, vi):
    nw, wk, rows, pf, swap = FVARIANTS[vi]
    M, K = SHAPES[vi % len(SHAPES)]
    split = SPLITS[(vi // 2) % len(SPLITS)]
    N = 300 + 16 * (vi % 7)                      # several tiles + a ragged tail
    cfg = dict(swap_ab=swap, split_k=split, waves_n=nw // wk, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=4, w_layout=1)
    return fmt, M, N, K, cfg


FUSED_CASES = cases("fused", [(f, vi) for f in FMTS for vi in range(len(FVARIANTS))], _fused_args)


@pytest.mark.parametrize("fmt,vi", FUSED_CASES)
def test_every_fused_instantiation_matches_oracle(fmt, vi):
    _, M, N, K, cfg = _fused_args(fmt, vi)
    wk = cfg["waves_k"]
    x, w = make_inputs(K, N, M, 0.02, seed=4000 + vi)
    xb = bf16_bits(x)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    w_p, w_s = _weights(fmt, r)
    a_p, a_s, y, ws = _forward(plan, fmt, xb, w_p, w_s)
    _check(fmt, r, plan, a_p, a_s, y, str(cfg), waves_k=wk)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_special_rows(fmt):
    """Zero rows, negative zeros, tiny rows on both sides of the reciprocal
    path's lower scale limit, saturating values, and bf16 subnormals."""
    M, N, K = 8, 320, 2048
    xr = np.zeros((M, K))
    xr[1, :] = np.linspace(-3, 3, K)
    xr[2, 7] = -1e-38
    xr[3, :] = 2.0 ** -130
    xr[4, ::2] = -0.0
    xr[5, :] = 448.0 * np.sign(np.sin(np.arange(K)))
    xr[5, 3] = 1e30
    xr[6, :] = np.linspace(-1, 1, K) * 2.0 ** -88
    xr[7, :] = np.linspace(-1, 1, K) * 2.0 ** -92
    xb = torch.from_numpy(xr.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, w = make_inputs(K, N, 1, 0.02, seed=77)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(swap_ab=1, split_k=2, waves_n=2, waves_k=2, a_mode=4,
                                                         w_layout=1))
    w_p, w_s = _weights(fmt, r)
    a_p, a_s, y, _ = _forward(plan, fmt, xb, w_p, w_s)
    n = ql.qlinear_packed_act_bytes(M, K)
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(_codes_u8(fmt, r["a_q"])))
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), np.asarray(r["s_a"], np.float32).view(np.uint32))
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(y, r["y_ref"])
    else:
        st = fp8_check(fmt, r, y, 2, 2)
        assert fp8_ok(st), st


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 6144, 4096), (4, 4096, 4096), (1, 4096, 12288)])
def test_fused_equals_two_launch_forward(fmt, M, N, K):
    """At decode shapes the fused launch and quantizer + GEMM give the same
    codes, scales and (INT8) outputs; FP8 both inside the oracle bound."""
    x, w = make_inputs(K, N, M, 0.02, seed=M * 7 + N)
    xb = bf16_bits(x)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    w_p, w_s = _weights(fmt, r)
    base = dict(swap_ab=0, split_k=1, waves_n=1, waves_k=4, rows_per_wave=16, prefetch=2, w_layout=1)
    pf = ql.qlinear_plan_with_config(fmt, M, N, K, dict(base, a_mode=4))
    pu = ql.qlinear_plan_with_config(fmt, M, N, K, dict(base, a_mode=2))
    af, sf, yf, _ = _forward(pf, fmt, xb, w_p, w_s)
    au, su, yu, _ = _forward(pu, fmt, xb, w_p, w_s)
    n = ql.qlinear_packed_act_bytes(M, K)
    assert torch.equal(af[:n].view(torch.uint8), au[:n].view(torch.uint8))
    assert torch.equal(sf, su)
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(yf, yu) and np.array_equal(yf, r["y_ref"])
    else:
        assert fp8_ok(fp8_check(fmt, r, yf, 1, 4)) and fp8_ok(fp8_check(fmt, r, yu, 1, 4))


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_graph_replays_match_eager(fmt):
    M, N, K = 2, 1536, 4096
    x, w = make_inputs(K, N, M, 0.02, seed=41)
    xb = bf16_bits(x)
    r = oracle.reference(fmt, xb, bf16_bits(w))
    w_p, w_s = _weights(fmt, r)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(swap_ab=1, split_k=4, waves_n=2, waves_k=2, a_mode=4,
                                                         w_layout=1))
    xd = dev_bf16(xb)
    a_p = ql.act_buffer(plan)
    a_s = ql.act_scale_buffer(plan)      # Block_FP8: the [M, K/128] group scales
    y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    ws = plan.new_workspace()
    ql.qlinear_forward(plan, xd, a_p, a_s, w_p, w_s, y, ws)
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ql.qlinear_graph_begin(s)
        ql.qlinear_forward(plan, xd, a_p, a_s, w_p, w_s, y, ws, stream=s)
        g = ql.qlinear_graph_end(s)
    for i in range(4):
        y.fill_(0)
        a_p.view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        if fmt == ql.W8A8_INT8:
            assert torch.equal(y, eager), i
        else:
            assert fp8_ok(fp8_check(fmt, r, host_bf16_bits(y), 4)), i
        n = ql.qlinear_packed_act_bytes(M, K)
        assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(_codes_u8(fmt, r["a_q"]))), i
        assert int(torch.count_nonzero(ws)) == 0
        _ = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays
