"""GPU parity of the MXFP8 path against the oracle's MX statement
(oracle/mx.py): the quantizer bit-exact (E4M3 codes and E8M0 bytes, row-major
and packed), the GEMM inside the oracle's acceptance rule -- within one bf16
ulp of the correctly rounded product, or inside the binary32 forward-error
bound over the block-scaled products -- for every instantiated shape,
split-K and Swap-AB, and at the full decode shapes."""

import itertools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from oracle import mx
from tests.gpu_util import (dev_bf16, fp4_bytes, host_bf16_bits, MIN_FRAC_WITHIN_ULP, pack_fp4_ref,
                            pack_mx_scales_ref, pack_ref, requires_gpu)
from tests.instantiations import cases
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]

# swap x (waves_n, waves_k) x rows per wave x batch x activation mode (2 packed from L2, 3 staged in LDS)
MXV = list(itertools.product([0, 1], [(4, 1), (2, 2), (1, 4), (8, 1), (1, 8), (2, 4), (16, 1), (1, 16), (4, 4)],
                             [16, 32, 64], [1, 2], [2, 3]))
SPLITS = [1, 2, 4, 8]
MS = [1, 5, 13, 20, 29, 32, 40, 64]


def _quant(xb, packed=False):
    x = dev_bf16(xb)
    q, s = (ql.quantize_act_packed if packed else ql.quantize_act)(ql.MXFP8, x)
    torch.cuda.synchronize()
    return q.view(torch.uint8).cpu().numpy(), s.cpu().numpy()


def _weights(r):
    K = r["w_q"].shape[1]
    w_q = torch.from_numpy(np.ascontiguousarray(r["w_q"], dtype=np.uint8)).cuda().view(torch.float8_e4m3fn)
    return ql.pack_weight(w_q), torch.from_numpy(pack_mx_scales_ref(r["s_w"], K)).cuda()


def _acts(r):
    K = r["a_q"].shape[1]
    a_p = torch.from_numpy(pack_ref(r["a_q"])).cuda().view(torch.float8_e4m3fn)
    return a_p, torch.from_numpy(pack_mx_scales_ref(r["s_a"], K)).cuda()


def _mx_check(r, y_bits, split, waves_k):
    K = r["a_q"].shape[1]
    d = oracle.summation_depth(K, split=split, waves_k=waves_k)
    B = mx.MxBound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], d)
    return oracle.check_fp8_parity(y_bits, r["y_ref"], r["y_true"], B)


def _run(plan, a_p, a_s, w_p, w_s):
    y = torch.full((plan.M, plan.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = plan.new_workspace()
    ql.qlinear_run(plan, a_p, a_s, w_p, w_s, y, ws)
    torch.cuda.synchronize()
    return host_bf16_bits(y), ws


@pytest.mark.parametrize("M,K", [(1, 4096), (5, 128), (32, 12288), (17, 1024), (3, 25600), (64, 4096)])
def test_mx_act_quantizer_bit_exact(M, K):
    x, _ = make_inputs(K, 8, M, 0.02, seed=M + K)
    xb = bf16_bits(x)
    cq, cs = mx.mx_quantize(xb)
    q, s = _quant(xb)
    assert np.array_equal(q.reshape(M, K), cq) and np.array_equal(s, cs)
    qp, sp = _quant(xb, packed=True)
    n = ql.qlinear_packed_act_bytes(M, K)
    ns = ql.qlinear_packed_mx_scale_bytes(M, K)
    assert np.array_equal(qp[:n], pack_ref(cq)) and np.array_equal(sp[:ns], pack_mx_scales_ref(cs, K))


def test_mx_quantizer_special_blocks():
    """All-zero and negative-zero blocks, bf16 subnormals, tiny normals (the
    -127 clamp), amax on and just below a power of two, values that clamp to
    448, a huge outlier beside small values, and random signs."""
    K = 256
    rows = np.zeros((8, K), np.float64)
    rows[1, :] = -0.0
    rows[2, :32] = np.linspace(1, 127, 32) * 2.0 ** -133          # bf16 subnormals
    rows[2, 32:64] = -(2.0 ** -126) * np.linspace(1, 1.9, 32)     # tiny normals
    rows[3, :32] = np.linspace(-1.0, 1.0, 32)                     # amax exactly 2^0
    rows[3, 32:64] = np.linspace(-0.99609375, 0.5, 32)            # amax just below
    rows[3, 64:96] = np.linspace(-1.9, 1.75, 32)                  # 1.9 * 256 clamps to 448
    rows[4, :] = np.sin(np.arange(K)) * 1e-3
    rows[4, 5] = 1e30
    rows[5, :] = np.random.default_rng(1).standard_normal(K) * 3e4
    rows[6, ::3] = 448.0
    rows[6, 1::3] = -2.0 ** -20
    rows[7, :] = np.random.default_rng(2).standard_normal(K)
    xb = torch.from_numpy(rows.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xb[1, :] = 0x8000
    cq, cs = mx.mx_quantize(xb)
    for packed in (False, True):
        q, s = _quant(xb, packed)
        if packed:
            assert np.array_equal(s[:ql.qlinear_packed_mx_scale_bytes(8, K)], pack_mx_scales_ref(cs, K))
        else:
            assert np.array_equal(s, cs)
        got = q[:ql.qlinear_packed_act_bytes(8, K)] if packed else q.reshape(8, K)
        assert np.array_equal(got, pack_ref(cq) if packed else cq), packed
    assert cs[0, 0] == 0 and np.all(cq[1] == 0x80)


@pytest.mark.parametrize("N,K", [(300, 512), (4096, 4096), (1000, 12288)])
def test_mx_weight_quantizer_bit_exact(N, K):
    _, w = make_inputs(K, N, 1, 0.02, seed=N)
    wb = bf16_bits(w)
    w_q, w_s = ql.quantize_weight(ql.MXFP8, w.cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(N).integers(0, N, 64))
    cq, cs = mx.mx_quantize(wb[rows])
    assert np.array_equal(w_q.view(torch.uint8).cpu().numpy()[rows], cq)
    assert np.array_equal(w_s.cpu().numpy()[rows], cs)


@pytest.mark.parametrize("R,K", [(37, 384), (16, 128), (1, 4096), (300, 1024)])
def test_mx_scale_packing_matches_the_layout_definition(R, K):
    s = np.random.default_rng(R).integers(0, 255, (R, K // 32), dtype=np.uint8)
    out = ql.pack_mx_scales(torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    n = ql.qlinear_packed_mx_scale_bytes(R, K)
    assert n == -(-R // 16) * (K // 128) * 64
    assert np.array_equal(out.cpu().numpy()[:n], pack_mx_scales_ref(s, K))


def _mx_args(vi):
    swap, (wn, wk), rows, pf, amode = MXV[vi]
    M = MS[vi % len(MS)]
    K = [1024, 1152, 2048][vi % 3]
    N = 300 + 16 * (vi % 7)                      # several tiles + a ragged tail
    split = SPLITS[(vi // 2) % len(SPLITS)]
    cfg = dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=amode, w_layout=1)
    return ql.MXFP8, M, N, K, cfg


MX_CASES = cases("mxfp8", [(vi,) for vi in range(len(MXV))], _mx_args)


@pytest.mark.parametrize("vi", [c[0] for c in MX_CASES])
def test_every_mx_instantiation_matches_oracle(vi):
    _, M, N, K, cfg = _mx_args(vi)
    wk = cfg["waves_k"]
    plan = ql.qlinear_plan_with_config(ql.MXFP8, M, N, K, cfg)
    x, w = make_inputs(K, N, M, 0.02, seed=7000 + vi)
    r = mx.mx_reference(bf16_bits(x), bf16_bits(w))
    w_p, w_s = _weights(r)
    a_p, a_s = _acts(r)
    y, ws = _run(plan, a_p, a_s, w_p, w_s)
    st = _mx_check(r, y, plan.facts["chunks"], wk)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("lab,N,K", [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096),
                                     ("down", 4096, 12288)])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_mx_planner_plans_at_full_size(lab, N, K, M):
    """The planner's forward at the 8B decode shapes, weights quantized on the
    GPU; codes and scales checked whole, outputs on 64 sampled columns."""
    ql.load_default_table()
    x, w = make_inputs(K, N, M, 0.02, seed=17 + M)
    xb, wb = bf16_bits(x), bf16_bits(w)
    plan = ql.qlinear_plan_layouts(ql.MXFP8, M, N, K, 1, 1)
    w_q, w_s = ql.quantize_weight(ql.MXFP8, w.cuda())
    a_p = ql.act_buffer(plan)
    a_s = ql.act_scale_buffer(plan)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_p, a_s, ql.pack_weight(w_q), ql.pack_mx_scales(w_s), y,
                       plan.new_workspace())
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(M + N).choice(N, 64, replace=False))
    r = mx.mx_reference(xb, wb[cols])
    n = ql.qlinear_packed_act_bytes(M, K)
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(r["a_q"]))
    ns = ql.qlinear_packed_mx_scale_bytes(M, K)
    assert np.array_equal(a_s.cpu().numpy()[:ns], pack_mx_scales_ref(r["s_a"], K))
    st = _mx_check(r, host_bf16_bits(y)[:, cols], plan.facts["chunks"], plan.config["waves_k"])
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


def test_mx_forward_equals_quantize_then_run_and_graph_replays():
    M, N, K = 12, 2048, 4096
    x, w = make_inputs(K, N, M, 0.02, seed=99)
    r = mx.mx_reference(bf16_bits(x), bf16_bits(w))
    w_p, w_s = _weights(r)
    plan = ql.qlinear_plan_with_config(ql.MXFP8, M, N, K, dict(swap_ab=1, split_k=1, waves_n=2, waves_k=2,
                                                               rows_per_wave=16, prefetch=2, a_mode=3, w_layout=1))
    a_p, a_s = _acts(r)
    y_run, _ = _run(plan, a_p, a_s, w_p, w_s)
    xd = x.cuda()
    a_q = ql.act_buffer(plan)
    s_q = ql.act_scale_buffer(plan)
    y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, xd, a_q, s_q, w_p, w_s, y)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y), y_run)              # same codes, same kernel, split 1
    st = _mx_check(r, y_run, 1, 2)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, st
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ql.qlinear_graph_begin(s)
        ql.qlinear_forward(plan, xd, a_q, s_q, w_p, w_s, y, stream=s)
        g = ql.qlinear_graph_end(s)
    for i in range(3):
        y.fill_(0)
        a_q.view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        assert np.array_equal(host_bf16_bits(y), y_run), i
        _ = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays


# ---------------------------------------------------------------- MXFP4 weights

def _weights4(r):
    K = r["w_q"].shape[1]
    return (torch.from_numpy(pack_fp4_ref(r["w_q"])).cuda(),
            torch.from_numpy(pack_mx_scales_ref(r["s_w"], K)).cuda())


def _mx4_check(r, y_bits, split, waves_k):
    K = r["a_q"].shape[1]
    d = oracle.summation_depth(K, split=split, waves_k=waves_k)
    B = mx.MxBound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], d, fp4=True)
    return oracle.check_fp8_parity(y_bits, r["y_ref"], r["y_true"], B)


@pytest.mark.parametrize("N,K", [(300, 512), (4096, 4096), (1000, 12288)])
def test_mx4_weight_quantizer_bit_exact(N, K):
    _, w = make_inputs(K, N, 1, 0.02, seed=N + 1)
    w_q, w_s = ql.quantize_weight(ql.MXFP4, w.cuda())
    torch.cuda.synchronize()
    assert tuple(w_q.shape) == (N, K // 2)
    rows = np.unique(np.random.default_rng(N).integers(0, N, 64))
    cq, cs = mx.mx4_quantize(bf16_bits(w)[rows])
    assert np.array_equal(w_q.cpu().numpy()[rows], fp4_bytes(cq))
    assert np.array_equal(w_s.cpu().numpy()[rows], cs)


def test_mx4_weight_quantizer_rounding_ties_and_special_blocks():
    """Blocks whose amax is 4 (scale 2^0), so w / 2^e hits every E2M1 rounding
    tie exactly (0.25, 0.75, ..., 5) and their neighbours; an all-zero block,
    negative zeros, bf16 subnormals, a huge outlier."""
    K = 256
    rows = np.zeros((4, K), np.float64)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for t in ties:
        vals += [t, -t, t * (1 - 2 ** -7), t * (1 + 2 ** -7)]
    rows[0, :32] = ([4.0] + vals + [0.0] * 32)[:32]
    rows[0, 32:64] = ([-4.0] + vals[::-1] + [0.0] * 32)[:32]
    rows[0, 64:96] = [5.0, 5.5, 6.0, 5.9] * 8           # amax 6: scale 2^0; 5.0 is the 4 / 6 tie (-> 4)
    rows[1, 32:64] = -0.0
    rows[2, :32] = np.linspace(1, 127, 32) * 2.0 ** -133
    rows[3, :] = np.sin(np.arange(K)) * 1e-3
    rows[3, 7] = 1e30
    wb = torch.from_numpy(rows.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wb[1, 32:64] = 0x8000
    w_q, w_s = ql.quantize_weight(ql.MXFP4, dev_bf16(wb))
    torch.cuda.synchronize()
    cq, cs = mx.mx4_quantize(wb)
    assert np.array_equal(w_q.cpu().numpy(), fp4_bytes(cq))
    assert np.array_equal(w_s.cpu().numpy(), cs)


@pytest.mark.parametrize("N,K", [(37, 384), (16, 128), (300, 1024)])
def test_mx4_weight_packing_matches_the_layout_definition(N, K):
    codes = np.random.default_rng(N).integers(0, 16, (N, K), dtype=np.uint8)
    out = ql.pack_weight_fp4(torch.from_numpy(fp4_bytes(codes)).cuda())
    torch.cuda.synchronize()
    n = ql.qlinear_packed_weight_bytes_fp4(N, K)
    assert n == -(-N // 16) * (K // 128) * 1024
    assert np.array_equal(out.cpu().numpy()[:n], pack_fp4_ref(codes))


def _mx4_args(vi):
    swap, (wn, wk), rows, pf, amode = MXV[vi]
    M = MS[(vi + 3) % len(MS)]
    K = [1024, 1152, 2048][(vi + 1) % 3]
    N = 300 + 16 * (vi % 7)
    split = SPLITS[(vi // 2) % len(SPLITS)]
    cfg = dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=amode, w_layout=1)
    return ql.MXFP4, M, N, K, cfg


MX4_CASES = cases("mxfp4", [(vi,) for vi in range(len(MXV))], _mx4_args)


@pytest.mark.parametrize("vi", [c[0] for c in MX4_CASES])
def test_every_mx4_instantiation_matches_oracle(vi):
    _, M, N, K, cfg = _mx4_args(vi)
    wk = cfg["waves_k"]
    plan = ql.qlinear_plan_with_config(ql.MXFP4, M, N, K, cfg)
    x, w = make_inputs(K, N, M, 0.02, seed=9000 + vi)
    r = mx.mx4_reference(bf16_bits(x), bf16_bits(w))
    w_p, w_s = _weights4(r)
    a_p, a_s = _acts(r)
    y, ws = _run(plan, a_p, a_s, w_p, w_s)
    st = _mx4_check(r, y, plan.facts["chunks"], wk)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("lab,N,K", [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096),
                                     ("down", 4096, 12288)])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_mx4_planner_plans_at_full_size(lab, N, K, M):
    ql.load_default_table()
    x, w = make_inputs(K, N, M, 0.02, seed=23 + M)
    xb, wb = bf16_bits(x), bf16_bits(w)
    plan = ql.qlinear_plan_layouts(ql.MXFP4, M, N, K, 1, 1)
    w_q, w_s = ql.quantize_weight(ql.MXFP4, w.cuda())
    a_p = ql.act_buffer(plan)
    a_s = ql.act_scale_buffer(plan)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_p, a_s, ql.pack_weight_fp4(w_q), ql.pack_mx_scales(w_s), y,
                       plan.new_workspace())
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(M + N + 1).choice(N, 64, replace=False))
    r = mx.mx4_reference(xb, wb[cols])
    st = _mx4_check(r, host_bf16_bits(y)[:, cols], plan.facts["chunks"], plan.config["waves_k"])
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


# ---------------------------------------------------------------- MXFP8 beyond the decode range

TILED_MX = list(itertools.product([0, 1], [(64, 128), (64, 256), (128, 128), (128, 256), (256, 128)], [1, 2, 4],
                                  [1, 2]))


def _mx_tiled_args(vi):
    swap, (bm, bn), pf, split = TILED_MX[vi]
    M = [40, 100, 200, 257][vi % 4]
    K = [1024, 1152][vi % 2]
    N = 300 + 16 * (vi % 5)
    cfg = dict(algo=ql.ALGO_TILED, swap_ab=swap, split_k=split, tile_m=bm, tile_n=bn, prefetch=pf, w_lds=0,
               a_mode=2, w_layout=1)
    return ql.MXFP8, M, N, K, cfg


MX_TILED_CASES = cases("mxfp8_tiled", [(vi,) for vi in range(len(TILED_MX))], _mx_tiled_args)


@pytest.mark.parametrize("vi", [c[0] for c in MX_TILED_CASES])
def test_every_mx_tiled_instantiation_matches_oracle(vi):
    _, M, N, K, cfg = _mx_tiled_args(vi)
    plan = ql.qlinear_plan_with_config(ql.MXFP8, M, N, K, cfg)
    x, w = make_inputs(K, N, M, 0.02, seed=11000 + vi)
    r = mx.mx_reference(bf16_bits(x), bf16_bits(w))
    w_p, w_s = _weights(r)
    a_p, a_s = _acts(r)
    y, ws = _run(plan, a_p, a_s, w_p, w_s)
    st = _mx_check(r, y, plan.facts["chunks"], 1)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("M", [128, 1024])
def test_mx_planner_large_m_plans(M):
    """Beyond 64 tokens the planner sends MXFP8 to the tiled kernel; the 14B
    QKV shape, 64 sampled columns (and 128 sampled rows at M = 1024)."""
    N, K = 7168, 5120
    x, w = make_inputs(K, N, M, 0.02, seed=M)
    plan = ql.qlinear_plan_layouts(ql.MXFP8, M, N, K, 1, 1)
    assert plan.config["algo"] == ql.ALGO_TILED
    w_q, w_s = ql.quantize_weight(ql.MXFP8, w.cuda())
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), ql.act_buffer(plan), ql.act_scale_buffer(plan), ql.pack_weight(w_q),
                       ql.pack_mx_scales(w_s), y, plan.new_workspace())
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    cols = np.sort(rng.choice(N, 64, replace=False))
    rows = np.sort(rng.choice(M, min(M, 128), replace=False))
    r = mx.mx_reference(bf16_bits(x[torch.from_numpy(rows)]), bf16_bits(w[torch.from_numpy(cols)]))
    st = _mx_check(r, host_bf16_bits(y)[np.ix_(rows, cols)], plan.facts["chunks"], 1)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


# ---------------------------------------------------------------- MXFP4 beyond the decode range

def _mx4_tiled_args(vi):
    swap, (bm, bn), pf, split = TILED_MX[vi]
    M = [40, 100, 200, 257][(vi + 1) % 4]
    K = [1024, 1152][(vi + 1) % 2]
    N = 300 + 16 * (vi % 5)                        # several tiles + a ragged tail
    cfg = dict(algo=ql.ALGO_TILED, swap_ab=swap, split_k=split, tile_m=bm, tile_n=bn, prefetch=pf, w_lds=0,
               a_mode=2, w_layout=1)
    return ql.MXFP4, M, N, K, cfg


MX4_TILED_CASES = cases("mxfp4_tiled", [(vi,) for vi in range(len(TILED_MX))], _mx4_tiled_args)


@pytest.mark.parametrize("vi", [c[0] for c in MX4_TILED_CASES])
def test_every_mx4_tiled_instantiation_matches_oracle(vi):
    """E2M1 weights through the tiled kernel (1 KB weight tiles in the LDS
    stage), every instantiated tile, ring depth, Swap-AB and split-K."""
    _, M, N, K, cfg = _mx4_tiled_args(vi)
    plan = ql.qlinear_plan_with_config(ql.MXFP4, M, N, K, cfg)
    x, w = make_inputs(K, N, M, 0.02, seed=12000 + vi)
    r = mx.mx4_reference(bf16_bits(x), bf16_bits(w))
    w_p, w_s = _weights4(r)
    a_p, a_s = _acts(r)
    y, ws = _run(plan, a_p, a_s, w_p, w_s)
    st = _mx4_check(r, y, plan.facts["chunks"], 1)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("M", [65, 256, 1024])
def test_mx4_planner_large_m_plans(M):
    """Beyond 64 tokens the planner sends MXFP4 to the tiled kernel; the 14B
    QKV shape through the forward (MXFP8 quantizer + GEMM), 64 sampled
    columns and up to 128 sampled rows."""
    N, K = 7168, 5120
    x, w = make_inputs(K, N, M, 0.02, seed=M + 5)
    plan = ql.qlinear_plan_layouts(ql.MXFP4, M, N, K, 1, 1)
    assert plan.config["algo"] == ql.ALGO_TILED
    w_q, w_s = ql.quantize_weight(ql.MXFP4, w.cuda())
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), ql.act_buffer(plan), ql.act_scale_buffer(plan), ql.pack_weight_fp4(w_q),
                       ql.pack_mx_scales(w_s), y, plan.new_workspace())
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    cols = np.sort(rng.choice(N, 64, replace=False))
    rows = np.sort(rng.choice(M, min(M, 128), replace=False))
    r = mx.mx4_reference(bf16_bits(x[torch.from_numpy(rows)]), bf16_bits(w[torch.from_numpy(cols)]))
    st = _mx4_check(r, host_bf16_bits(y)[np.ix_(rows, cols)], plan.facts["chunks"], 1)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)
