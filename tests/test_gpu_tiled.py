"""GPU parity of the tiled (M > 32) GEMM against the oracle.

Every instantiation (format x orientation x tile x weight layout) runs on
ragged shapes that span several tiles, with and without split-K; INT8 must be
bit-exact on the raw int32 accumulators and on Y, FP8 / Block_FP8 inside the
oracle's bound.  The large-M workloads (14B-class shapes at M = 64..4096) run
at full size with the planner's configuration, checked on sampled columns.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import (dev_codes, dev_f32, fp8_check, fp8_ok, host_bf16_bits, host_codes,
                            MIN_FRAC_WITHIN_ULP, requires_gpu, run_gemm)
from tests.test_gpu_gemm import _assert_parity, _dev_packed_act
from tests.instantiations import cases
from workloads import bf16_bits, config_by_name, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]
TILES = [(64, 128), (64, 256), (128, 128), (128, 256), (256, 128)]
# swap x tile x (packed weights, packed activations) x ring depth
TVARIANTS = list(itertools.product([0, 1], TILES, [(0, 0), (1, 0), (1, 1)], [1, 2, 4]))


def _ref(fmt, M, N, K, seed):
    x, w = make_inputs(K, N, M, 0.02, seed=seed)
    return oracle.reference(fmt, bf16_bits(x), bf16_bits(w))


def _tiled_args(fmt, M, vi):
    swap, (bm, bn), (packed, apacked), pf = TVARIANTS[vi]
    split = [1, 2, 4][(vi + M) % 3]
    N = 300 if bn == 128 else 520                         # several tiles + a ragged tail
    K = 1152 if fmt == ql.BLOCK_FP8 or vi % 2 else 1040   # 1040: ragged last K block (9 blocks: ring wraps)
    cfg = dict(algo=ql.ALGO_TILED, swap_ab=swap, split_k=split, tile_m=bm, tile_n=bn, w_layout=packed, prefetch=pf,
               a_mode=2 * apacked)
    return fmt, M, N, K, cfg


TILED_CASES = cases("tiled", [(f, M, vi) for f in FMTS for M in (40, 200) for vi in range(len(TVARIANTS))],
                    _tiled_args)


@pytest.mark.parametrize("fmt,M,vi", TILED_CASES)
def test_every_tiled_instantiation_matches_oracle(fmt, M, vi):
    _, _, N, K, cfg = _tiled_args(fmt, M, vi)
    packed, apacked = cfg["w_layout"], cfg["a_mode"] // 2
    r = _ref(fmt, M, N, K, seed=3000 + vi * 5 + M)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    a_q, s_a, w_q, s_w = (dev_codes(fmt, r["a_q"]), dev_f32(r["s_a"]), dev_codes(fmt, r["w_q"]), dev_f32(r["s_w"]))
    if packed:
        w_q = ql.pack_weight(w_q)
    if apacked:
        a_q = _dev_packed_act(fmt, r)
    y, acc, ws = run_gemm(plan, a_q, s_a, w_q, s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg))
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


DMA_VARIANTS = list(itertools.product([0, 1], [(128, 128), (128, 256), (256, 128)], [2, 3])) + \
    [(0, (256, 256), 2), (1, (256, 256), 2)]     # the 8-wave tile


@pytest.mark.parametrize("fmt", [ql.FP8_DYNAMIC, ql.W8A8_INT8])
@pytest.mark.parametrize("M", [40, 300])
@pytest.mark.parametrize("vi", range(len(DMA_VARIANTS)))
def test_tiled_lds_dma_ring_matches_oracle(fmt, M, vi):
    """Packed operands streamed into an LDS ring by LDS-DMA (w_lds = 1), with
    ragged M, N and K (a last K block of 16 bytes) and split-K."""
    swap, (bm, bn), ns = DMA_VARIANTS[vi]
    split = [1, 2, 4][(vi + M) % 3]
    N, K = 520 + 16 * vi, 1040 if vi % 2 else 1152
    r = _ref(fmt, M, N, K, seed=5000 + vi * 3 + M)
    cfg = dict(algo=ql.ALGO_TILED, swap_ab=swap, split_k=split, tile_m=bm, tile_n=bn, w_layout=1, a_mode=2,
               w_lds=1, prefetch=ns)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    a_q, s_a, w_q, s_w = (dev_codes(fmt, r["a_q"]), dev_f32(r["s_a"]), dev_codes(fmt, r["w_q"]), dev_f32(r["s_w"]))
    y, acc, ws = run_gemm(plan, _dev_packed_act(fmt, r), s_a, ql.pack_weight(w_q), s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg))
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("fmt", FMTS)
def test_tiled_matches_decode_bitwise_for_int8_and_closely_for_fp8(fmt):
    """The same M = 32 problem through both algorithms: INT8 identical bits,
    FP8 both inside the oracle bound (their summation orders differ)."""
    M, N, K = 32, 384, 1280
    r = _ref(fmt, M, N, K, seed=77)
    a_q, s_a, w_q, s_w = (dev_codes(fmt, r["a_q"]), dev_f32(r["s_a"]), dev_codes(fmt, r["w_q"]), dev_f32(r["s_w"]))
    pd = ql.qlinear_plan_with_config(fmt, M, N, K, dict(swap_ab=1, split_k=2, a_mode=0))
    pt = ql.qlinear_plan_with_config(fmt, M, N, K, dict(algo=ql.ALGO_TILED, swap_ab=0, split_k=1, tile_m=64,
                                                        tile_n=128, prefetch=4))
    yd, accd, _ = run_gemm(pd, a_q, s_a, w_q, s_w)
    yt, acct, _ = run_gemm(pt, a_q, s_a, w_q, s_w)
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(accd, acct) and np.array_equal(yd, yt)
    else:
        assert fp8_ok(fp8_check(fmt, r, yd, 2)) and fp8_ok(fp8_check(fmt, r, yt, 1))


def test_planner_routes_large_m_to_the_tiled_algorithm():
    p = ql.qlinear_plan(ql.FP8_DYNAMIC, 33, 4096, 4096)
    assert p.config["algo"] == ql.ALGO_TILED and p.facts["threads"] == 512   # 8-wave tiles
    p = ql.qlinear_plan(ql.FP8_DYNAMIC, 32, 4096, 4096)
    assert p.config["algo"] == ql.ALGO_DECODE


def _large_points():
    cfg = config_by_name("fp8_dynamic_14b_large_m")
    pts = []
    for (lab, N, K) in cfg.shapes:
        for M in cfg.ms:
            if M == 4096 and lab != "qkv":
                continue              # one 4096-token shape keeps the suite short
            pts.append((lab, N, K, M))
    return pts


_LARGE = {}


@pytest.mark.parametrize("lab,N,K,M", _large_points())
def test_large_m_workloads_sampled_columns(lab, N, K, M):
    """14B-class FP8 shapes at full size with the planner's configuration
    (packed weights and activations; tiled, or at M = 64 possibly the
    weight-streaming kernel); the oracle recomputes 64 sampled output columns."""
    cfg = config_by_name("fp8_dynamic_14b_large_m")
    fmt = cfg.fmt
    key = (lab, N, K)
    if key not in _LARGE:
        _LARGE.clear()
        x, w = make_inputs(K, N, max(cfg.ms), cfg.sigma_w, seed=cfg.seed)
        w_q, w_s = ql.quantize_weight(fmt, w.cuda())
        _LARGE[key] = (x, w, ql.pack_weight(w_q), w_s)
    x, w, w_p, w_s = _LARGE[key]
    xm = x[:M]
    a_q, a_s = ql.quantize_act(fmt, xm.cuda())
    a_p, _ = ql.quantize_act_packed(fmt, xm.cuda())
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, 1, 1)
    # the table may serve M = 64 with the weight-streaming kernel (four token tiles)
    assert plan.config["algo"] == ql.ALGO_TILED or M <= 64
    assert plan.config["a_mode"] == 2
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_run(plan, a_p, a_s, w_p, w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    yb = host_bf16_bits(y)
    rng = np.random.default_rng(M + N)
    cols = np.sort(rng.choice(N, 64, replace=False))
    rows = np.sort(rng.choice(M, min(M, 256), replace=False))
    r = oracle.reference(fmt, bf16_bits(xm[torch.from_numpy(rows)]), bf16_bits(w[torch.from_numpy(cols)]))
    assert np.array_equal(host_codes(fmt, a_q)[rows], r["a_q"])
    st = fp8_check(fmt, r, yb[np.ix_(rows, cols)], plan.facts["chunks"])
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)
