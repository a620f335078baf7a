"""GPU parity of decode plans with a row tile (tile_n of a decode plan): a
workgroup owns a multiple of 8 rows of N that need not fill its waves' row
groups, so its last row group is partly masked and, for a tile that is not a
multiple of 16, starts inside a packed 16-row weight tile.

Every output is written exactly once (Y starts as NaN), INT8 accumulators and
outputs are bit-exact, FP8_Dynamic and Block_FP8 outputs pass the oracle's
acceptance rule (Block_FP8: row groups that straddle a 128-row weight-scale
block); ragged N (a partial last tile), ragged K, split-K and every
activation mode are covered.
"""

import itertools

import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import requires_gpu, run_gemm
from tests.test_gpu_fused import _check as _check_fused, _forward, _weights
from tests.test_gpu_gemm import _assert_parity, _dev, _dev_packed_act
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]

# (row tile, rows per wave, waves_n, waves_k, prefetch)
TILES = [(8, 16, 1, 4, 2), (24, 32, 1, 4, 2), (40, 64, 1, 4, 1), (24, 16, 2, 2, 2), (48, 64, 1, 4, 1),
         (56, 32, 2, 4, 1)]
# (weight layout, activation mode): row-major W and A; packed W, packed A per block; packed A staged in LDS
LAYOUTS = [(0, 0), (1, 0), (1, 2), (1, 3)]
# row-major weights are instantiated for 4-wave workgroups of up to 32 rows a wave only, and
# Block_FP8 with two token tiles for up to 32 rows a wave (its per-block scales take registers)
CASES = [c for c in itertools.product([ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8], [3, 17, 32], range(len(TILES)),
                                      [0, 1], range(len(LAYOUTS)))
         if (LAYOUTS[c[4]][0] == 1 or (TILES[c[2]][1] <= 32 and TILES[c[2]][2] * TILES[c[2]][3] == 4))
         and not (c[0] == ql.BLOCK_FP8 and c[1] > 16 and TILES[c[2]][1] == 64)]


def _ref(fmt, M, N, K, seed):
    x, w = make_inputs(K, N, M, 0.02, seed=seed)
    return oracle.reference(fmt, bf16_bits(x), bf16_bits(w))


@pytest.mark.parametrize("fmt,M,ti,swap,li", CASES)
def test_row_tile_plans_match_oracle(fmt, M, ti, swap, li):
    rt, rows, wn, wk, pf = TILES[ti]
    w_layout, a_mode = LAYOUTS[li]
    split = [1, 2][(ti + li + M) % 2]
    N = 1000                                              # 1000 % rt != 0 for most tiles: a partial last tile
    K = 1040 if (ti + swap) % 2 and fmt != ql.BLOCK_FP8 else 1152   # 1040: ragged last K block
    cfg = dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=a_mode, w_lds=0, w_layout=w_layout, tile_n=rt)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    assert plan.facts["workgroups"] == -(-N // rt) * plan.facts["chunks"]
    r = _ref(fmt, M, N, K, seed=7000 + 31 * ti + 7 * li + M + swap)
    a_q, s_a, w_q, s_w = _dev(fmt, r)
    if w_layout:
        w_q = ql.pack_weight(w_q)
    if a_mode >= 2:
        a_q = _dev_packed_act(fmt, r)
    y, acc, ws = run_gemm(plan, a_q, s_a, w_q, s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg))
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("fmt", [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8])
@pytest.mark.parametrize("rt,rows,wn,wk", [(24, 32, 1, 4), (40, 64, 1, 8), (8, 16, 1, 8)])
def test_row_tile_fused_quantization_matches_oracle(fmt, rt, rows, wn, wk):
    """The quantizer fused into the GEMM launch (a_mode 4) with a row tile:
    codes and scales bit-exact, outputs as for the two-launch path."""
    M, N, K = 2, 1000, 4096
    x, w = make_inputs(K, N, M, 0.02, seed=91 + rt)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    cfg = dict(swap_ab=0, split_k=1, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=1, a_mode=4,
               w_layout=1, tile_n=rt)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    w_p, w_s = _weights(fmt, r)
    a_p, a_s, y, _ = _forward(plan, fmt, bf16_bits(x), w_p, w_s)
    _check_fused(fmt, r, plan, a_p, a_s, y, str(cfg))


@pytest.mark.parametrize("fmt", [ql.FP8_DYNAMIC, ql.W8A8_INT8])
@pytest.mark.parametrize("rt,rows,wn,wk,split", [(24, 32, 1, 4, 1), (40, 64, 1, 8, 4), (8, 16, 1, 4, 1)])
def test_row_tile_given_amax_matches_oracle(fmt, rt, rows, wn, wk, split):
    """A given-amax plan (a_mode 5: each workgroup quantizes its own K chunk
    with the per-token amax its producer folded) with a row tile: codes,
    scales and outputs as the oracle's, the amax words cleared, twice in a row."""
    from tests.test_gpu_chain import _check_consumer, _consume, _given_amax, _weights as _chain_weights
    M, N, K = 9, 1000, 1152
    x, _ = make_inputs(K, N, M, 0.02, seed=400 + rt + split, with_weight=False)
    xb = bf16_bits(x)
    w_full, w_p, w_s = _chain_weights(fmt, N, K, seed=rt + split)
    cfg = dict(swap_ab=0, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=1, a_mode=5,
               w_lds=0, w_layout=1, tile_n=rt)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    for rep in range(2):
        amax = _given_amax(xb, M, seed=rep)
        a_q, a_s, y = _consume(fmt, plan, x.cuda(), amax, w_p, w_s)
        _check_consumer(fmt, plan, xb, w_full, a_q, a_s, y, str(cfg))
        assert int(torch.count_nonzero(amax)) == 0
