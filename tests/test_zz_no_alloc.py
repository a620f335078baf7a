"""qlinear_forward_noalloc against qlinear_forward (through the C ABI).

The no-allocation entry point takes a split-K plan's workspace from the
library's per-GPU scratch array instead of a caller buffer.  Its results
must be those of qlinear_forward: bit-exact codes, scales and INT8 output,
FP8 output within the oracle's bound -- on two calls in a row, the second
with a smaller input (the scratch keeps the last call's contents, so the
second call checks that the first left it clean), in eager launches and as
replays of a captured graph.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import fp8_check, host_bf16_bits, requires_gpu
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(fmt, M, N, K, cfg, seed):
    x, w = make_inputs(K, N, M, 0.02, seed=seed)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    assert plan.workspace_bytes > 0, "the case must exercise the split-K workspace"
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    if cfg.get("w_layout"):
        w_q = ql.pack_weight(w_q)
    return x.cuda(), r, plan, w_q, w_s


def _buffers(fmt, plan):
    a_q = ql.act_buffer(plan)
    a_s = torch.empty(ql.act_scale_shape(fmt, plan.M, plan.K), dtype=torch.float32, device="cuda")
    y = torch.full((plan.M, plan.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    return a_q, a_s, y


def _check_pair(fmt, r, plan, ref, got):
    (aq0, as0, y0), (aq1, as1, y1) = ref, got
    assert torch.equal(aq0.view(torch.uint8), aq1.view(torch.uint8))
    assert torch.equal(as0, as1)
    y0b, y1b = host_bf16_bits(y0), host_bf16_bits(y1)
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(y1b, y0b)
        assert np.array_equal(y1b, r["y_ref"])
    else:
        for yb in (y0b, y1b):
            st = fp8_check(fmt, r, yb, plan.facts["chunks"])
            assert st["ok"], st


def _forward_both(fmt, xd, plan, w_q, w_s):
    ref = _buffers(fmt, plan)
    ql.qlinear_forward(plan, xd, *ref[:2], w_q, w_s, ref[2], plan.new_workspace())
    got = _buffers(fmt, plan)
    ql.qlinear_forward_noalloc(plan, xd, *got[:2], w_q, w_s, got[2])
    torch.cuda.synchronize()
    return ref, got


SPLIT = dict(swap_ab=0, waves_n=4, waves_k=1, rows_per_wave=16, prefetch=2, a_mode=0, w_lds=0, w_layout=0)


@pytest.mark.parametrize("fmt", [ql.W8A8_INT8, ql.FP8_DYNAMIC, ql.BLOCK_FP8])
def test_noalloc_matches_forward_two_calls(fmt):
    big = _case(fmt, 24, 1040, 8192, dict(SPLIT, split_k=8), seed=1)
    small = _case(fmt, 3, 496, 2048, dict(SPLIT, split_k=4, swap_ab=1), seed=2)
    for xd, r, plan, w_q, w_s in (big, small):
        ref, got = _forward_both(fmt, xd, plan, w_q, w_s)
        _check_pair(fmt, r, plan, ref, got)


@pytest.mark.parametrize("fmt", [ql.W8A8_INT8, ql.FP8_DYNAMIC])
def test_noalloc_fused_quantization_split(fmt):
    """One-launch plans (the quantizer inside the GEMM) with split-K."""
    cfg = dict(swap_ab=0, split_k=4, waves_n=1, waves_k=4, rows_per_wave=16, prefetch=2, a_mode=4, w_lds=0,
               w_layout=1)
    for M, N, K, seed in ((4, 2048, 4096, 3), (2, 1024, 2048, 4)):
        xd, r, plan, w_q, w_s = _case(fmt, M, N, K, cfg, seed)
        ref, got = _forward_both(fmt, xd, plan, w_q, w_s)
        _check_pair(fmt, r, plan, ref, got)


def test_noalloc_graph_replays_match_eager():
    fmt = ql.W8A8_INT8
    xd, r, plan, w_q, w_s = _case(fmt, 16, 2048, 4096, dict(SPLIT, split_k=16), seed=5)
    a_q, a_s, y = _buffers(fmt, plan)
    ql.qlinear_forward_noalloc(plan, xd, a_q, a_s, w_q, w_s, y)   # first call on the GPU: outside capture
    torch.cuda.synchronize()
    eager = host_bf16_bits(y)
    assert np.array_equal(eager, r["y_ref"])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ql.qlinear_graph_begin(s)
        ql.qlinear_forward_noalloc(plan, xd, a_q, a_s, w_q, w_s, y, stream=s)
        g = ql.qlinear_graph_end(s)
    for i in range(4):
        with torch.cuda.stream(s):
            y.fill_(float("nan"))
            g.launch(s)
        s.synchronize()
        assert np.array_equal(host_bf16_bits(y), eager), i
        # eager work of the program between replays, on the scratch too
        small = _case(fmt, 2, 512, 1024, dict(SPLIT, split_k=8), seed=6 + i)
        ref, got = _forward_both(fmt, small[0], small[2], small[3], small[4])
        _check_pair(fmt, small[1], small[2], ref, got)
    del g


def test_noalloc_rejects_plans_beyond_the_scratch():
    fmt = ql.W8A8_INT8
    M, N, K = 64, 70016, 256
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(SPLIT, split_k=2, w_layout=1))
    assert plan.workspace_bytes > ql.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    a_q, a_s, y = _buffers(fmt, plan)
    w_q = torch.zeros(N, K, dtype=torch.int8, device="cuda")
    w_s = torch.ones(N, dtype=torch.float32, device="cuda")
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_forward_noalloc(plan, x, a_q, a_s, w_q, w_s, y)
    assert e.value.status == 2 and "scratch" in str(e.value)
