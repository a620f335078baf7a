"""The gated MLP as a chain: gate_up (SiLU-and-mul epilogue folding the
per-token amax of H) -> down (a_mode 5: each workgroup quantizes its own K
chunk of H with the given amax, in the GEMM launch).

Checked against the oracle: H within the SiLU-and-mul rule; the amax words
equal max |H| per token of the GPU's own H, bit for bit; down's codes and
scales equal ``oracle.quantize_act`` of that H bit for bit; down's Y is
bit-exact (INT8) or within the FP8 rule against the oracle linear on that H;
the amax words are all zero after the consumer.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import amax_words, filled_amax_buffer, fp8_check, fp8_ok, host_bf16_bits, pack_ref, requires_gpu
from workloads import bf16_bits, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8]


def _weights(fmt, N, K, seed, sigma=0.02):
    _, w = make_inputs(K, N, 1, sigma, seed=seed)
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    return w, ql.pack_weight(w_q), w_s


def _consume(fmt, plan, hd, amax, w_p, w_s):
    a_q = ql.act_buffer(plan)
    a_s = torch.empty(plan.M, dtype=torch.float32, device="cuda")
    y = torch.full((plan.M, plan.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward_amax(plan, hd, amax, a_q, a_s, w_p, w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    return a_q, a_s, y


def _check_consumer(fmt, plan, h_bits, w_down, a_q, a_s, y, label):
    M, K = h_bits.shape
    r = oracle.reference(fmt, h_bits, bf16_bits(w_down))
    codes = np.asarray(r["a_q"]).view(np.uint8) if fmt != ql.W8A8_INT8 else np.asarray(r["a_q"]).astype(np.int8).view(np.uint8)
    n = ql.qlinear_packed_act_bytes(M, K)
    assert np.array_equal(a_q.view(torch.uint8)[:n].cpu().numpy(), pack_ref(codes)), label
    assert np.array_equal(a_s.cpu().numpy(), np.asarray(r["s_a"], np.float32)), label
    yb = host_bf16_bits(y)
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(yb, r["y_ref"]), label
    else:
        st = fp8_check(fmt, r, yb, plan.facts["chunks"])
        assert fp8_ok(st), (label, st)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 3, 8, 16, 24])
def test_chain_matches_oracle(fmt, M):
    I, K, N2 = 640, 1024, 384                      # gate_up [2I, K], down [N2, I]
    x, w_gu = make_inputs(K, 2 * I, M, 0.02, seed=M + 10 * fmt)
    w_down, wd_p, wd_s = _weights(fmt, N2, I, seed=M + 7)
    wg_q, wg_s = ql.quantize_weight(fmt, w_gu.cuda())
    glu = ql.qlinear_plan_glu(fmt, M, 2 * I, K, 2)
    h = torch.full((M, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    amax = ql.amax_buffer(M)
    ql.qlinear_forward_glu_amax(glu, x.cuda(), ql.act_buffer(glu),
                                torch.empty(M, dtype=torch.float32, device="cuda"), ql.pack_weight(wg_q), wg_s, h,
                                amax, glu.new_workspace())
    torch.cuda.synchronize()
    h_bits = host_bf16_bits(h)
    # H itself against the oracle's SiLU-and-mul rule
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w_gu))
    h_ref, h_true, bound = oracle.glu_reference(fmt, r, split=glu.facts["chunks"])
    st = oracle.check_fp8_parity(h_bits, h_ref, h_true, bound)
    assert fp8_ok(st), st
    # the maxima over the replicas: max |H| per token of this H, exactly; the
    # counters zero; nothing written past the M tokens of any replica
    words = amax.cpu().numpy().view(np.uint32)
    assert np.array_equal(ql.amax_of_buffer(amax, M), amax_words(h_bits))
    reps = words[:ql.AMAX_REPLICAS * ql.AMAX_LINE].reshape(ql.AMAX_REPLICAS, ql.AMAX_LINE)
    assert not reps[:, M:].any() and not words[ql.AMAX_REPLICAS * ql.AMAX_LINE:].any()
    assert np.count_nonzero(reps[:, :M].any(axis=1)) > 1, "the producer waves spread over replicas"
    down = ql.qlinear_plan_layouts(fmt, M, N2, I, 1, 3)
    assert (down.config["a_mode"] == 5) == (M <= 16)
    a_q, a_s, y = _consume(fmt, down, h, amax, wd_p, wd_s)
    _check_consumer(fmt, down, h_bits, w_down, a_q, a_s, y, (fmt, M, down.config))
    assert int(torch.count_nonzero(amax)) == 0, "the consumer leaves the amax words zero"


def _given_amax(x_bits, M, seed=0):
    return filled_amax_buffer(amax_words(x_bits), seed=seed)


# a_mode 5 instantiations: waves (n x k), rows per wave, batch, swap
MODE5 = list(itertools.product([(1, 4), (2, 2), (4, 1), (1, 8), (2, 4), (1, 16), (4, 4)], [16, 32, 64], [1, 2],
                               [0, 1]))


def _mode5_available(fmt, M, N, K, cfg):
    try:
        return ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    except ql.QLinearError as e:
        assert e.status == 2, e
        return None


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [2, 13])
@pytest.mark.parametrize("split", [1, 4])
def test_every_mode5_instantiation(fmt, M, split):
    """Every instantiated a_mode 5 shape, on a ragged N with several tiles,
    against the oracle, twice in a row (the second run must find the words
    the first one cleared, refilled)."""
    N, K = 600, 1152                      # 13 x 1152 values fit one workgroup at split 1
    x, _ = make_inputs(K, N, M, 0.02, seed=M * 31 + split, with_weight=False)
    xb = bf16_bits(x)
    w_full, w_p, w_s = _weights(fmt, N, K, seed=M + split)
    ran = 0
    for (wn, wk), rows, pf, swap in MODE5:
        cfg = dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=pf, a_mode=5,
                   w_lds=0, w_layout=1)
        plan = _mode5_available(fmt, M, N, K, cfg)
        if plan is None:
            continue
        for rep in range(2):
            amax = _given_amax(xb, M, seed=rep)
            a_q, a_s, y = _consume(fmt, plan, x.cuda(), amax, w_p, w_s)
            _check_consumer(fmt, plan, xb, w_full, a_q, a_s, y, cfg)
            assert int(torch.count_nonzero(amax)) == 0
        ran += 1
    assert ran >= 20, ran


@pytest.mark.parametrize("fmt", FMTS)
def test_consumer_without_mode5_clears_the_words(fmt):
    """A plan that quantizes separately (M > 16) still leaves the words zero."""
    M, N, K = 24, 256, 512
    x, _ = make_inputs(K, N, M, 0.02, seed=5, with_weight=False)
    w_full, w_p, w_s = _weights(fmt, N, K, seed=6)
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, 1, 3)
    assert plan.config["a_mode"] != 5
    amax = _given_amax(bf16_bits(x), M)
    a_q, a_s, y = _consume(fmt, plan, x.cuda(), amax, w_p, w_s)
    _check_consumer(fmt, plan, bf16_bits(x), w_full, a_q, a_s, y, plan.config)
    assert int(torch.count_nonzero(amax)) == 0


def test_mode5_plan_refuses_plain_forward():
    plan = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 4, 256, 512, 1, 3)
    assert plan.config["a_mode"] == 5
    x = torch.zeros(4, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_forward(plan, x, ql.act_buffer(plan), torch.empty(4, device="cuda"),
                           torch.zeros(ql.qlinear_packed_weight_bytes(256, 512), dtype=torch.uint8,
                                       device="cuda").view(torch.float8_e4m3fn),
                           torch.ones(256, device="cuda"), torch.empty(4, 256, dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 1


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [2, 24])
def test_chain_graph_replays(fmt, M):
    """gate_up (amax fold) -> down (mode 5 at M <= 16, else the quantizer and
    a GEMM that clears the buffer) captured once and replayed four times with
    unrelated eager work between: every replay gives the eager outputs, and
    leaves the amax buffer zero for the next."""
    I, K, N2 = 640, 1024, 384
    x, w_gu = make_inputs(K, 2 * I, M, 0.02, seed=M + 100 * fmt)
    _, wd_p, wd_s = _weights(fmt, N2, I, seed=M + 9)
    wg_q, wg_s = ql.quantize_weight(fmt, w_gu.cuda())
    wg_p = ql.pack_weight(wg_q)
    glu = ql.qlinear_plan_glu(fmt, M, 2 * I, K, 2)
    down = ql.qlinear_plan_layouts(fmt, M, N2, I, 1, 3)
    xd = x.cuda()
    h = torch.empty(M, I, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(M, N2, dtype=torch.bfloat16, device="cuda")
    amax = ql.amax_buffer(M)
    bufs = dict(ga=ql.act_buffer(glu), gs=torch.empty(M, dtype=torch.float32, device="cuda"), gw=glu.new_workspace(),
                da=ql.act_buffer(down), ds=torch.empty(M, dtype=torch.float32, device="cuda"), dw=down.new_workspace())

    def chain(stream=None):
        ql.qlinear_forward_glu_amax(glu, xd, bufs["ga"], bufs["gs"], wg_p, wg_s, h, amax, bufs["gw"], stream=stream)
        ql.qlinear_forward_amax(down, h, amax, bufs["da"], bufs["ds"], wd_p, wd_s, y, bufs["dw"], stream=stream)

    chain()
    torch.cuda.synchronize()
    h_eager, y_eager = h.clone(), y.clone()
    assert int(torch.count_nonzero(amax)) == 0
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ql.qlinear_graph_begin(s)
        chain(stream=s)
        g = ql.qlinear_graph_end(s)
    for i in range(4):
        h.fill_(0)
        y.fill_(0)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        if fmt == ql.W8A8_INT8:
            assert torch.equal(h, h_eager) and torch.equal(y, y_eager), i
        else:
            # the same plans on the same inputs: only a split-K summation order can differ
            # (fp32 atomics), and with it a last bit of H, a code of down's input, a bit of Y
            if glu.facts["chunks"] == 1:
                assert torch.equal(h, h_eager), i
            ref = y_eager.float().abs().max()
            assert float((y.float() - y_eager.float()).abs().max()) <= 2 ** -6 * float(ref), i
        assert int(torch.count_nonzero(amax)) == 0, i
        _ = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays
