"""GPU parity of the decode GEMM against the oracle.

INT8: the int32 accumulator and the bf16 output are bit-exact.  FP8_Dynamic
and Block_FP8: the bf16 output passes the oracle's acceptance rule (within
1 bf16 ulp of the single-rounded result, or within the binary32 summation
bound of the exact result; normwise error <= 1e-2), and the fp32
accumulator lies within the summation bound of the exact sum.
"""

import itertools
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import (MIN_FRAC_WITHIN_ULP, amax_words, dev_bf16, dev_codes, dev_f32, filled_amax_buffer, fp8_check,
                            fp8_ok, host_bf16_bits, host_codes, pack_ref, requires_gpu, run_gemm)
from tests.instantiations import cases
from workloads import CONFIGS, bf16_bits, config_by_name, decode_points, decode_workloads, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]


def _ref(fmt, M, N, K, seed, sigma=0.02):
    x, w = make_inputs(K, N, M, sigma, seed=seed)
    return oracle.reference(fmt, bf16_bits(x), bf16_bits(w))


def _dev_packed_act(fmt, r):
    """Oracle activation codes in the packed layout (restated on the host, not by the GPU quantizer)."""
    codes = np.asarray(r["a_q"]).view(np.uint8) if fmt != ql.W8A8_INT8 else np.asarray(r["a_q"]).astype(np.int8).view(np.uint8)
    t = torch.from_numpy(pack_ref(codes)).cuda()
    return t.view(torch.int8) if fmt == ql.W8A8_INT8 else t.view(torch.float8_e4m3fn)


def _dev(fmt, r):
    return (dev_codes(fmt, r["a_q"]), dev_f32(r["s_a"]), dev_codes(fmt, r["w_q"]), dev_f32(r["s_w"]))


def _assert_parity(fmt, r, y, acc, split, label="", waves_k=16):
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(acc.astype(np.int64), r["S"]), label
        bad = np.argwhere(y != r["y_ref"])
        assert bad.size == 0, (label, bad[:5])
        return
    st = fp8_check(fmt, r, y, split, waves_k)
    assert fp8_ok(st), (label, st)
    K = r["a_q"].shape[1]
    d = oracle.summation_depth(K, split=split, waves_k=waves_k)
    # the raw accumulator against the exact sum: the bound is evaluated where
    # its binary32 part alone does not already cover the difference
    if fmt == ql.FP8_DYNAMIC:
        B, ref = oracle.accumulator_bound(fmt, r["a_q"], r["w_q"], d), r["S"]
    else:
        B, ref = oracle.Fp8Bound(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], d), r["y_true"]
    diff = np.abs(acc.astype(np.float64) - ref)
    open_ = np.argwhere(diff > B.base)
    assert np.all(diff[open_[:, 0], open_[:, 1]] <= B.at(open_[:, 0], open_[:, 1]) + 1e-30), label


# every kernel instantiation: swap x rows/wave x prefetch x activation LDS staging x weight mode
# (0 row-major direct, 1 row-major through the LDS transpose, 2 packed tiles), both token tiles
# (instantiations that would spill registers do not exist)
VARIANTS = [v for v in itertools.product([0, 1], [16, 32], [2, 4], [0, 1, 2, 3], [0, 1, 2])
            if v[3] < 2 or v[4] == 2]         # packed activations (a_mode 2, 3) go with packed weights
SPLITS = [1, 2, 4, 8]
WAVES_K = [1, 2, 4]


def _variant_args(fmt, M, vi):
    swap, rows, pf, alds, wmode = VARIANTS[vi]
    split = SPLITS[(vi + M) % len(SPLITS)]
    wk = WAVES_K[(vi // 2 + M) % len(WAVES_K)]
    N = 300 if rows == 16 else 520                      # several tiles + a ragged tail
    K = 1152 if fmt == ql.BLOCK_FP8 or vi % 3 else 1040  # 1040: ragged last K block
    cfg = dict(swap_ab=swap, split_k=split, waves_n=4 // wk, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=alds, w_lds=int(wmode == 1), w_layout=int(wmode == 2))
    return fmt, M, N, K, cfg


# the instantiated points of fmt x M x VARIANTS (shapes that would spill or
# exceed the LDS are not instantiated; the manifest test watches the list)
VARIANT_CASES = cases("gemm_variants", [(f, M, vi) for f in FMTS for M in (5, 29) for vi in range(len(VARIANTS))],
                      _variant_args)


@pytest.mark.parametrize("fmt,M,vi", VARIANT_CASES)
def test_every_instantiation_matches_oracle(fmt, M, vi):
    _, _, N, K, cfg = _variant_args(fmt, M, vi)
    wmode = VARIANTS[vi][4]
    alds = cfg["a_mode"]
    r = _ref(fmt, M, N, K, seed=vi * 7 + M)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    a_q, s_a, w_q, s_w = _dev(fmt, r)
    if wmode == 2:
        w_q = ql.pack_weight(w_q)
    if alds >= 2:
        a_q = _dev_packed_act(fmt, r)
    y, acc, ws = run_gemm(plan, a_q, s_a, w_q, s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg))
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


# packed-weight shapes with wider workgroups: waves per workgroup x rows per wave x batch size
WIDE = list(itertools.product([4, 8, 16], [16, 32, 64], [1, 2], [0, 1], [0, 2, 3]))   # ... x activation mode


def _wide_args(fmt, M, wi):
    nw, rows, pf, swap, amode = WIDE[wi]
    wks = [k for k in (1, 2, 4, 8, 16) if k <= nw]
    wk = wks[(wi + M) % len(wks)]
    split = SPLITS[(wi + 2 * M) % len(SPLITS)]
    N = 300 + 16 * wi                                    # several tiles + a ragged tail
    K = 1152 if fmt == ql.BLOCK_FP8 or wi % 3 else 1040  # 1040: ragged last K block
    cfg = dict(swap_ab=swap, split_k=split, waves_n=nw // wk, waves_k=wk, rows_per_wave=rows, prefetch=pf,
               a_mode=amode, w_lds=0, w_layout=1)
    return fmt, M, N, K, cfg


WIDE_CASES = cases("gemm_wide", [(f, M, wi) for f in FMTS for M in (5, 29, 61) for wi in range(len(WIDE))],
                   _wide_args)


@pytest.mark.parametrize("fmt,M,wi", WIDE_CASES)
def test_wide_workgroup_instantiations_match_oracle(fmt, M, wi):
    _, _, N, K, cfg = _wide_args(fmt, M, wi)
    wk, amode = cfg["waves_k"], cfg["a_mode"]
    r = _ref(fmt, M, N, K, seed=1000 + wi * 7 + M)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    a_q, s_a, w_q, s_w = _dev(fmt, r)
    if amode >= 2:
        a_q = _dev_packed_act(fmt, r)
    y, acc, ws = run_gemm(plan, a_q, s_a, ql.pack_weight(w_q), s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg), waves_k=wk)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 16, 17, 24, 32])
def test_token_counts_and_tiles(fmt, M):
    N, K = 1024, 2048
    r = _ref(fmt, M, N, K, seed=M)
    for cfg in (dict(swap_ab=0, split_k=1, waves_n=1, waves_k=4, a_mode=0),
                dict(swap_ab=1, split_k=4, waves_n=2, waves_k=2, rows_per_wave=32, a_mode=1),
                dict(swap_ab=1, split_k=16, waves_n=4, waves_k=1, prefetch=4, a_mode=1, w_lds=1),
                dict(swap_ab=0, split_k=1, waves_n=1, waves_k=4, rows_per_wave=32, a_mode=0, w_lds=1)):
        plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
        y, acc, _ = run_gemm(plan, *_dev(fmt, r))
        _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(cfg))




@pytest.mark.parametrize("N,K", [(300, 1040), (16, 128), (4096, 4096), (33, 16), (1, 2064)])
def test_pack_weight_matches_layout_definition(N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    packed = ql.pack_weight(torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    assert packed.numel() == ql.qlinear_packed_weight_bytes(N, K)
    assert np.array_equal(packed.cpu().numpy().view(np.uint8), pack_ref(q))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 8, 32])
def test_packed_plans_match_row_major(fmt, M):
    """Heuristic / table plans for packed weights agree with the oracle on a multi-tile ragged shape."""
    N, K = 1000, 3072 if fmt == ql.BLOCK_FP8 else 3088
    r = _ref(fmt, M, N, K, seed=M + 40)
    a_q, s_a, w_q, s_w = _dev(fmt, r)
    plan = ql.qlinear_plan_packed(fmt, M, N, K)
    assert plan.config["w_layout"] == 1
    y, acc, ws = run_gemm(plan, a_q, s_a, ql.pack_weight(w_q), s_w)
    _assert_parity(fmt, r, y, acc, plan.facts["chunks"], label=str(plan.config))


def test_int8_all_variants_bitwise_identical_and_deterministic():
    M, N, K = 12, 700, 3072
    r = _ref(ql.W8A8_INT8, M, N, K, seed=99)
    d = _dev(ql.W8A8_INT8, r)
    outs = []
    packed = ql.pack_weight(d[2])
    for swap, split, wk, rows, alds, wmode in itertools.product([0, 1], [1, 8, 32], [1, 4], [16, 32], [0, 1],
                                                                [0, 1, 2]):
        cfg = dict(swap_ab=swap, split_k=split, waves_n=4 // wk, waves_k=wk, rows_per_wave=rows, a_mode=alds,
                   w_lds=int(wmode == 1), w_layout=int(wmode == 2))
        try:
            plan = ql.qlinear_plan_with_config(ql.W8A8_INT8, M, N, K, cfg)
        except ql.QLinearError:
            continue
        args = (d[0], d[1], packed if wmode == 2 else d[2], d[3])
        for _ in range(2):
            y, _, _ = run_gemm(plan, *args, acc=False)
            outs.append(y)
    assert len(outs) >= 100
    for y in outs[1:]:
        assert np.array_equal(y, outs[0])
    assert np.array_equal(outs[0], r["y_ref"])


@pytest.mark.parametrize("fmt", FMTS)
def test_split_k_workspace_reuse_across_runs(fmt):
    M, N, K = 8, 512, 4096
    r = _ref(fmt, M, N, K, seed=5)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(split_k=8, swap_ab=1))
    d = _dev(fmt, r)
    ws = plan.new_workspace()
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        y.fill_(0)
        ql.qlinear_run(plan, *d, y, ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0
        st = fp8_check(fmt, r, host_bf16_bits(y), 8) if fmt != ql.W8A8_INT8 else None
        if st is None:
            assert np.array_equal(host_bf16_bits(y), r["y_ref"])
        else:
            assert fp8_ok(st), st


@pytest.mark.parametrize("fmt", FMTS)
def test_forward_quantizes_and_runs(fmt):
    M, N, K = 9, 640, 2048
    x, w = make_inputs(K, N, M, 0.02, seed=21)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    plan = ql.qlinear_plan(fmt, M, N, K)
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    a_q = torch.empty(M, K, dtype=ql.code_dtype(fmt), device="cuda")
    a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_q, a_s, w_q, w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(fmt, a_q), r["a_q"])
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(host_bf16_bits(y), r["y_ref"])
    else:
        assert fp8_ok(fp8_check(fmt, r, host_bf16_bits(y), plan.facts["chunks"]))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [3, 24, 40])
def test_forward_with_packed_operands(fmt, M):
    """qlinear_forward on a packed-weight, packed-activation plan quantizes into
    the packed layout itself (decode and tiled algorithms)."""
    N, K = 520, 2048
    x, w = make_inputs(K, N, M, 0.02, seed=22 + M)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, 1, 1)
    assert plan.config["a_mode"] >= 2
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    a_p = ql.act_buffer(plan)
    a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ql.qlinear_forward(plan, x.cuda(), a_p, a_s, ql.pack_weight(w_q), w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    n = ql.qlinear_packed_act_bytes(M, K)
    codes = np.asarray(r["a_q"]).astype(np.int8).view(np.uint8) if fmt == ql.W8A8_INT8 else np.asarray(r["a_q"])
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(codes))
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(host_bf16_bits(y), r["y_ref"])
    else:
        assert fp8_ok(fp8_check(fmt, r, host_bf16_bits(y), plan.facts["chunks"]))


def test_k_zero_gives_zeros_and_empty_shapes_are_no_ops():
    plan = ql.qlinear_plan(ql.FP8_DYNAMIC, 4, 100, 0)
    y = torch.full((4, 100), 3.0, dtype=torch.bfloat16, device="cuda")
    e = torch.empty(16, dtype=torch.uint8, device="cuda")
    f = torch.empty(16, dtype=torch.float32, device="cuda")
    ql.qlinear_run(plan, e, f, e, f, y)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0
    for M, N in ((0, 64), (4, 0)):
        p = ql.qlinear_plan(ql.W8A8_INT8, M, N, 256)
        yy = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ql.qlinear_run(p, e, f, e, f, yy)


@pytest.mark.parametrize("fmt", FMTS)
def test_graph_capture_replays_match_eager(fmt):
    M, N, K = 16, 1536, 4096
    x, w = make_inputs(K, N, M, 0.02, seed=31)
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(split_k=4, swap_ab=1))
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    xd = x.cuda()
    a_q = torch.empty(M, K, dtype=ql.code_dtype(fmt), device="cuda")
    a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
    y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    ws = plan.new_workspace()
    ql.qlinear_forward(plan, xd, a_q, a_s, w_q, w_s, y, ws)
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ql.qlinear_graph_begin(s)
        ql.qlinear_forward(plan, xd, a_q, a_s, w_q, w_s, y, ws, stream=s)
        g = ql.qlinear_graph_end(s)
    for i in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        if fmt == ql.W8A8_INT8:
            assert torch.equal(y, eager), i
        else:
            r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
            assert fp8_ok(fp8_check(fmt, r, host_bf16_bits(y), 4)), i
        assert int(torch.count_nonzero(ws)) == 0
        _ = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays


# ---------------------------------------------------------------- full-size workloads

def _full_points():
    pts = []
    for cfg in decode_workloads():
        for (lab, N, K, M) in decode_points(cfg):
            if len(cfg.shapes) == 1 or M in (1, 8, 32) or (cfg.name == "fp8_dynamic_8b" and lab == "o"):
                pts.append((cfg.name, lab, N, K, M))
    return pts


_W_CACHE = {}


def _weights(wname, lab, N, K):
    key = (wname, lab)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        cfg = config_by_name(wname)
        x, w = make_inputs(K, N, max(cfg.ms), cfg.sigma_w, seed=cfg.seed)
        w_q, w_s = ql.quantize_weight(cfg.fmt, w.cuda())
        _W_CACHE[key] = (x, w, w_q, w_s)
    return _W_CACHE[key]


@pytest.mark.parametrize("wname,lab,N,K,M", _full_points())
def test_full_size_workloads_sampled_columns(wname, lab, N, K, M):
    """Configured workloads at full size with the plan the bench uses; the
    oracle recomputes sampled output columns one by one (it quantizes just the
    weight rows, or 128-row blocks, those columns need)."""
    fmt = config_by_name(wname).fmt
    ql.load_default_table()
    x, w, w_q, w_s = _weights(wname, lab, N, K)
    xm = x[:M]
    a_q, a_s = ql.quantize_act(fmt, xm.cuda())
    a_p, _ = ql.quantize_act_packed(fmt, xm.cuda())
    w_p = ql.pack_weight(w_q)
    ys = []
    for w_layout, a_packed in ((0, 0), (1, 0), (1, 1)):
        plan = ql.qlinear_plan_layouts(fmt, M, N, K, w_layout, a_packed)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ql.qlinear_run(plan, a_p if a_packed else a_q, a_s, w_p if w_layout else w_q, w_s, y, plan.new_workspace())
        torch.cuda.synchronize()
        ys.append((plan, host_bf16_bits(y)))
    rng = np.random.default_rng(sum(map(ord, wname)) * 1000 + M)
    if fmt == ql.BLOCK_FP8:
        nbs = rng.choice(-(-N // 128), 2, replace=False)
        cols = np.concatenate([np.arange(nb * 128, min(N, nb * 128 + 128)) for nb in nbs])
    else:
        cols = np.sort(rng.choice(N, 96, replace=False))
    r = oracle.reference(fmt, bf16_bits(xm), bf16_bits(w[torch.from_numpy(cols)]))
    assert np.array_equal(host_codes(fmt, a_q), r["a_q"])
    for plan, yb in ys:
        ysel = yb[:, cols]
        if fmt == ql.W8A8_INT8:
            assert np.array_equal(ysel, r["y_ref"]), plan.config
        else:
            st = fp8_check(fmt, r, ysel, plan.facts["chunks"])
            assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (plan.config, st)


def _table_entries():
    path = ql.DEFAULT_TABLE
    if not os.path.exists(path):
        return []
    out = []
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        v = [int(t) for t in f[:16]]
        kind = f[17] if len(f) > 17 else ""
        out.append(tuple(v) + ({"": 0, "fwd": 1, "glu": 2, "amx": 3}[kind],))
    return out


_TABLE_FIELDS = ("algo", "swap_ab", "split_k", "waves_n", "waves_k", "rows_per_wave", "prefetch",
                 "a_mode", "w_lds", "w_layout", "tile_m", "tile_n")


def _shape_config(fmt, N, K):
    for cfg in CONFIGS:
        if cfg.fmt != fmt:
            continue
        for (lab, n, k) in cfg.shapes:
            if (n, k) == (N, K):
                return cfg.name, lab
    raise KeyError((fmt, N, K))


@pytest.mark.parametrize("entry", _table_entries(),
                         ids=lambda e: "f%d-M%d-N%d-K%d-L%d%s" % (e[0], e[1], e[2], e[3], e[13],
                                                                  ["", "-fwd", "-glu", "-amx"][e[16]]))
def test_every_table_entry_matches_oracle(entry):
    """Each configuration the shipped sweep table selects, run at its own
    (format, M, N, K) and weight layout, against the oracle on sampled columns
    (forward entries through qlinear_forward, which also quantizes)."""
    fmt, M, N, K = entry[:4]
    cfg = dict(zip(_TABLE_FIELDS, entry[4:16]))
    wname, lab = _shape_config(fmt, N, K)
    x, w, w_q, w_s = _weights(wname, lab, N, K)
    xm = x[:M]
    if entry[16] == 2:
        _check_glu_entry(fmt, M, N, K, cfg, xm, w, w_q, w_s)
        return
    a_q, a_s = ql.quantize_act(fmt, xm.cuda())
    plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    w_use = ql.pack_weight(w_q) if cfg["w_layout"] else w_q
    if fmt == ql.MXFP4:
        w_use = ql.pack_weight_fp4(w_q)
    if fmt in ql.MX_FORMATS:
        w_s = ql.pack_mx_scales(w_s)
    if entry[16] == 3:
        # given-amax forward: the amax words of X from the host, cleared by the run
        a_f = ql.act_buffer(plan)
        s_f = torch.empty_like(a_s)
        amax = filled_amax_buffer(amax_words(bf16_bits(xm)), seed=M + N)
        ql.qlinear_forward_amax(plan, xm.cuda(), amax, a_f, s_f, w_use, w_s, y, plan.new_workspace())
        torch.cuda.synchronize()
        assert torch.equal(s_f, a_s) and int(torch.count_nonzero(amax)) == 0
    elif entry[16]:
        a_f = ql.act_buffer(plan)
        s_f = torch.empty_like(a_s)
        ql.qlinear_forward(plan, xm.cuda(), a_f, s_f, w_use, w_s, y, plan.new_workspace())
        torch.cuda.synchronize()
        assert torch.equal(s_f, a_s)
    else:
        if cfg["a_mode"] >= 2:
            a_q, a_p_s = ql.quantize_act_packed(fmt, xm.cuda())
            if fmt in ql.MX_FORMATS:
                a_s = a_p_s
        ql.qlinear_run(plan, a_q, a_s, w_use, w_s, y, plan.new_workspace())
        torch.cuda.synchronize()
    yb = host_bf16_bits(y)
    rng = np.random.default_rng(N + 7 * M)
    if fmt == ql.BLOCK_FP8:
        nb = int(rng.integers(0, -(-N // 128)))
        cols = np.arange(nb * 128, min(N, nb * 128 + 128))
    else:
        cols = np.sort(rng.choice(N, 64, replace=False))
    rows = np.sort(rng.choice(M, 256, replace=False)) if M > 256 else np.arange(M)
    ysel = yb[np.ix_(rows, cols)]
    if fmt in ql.MX_FORMATS:
        ref = oracle.mx4_reference if fmt == ql.MXFP4 else oracle.mx_reference
        r = ref(bf16_bits(xm[torch.from_numpy(rows)]), bf16_bits(w[torch.from_numpy(cols)]))
        d = oracle.summation_depth(K, split=plan.facts["chunks"], waves_k=16)
        B = oracle.MxBound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], d, fp4=fmt == ql.MXFP4)
        st = oracle.check_fp8_parity(ysel, r["y_ref"], r["y_true"], B)
        assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)
        return
    r = oracle.reference(fmt, bf16_bits(xm[torch.from_numpy(rows)]), bf16_bits(w[torch.from_numpy(cols)]))
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(ysel, r["y_ref"]), cfg
    else:
        st = fp8_check(fmt, r, ysel, plan.facts["chunks"])
        assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)


def _check_glu_entry(fmt, M, N, K, cfg, xm, w, w_q, w_s):
    """A SiLU-and-mul table entry: forward with the merged gate/up weight,
    64 sampled output columns (whole 128-row blocks for Block_FP8) against
    the oracle's glu_reference."""
    I = N // 2
    plan = ql.qlinear_plan_glu_with_config(fmt, M, N, K, cfg)
    y = torch.empty(M, I, dtype=torch.bfloat16, device="cuda")
    a_p = ql.act_buffer(plan)
    a_s = torch.empty(ql.act_scale_shape(fmt, M, K), dtype=torch.float32, device="cuda")
    ql.qlinear_forward(plan, xm.cuda(), a_p, a_s, ql.pack_weight(w_q), w_s, y, plan.new_workspace())
    torch.cuda.synchronize()
    h = host_bf16_bits(y)
    rng = np.random.default_rng(N + M)
    if fmt == ql.BLOCK_FP8:
        nb = int(rng.integers(0, I // 128))
        cols = np.arange(nb * 128, nb * 128 + 128)
    else:
        cols = np.sort(rng.choice(I, 64, replace=False))
    r = oracle.reference(fmt, bf16_bits(xm), bf16_bits(w[torch.from_numpy(np.concatenate([cols, I + cols]))]))
    h_ref, h_true, bound = oracle.glu_reference(fmt, r, split=plan.facts["chunks"])
    st = oracle.check_fp8_parity(h[:, cols], h_ref, h_true, bound)
    assert st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP, (cfg, st)


def test_concurrent_plans_on_two_streams_match_serial_runs():
    """Two split-K plans (their own workspaces) enqueued alternately on two
    streams of default priority, several times each without waiting: every
    output equals its serial run (INT8 bit-exact; FP8 against the oracle)."""
    cases = []
    for fmt, (M, N, K), split in ((ql.W8A8_INT8, (8, 4096, 2048), 4), (ql.FP8_DYNAMIC, (5, 3072, 4096), 8)):
        r = _ref(fmt, M, N, K, seed=N + split)
        a_q, s_a, w_q, s_w = _dev(fmt, r)
        plan = ql.qlinear_plan_with_config(fmt, M, N, K, dict(split_k=split, waves_n=2, waves_k=2))
        y_serial, _, _ = run_gemm(plan, a_q, s_a, w_q, s_w, acc=False)
        cases.append((fmt, r, plan, (a_q, s_a, w_q, s_w), y_serial))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty(c[2].M, c[2].N, dtype=torch.bfloat16, device="cuda") for _ in range(3)] for c in cases]
    wss = [c[2].new_workspace() for c in cases]
    torch.cuda.synchronize()
    for it in range(3):
        for ci, (fmt, r, plan, ops, _) in enumerate(cases):
            with torch.cuda.stream(streams[ci]):
                ql.qlinear_run(plan, *ops, outs[ci][it], wss[ci], stream=streams[ci])
    torch.cuda.synchronize()
    for ci, (fmt, r, plan, ops, y_serial) in enumerate(cases):
        for it in range(3):
            yb = host_bf16_bits(outs[ci][it])
            if fmt == ql.W8A8_INT8:
                assert np.array_equal(yb, y_serial) and np.array_equal(yb, r["y_ref"]), it
            else:
                assert fp8_ok(fp8_check(fmt, r, yb, plan.facts["chunks"], 2)), it
        assert int(torch.count_nonzero(wss[ci])) == 0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("split", [64, 128, 256])
def test_split_k_up_to_256(fmt, split):
    """The pages' split_k range reaches 256: a long-K, small-N shape (256 K
    blocks, so chunks of 4, 2 and 1 blocks) in row-major and packed layouts;
    INT8 bit-exact, FP8 within the bound, workspace left all-zero."""
    M, N, K = 5, 200, 32768
    r = _ref(fmt, M, N, K, seed=split + fmt)
    a_q, s_a, w_q, s_w = _dev(fmt, r)
    for packed in (0, 1):
        cfg = dict(swap_ab=int(split == 128), split_k=split, waves_n=4 if packed else 2,
                   waves_k=1 if packed else 2, rows_per_wave=16, prefetch=2, a_mode=2 if packed else 0, w_lds=0,
                   w_layout=packed)
        plan = ql.qlinear_plan_with_config(fmt, M, N, K, cfg)
        assert plan.facts["chunks"] == split
        y, acc, ws = run_gemm(plan, _dev_packed_act(fmt, r) if packed else a_q, s_a,
                              ql.pack_weight(w_q) if packed else w_q, s_w)
        _assert_parity(fmt, r, y, acc, split, label=str(cfg), waves_k=cfg["waves_k"])
        assert int(torch.count_nonzero(ws)) == 0, "split-K workspace not left all-zero"
