"""Pins of the oracle's quantizers, contraction, epilogue and tolerance (CPU only).

Each check compares the oracle with something other than itself: the
exact-rational restatement in ``tests/exact_ref.py``, closed forms, one-hot
layout probes, and invariants that any correct implementation satisfies.
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from oracle import FMT_BLOCK_FP8, FMT_FP8_DYNAMIC, FMT_W8A8_INT8
from tests import exact_ref as X
from workloads import make_inputs, bf16_bits

FMTS = [FMT_FP8_DYNAMIC, FMT_W8A8_INT8, FMT_BLOCK_FP8]
KIND = {FMT_FP8_DYNAMIC: "fp8", FMT_W8A8_INT8: "int8", FMT_BLOCK_FP8: "fp8"}


def _bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _frac_of_bits(bits):
    return [F(float(v)) for v in oracle.bf16_bits_to_f32(bits).ravel().tolist()]


def _negzero(bits):
    return [bool(b == 0x8000) for b in np.asarray(bits).ravel().tolist()]


def _groups_act(fmt, M, K):
    if fmt == FMT_BLOCK_FP8:
        return [(m, slice(g * 128, (g + 1) * 128), (m, g)) for m in range(M) for g in range(K // 128)]
    return [(m, slice(0, K), (m,)) for m in range(M)]


# --------------------------------------------------------------- brute force

def _brute_linear(fmt, x_bits, w_bits):
    """Exact-rational restatement: codes, scales, exact sums and y_ref values."""
    kind, Q = KIND[fmt], oracle.qmax_of(fmt)
    M, K = x_bits.shape
    N = w_bits.shape[0]
    xf = np.array(_frac_of_bits(x_bits), dtype=object).reshape(M, K)
    wf = np.array(_frac_of_bits(w_bits), dtype=object).reshape(N, K)
    xz = np.array(_negzero(x_bits)).reshape(M, K)
    wz = np.array(_negzero(w_bits)).reshape(N, K)
    aval = np.empty((M, K), dtype=object)
    wval = np.empty((N, K), dtype=object)
    if fmt == FMT_BLOCK_FP8:
        G = K // 128
        sa = np.empty((M, G), dtype=object)
        for m in range(M):
            for g in range(G):
                cs = slice(g * 128, (g + 1) * 128)
                codes, s = X.quantize_group(list(xf[m, cs]), list(xz[m, cs]), Q, kind)
                aval[m, cs] = [c[0] for c in codes]
                sa[m, g] = s
        NB = -(-N // 128)
        sw = np.empty((NB, G), dtype=object)
        for nb in range(NB):
            rs = slice(nb * 128, min(N, nb * 128 + 128))
            for g in range(G):
                cs = slice(g * 128, (g + 1) * 128)
                blk = wf[rs, cs]
                codes, s = X.quantize_group(list(blk.ravel()), list(wz[rs, cs].ravel()), Q, kind)
                wval[rs, cs] = np.array([c[0] for c in codes], dtype=object).reshape(blk.shape)
                sw[nb, g] = s
        y = np.empty((M, N), dtype=object)
        for m in range(M):
            for n in range(N):
                tot = F(0)
                for g in range(G):
                    cs = slice(g * 128, (g + 1) * 128)
                    tot += X.dot_frac(aval[m, cs], wval[n, cs]) * sa[m, g] * sw[n // 128, g]
                y[m, n] = X.rbf16(X.r32(tot))
        return aval, sa, wval, sw, None, y
    sa = np.empty(M, dtype=object)
    sw = np.empty(N, dtype=object)
    for m in range(M):
        codes, s = X.quantize_group(list(xf[m]), list(xz[m]), Q, kind)
        aval[m] = codes if kind == "int8" else [c[0] for c in codes]
        sa[m] = s
    for n in range(N):
        codes, s = X.quantize_group(list(wf[n]), list(wz[n]), Q, kind)
        wval[n] = codes if kind == "int8" else [c[0] for c in codes]
        sw[n] = s
    acc = np.empty((M, N), dtype=object)
    y = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc[m, n] = X.dot_int(aval[m], wval[n]) if kind == "int8" else X.dot_frac(aval[m], wval[n])
            y[m, n] = X.rbf16(X.r32(X.r32(X.r32(acc[m, n]) * sa[m]) * sw[n]))
    return aval, sa, wval, sw, acc, y


def _code_values(fmt, q):
    return [F(int(v)) for v in np.asarray(q, np.int8).ravel()] if fmt == FMT_W8A8_INT8 else \
        [X.E4M3[int(c)] for c in np.asarray(q, np.uint8).ravel()]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 3, 128), (3, 5, 256), (4, 8, 384), (2, 130, 256)])
def test_brute_force_tiny(fmt, shape):
    M, N, K = shape
    if N > 8 and fmt != FMT_BLOCK_FP8:
        N = 8
    x, w = make_inputs(K, N, M, 0.02, seed=M * 100 + N + K)
    xb, wb = bf16_bits(x), bf16_bits(w)
    r = oracle.reference(fmt, xb, wb)
    aval, sa, wval, sw, acc, y = _brute_linear(fmt, xb, wb)
    assert _code_values(fmt, r["a_q"]) == list(aval.ravel())
    assert _code_values(fmt, r["w_q"]) == list(wval.ravel())
    assert [F(float(v)) for v in np.ravel(r["s_a"])] == list(np.ravel(sa))
    assert [F(float(v)) for v in np.ravel(r["s_w"])] == list(np.ravel(sw))
    if fmt != FMT_BLOCK_FP8:
        assert [F(v) for v in np.ravel(r["S"]).tolist()] == list(acc.ravel())
    ours = [F(float(v)) for v in oracle.bf16_bits_to_f32(r["y_ref"]).ravel()]
    assert ours == list(y.ravel())


def test_fp8_sign_of_zero_codes_follow_input_sign():
    x = _bits([[1.0, -1e-6, 1e-6, -0.0, 0.0, -2.0 ** -22]])
    q, s = oracle.quantize_act(FMT_FP8_DYNAMIC, np.pad(x, ((0, 0), (0, 10))))
    assert q[0, :6].tolist() == [0x7E, 0x80, 0x00, 0x80, 0x00, 0x80]


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("fmt,K", [(FMT_W8A8_INT8, 2048), (FMT_W8A8_INT8, 25600),
                                   (FMT_FP8_DYNAMIC, 4096), (FMT_FP8_DYNAMIC, 17408),
                                   (FMT_BLOCK_FP8, 1024)])
def test_closed_form_constant_inputs(fmt, K):
    c, wv = 0.75, -0.03125
    x = _bits(np.full((3, K), c))
    w = _bits(np.full((5, K), wv))
    r = oracle.reference(fmt, x, w)
    code = 127 if fmt == FMT_W8A8_INT8 else 448
    assert np.all(oracle.dequant_codes(fmt, r["a_q"]) == code)
    assert np.all(oracle.dequant_codes(fmt, r["w_q"]) == -code)
    sa, sw = X.r32(F(c) / code), X.r32(abs(F(wv)) / code)
    if fmt == FMT_BLOCK_FP8:
        G = K // 128
        assert np.all(r["S"] == -code * code * 128)
        y = X.rbf16(X.r32(G * (-code * code * 128) * sa * sw))
    else:
        assert np.all(r["S"] == -code * code * K)          # 16129 K or 200704 K
        y = X.rbf16(X.r32(X.r32(X.r32(-code * code * K) * sa) * sw))
    assert np.all(oracle.bf16_bits_to_f32(r["y_ref"]) == float(y))


def test_closed_form_alternating_signs_int8():
    K = 1024
    row = np.where(np.arange(K) % 4 == 0, -1.0, 1.0)          # 256 negative, 768 positive
    x = _bits(np.tile(row, (2, 1)) * 0.5)
    w = _bits(np.full((3, K), 0.25))
    r = oracle.reference(FMT_W8A8_INT8, x, w)
    assert np.all(r["S"] == 16129 * (768 - 256))


# --------------------------------------------------------------- layout pins

@pytest.mark.parametrize("fmt", FMTS)
def test_layout_one_hot_rows(fmt):
    rng = np.random.default_rng(5)
    M, N, K = 5, 300, 512
    j = rng.integers(0, K, N)
    wv = np.zeros((N, K))
    wv[np.arange(N), j] = 1.0
    x, _ = make_inputs(K, 1, M, 0.02, seed=9, with_weight=False)
    xb, wb = bf16_bits(x), _bits(wv)
    r = oracle.reference(fmt, xb, wb)
    Q = int(oracle.qmax_of(fmt))
    assert np.all(oracle.dequant_codes(fmt, r["w_q"])[np.arange(N), j] == Q)
    a = oracle.dequant_codes(fmt, r["a_q"])
    for n in range(0, N, 7):
        for m in range(M):
            if fmt == FMT_BLOCK_FP8:
                g = j[n] // 128
                want = X.rbf16(X.r32(F(a[m, j[n]]) * Q * F(float(r["s_a"][m, g]))
                                     * F(float(r["s_w"][n // 128, g]))))
            else:
                want = X.rbf16(X.r32(X.r32(X.r32(F(a[m, j[n]]) * Q) * F(float(r["s_a"][m])))
                                     * F(float(r["s_w"][n]))))
            assert F(float(oracle.bf16_bits_to_f32(r["y_ref"][m, n]))) == want, (m, n)


def test_block_weight_scale_indexing_ragged_n():
    """Every 128x128 block gets its own scale; the last block row is ragged."""
    N, K = 300, 384
    wv = np.zeros((N, K))
    for nb in range(3):
        for g in range(3):
            r1 = min(N, nb * 128 + 128)
            wv[nb * 128:r1, g * 128:(g + 1) * 128] = 2.0 ** (nb * 3 + g - 4)
    q, s = oracle.quantize_weight(FMT_BLOCK_FP8, _bits(wv))
    assert s.shape == (3, 3)
    for nb in range(3):
        for g in range(3):
            assert s[nb, g] == np.float32(2.0 ** (nb * 3 + g - 4)) / np.float32(448)
    assert np.all(q == 0x7E)


# --------------------------------------------------------------- variant invariants

@pytest.mark.parametrize("fmt", [FMT_FP8_DYNAMIC, FMT_W8A8_INT8])
def test_split_and_swap_orders_agree_bitwise(fmt):
    rng = np.random.default_rng(6)
    M, N, K = 7, 33, 2048
    x, w = make_inputs(K, N, M, 0.02, seed=11)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    S = r["S"]
    assert np.array_equal(oracle.contract_swap_ab(fmt, r["a_q"], r["w_q"]), S)
    for _ in range(5):
        nch = int(rng.integers(2, 9))
        cuts = np.sort(rng.choice(np.arange(1, K // 16), nch - 1, replace=False)) * 16
        bounds = [0] + cuts.tolist() + [K]
        order = rng.permutation(nch).tolist()
        assert np.array_equal(oracle.contract_split_order(fmt, r["a_q"], r["w_q"], bounds, order), S)


def test_int8_sum_order_independent_under_k_permutation():
    rng = np.random.default_rng(7)
    x, w = make_inputs(512, 9, 4, 0.02, seed=12)
    r = oracle.reference(FMT_W8A8_INT8, bf16_bits(x), bf16_bits(w))
    p = rng.permutation(512)
    S2 = oracle.contract_exact(FMT_W8A8_INT8, r["a_q"][:, p], r["w_q"][:, p])
    assert np.array_equal(S2, r["S"])


def test_exact_contraction_matches_integer_and_rational_dot_at_full_shape():
    """fp64 BLAS equals exact integer / rational dots on sampled outputs of a real shape."""
    rng = np.random.default_rng(8)
    K, N, M = 25600, 64, 4
    x, w = make_inputs(K, N, M, 0.015, seed=13)
    r = oracle.reference(FMT_W8A8_INT8, bf16_bits(x), bf16_bits(w))
    a = r["a_q"].astype(np.int64)
    ww = r["w_q"].astype(np.int64)
    for _ in range(40):
        m, n = int(rng.integers(M)), int(rng.integers(N))
        assert int(np.dot(a[m], ww[n])) == int(r["S"][m, n])
    r8 = oracle.reference(FMT_FP8_DYNAMIC, bf16_bits(x)[:, :4096], bf16_bits(w)[:, :4096])
    av = [X.E4M3[int(c)] for c in r8["a_q"][1]]
    for n in range(0, N, 9):
        wv = [X.E4M3[int(c)] for c in r8["w_q"][n]]
        assert X.dot_frac(av, wv) == F(float(r8["S"][1, n]))


# --------------------------------------------------------------- quantizer invariants

@pytest.mark.parametrize("fmt", FMTS)
def test_quantizer_invariants(fmt):
    x, _ = make_inputs(4096, 1, 16, 0.02, seed=14, with_weight=False)
    xb = bf16_bits(x)
    q, s = oracle.quantize_act(fmt, xb)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    vals = oracle.dequant_codes(fmt, q)
    Q = oracle.qmax_of(fmt)
    if fmt == FMT_BLOCK_FP8:
        vg = vals.reshape(16, 32, 128)
        assert np.all(np.max(np.abs(vg), axis=2) == Q)
        sfull = np.repeat(s, 128, axis=1).astype(np.float64)
    else:
        assert np.all(np.max(np.abs(vals), axis=1) == Q)
        sfull = s.astype(np.float64)[:, None]
    err = np.abs(xf - vals * sfull)
    # the code rounds fl(x/s), which is within one binary32 rounding of x/s
    if fmt == FMT_W8A8_INT8:
        assert np.all(err <= sfull * 0.5 + np.abs(xf) * 2 ** -23)
    else:
        t = np.abs(xf / sfull)
        big = t >= 2 ** -6
        assert np.all(err[big] <= np.abs(xf[big]) * (2 ** -4 + 2 ** -22))
        assert np.all(err[~big] <= (2 ** -10 * sfull * np.ones_like(xf))[~big] * (1 + 2 ** -20))
    # re-quantizing the dequantized values with the same scales reproduces the codes
    deq = (vals.astype(np.float32) * sfull.astype(np.float32)).astype(np.float32)
    t2 = (deq / sfull.astype(np.float32)).astype(np.float32)
    if fmt == FMT_W8A8_INT8:
        assert np.array_equal(np.clip(np.rint(t2), -127, 127).astype(np.int8), q)
    else:
        assert np.array_equal(oracle.dequant_codes(fmt, oracle.e4m3_encode(np.clip(t2, -448, 448))), vals)


def test_max_code_is_exactly_q_for_every_bf16_amax():
    """For every positive finite bf16 amax with a normal scale, fl(amax/fl(amax/Q)) rounds to Q."""
    bits = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    for Q in (np.float32(127), np.float32(448)):
        s = (bits / Q).astype(np.float32)
        normal = s >= np.float32(2.0 ** -126)
        t = (bits[normal] / s[normal]).astype(np.float32)
        assert np.all(np.rint(t) == Q) if Q == 127 else np.all(np.abs(t - Q) <= Q * 2 ** -20)
        if Q == 448:
            assert np.all(oracle.e4m3_encode(np.clip(t, -448, 448)) == 0x7E)


def test_zero_rows_and_groups_get_unit_scale():
    x = np.zeros((3, 256))
    x[1, 5] = 2.0
    xb = _bits(x)
    for fmt in FMTS:
        q, s = oracle.quantize_act(fmt, xb)
        assert np.all(oracle.dequant_codes(fmt, q)[0] == 0)
        if fmt == FMT_BLOCK_FP8:
            assert s[0].tolist() == [1.0, 1.0] and s[1, 1] == 1.0
        else:
            assert s[0] == 1.0 and s[2] == 1.0


def test_subnormal_scale_is_kept():
    x = _bits(np.array([[1e-37, -5e-38] + [0.0] * 126]))
    q, s = oracle.quantize_act(FMT_W8A8_INT8, x)
    assert 0 < s[0] < 2 ** -126                  # binary32 subnormal scale
    assert s[0] == np.float32(oracle.bf16_bits_to_f32(x)[0, 0]) / np.float32(127)
    assert int(q[0, 0]) == 127


# --------------------------------------------------------------- tolerance self-test

@pytest.mark.parametrize("fmt", [FMT_FP8_DYNAMIC, FMT_BLOCK_FP8])
def test_tolerance_accepts_emulated_fp32_orders_and_rejects_dropped_tile(fmt):
    rng = np.random.default_rng(15)
    M, N, K = 4, 48, 1024
    x, w = make_inputs(K, N, M, 0.02, seed=16)
    r = oracle.reference(fmt, bf16_bits(x), bf16_bits(w))
    for bounds in ([0, K], [0, 384, K], [0, 256, 512, 768, K]):
        order = rng.permutation(len(bounds) - 1).tolist()
        yb = oracle.emulate_fp32_accumulation(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], bounds, order, rng)
        d = oracle.summation_depth(K, split=len(bounds) - 1)
        for mc in (False, True):      # binary32-only bound, and with the matrix-core allowance
            B = oracle.tolerance_bound(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], d, matrix_core=mc)
            st = oracle.check_fp8_parity(yb, r["y_ref"], r["y_true"], B)
            assert st["ok"], st
    # a kernel that drops one 128-wide K tile must fail on nearly every element
    wq = r["w_q"].copy()
    wq[:, 256:384] = 0
    yb = oracle.emulate_fp32_accumulation(fmt, r["a_q"], wq, r["s_a"], r["s_w"], [0, K], [0], rng)
    B = oracle.tolerance_bound(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], oracle.summation_depth(K))
    st = oracle.check_fp8_parity(yb, r["y_ref"], r["y_true"], B)
    assert not st["ok"] and st["n_fail"] >= 0.9 * st["n"], st


def test_tolerance_rejects_wrong_scale_and_sign():
    x, w = make_inputs(512, 32, 4, 0.02, seed=17)
    r = oracle.reference(FMT_FP8_DYNAMIC, bf16_bits(x), bf16_bits(w))
    B = oracle.tolerance_bound(FMT_FP8_DYNAMIC, r["a_q"], r["w_q"], r["s_a"], r["s_w"], oracle.summation_depth(512))
    yf = oracle.bf16_bits_to_f32(r["y_ref"])
    for bad in (-yf, yf * 1.01, np.roll(yf, 1, axis=1)):
        st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(bad), r["y_ref"], r["y_true"], B)
        assert not st["ok"]
