"""Pins of the MXFP8 oracle (oracle/mx.py) against things other than itself:
the bf16 bit fields, an exact-rational restatement (tests/exact_ref.py),
hand-computed closed forms, a one-hot layout probe, and invariants that the
MX definition implies (power-of-two scale invariance, the range of a block's
largest element, round-trip error, re-quantization fixed point)."""

from fractions import Fraction as F
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mx
from tests import exact_ref as X
from workloads import bf16_bits, make_inputs


def _frac_of_bits(bits):
    u = int(bits)
    sign = -1 if u & 0x8000 else 1
    ex, m = (u >> 7) & 0xFF, u & 0x7F
    return sign * (F(m, 128) * F(2) ** -126 if ex == 0 else (1 + F(m, 128)) * F(2) ** (ex - 127))


def _bf(values):
    """bf16 bit patterns (uint16) of float values (numpy or torch), RNE."""
    t = values if isinstance(values, torch.Tensor) else torch.from_numpy(np.asarray(values, np.float32))
    return bf16_bits(t.float().to(torch.bfloat16))


def test_shared_exponent_from_the_bit_fields_for_every_bf16():
    """e = floor(log2 amax) - 8 read off the bf16 exponent field (normal) or the
    leading mantissa bit (subnormal), clamped at -127, for all positive finite bf16."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    ex, m = (bits >> 7) & 0xFF, bits & 0x7F
    lead = np.array([int(v).bit_length() - 1 for v in m])
    fl2 = np.where(ex > 0, ex.astype(np.int64) - 127, lead - 133)
    want = np.maximum(fl2 - 8, -127)
    amax = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = mx.mx_shared_exponent(amax)
    assert np.array_equal(got, want)
    ratio = amax / np.ldexp(1.0, got)
    unclamped = fl2 - 8 >= -127
    assert np.all((ratio[unclamped] >= 256) & (ratio[unclamped] < 512))
    assert np.all(ratio[~unclamped] < 256)
    assert mx.mx_shared_exponent(0.0) == -127


def test_quantizer_matches_exact_rational_blocks():
    rng = np.random.default_rng(3)
    rows = []
    for kind in range(6):
        v = rng.standard_normal(96) * [1.0, 1e-3, 40.0, 1e-36, 3e4, 1.0][kind]
        if kind == 5:
            v[:32] = 0.0
            v[40] = -0.0
            v[64:] = 448.0 * np.sign(rng.standard_normal(32))
        rows.append(v)
    xb = _bf(np.asarray(rows, np.float32))
    xb[5, 33] = 0x8000                                   # -0.0 inside a nonzero block
    codes, scales = mx.mx_quantize(xb)
    dec = oracle.e4m3_decode(codes)
    for r in range(xb.shape[0]):
        for b in range(xb.shape[1] // 32):
            blk = xb[r, 32 * b:32 * b + 32]
            vals = [_frac_of_bits(u) for u in blk]
            nz = [int(u) == 0x8000 for u in blk]
            want, e = X.mx_quantize_block(vals, nz)
            assert int(scales[r, b]) == e + 127
            for j, (val, neg) in enumerate(want):
                c = int(codes[r, 32 * b + j])
                assert F(float(dec[r, 32 * b + j])) == (-val if neg and val > 0 else val) or \
                    (val == 0 and dec[r, 32 * b + j] == 0)
                assert bool(c & 0x80) == neg, (r, b, j)


def test_all_zero_block_gets_the_smallest_scale_and_zero_codes():
    xb = np.zeros((2, 64), np.uint16)
    xb[1, 32:] = 0x3F80                                  # 1.0
    codes, scales = mx.mx_quantize(xb)
    assert list(scales[0]) == [0, 0] and scales[1, 0] == 0 and scales[1, 1] == 127 - 8
    assert not codes[0].any() and not codes[1, :32].any()
    assert np.all(codes[1, 32:] == 0x78)                 # 1.0 / 2**-8 = 256 = E4M3 0.1111.000


@pytest.mark.parametrize("k", [-20, -3, 1, 7, 30])
def test_power_of_two_scaling_moves_only_the_exponent(k):
    x, _ = make_inputs(256, 8, 16, 0.02, seed=5)
    xb = bf16_bits(x)
    xs = _bf(x.double() * 2.0 ** k)      # exact: bf16 times a power of two, in range
    c0, s0 = mx.mx_quantize(xb)
    c1, s1 = mx.mx_quantize(xs)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_largest_element_of_every_block_lies_in_256_448():
    x, w = make_inputs(4096, 64, 32, 0.02, seed=8)
    for b in (bf16_bits(x), bf16_bits(w)):
        codes, scales = mx.mx_quantize(b)
        dec = np.abs(oracle.e4m3_decode(codes)).reshape(codes.shape[0], -1, 32).max(axis=2)
        assert np.all((dec >= 256) & (dec <= 448))


def test_round_trip_error_and_requantization_fixed_point():
    x, _ = make_inputs(2048, 8, 32, 0.02, seed=11)
    xb = bf16_bits(x)
    codes, scales = mx.mx_quantize(xb)
    v = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    d = mx.mx_dequantize(codes, scales)
    X2 = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    t = np.abs(v) / X2
    err = np.abs(v - d) / X2
    # half the E4M3 spacing at |t| (normals), the subnormal half-quantum, the clamp
    half = np.where(t >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(t, 2.0 ** -6))).astype(int) - 4),
                    2.0 ** -10)
    assert np.all(np.where(t > 448, err <= t - 448, err <= half))
    c2, s2 = mx.mx_quantize(_bf(d.astype(np.float32)))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_contraction_equals_exact_rational_sum():
    rng = np.random.default_rng(12)
    M, N, K = 3, 5, 128
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x3C                         # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0x41
    sa = rng.integers(100, 160, (M, K // 32), dtype=np.uint8)
    sw = rng.integers(60, 200, (N, K // 32), dtype=np.uint8)
    y = mx.mx_contract_exact(a, sa, w, sw)
    for m in range(M):
        for n in range(N):
            s = sum(X.E4M3[int(a[m, k])] * X.E4M3[int(w[n, k])] * F(2) ** (int(sa[m, k // 32]) + int(sw[n, k // 32]) - 254)
                    for k in range(K))
            assert y[m, n] == float(s), (m, n)          # fsum is correctly rounded, as is float(Fraction)


def test_closed_form_constant_inputs():
    """X = 1.0 and W = bf16(0.02) = 1.28125 * 2**-6 everywhere: X codes are 256
    at scale 2**-8; W at scale 2**-14 is 328, which rounds to 320 (E4M3 keeps
    three mantissa bits), so every product is 0.01953125 and Y = K * 0.01953125."""
    M, N, K = 2, 3, 256
    xb = np.full((M, K), 0x3F80, np.uint16)
    wb = np.full((N, K), 0x3CA4, np.uint16)
    assert _frac_of_bits(0x3CA4) == F(41, 32) * F(2) ** -6
    r = mx.mx_reference(xb, wb)
    assert np.all(r["a_q"] == 0x78) and np.all(r["s_a"] == 119)
    assert np.all(r["w_q"] == 0x7A) and np.all(r["s_w"] == 113)
    assert np.all(r["y_true"] == K * 0.01953125)
    assert np.all(r["y_ref"] == 0x40A0)                  # 5.0 in bf16


def test_layout_one_hot_weight_rows():
    """W row n holds 1.0 at column j(n) only: its block there has scale 2**-8
    and code 256, every other block is all-zero, so Y[m, n] is the decoded
    activation A[m, j(n)] (code times its own block's scale) exactly."""
    M, K = 4, 512
    js = [0, 31, 32, 100, 255, 256, 384, 511]
    x, _ = make_inputs(K, 8, M, 0.02, seed=21)
    xb = bf16_bits(x)
    wb = np.zeros((len(js), K), np.uint16)
    for n, j in enumerate(js):
        wb[n, j] = 0x3F80
    r = mx.mx_reference(xb, wb)
    a = mx.mx_dequantize(r["a_q"], r["s_a"])
    assert np.array_equal(r["y_true"], a[:, js])


def test_tolerance_accepts_binary32_order_and_rejects_a_dropped_block():
    M, N, K = 8, 64, 2048
    x, w = make_inputs(K, N, M, 0.02, seed=13)
    r = mx.mx_reference(bf16_bits(x), bf16_bits(w))
    depth = oracle.summation_depth(K, split=2, waves_k=4)
    B = mx.mx_tolerance_bound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], depth)
    a = mx.mx_dequantize(r["a_q"], r["s_a"])
    wd = mx.mx_dequantize(r["w_q"], r["s_w"])
    # binary32 evaluation: exact 128-K steps, added in binary32 in K order
    acc = np.zeros((M, N), np.float32)
    for kb in range(K // 128):
        acc = (acc + (a[:, kb * 128:(kb + 1) * 128] @ wd[:, kb * 128:(kb + 1) * 128].T).astype(np.float32)).astype(np.float32)
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(acc), r["y_ref"], r["y_true"], B)
    assert st["ok"] and st["frac_within_ulp"] > 0.99, st
    drop = (acc - (a[:, 64:96] @ wd[:, 64:96].T).astype(np.float32)).astype(np.float32)
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(drop), r["y_ref"], r["y_true"], B)
    assert not st["ok"] and st["n_fail"] > 0.5 * M * N, st


# ---------------------------------------------------------------- MXFP4 weights

def test_e2m1_codec_matches_generic_rounding():
    """Every multiple of 1/256 in [-6, 6] and random values: the encoder's code
    decodes to the exact-rational round-to-nearest-even E2M1 value, sign kept."""
    v = np.concatenate([np.arange(-1536, 1537) / 256.0, np.random.default_rng(4).uniform(-6, 6, 4000), [-0.0]])
    codes = oracle.e2m1_encode(v)
    dec = oracle.e2m1_decode(codes)
    for x, c, d in zip(v, codes, dec):
        want = X.re2m1(F(float(x)))
        assert F(float(d)) == want or (want == 0 and d == 0), (x, c)
        assert bool(c & 0x8) == bool(np.signbit(x)), x
    assert list(oracle.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_mx4_shared_exponent_from_the_bit_fields_for_every_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    ex, m = (bits >> 7) & 0xFF, bits & 0x7F
    lead = np.array([int(v).bit_length() - 1 for v in m])
    fl2 = np.where(ex > 0, ex.astype(np.int64) - 127, lead - 133)
    amax = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(mx.mx4_shared_exponent(amax), np.maximum(fl2 - 2, -127))


def test_mx4_quantizer_matches_exact_rational_blocks():
    rng = np.random.default_rng(5)
    rows = np.stack([rng.standard_normal(96) * s for s in (1.0, 1e-3, 0.02, 1e-37, 3e4)])
    rows[1, :32] = 0.0
    wb = _bf(rows.astype(np.float32))
    wb[1, 40] = 0x8000
    codes, scales = mx.mx4_quantize(wb)
    dec = oracle.e2m1_decode(codes)
    for r in range(wb.shape[0]):
        for b in range(3):
            blk = wb[r, 32 * b:32 * b + 32]
            want, e = X.mx4_quantize_block([_frac_of_bits(u) for u in blk], [int(u) == 0x8000 for u in blk])
            assert int(scales[r, b]) == e + 127
            for j, (val, neg) in enumerate(want):
                assert F(float(abs(dec[r, 32 * b + j]))) == abs(val)
                assert bool(codes[r, 32 * b + j] & 0x8) == neg, (r, b, j)


def test_mx4_largest_element_of_every_block_lies_in_4_6():
    _, w = make_inputs(4096, 64, 1, 0.02, seed=8)
    codes, _ = mx.mx4_quantize(bf16_bits(w))
    big = np.abs(oracle.e2m1_decode(codes)).reshape(64, -1, 32).max(axis=2)
    assert np.all((big >= 4) & (big <= 6))


def test_mx4_contraction_equals_exact_rational_sum():
    rng = np.random.default_rng(14)
    M, N, K = 3, 4, 128
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    w = rng.integers(0, 16, (N, K), dtype=np.uint8)
    sa = rng.integers(100, 160, (M, K // 32), dtype=np.uint8)
    sw = rng.integers(60, 200, (N, K // 32), dtype=np.uint8)
    y = mx.mx4_contract_exact(a, sa, w, sw)
    e2m1 = {c: (-1 if c & 8 else 1) * [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)][c & 7] for c in range(16)}
    for m in range(M):
        for n in range(N):
            s = sum(X.E4M3[int(a[m, k])] * e2m1[int(w[n, k])] * F(2) ** (int(sa[m, k // 32]) + int(sw[n, k // 32]) - 254)
                    for k in range(K))
            assert y[m, n] == float(s), (m, n)


def test_mx4_closed_form_constant_inputs():
    """X = 1.0 (MXFP8: code 256 at 2**-8) and W = bf16(0.02) = 1.28125 * 2**-6:
    W's exponent is -6 - 2 = -8, w / 2**-8 = 5.125 rounds to 6 (code 7), so
    every product is 6 * 2**-8 and Y = K * 0.0234375."""
    M, N, K = 2, 3, 256
    r = mx.mx4_reference(np.full((M, K), 0x3F80, np.uint16), np.full((N, K), 0x3CA4, np.uint16))
    assert np.all(r["w_q"] == 7) and np.all(r["s_w"] == 119)
    assert np.all(r["y_true"] == K * 0.0234375)


def test_mx4_tolerance_accepts_binary32_order_and_rejects_a_dropped_block():
    M, N, K = 8, 64, 2048
    x, w = make_inputs(K, N, M, 0.02, seed=15)
    r = mx.mx4_reference(bf16_bits(x), bf16_bits(w))
    B = mx.mx4_tolerance_bound(r["a_q"], r["s_a"], r["w_q"], r["s_w"], oracle.summation_depth(K, 2, 4))
    a = mx.mx_dequantize(r["a_q"], r["s_a"])
    wd = (oracle.e2m1_decode(r["w_q"]).reshape(N, -1, 32)
          * np.ldexp(1.0, r["s_w"].astype(int) - 127)[:, :, None]).reshape(N, K)
    acc = np.zeros((M, N), np.float32)
    for kb in range(K // 128):
        acc = (acc + (a[:, kb * 128:(kb + 1) * 128] @ wd[:, kb * 128:(kb + 1) * 128].T).astype(np.float32)).astype(np.float32)
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(acc), r["y_ref"], r["y_true"], B)
    assert st["ok"] and st["frac_within_ulp"] > 0.99, st
    drop = (acc - (a[:, 64:96] @ wd[:, 64:96].T).astype(np.float32)).astype(np.float32)
    st = oracle.check_fp8_parity(oracle.bf16_bits_from_f32(drop), r["y_ref"], r["y_true"], B)
    assert not st["ok"] and st["n_fail"] > 0.5 * M * N, st
