"""Pins of the oracle's floating-point helpers and E4M3 codec (CPU only)."""

import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from tests import exact_ref as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_golden_e4m3_ocp_values_decode_and_encode():
    rows = _load_golden_e4m3()
    assert len(rows) >= 12
    for code, val in rows:
        dec = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        if val == "nan":
            assert np.isnan(dec)
            continue
        v = float(F(val))
        assert dec == v, (hex(code), val, dec)
        enc = oracle.e4m3_encode(np.array([v], np.float32))[0]
        if v == 0.0 and code == 0x80:
            enc = oracle.e4m3_encode(np.array([-0.0], np.float32))[0]
        assert enc == code, (hex(code), val, hex(enc))


def test_e4m3_decode_matches_exact_table_all_codes():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = X.E4M3[c]
        if ref is None:
            assert np.isnan(dec[c])
        else:
            assert dec[c] == float(ref)
    assert set(np.where(np.isnan(dec))[0].tolist()) == {0x7F, 0xFF}


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _midpoint_probe_values():
    """Every binary32 value within +-4 ulp of each midpoint between adjacent E4M3 values."""
    pos = sorted({float(v) for v in X.E4M3.values() if v is not None and v >= 0})
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])] + pos
    out = []
    for m in mids:
        b = int(np.array([m], np.float32).view(np.uint32)[0])
        for d in range(-4, 5):
            if b + d >= 0:
                out.append(np.array([b + d], np.uint32).view(np.float32)[0])
    v = np.array(out, np.float32)
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_torch_cast_on_midpoints_and_random():
    rng = np.random.default_rng(1)
    probes = [_midpoint_probe_values(),
              rng.uniform(-448, 448, 1_000_000).astype(np.float32),
              (rng.standard_normal(300_000) * rng.choice([1e-4, 1e-2, 1, 30], 300_000)).astype(np.float32)]
    for v in probes:
        v = np.clip(v, -448, 448).astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_matches_torch_on_every_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_matches_exact_rounding_on_sample():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-448, 448, 2000), rng.uniform(-0.05, 0.05, 2000)]).astype(np.float32)
    codes = oracle.e4m3_encode(v)
    for x, c in zip(v.tolist(), codes.tolist()):
        ref = X.re4m3(F(x))
        assert X.E4M3[c] == ref, (x, hex(c))
        assert (c >> 7) == (1 if np.signbit(np.float32(x)) else 0)


def test_e4m3_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0], np.float32))


def test_bf16_rounding_matches_exact_and_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000),
                        np.array([0.0, -0.0, 1.0, 3.0e38, 1e-40, -2.5e-39])]).astype(np.float32)
    ours = oracle.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    for xv in x[:3000].tolist():
        b = oracle.bf16_bits_from_f32(np.array([xv], np.float32))
        assert F(float(oracle.bf16_bits_to_f32(b)[0])) == X.rbf16(F(xv))


def test_ulp_bf16_closed_forms():
    vals = np.array([1.0, 1.5, 2.0, 255.0, 256.0, -3.0, 0.0, 2.0 ** -126, 2.0 ** -130], np.float32)
    want = [2 ** -7, 2 ** -7, 2 ** -6, 1.0, 2.0, 2 ** -6, 2 ** -133, 2 ** -133, 2 ** -133]
    got = oracle.ulp_bf16(oracle.bf16_bits_from_f32(vals))
    assert got.tolist() == want


def test_f32_rounding_matches_exact():
    rng = np.random.default_rng(4)
    ints = rng.integers(-2 ** 40, 2 ** 40, 5000)
    for i, r in zip(ints.tolist(), oracle.f32(ints).tolist()):
        assert F(r) == X.r32(F(i))
