"""Operands that probe how the matrix core rounds an E4M3 dot product.

A decode GEMM plan with K = 128 and one wave per K range runs exactly one
16x16x128 E4M3 matrix instruction per output element, with a zero
accumulator input; its raw fp32 accumulator (``qlinear_run_debug_acc``) is
that instruction's result.  With K = 256 or 512 the same wave chains two or
four instructions through the accumulator input.  These generators build A
(16 rows) and W (N rows) code matrices whose rows mix realistic, extreme and
adversarial patterns -- one dominant product among many small ones of both
signs, exact cancellation with a small residue, subnormal products, every
finite code -- so that every output element is a probe of a different kind.

Everything here is host-side numpy; the exact sum of each probe is an fp64
dot product of the decoded values (every E4M3 product is a multiple of
2**-18 below 2**17.7, so any sum of up to 2**17 of them is exact in binary64).
"""

import numpy as np

import oracle

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # every code but NaN
ONE, MAX = 0x38, 0x7E            # 1.0 and 448


def _enc(v):
    return oracle.e4m3_encode(np.clip(np.asarray(v, np.float32), -448.0, 448.0))


def _codes_with_exponent(rng, lo, hi, size, signed=True):
    """Random codes whose exponent field lies in [lo, hi] (0 = subnormal)."""
    e = rng.integers(lo, hi + 1, size=size)
    m = rng.integers(0, 8, size=size)
    m = np.where((e == 15) & (m == 7), 6, m)          # not NaN
    c = (e << 3) | m
    if signed:
        c = c | (rng.integers(0, 2, size=size) << 7)
    return c.astype(np.uint8)


def probe_a_rows(rng, K):
    """16 activation rows of K codes."""
    rows = []
    rows.append(np.full(K, ONE, np.uint8))                                    # 0 ones
    rows.append(np.where(np.arange(K) % 2, ONE | 0x80, ONE).astype(np.uint8))  # 1 alternating +-1
    for s in (1.0, 1.0):                                                      # 2, 3 realistic
        x = rng.standard_normal(K)
        x[rng.choice(K, max(1, K // 100), replace=False)] *= 20
        rows.append(_enc(x * 448.0 / np.max(np.abs(x))))
    rows.append(rng.choice(FINITE, K))                                        # 4, 5 every finite code
    rows.append(rng.choice(FINITE, K))
    rows.append(rng.choice(FINITE[FINITE < 0x80], K))                         # 6 positive codes
    rows.append((rng.integers(0, 16, K) << 3 | rng.integers(0, 2, K) << 7).astype(np.uint8))  # 7 powers of two
    r = np.full(K, ONE, np.uint8); r[0] = MAX; rows.append(r)                 # 8 448 first, then ones
    r = np.full(K, ONE, np.uint8); r[-1] = MAX; rows.append(r)                # 9 448 last
    rows.append(_codes_with_exponent(rng, 0, 0, K))                           # 10 subnormal
    rows.append(_codes_with_exponent(rng, 6, 7, K))                           # 11 [0.5, 2)
    for s in (1.0, 30.0, 448.0, 0.05):                                        # 12..15 scaled normals
        rows.append(_enc(rng.standard_normal(K) * s))
    return np.stack(rows).astype(np.uint8)


N_FAMILIES = 12


def probe_w_row(rng, fam, K):
    """One weight row of family ``fam``."""
    if fam == 0:                                       # ones
        return np.full(K, ONE, np.uint8)
    if fam == 1:                                       # per-channel quantized N(0, 1)
        x = rng.standard_normal(K)
        return _enc(x * 448.0 / np.max(np.abs(x)))
    if fam == 2:                                       # every finite code
        return rng.choice(FINITE, K)
    if fam == 3:                                       # one dominant, small rest of both signs
        r = _codes_with_exponent(rng, 0, 3, K)
        r[rng.integers(K)] = MAX | (rng.integers(2) << 7)
        return r
    if fam == 4:                                       # cancelling pairs + one small residue
        h = K // 2
        c = rng.choice(FINITE[FINITE < 0x80], h)
        r = np.concatenate([c, c | 0x80]).astype(np.uint8)
        r[rng.integers(K)] = _codes_with_exponent(rng, 0, 4, 1)[0]
        return r
    if fam == 5:                                       # one big and one small, zeros elsewhere
        r = np.zeros(K, np.uint8)
        i, j = rng.choice(K, 2, replace=False)
        r[i] = MAX | (rng.integers(2) << 7)
        r[j] = rng.choice(FINITE)
        return r
    if fam == 6:                                       # 448 then K-1 copies of one small code
        r = np.full(K, rng.choice(FINITE), np.uint8)
        r[rng.integers(K)] = MAX
        return r
    if fam == 7:                                       # subnormal
        return _codes_with_exponent(rng, 0, 0, K)
    if fam == 8:                                       # one magnitude, alternating signs
        c = rng.choice(FINITE[FINITE < 0x80])
        return np.where(np.arange(K) % 2, c | 0x80, c).astype(np.uint8)
    if fam == 9:                                       # powers of two, any exponent
        return (rng.integers(0, 16, K) << 3 | rng.integers(0, 2, K) << 7).astype(np.uint8)
    if fam == 10:                                      # sparse
        r = rng.choice(FINITE, K)
        r[rng.random(K) < 0.9] = 0
        return r
    if fam == 11:                                      # large values of both signs (heavy cancellation)
        return _codes_with_exponent(rng, 12, 15, K)
    raise ValueError(fam)


def probe_operands(seed, N, K):
    """A codes [16, K] and W codes [N, K] (uint8); W row n is of family n % N_FAMILIES."""
    rng = np.random.default_rng(seed)
    a = probe_a_rows(rng, K)
    w = np.stack([probe_w_row(rng, n % N_FAMILIES, K) for n in range(N)]).astype(np.uint8)
    return a, w


def exact_sums(a_codes, w_codes, block=128):
    """Exact dot products, absolute sums and the largest |product| per 128-wide
    block: S [M, N], A [M, N], P [M, N] (fp64; A and S are exact)."""
    a = oracle.e4m3_decode(a_codes)
    w = oracle.e4m3_decode(w_codes)
    S = a @ w.T
    A = np.abs(a) @ np.abs(w).T
    K = a.shape[1]
    P = np.zeros_like(S)
    for k0 in range(0, K, block):
        pa, pw = a[:, k0:k0 + block], w[:, k0:k0 + block]
        P = np.maximum(P, np.max(np.abs(pa[:, None, :] * pw[None, :, :]), axis=2))
    return S, A, P


N_FP4_FAMILIES = 6


def probe_fp4_row(rng, fam, K):
    """One E2M1 weight row (codes 0..15, one a byte) of family ``fam``."""
    if fam == 0:                                       # every code
        return rng.integers(0, 16, K).astype(np.uint8)
    if fam == 1:                                       # one dominant (+-6), the rest +-0.5
        r = (rng.integers(0, 2, K) << 3 | 1).astype(np.uint8)
        r[rng.integers(K)] = 7 | (rng.integers(2) << 3)
        return r
    if fam == 2:                                       # +-6 and +-0.5 only, random
        return np.where(rng.random(K) < 0.5, 7, 1).astype(np.uint8) | (rng.integers(0, 2, K) << 3).astype(np.uint8)
    if fam == 3:                                       # sparse
        r = rng.integers(0, 16, K).astype(np.uint8)
        r[rng.random(K) < 0.85] = 0
        return r
    if fam == 4:                                       # one magnitude, alternating signs
        c = int(rng.integers(1, 8))
        return np.where(np.arange(K) % 2, c | 8, c).astype(np.uint8)
    if fam == 5:                                       # ones
        return np.full(K, 2, np.uint8)
    raise ValueError(fam)


def probe_fp4_operands(seed, N, K):
    """E4M3 A codes [16, K] and E2M1 W codes [N, K]; W row n is of family n % N_FP4_FAMILIES."""
    rng = np.random.default_rng(seed)
    a = probe_a_rows(rng, K)
    w = np.stack([probe_fp4_row(rng, n % N_FP4_FAMILIES, K) for n in range(N)]).astype(np.uint8)
    return a, w
