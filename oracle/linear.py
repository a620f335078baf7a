"""Exact contraction, scale epilogue and FP8 tolerance (test infrastructure only).

What is computed -- Summary, "Put algorithm selection inside the search
space": a GEMM whose quantized variants "add scaling logic", with an fp32
accumulator (Noticias, "¿Como se implementa el kernel?", the listing's
accumulator dtype).  The scaled linear is

    Y[m, n] = s_a[m] * s_w[n] * sum_k A_q[m, k] * W_q[n, k]

and for Block_FP8 the scales vary along K, so they enter per 128-wide group g:

    Y[m, n] = sum_g s_a[m, g] * s_w[n // 128, g] * S_g[m, n],
    S_g[m, n] = sum_{k in group g} A_q[m, k] * W_q[n, k].

Exactness of the contraction (why fp64 BLAS is an exact oracle here):
  * INT8: |A_q * W_q| <= 127**2 = 16129, so every partial sum of K <= 2**37
    terms is an integer below 2**53 and float64 arithmetic on it is exact in
    any order, with or without FMA.
  * E4M3: every value is a multiple of 2**-9 with magnitude <= 448, so every
    product is a multiple of 2**-18 with magnitude < 2**17.7; any partial sum
    of K <= 2**17 such products is a multiple of 2**-18 below 2**35, which
    binary64 (53-bit significand) holds exactly.
So ``A @ W.T`` in float64 returns the exact sum S regardless of the blocking
the BLAS library picks.

Split-K and Swap-AB are different evaluation orders of the same sum (the
page's split_k / swap_ab tunables); ``contract_split_order`` and
``contract_swap_ab`` evaluate those orders explicitly for the invariant pins.
"""

import numpy as np

from . import matrix_core as mc
from .fpbits import f32, bf16_bits_from_f32, bf16_bits_to_f32, ulp_bf16
from .quant import (FMT_BLOCK_FP8, FMT_W8A8_INT8, GROUP, dequant_codes,
                    quantize_act, quantize_weight)

U32 = 2.0 ** -24    # unit roundoff of binary32


def _check_exact_range(fmt, K):
    if fmt == FMT_W8A8_INT8:
        assert 16129 * K < 2 ** 53
    else:
        assert K <= 2 ** 17


def contract_exact(fmt, a_q, w_q):
    """Exact sum S = A_q . W_q^T.

    INT8 -> int64 [M, N].  FP8_Dynamic -> float64 [M, N] (exact).
    Block_FP8 -> float64 [G, M, N], one exact partial per 128-wide K group.
    """
    M, K = a_q.shape
    _check_exact_range(fmt, K)
    a = dequant_codes(fmt, a_q)
    w = dequant_codes(fmt, w_q)
    if fmt == FMT_BLOCK_FP8:
        G = K // GROUP
        return np.stack([a[:, g * GROUP:(g + 1) * GROUP] @ w[:, g * GROUP:(g + 1) * GROUP].T
                         for g in range(G)]) if G else np.zeros((0, M, w.shape[0]))
    s = a @ w.T
    if fmt == FMT_W8A8_INT8:
        s64 = s.astype(np.int64)
        assert np.all(np.abs(s64) < 2 ** 31), "int32 accumulator would overflow"
        return s64
    return s


def contract_abs(fmt, a_q, w_q):
    """Exact sum of |products|, same shape conventions as ``contract_exact``."""
    a = np.abs(dequant_codes(fmt, a_q))
    w = np.abs(dequant_codes(fmt, w_q))
    if fmt == FMT_BLOCK_FP8:
        G = a.shape[1] // GROUP
        return np.stack([a[:, g * GROUP:(g + 1) * GROUP] @ w[:, g * GROUP:(g + 1) * GROUP].T
                         for g in range(G)])
    return a @ w.T


def _block_scale(s_a, s_w, N):
    """Per-group scale product s_a[m,g] * s_w[n//128, g] as float64 [G, M, N]."""
    sw_rows = np.repeat(s_w.astype(np.float64), GROUP, axis=0)[:N]     # [N, G]
    return s_a.astype(np.float64).T[:, :, None] * sw_rows.T[:, None, :]


def epilogue(fmt, S, s_a, s_w):
    """Scale epilogue.  Returns (y_ref_bits uint16 [M,N], y_true float64 [M,N]).

    Fixed op order (the pages are silent; one order is pinned because the
    Summary warns that one formula may follow different accumulation paths):
      INT8:        y = bf16( fl( fl( f32(acc) * s_a[m] ) * s_w[n] ) )   -- the
                   bit-exact contract; f32(acc) rounds (|acc| may exceed 2**24).
      FP8_Dynamic: y_ref = bf16( fl( fl( fl(S) * s_a[m] ) * s_w[n] ) ),
                   y_true = S * s_a * s_w in float64.
      Block_FP8:   y_true = sum_g S_g * s_a[m,g] * s_w[n//128,g] in float64,
                   y_ref = bf16( fl(y_true) ).
    For INT8 y_true is returned as the float64 product as well (informational).
    """
    if fmt == FMT_BLOCK_FP8:
        N = S.shape[2]
        y_true = np.sum(S * _block_scale(s_a, s_w, N), axis=0) if S.shape[0] else \
            np.zeros(S.shape[1:], np.float64)
        return bf16_bits_from_f32(f32(y_true)), y_true
    sa = np.asarray(s_a, np.float32)[:, None]
    sw = np.asarray(s_w, np.float32)[None, :]
    t = (f32(S) * sa).astype(np.float32)
    t = (t * sw).astype(np.float32)
    y_true = np.asarray(S, np.float64) * sa.astype(np.float64) * sw.astype(np.float64)
    return bf16_bits_from_f32(t), y_true


def reference(fmt, x_bits, w_bits):
    """End to end: quantize X and W, contract exactly, apply the epilogue.

    Returns a dict with a_q, s_a, w_q, s_w, S (exact), y_ref (bf16 bits) and
    y_true (float64).
    """
    a_q, s_a = quantize_act(fmt, x_bits)
    w_q, s_w = quantize_weight(fmt, w_bits)
    S = contract_exact(fmt, a_q, w_q)
    y_ref, y_true = epilogue(fmt, S, s_a, s_w)
    return dict(a_q=a_q, s_a=s_a, w_q=w_q, s_w=s_w, S=S, y_ref=y_ref, y_true=y_true)


# ----------------------------------------------------------------------------
# FP8 tolerance.  A GPU accumulates E4M3 products in binary32 in an order of
# its own (matrix-core internal sums, per-chunk sums, atomic split-K combine),
# so its result is one of many correctly-rounded-per-step evaluations.
# ----------------------------------------------------------------------------

def summation_depth(K, split=1, waves_k=8):
    """Conservative count of binary32 roundings any product passes through.

    128 inside one matrix-core K=128 step, +3 for the Block_FP8 per-group
    scale multiply/add, one per 128-wide K step of the longest chunk, the
    in-workgroup reduction over at most ``waves_k`` partials, and one per
    split-K chunk combined by atomics.  Over-estimating only widens the bound.
    """
    return 128 + 3 + -(-K // GROUP) + waves_k + split


class Fp8Bound:
    """Forward-error bound of a GPU evaluation of the FP8 linear, per element:

        B[m, n] = (gamma_d * sum_k |p_k| + allowance[m, n]) * scales * (1 + 4u)

    gamma_d = d*u / (1 - d*u) is the classic bound for a sum evaluated with
    at most d binary32 roundings per term (u = 2**-24); ``allowance`` is the
    matrix instruction's own cut of small products (``matrix_core``), summed
    over its 128-wide K blocks.  The scales multiply both (Block_FP8: per
    128-wide group, whose partial sum the kernel scales before adding it).
    ``matrix_core=False`` gives the pure binary32 bound.

    The gamma part is one exact fp64 matmul on |A_q|, |W_q| for every
    element; the allowance is evaluated only where asked (``at``), since a
    check needs it only for elements that the cheaper clauses leave open.
    """

    def __init__(self, fmt, a_q, w_q, s_a, s_w, depth, matrix_core=True):
        self.fmt, self.a_q, self.w_q = fmt, np.asarray(a_q), np.asarray(w_q)
        self.s_a, self.s_w = np.asarray(s_a), np.asarray(s_w)
        self.matrix_core = matrix_core
        self.gamma = depth * U32 / (1.0 - depth * U32)
        absS = contract_abs(fmt, a_q, w_q)
        N = self.w_q.shape[0]
        if fmt == FMT_BLOCK_FP8:
            self._scale = _block_scale(s_a, s_w, N)                           # [G, M, N]
            self.base = self.gamma * np.sum(absS * self._scale, axis=0) * (1.0 + 4.0 * U32)
        else:
            self._scale = np.asarray(s_a, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :]
            self.base = self.gamma * absS * self._scale * (1.0 + 4.0 * U32)
        self.shape = self.base.shape

    def _operands(self):
        a = dequant_codes(self.fmt, self.a_q)
        w = dequant_codes(self.fmt, self.w_q)
        return (a, mc.e4m3_exponent(self.a_q.view(np.uint8)),
                w, mc.e4m3_exponent(self.w_q.view(np.uint8)))

    def allowance_at(self, mi, ni):
        """Scaled matrix-core allowance at the pairs (mi[j], ni[j])."""
        mi, ni = np.asarray(mi, np.int64), np.asarray(ni, np.int64)
        if not self.matrix_core or self.fmt == FMT_W8A8_INT8 or mi.size == 0:
            return np.zeros(mi.shape)
        per_block = mc.allowance_pairs(*self._operands(), mi, ni)    # [L, G]
        if self.fmt == FMT_BLOCK_FP8:
            return np.sum(per_block * self._scale[:, mi, ni].T, axis=1)
        return per_block.sum(axis=1) * self._scale[mi, ni]

    def at(self, mi, ni):
        mi, ni = np.asarray(mi, np.int64), np.asarray(ni, np.int64)
        return self.base[mi, ni] + self.allowance_at(mi, ni) * (1.0 + 4.0 * U32)

    def full(self):
        M, N = self.shape
        mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return self.at(mi.reshape(-1), ni.reshape(-1)).reshape(M, N)


def tolerance_bound(fmt, a_q, w_q, s_a, s_w, depth, matrix_core=True):
    """The bound of ``Fp8Bound`` for every element, float64 [M, N]."""
    return Fp8Bound(fmt, a_q, w_q, s_a, s_w, depth, matrix_core).full()


def accumulator_bound(fmt, a_q, w_q, depth):
    """Bound on |acc - S| of the raw FP8_Dynamic accumulator (unit scales):
    an ``Fp8Bound`` whose ``at`` gives gamma_d * sum |p| + the allowance."""
    return Fp8Bound(fmt, a_q, w_q, np.ones(a_q.shape[0], np.float32), np.ones(w_q.shape[0], np.float32), depth)


def check_fp8_parity(y_gpu_bits, y_ref_bits, y_true, bound, rel_limit=1e-2):
    """Apply the FP8 acceptance rule; returns a dict of statistics and ``ok``.

    Element (m, n) passes if |y_gpu - y_ref| <= 1 ulp_bf16(y_ref), or if
    |y_gpu - y_true| <= ulp_bf16(y_gpu)/2 + B[m, n].  Additionally the
    normwise error max|y_gpu - y_ref| / max|y_ref| must be <= rel_limit.
    ``bound`` is an array B, or an object with ``at(mi, ni)`` (``Fp8Bound``)
    that is evaluated only at the elements the first clause leaves open.
    """
    yg = bf16_bits_to_f32(y_gpu_bits).astype(np.float64)
    yr = bf16_bits_to_f32(y_ref_bits).astype(np.float64)
    d_ref = np.abs(yg - yr)
    within_ulp = d_ref <= ulp_bf16(y_ref_bits)
    open_ = np.argwhere(~within_ulp)
    if hasattr(bound, "at"):
        b_open = bound.at(open_[:, 0], open_[:, 1]) if open_.size else np.zeros(0)
    else:
        b_open = np.asarray(bound)[~within_ulp]
    yt_open = np.asarray(y_true, np.float64)[~within_ulp]
    within_b_open = np.abs(yg[~within_ulp] - yt_open) <= 0.5 * ulp_bf16(np.asarray(y_gpu_bits)[~within_ulp]) + b_open
    ok_elem = within_ulp.copy()
    ok_elem[~within_ulp] = within_b_open
    finite = np.isfinite(yg)
    denom = np.max(np.abs(yr)) if yr.size else 0.0
    normwise = float(np.max(d_ref) / denom) if denom > 0 else float(np.max(d_ref, initial=0.0))
    n = ok_elem.size
    st = dict(ok=bool(np.all(ok_elem & finite) and normwise <= rel_limit),
              n=n, n_fail=int(np.sum(~(ok_elem & finite))),
              frac_within_ulp=float(np.mean(within_ulp)) if n else 1.0,
              n_needed_bound=int(np.sum(within_b_open)),
              normwise=normwise)
    _STATS.append(st)
    return st


# Every check made in this process, in order (the parity tests summarise them).
_STATS = []


def parity_statistics():
    """The statistics dicts of every ``check_fp8_parity`` call so far."""
    return list(_STATS)


# ----------------------------------------------------------------------------
# Evaluation orders of the variants (for the invariant pins).
# ----------------------------------------------------------------------------

def contract_split_order(fmt, a_q, w_q, bounds, order):
    """Split-K order: exact partial sums over K-chunks, combined in ``order``.

    bounds: chunk edges [k0=0, k1, ..., K]; order: permutation of chunk ids in
    which the partials are added ("atomic" arrival order).  Not for Block_FP8
    (use contract_exact's per-group partials there).
    """
    parts = [contract_exact(fmt, a_q[:, bounds[i]:bounds[i + 1]], w_q[:, bounds[i]:bounds[i + 1]])
             for i in range(len(bounds) - 1)]
    total = np.zeros_like(parts[0])
    for i in order:
        total = total + parts[i]
    return total


def contract_swap_ab(fmt, a_q, w_q):
    """Swap-AB order: compute (W_q . A_q^T)^T, the transpose identity A@B = (B^T@A^T)^T."""
    if fmt == FMT_BLOCK_FP8:
        raise ValueError("use per-group partials for Block_FP8")
    return contract_exact(fmt, w_q, a_q).T


def emulate_fp32_accumulation(fmt, a_q, w_q, s_a, s_w, bounds, order, rng=None):
    """Emulate a binary32 GPU evaluation of the FP8 linear.

    Within each 128-wide K step the 128 products are summed in binary32 in a
    random order (a stand-in for the matrix core's internal order); the step
    sums are added sequentially in binary32 within each chunk; the chunk
    partials are combined in ``order`` in binary32; the epilogue follows the
    fixed order.  Block_FP8 scales each 128-step sum by (s_a * s_w) before
    adding it.  Returns bf16 bits [M, N].  Slow: small shapes only.
    """
    rng = rng or np.random.default_rng(0)
    a = dequant_codes(fmt, a_q)
    w = dequant_codes(fmt, w_q)
    M, K = a.shape
    N = w.shape[0]
    parts = []
    for c in range(len(bounds) - 1):
        acc = np.zeros((M, N), np.float32)
        for k0 in range(bounds[c], bounds[c + 1], GROUP):
            k1 = min(k0 + GROUP, bounds[c + 1])
            prods = (a[:, None, k0:k1] * w[None, :, k0:k1]).astype(np.float32)  # exact products
            perm = rng.permutation(k1 - k0)
            step = np.zeros((M, N), np.float32)
            for j in perm:
                step = (step + prods[:, :, j]).astype(np.float32)
            if fmt == FMT_BLOCK_FP8:
                g = k0 // GROUP
                sw_rows = np.repeat(s_w[:, g], GROUP)[:N].astype(np.float32)
                step = (step * s_a[:, g][:, None].astype(np.float32)).astype(np.float32)
                step = (step * sw_rows[None, :]).astype(np.float32)
            acc = (acc + step).astype(np.float32)
        parts.append(acc)
    tot = np.zeros((M, N), np.float32)
    for i in order:
        tot = (tot + parts[i]).astype(np.float32)
    if fmt == FMT_BLOCK_FP8:
        return bf16_bits_from_f32(tot)
    t = (tot * np.asarray(s_a, np.float32)[:, None]).astype(np.float32)
    t = (t * np.asarray(s_w, np.float32)[None, :]).astype(np.float32)
    return bf16_bits_from_f32(t)
