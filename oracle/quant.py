"""Symmetric absmax quantizers of the three formats (test infrastructure only).

Formats and scale granularity -- Summary, "Put algorithm selection inside the
search space" (last paragraph) and Noticias, "El backend lineal de Helion /
Alcance":
  * FP8_Dynamic: FP8 activations scaled per token, weights per output channel.
  * W8A8_INT8:   INT8 activations per token, weights per output channel.
  * Block_FP8:   FP8 with 1x128 activation groups and 128x128 weight blocks.

Readings (the pages give no formula):
  * symmetric absmax scaling, no zero point: s = fl(amax / Q) with Q = 127
    (INT8) or 448 (largest finite E4M3);
  * each code is computed by IEEE binary32 division fl(x / s) -- a division,
    not a multiply by a reciprocal -- then rounded half-to-even: INT8 clamps to
    [-127, 127]; FP8 clamps to [-448, 448] before the E4M3 rounding;
  * an all-zero row / group / block gets s = 1 and all-zero codes;
  * binary32 subnormal scales are kept (no flush to zero).
Inputs are bf16 (given as uint16 bit patterns); widening to binary32 is exact,
so amax is exact.
"""

import numpy as np

from .fpbits import bf16_bits_to_f32
from .e4m3 import e4m3_encode, e4m3_decode, E4M3_MAX

FMT_FP8_DYNAMIC = 0
FMT_W8A8_INT8 = 1
FMT_BLOCK_FP8 = 2
FORMATS = (FMT_FP8_DYNAMIC, FMT_W8A8_INT8, FMT_BLOCK_FP8)
GROUP = 128


def qmax_of(fmt):
    """Largest code magnitude Q of the format (127 for INT8, 448 for E4M3)."""
    return 127.0 if fmt == FMT_W8A8_INT8 else E4M3_MAX


def _quantize_groups(x, fmt):
    """Quantize every row of the 2-D binary32 array ``x`` as one scaling group.

    Returns (codes [R, C], scales float32 [R]).  Codes are int8 for INT8 and
    E4M3 bytes (uint8) for the FP8 formats.
    """
    x = np.asarray(x, dtype=np.float32)
    Q = np.float32(qmax_of(fmt))
    amax = np.max(np.abs(x), axis=1) if x.shape[1] > 0 else np.zeros(x.shape[0], np.float32)
    s = (amax.astype(np.float32) / Q).astype(np.float32)       # one binary32 division
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    t = (x / s[:, None]).astype(np.float32)                      # one binary32 division per element
    if fmt == FMT_W8A8_INT8:
        q = np.clip(np.rint(t), -127, 127).astype(np.int8)
    else:
        q = e4m3_encode(np.clip(t, -E4M3_MAX, E4M3_MAX))
    return q, s


def quantize_act(fmt, x_bits):
    """Dynamic activation quantizer.

    x_bits: uint16 [M, K] bf16 bit patterns.
    Returns (A_q [M, K], s_a): s_a is float32 [M] (per token) or [M, K/128]
    (Block_FP8, one scale per 1x128 group along K, row-major).
    """
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    if fmt == FMT_BLOCK_FP8:
        if K % GROUP:
            raise ValueError("Block_FP8 needs K % 128 == 0")
        G = K // GROUP
        q, s = _quantize_groups(x.reshape(M * G, GROUP), fmt)
        return q.reshape(M, K), s.reshape(M, G)
    return _quantize_groups(x, fmt)


def quantize_weight(fmt, w_bits):
    """Offline weight quantizer.

    w_bits: uint16 [N, K] bf16 bit patterns (row n = output channel n).
    Returns (W_q [N, K], s_w): s_w is float32 [N] (per output channel) or
    [ceil(N/128), K/128] for Block_FP8 (one scale per 128x128 block; the last
    block row may hold fewer than 128 channels).
    """
    w = bf16_bits_to_f32(w_bits)
    N, K = w.shape
    if fmt != FMT_BLOCK_FP8:
        return _quantize_groups(w, fmt)
    if K % GROUP:
        raise ValueError("Block_FP8 needs K % 128 == 0")
    NB, G = -(-N // GROUP), K // GROUP
    q = np.zeros((N, K), dtype=np.uint8)
    s = np.zeros((NB, G), dtype=np.float32)
    for nb in range(NB):
        r0, r1 = nb * GROUP, min(N, (nb + 1) * GROUP)
        for g in range(G):
            blk = w[r0:r1, g * GROUP:(g + 1) * GROUP]
            qb, sb = _quantize_groups(blk.reshape(1, -1), fmt)
            q[r0:r1, g * GROUP:(g + 1) * GROUP] = qb.reshape(blk.shape)
            s[nb, g] = sb[0]
    return q, s


def dequant_codes(fmt, q):
    """Real values of the codes as float64 (E4M3 decode, or the int8 value)."""
    if fmt == FMT_W8A8_INT8:
        return np.asarray(q, dtype=np.int8).astype(np.float64)
    return e4m3_decode(q)
