"""Helpers shared by the GPU parity tests: moving oracle data to the device and back."""

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> device bf16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_codes(fmt, q):
    """Oracle codes -> device tensor (int8, or float8_e4m3fn from the raw bytes)."""
    if fmt == oracle.FMT_W8A8_INT8:
        return torch.from_numpy(np.ascontiguousarray(q).astype(np.int8)).cuda()
    return torch.from_numpy(np.ascontiguousarray(q).astype(np.uint8)).cuda().view(torch.float8_e4m3fn)


def host_codes(fmt, t):
    """Device codes -> numpy array in the oracle's convention (int8 / uint8 bytes)."""
    if fmt == oracle.FMT_W8A8_INT8:
        return t.cpu().numpy().astype(np.int8)
    return t.view(torch.uint8).cpu().numpy()


def host_bf16_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_gemm(plan, a_q, s_a, w_q, s_w, acc=True):
    """Run a plan once; returns (y_bits, acc numpy or None, workspace tensor or None)."""
    M, N = plan.M, plan.N
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    y.fill_(float("nan"))
    ws = plan.new_workspace()
    if acc:
        a = torch.empty(M, N, dtype=torch.int32 if plan.fmt == ql.W8A8_INT8 else torch.float32, device="cuda")
        ql.qlinear_run_debug_acc(plan, a_q, s_a, w_q, s_w, y, a, ws)
    else:
        ql.qlinear_run(plan, a_q, s_a, w_q, s_w, y, ws)
    torch.cuda.synchronize()
    return host_bf16_bits(y), (a.cpu().numpy() if acc else None), ws


# Lowest fraction of outputs within 1 bf16 ulp of y_ref that an FP8 parity
# check may show (the other outputs must meet the oracle's bound clause).
# Measured on MI355X over every GPU parity check: lowest 0.9844 (one element
# of a 64-element sample), 0.9978 of all 30.9 M checked elements -- the
# matrix core cuts small products (oracle/matrix_core.py), so a few outputs
# land a bf16 ulp away.
MIN_FRAC_WITHIN_ULP = 0.98


def fp8_ok(st):
    """The acceptance rule held, and enough outputs lie within 1 ulp."""
    return st["ok"] and st["frac_within_ulp"] >= MIN_FRAC_WITHIN_ULP


def fp8_check(fmt, r, y_bits, split, waves_k=16):
    """Apply the oracle's FP8 acceptance rule to a GPU result (``waves_k``: the
    partial sums a workgroup reduces, at most 16 in any plan)."""
    K = r["a_q"].shape[1]
    d = oracle.summation_depth(K, split=split, waves_k=waves_k)
    B = oracle.Fp8Bound(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], d)
    return oracle.check_fp8_parity(y_bits, r["y_ref"], r["y_true"], B)


def pack_ref(q):
    """The packed tile layout (weights and activations alike), restated from its definition:
    tile (t, kb) holds rows 16t.., K bytes 128kb..; tile byte h*1024 + l*16 + j =
    Q[16t + l%16][128kb + 64h + 16(l//16) + j], zero padded."""
    q = np.ascontiguousarray(q).view(np.uint8)
    N, K = q.shape
    NT, G = -(-N // 16), -(-K // 128)
    pad = np.zeros((NT * 16, G * 128), np.uint8)
    pad[:N, :K] = q
    arr = pad.reshape(NT, 16, G, 128)
    out = np.zeros((NT, G, 2, 64, 16), np.uint8)
    for h in range(2):
        for g in range(4):
            out[:, :, h, 16 * g:16 * g + 16, :] = arr[:, :, :, 64 * h + 16 * g:64 * h + 16 * g + 16].transpose(0, 2, 1, 3)
    return out.reshape(-1)


def pack_mx_scales_ref(s, K):
    """The lane-order MXFP8 scale layout, restated from its definition: the 64
    bytes of (16-row group t, K block kb) at (t*G + kb)*64, byte l =
    S[16t + l%16][4kb + l//16], zero past the last row."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    R = s.shape[0]
    T, G = -(-R // 16), K // 128
    out = np.zeros((T, G, 64), np.uint8)
    for t in range(T):
        for kb in range(G):
            for l in range(64):
                row = 16 * t + l % 16
                if row < R:
                    out[t, kb, l] = s[row, 4 * kb + l // 16]
    return out.reshape(-1)


def fp4_bytes(codes):
    """E2M1 codes [N, K] (one a byte) -> row-major pairs [N, K/2], low nibble = even K."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def pack_fp4_ref(codes):
    """The packed MXFP4 weight layout, restated from its definition: 1 KB per
    (16-row group t, K block kb) at (t*G + kb)*1024; lane l's 16 bytes hold row
    16t + l%16, K [128kb + 32(l//16), +32) as pairs; zero past the last row."""
    b = fp4_bytes(codes)
    N, K = b.shape[0], b.shape[1] * 2
    T, G = -(-N // 16), K // 128
    out = np.zeros((T, G, 64, 16), np.uint8)
    for t in range(T):
        for kb in range(G):
            for l in range(64):
                row = 16 * t + l % 16
                if row < N:
                    out[t, kb, l] = b[row, 64 * kb + 16 * (l // 16):64 * kb + 16 * (l // 16) + 16]
    return out.reshape(-1)


def amax_words(x_bits):
    """max |x| per row of bf16 bit patterns, as binary32 bit patterns."""
    return ((np.asarray(x_bits).astype(np.uint32) & 0x7FFF) << 16).max(axis=1).astype(np.uint32)


def filled_amax_buffer(maxima, seed=0):
    """An amax buffer holding the given per-token maxima the way producer
    waves leave it: each token's maximum in one random replica, the other
    replicas holding smaller (or zero) non-negative values."""
    rng = np.random.default_rng(seed)
    buf = ql.amax_buffer()
    words = np.zeros(buf.numel(), np.uint32)
    rep = words[:ql.AMAX_REPLICAS * ql.AMAX_LINE].reshape(ql.AMAX_REPLICAS, ql.AMAX_LINE)
    for m, v in enumerate(np.asarray(maxima, np.uint32)):
        below = rng.integers(0, int(v) + 1, ql.AMAX_REPLICAS, dtype=np.uint64).astype(np.uint32)
        below[rng.random(ql.AMAX_REPLICAS) < 0.5] = 0
        rep[:, m] = below
        rep[rng.integers(ql.AMAX_REPLICAS), m] = v
    buf.copy_(torch.from_numpy(words.view(np.int32)))
    return buf
