"""GPU parity of the activation and weight quantizers: bit-exact codes and scales."""

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import dev_bf16, host_codes, pack_ref, requires_gpu
from workloads import make_inputs, bf16_bits

pytestmark = [pytest.mark.gpu, requires_gpu]
FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8]


def _bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check_act(fmt, xb):
    """Row-major and packed quantizer outputs against the oracle (the packed
    layout restated independently from its definition)."""
    q_ref, s_ref = oracle.quantize_act(fmt, xb)
    a_q, a_s = ql.quantize_act(fmt, dev_bf16(xb))
    a_p, a_ps = ql.quantize_act_packed(fmt, dev_bf16(xb))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(fmt, a_q), q_ref)
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), np.asarray(s_ref, np.float32).view(np.uint32))
    n = ql.qlinear_packed_act_bytes(*xb.shape)
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(np.asarray(q_ref).view(np.uint8)))
    assert np.array_equal(a_ps.cpu().numpy().view(np.uint32), np.asarray(s_ref, np.float32).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K", [(1, 2048), (5, 4096), (32, 25600), (8, 12288), (3, 128), (7, 1152),
                                 (2, 40960), (64, 5120)])
def test_act_quantizer_bit_exact(fmt, M, K):
    x, _ = make_inputs(K, 1, M, 0.02, seed=M + K, with_weight=False)
    _check_act(fmt, bf16_bits(x))


@pytest.mark.parametrize("fmt", [ql.FP8_DYNAMIC, ql.W8A8_INT8])
@pytest.mark.parametrize("K", [16, 48, 1040, 4112])
def test_act_quantizer_ragged_k(fmt, K):
    x, _ = make_inputs(K, 1, 3, 0.02, seed=K, with_weight=False)
    _check_act(fmt, bf16_bits(x))


@pytest.mark.parametrize("fmt", FMTS)
def test_act_quantizer_special_rows(fmt):
    K = 256
    x = np.zeros((8, K))
    x[1, :] = np.linspace(-3, 3, K)                  # ordinary
    x[2, 7] = -1e-38                                 # subnormal scale
    x[3, :] = 2.0 ** -130                            # bf16 subnormal inputs
    x[4, ::2] = -0.0                                 # negative zeros only -> zero row
    x[5, :] = 448.0 * np.sign(np.sin(np.arange(K))) # ties and max magnitudes
    x[5, 3] = 1e30
    x[6, :] = np.linspace(-1, 1, K) * 2.0 ** -88     # smallest scales of the reciprocal path
    x[7, :] = np.linspace(-1, 1, K) * 2.0 ** -92     # scales just below it: the division path
    _check_act(fmt, _bits(x))


@pytest.mark.parametrize("fmt", FMTS)
def test_act_quantizer_rounding_ties(fmt):
    """Inputs placed exactly on code midpoints after division by the scale."""
    K = 256
    Q = 127.0 if fmt == ql.W8A8_INT8 else 448.0
    rng = np.random.default_rng(3)
    x = np.zeros((4, K))
    x[:, 0] = Q                                      # amax = Q -> s = 1 exactly
    if fmt == ql.W8A8_INT8:
        x[:, 1:] = (rng.integers(-126, 126, (4, K - 1)) + 0.5)
    else:
        x[:, 1:] = rng.choice([1.0625, 1.1875, 3.25 * 2 ** -9, 2 ** -10, 464.0 - 16, 2.0 ** -9 * 1.5], (4, K - 1))
    _check_act(fmt, _bits(x))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(300, 256), (4096, 2048), (128, 1024), (1000, 4096)])
def test_weight_quantizer_bit_exact(fmt, N, K):
    _, w = make_inputs(K, N, 1, 0.02, seed=N + K)
    wb = bf16_bits(w)
    q_ref, s_ref = oracle.quantize_weight(fmt, wb)
    w_q, w_s = ql.quantize_weight(fmt, dev_bf16(wb))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(fmt, w_q), q_ref)
    assert np.array_equal(w_s.cpu().numpy().view(np.uint32), np.asarray(s_ref, np.float32).view(np.uint32))


@pytest.mark.parametrize("fmt,N,K,sigma", [(ql.W8A8_INT8, 51200, 5120, 0.015), (ql.FP8_DYNAMIC, 24576, 4096, 0.02),
                                           (ql.BLOCK_FP8, 24576, 4096, 0.02), (ql.W8A8_INT8, 5120, 25600, 0.015)])
def test_weight_quantizer_full_size_sampled_rows(fmt, N, K, sigma):
    """Full-size weights quantized on the GPU; sampled rows (or 128-row blocks) checked by the oracle."""
    _, w = make_inputs(K, N, 1, sigma, seed=0)
    w_q, w_s = ql.quantize_weight(fmt, w.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    if fmt == ql.BLOCK_FP8:
        for nb in rng.choice(N // 128, 4, replace=False):
            rows = slice(nb * 128, nb * 128 + 128)
            q_ref, s_ref = oracle.quantize_weight(fmt, bf16_bits(w[rows]))
            assert np.array_equal(host_codes(fmt, w_q[rows]), q_ref)
            assert np.array_equal(w_s[nb].cpu().numpy(), s_ref[0])
    else:
        idx = np.sort(rng.choice(N, 64, replace=False))
        q_ref, s_ref = oracle.quantize_weight(fmt, bf16_bits(w[torch.from_numpy(idx)]))
        assert np.array_equal(host_codes(fmt, w_q[torch.from_numpy(idx).cuda()]), q_ref)
        assert np.array_equal(w_s[torch.from_numpy(idx).cuda()].cpu().numpy(), s_ref)


def test_quantizer_empty_inputs_are_no_ops():
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    a_q, a_s = ql.quantize_act(ql.W8A8_INT8, x)
    assert a_q.shape == (0, 256)


@pytest.mark.parametrize("fmt", FMTS)
def test_non_finite_rows_leave_the_other_rows_exact(fmt):
    """A row holding +inf, -inf and NaN is outside the quantizer's contract;
    every other row's codes and scales stay bit-exact, and the packed layout
    still holds the row-major codes of every row."""
    M, K = 6, 512
    x, _ = make_inputs(K, 1, M, 0.02, seed=77, with_weight=False)
    xb = np.array(bf16_bits(x), dtype=np.uint16)
    bad = 2
    xb[bad, 5], xb[bad, 300], xb[bad, 301] = 0x7F80, 0xFF80, 0x7FC0
    good = [m for m in range(M) if m != bad]
    q_ref, s_ref = oracle.quantize_act(fmt, xb[good])
    a_q, a_s = ql.quantize_act(fmt, dev_bf16(xb))
    a_p, a_ps = ql.quantize_act_packed(fmt, dev_bf16(xb))
    torch.cuda.synchronize()
    q = host_codes(fmt, a_q)
    assert np.array_equal(q[good], q_ref)
    s_bits = a_s.cpu().numpy().view(np.uint32)
    assert np.array_equal(s_bits[good], np.asarray(s_ref, np.float32).view(np.uint32))
    n = ql.qlinear_packed_act_bytes(M, K)
    assert np.array_equal(a_p[:n].view(torch.uint8).cpu().numpy(), pack_ref(np.asarray(q).view(np.uint8)))
    assert np.array_equal(a_ps.cpu().numpy().view(np.uint32)[good], s_bits[good])


def _e4m3_probe_inputs():
    """Every bf16 value; every binary32 within 64 ulp of each E4M3 value and of
    each midpoint between neighbouring values (both signs); values beyond the
    clamp; binary32 subnormals; random bit patterns."""
    v = oracle.e4m3_decode(np.arange(128, dtype=np.uint8))
    v = np.sort(v[np.isfinite(v)]).astype(np.float64)            # 0 .. 448, 127 values
    pts = np.concatenate([v, (v[1:] + v[:-1]) / 2]).astype(np.float32)
    b = pts.view(np.int32)[:, None] + np.arange(-64, 65, dtype=np.int32)[None, :]
    near = b[b >= 0].view(np.float32)
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    rng = np.random.default_rng(11)
    rnd = rng.integers(0, 2 ** 32, 4 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    extra = np.array([448.0, 448.5, 464.0, 464.5, 480.0, 1e30, np.inf, 1e-40, 1.4e-45, 0.0], np.float32)
    x = np.concatenate([near, -near, allbf, rnd, extra, -extra])
    return np.ascontiguousarray(x, np.float32)


def test_e4m3_encoder_matches_the_format_definition():
    """The conversion instruction the FP8 quantizers use, against the oracle's
    encoder (written from the OCP E4M3 definition) on the clamped inputs."""
    x = _e4m3_probe_inputs()
    xd = torch.from_numpy(x).cuda()
    codes = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    ql.qlinear_encode_e4m3(xd, codes)
    torch.cuda.synchronize()
    ref = oracle.e4m3_encode(np.clip(x, -448.0, 448.0))
    got = codes.cpu().numpy()
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(x[i]), hex(x[i:i + 1].view(np.uint32)[0]), int(got[i]), int(ref[i]))
                           for i in bad[:8]]
