"""Host-side logic of bench.py (CPU): the byte counts the roofline divides by,
the parsing of kernel names in profiler output, and the copy calibration of
the HBM counters."""

import math

import pytest
import torch

import bench
import quantized_gemm_decode_amd as ql
from workloads import config_by_name, decode_points

FMTS = [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8, ql.MXFP8, ql.MXFP4]


def _nbytes(shape, dtype):
    return math.prod(shape) * torch.empty((), dtype=dtype).element_size()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (32, 24576, 4096), (7, 300, 1280)])
def test_algorithmic_bytes_are_the_operand_buffers(fmt, M, N, K):
    """One GEMM reads W_q, s_w, A_q, s_a and writes bf16 Y: the sum of the
    buffer sizes the library's own shape helpers give for those operands."""
    want = (_nbytes(ql.weight_code_shape(fmt, N, K), ql.weight_code_dtype(fmt))
            + _nbytes(ql.weight_scale_shape(fmt, N, K), ql.scale_dtype(fmt))
            + _nbytes((M, K), ql.code_dtype(fmt))
            + _nbytes(ql.act_scale_shape(fmt, M, K), ql.scale_dtype(fmt))
            + _nbytes((M, N), torch.bfloat16))
    assert bench.algorithmic_bytes(fmt, M, N, K) == want
    # the quantizer reads bf16 X and writes the codes and scales
    assert bench.quantizer_bytes(fmt, M, K) == (_nbytes((M, K), torch.bfloat16) + _nbytes((M, K), ql.code_dtype(fmt))
                                                + _nbytes(ql.act_scale_shape(fmt, M, K), ql.scale_dtype(fmt)))
    # a fused launch reads X on top of what the two-launch GEMM moves
    assert bench.fused_kernel_bytes(fmt, M, N, K) == want + 2 * M * K


def test_fused_instantiation_names():
    fused = "void qlk::qgemm_decode_kernel<0, false, 1, 1, 4, 2, 4, 2, false>(qlk::DecodeArgs)"
    plain = "void qlk::qgemm_decode_kernel<0, false, 1, 1, 4, 2, 2, 2, false>(qlk::DecodeArgs)"
    glu = "void qlk::qgemm_decode_kernel<2, true, 1, 2, 4, 1, 4, 2, true>(qlk::DecodeArgs)"
    assert bench.is_fused_instantiation(fused) and bench.is_fused_instantiation(glu)
    assert not bench.is_fused_instantiation(plain)
    assert not bench.is_fused_instantiation("void qlk::qgemm_tiled_kernel<0, 1, 64, 128, 2, 2, 1, 0>(qlk::DecodeArgs)")


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Value\n")
        for i, (name, v) in enumerate(rows):
            f.write('%d,"%s",%r\n' % (i + 1, name, v))


def test_pmc_summary_applies_the_copy_calibration(tmp_path, monkeypatch):
    """Synthetic counter files for the single-linear workload: three GEMM
    dispatches, then three 256 MiB copies.  FETCH_SIZE of a copy reads half
    its bytes, so every fetched KiB counts twice; WRITE_SIZE reads 1:1."""
    wl = config_by_name("int8_linear_4096x2048")
    (lab, N, K, M), = decode_points(wl)
    gemm = "void qlk::qgemm_decode_kernel<1, false, 1, 1, 4, 2, 2, 2, false>(qlk::DecodeArgs)"
    copy = "void copy_kernel(unsigned char const*, unsigned char*)"
    fetch = [(gemm, 4000.0), (gemm, 4100.0), (gemm, 4200.0)] + [(copy, 131072.0)] * 3
    write = [(gemm, 64.0)] * 3 + [(copy, 262144.0)] * 3
    _csv(tmp_path / "f.csv", fetch)
    _csv(tmp_path / "w.csv", write)
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 64)
    out = bench.pmc_summary([wl], "fused", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))[wl.name]
    kv = dict(l.split() for l in out.splitlines() if l and not l.startswith("#"))
    want = 4100.0 * 1024 * 2 + 64.0 * 1024
    assert int(kv["traffic_bytes_per_step"]) == round(want)
    assert int(kv["algorithmic_bytes_per_step"]) == bench.algorithmic_bytes(wl.fmt, M, N, K)
    assert kv["kernel_sources_sha256"] == "0" * 64


def test_default_workloads_are_the_fp8_int8_decode_sweeps():
    """The default run measures the single INT8 linear and the three M = 1..32
    sweeps (FP8_Dynamic 8B, Block_FP8 8B, W8A8_INT8 32B) together."""
    wls = bench.resolve_workloads(bench.parse_args([]).workload)
    assert [w.name for w in wls] == list(bench.DECODE_SET)
    assert [w.fmt for w in wls] == [ql.W8A8_INT8, ql.FP8_DYNAMIC, ql.BLOCK_FP8, ql.W8A8_INT8]
    assert sum(len(decode_points(w)) for w in wls) == 85
    assert all(max(w.ms) <= 32 for w in wls)


def test_pmc_summary_splits_dispatches_by_workload(tmp_path, monkeypatch):
    """Two workloads profiled in one pass: each gets its own record, from its
    own dispatches in order."""
    wls = [config_by_name("int8_linear_4096x2048"), config_by_name("int8_linear_4096x2048")]
    gemm = "void qlk::qgemm_decode_kernel<1, false, 1, 1, 4, 2, 2, 2, false>(qlk::DecodeArgs)"
    copy = "void copy_kernel(unsigned char const*, unsigned char*)"
    fetch = [(gemm, 1000.0)] * 3 + [(gemm, 3000.0)] * 3 + [(copy, 131072.0)] * 3
    write = [(gemm, 0.0)] * 6 + [(copy, 262144.0)] * 3
    _csv(tmp_path / "f.csv", fetch)
    _csv(tmp_path / "w.csv", write)
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 64)
    wls2 = [wls[0], type(wls[1])(**{**wls[1].__dict__, "name": "other"})]
    out = bench.pmc_summary(wls2, "fused", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    kv = {n: dict(l.split() for l in t.splitlines() if l and not l.startswith("#")) for n, t in out.items()}
    assert int(kv[wls2[0].name]["traffic_bytes_per_step"]) == 1000 * 1024 * 2
    assert int(kv["other"]["traffic_bytes_per_step"]) == 3000 * 1024 * 2
