"""The C ABI from a plain C99 program (tests/native/abi_consumer.c), with no
Python or torch between the caller and the library: the header compiles as
C99 with warnings as errors, the host-side calls behave as documented, and
one linear run through the ABI from C (eager and as graph replays) matches
the oracle -- bit-exact for INT8 on the single-linear workload."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import quantized_gemm_decode_amd as ql
from tests.gpu_util import fp8_check, fp8_ok, requires_gpu
from workloads import bf16_bits, config_by_name, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "quantized_gemm_decode_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "abi_consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           os.path.join(HERE, "native", "abi_consumer.c"), "-o", exe,
           "-L" + PKG, "-lqlinear", "-Wl,-rpath," + PKG,
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_consumer_host_calls(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "host", ql.DEFAULT_TABLE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "host ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.gpu
@requires_gpu
@pytest.mark.parametrize("wname,fmt,M,N,K", [("int8_linear_4096x2048", ql.W8A8_INT8, 8, 4096, 2048),
                                             (None, ql.FP8_DYNAMIC, 5, 1536, 4096),
                                             (None, ql.BLOCK_FP8, 3, 640, 1024)])
def test_c_consumer_runs_one_linear(tmp_path, wname, fmt, M, N, K):
    exe = _build(tmp_path)
    sigma = config_by_name(wname).sigma_w if wname else 0.02
    x, w = make_inputs(K, N, M, sigma, seed=config_by_name(wname).seed if wname else 3)
    xb, wb = bf16_bits(x), bf16_bits(w)
    src, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([fmt, M, N, K], np.int64).tobytes())
        f.write(np.ascontiguousarray(xb, np.uint16).tobytes())
        f.write(np.ascontiguousarray(wb, np.uint16).tobytes())
    r = subprocess.run([exe, "gpu", str(src), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "gpu ok" in r.stdout, r.stdout + r.stderr
    y = np.fromfile(out, dtype=np.uint16).reshape(M, N)
    ref = oracle.reference(fmt, xb, wb)
    if fmt == ql.W8A8_INT8:
        assert np.array_equal(y, ref["y_ref"])
    else:
        # the program plans without a table, as this process does after clearing its own
        ql.qlinear_table_clear()
        try:
            chunks = ql.qlinear_plan(fmt, M, N, K).facts["chunks"]
        finally:
            ql.load_default_table()
        assert fp8_ok(fp8_check(fmt, ref, y, chunks))
