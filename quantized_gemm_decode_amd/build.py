"""Build libqlinear.so (the HIP kernels + C ABI) in-tree for gfx950.

Every translation unit is compiled with hipcc in parallel, then linked into
``quantized_gemm_decode_amd/libqlinear.so``.  Run ``python -m
quantized_gemm_decode_amd.build`` (or ``__graft_entry__.build()``).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlinear.so")

SOURCES = ["quant.hip", "decode_fp8.hip", "decode_int8.hip", "decode_block.hip", "decode_mx.hip", "decode_mx4.hip", "tiled_fp8.hip",
           "tiled_int8.hip", "tiled_block.hip", "tiled_mx.hip", "tiled_mx4.hip", "stream_read.hip", "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: hipcc must not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE division and fp32 subnormals are part of the quantizer's contract
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # the decode kernel's first 9 arguments (14 words) are preloaded into SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=9",
    "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _scratch_users(remarks):
    """Kernels whose register allocation spilled to scratch, from the resource remarks."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if n > 0:
                bad.append((name, n))
    return bad


def _compile(src):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    else:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    spills = _scratch_users(r.stderr)
    if spills:
        raise RuntimeError("%s: kernels spill registers to scratch (not allowed on the hot path): %s"
                           % (src, spills[:4]))
    return out


def build(verbose=False, jobs=None):
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
