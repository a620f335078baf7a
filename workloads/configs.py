"""The decode workloads: formats, GEMM shapes and token counts.

Token buckets {1, 2, 4, 8, 16, 24, 32} follow the Summary, "Hybrid dispatch
addresses runtime overhead" (token counts tuned separately up to the graph
threshold of 32).  The shapes are the QKV / O / gate_up / down projections of
dense 8B-class (hidden 4096, intermediate 12288) and 32B-class (hidden 5120,
intermediate 25600) models, plus a 14B-class set beyond the threshold.
"""

from dataclasses import dataclass

FP8_DYNAMIC, W8A8_INT8, BLOCK_FP8, MXFP8, MXFP4 = 0, 1, 2, 3, 4
FMT_NAMES = {FP8_DYNAMIC: "FP8_Dynamic", W8A8_INT8: "W8A8_INT8", BLOCK_FP8: "Block_FP8", MXFP8: "MXFP8",
             MXFP4: "MXFP4"}
DECODE_M = (1, 2, 4, 8, 16, 24, 32)


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: int
    shapes: tuple            # ((label, N, K), ...)
    ms: tuple                # token counts
    sigma_w: float = 0.02
    seed: int = 0
    notes: str = ""


CONFIGS = (
    Workload("int8_linear_4096x2048", W8A8_INT8, (("lin", 4096, 2048),), (8,),
             notes="single linear, bit-exact correctness anchor"),
    Workload("fp8_dynamic_8b", FP8_DYNAMIC,
             (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)),
             DECODE_M),
    Workload("block_fp8_8b", BLOCK_FP8,
             (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)),
             DECODE_M),
    Workload("int8_32b", W8A8_INT8,
             (("qkv", 10240, 5120), ("o", 5120, 8192), ("gate_up", 51200, 5120), ("down", 5120, 25600)),
             DECODE_M, sigma_w=0.015),
    Workload("mxfp8_8b", MXFP8,
             (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)),
             DECODE_M, notes="MX block-scaled E4M3 on the 8B shapes"),
    Workload("mxfp4_8b", MXFP4,
             (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)),
             DECODE_M, notes="MXFP4 weights, MXFP8 activations, on the 8B shapes"),
    Workload("fp8_dynamic_14b_large_m", FP8_DYNAMIC,
             (("qkv", 7168, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)),
             (64, 256, 1024, 4096)),
    Workload("mxfp8_14b_large_m", MXFP8,
             (("qkv", 7168, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)),
             (64, 256, 1024, 4096), notes="MXFP8 beyond the decode range (tiled kernel from M = 65)"),
    Workload("mxfp4_14b_large_m", MXFP4,
             (("qkv", 7168, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)),
             (64, 256, 1024, 4096), notes="MXFP4 weights beyond the decode range (tiled kernel from M = 65)"),
)


def decode_workloads(include_mx=False):
    """The workloads whose token counts stay within the decode range (M <= 32);
    the MXFP8 one only on request (its plans take packed operands only)."""
    return [c for c in CONFIGS if max(c.ms) <= 32 and (include_mx or c.fmt not in (MXFP8, MXFP4))]


def config_by_name(name):
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def decode_points(cfg):
    """All (label, N, K, M) points of a workload, in sweep order."""
    return [(lab, N, K, M) for (lab, N, K) in cfg.shapes for M in cfg.ms]
