"""The Python binding's operand size checks (CPU): the least bytes each
operand of a run must hold follow from the plan (operand layouts, format,
SiLU-and-mul output, workspace), and a smaller tensor is refused before any
pointer reaches the library."""

import pytest
import torch

import quantized_gemm_decode_amd as ql


def _bytes(t):
    return t.numel() * t.element_size()


@pytest.mark.parametrize("fmt", [ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8])
@pytest.mark.parametrize("layout", [(0, 0), (1, 0), (1, 1)])
def test_operand_bytes_follow_the_plan(fmt, layout):
    M, N, K = 24, 640, 2048
    plan = ql.qlinear_plan_layouts(fmt, M, N, K, *layout)
    need = plan.operand_bytes()
    packed_a = plan.config["a_mode"] >= 2
    assert need["a_q"] == (ql.qlinear_packed_act_bytes(M, K) if packed_a else M * K)
    assert need["w_q"] == (ql.qlinear_packed_weight_bytes(N, K) if layout[0] else N * K)
    assert need["a_scale"] == 4 * (M * K // 128 if fmt == ql.BLOCK_FP8 else M)
    assert need["w_scale"] == 4 * ((-(-N // 128)) * (K // 128) if fmt == ql.BLOCK_FP8 else N)
    assert need["y"] == 2 * M * N and need["x"] == 2 * M * K
    assert need["workspace"] == plan.workspace_bytes


def test_mx_and_glu_operand_bytes():
    M, N, K = 8, 512, 1024
    p = ql.qlinear_plan_layouts(ql.MXFP4, M, N, K, 1, 1)
    need = p.operand_bytes()
    assert need["w_q"] == ql.qlinear_packed_weight_bytes_fp4(N, K)
    assert need["w_scale"] == ql.qlinear_packed_mx_scale_bytes(N, K)
    assert need["a_scale"] == ql.qlinear_packed_mx_scale_bytes(M, K)
    g = ql.qlinear_plan_glu(ql.FP8_DYNAMIC, M, N, K, 1)
    assert g.operand_bytes()["y"] == 2 * M * (N // 2)
    z = ql.qlinear_plan_glu(ql.FP8_DYNAMIC, M, N, 0, 1)     # K = 0: only Y is written
    assert z.operand_bytes() == dict(z.operand_bytes(), y=2 * M * (N // 2), a_q=0, w_q=0, a_scale=0, w_scale=0)


def test_short_operands_are_refused():
    M, N, K = 8, 256, 512
    plan = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, M, N, K, 1, 1)
    need = plan.operand_bytes()
    ok = {k: torch.empty(max(v, 1), dtype=torch.uint8) for k, v in need.items()}
    plan.check_operands(**ok)
    for name in ("a_q", "a_scale", "w_q", "w_scale", "y"):
        short = dict(ok, **{name: torch.empty(need[name] - 1, dtype=torch.uint8)})
        with pytest.raises(ValueError, match=name):
            plan.check_operands(**short)
    assert _bytes(ok["y"]) == 2 * M * N


def test_quantizer_and_packer_outputs_are_checked():
    """Outputs sized from the input's shape: one byte short is refused before
    any pointer is formed (CPU tensors suffice for the size check)."""
    M, K, N = 5, 256, 40
    x = torch.empty(M, K, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="a_q"):
        ql.qlinear_quantize_act(ql.FP8_DYNAMIC, x, torch.empty(M * K - 1, dtype=torch.uint8),
                                torch.empty(M, dtype=torch.float32))
    with pytest.raises(ValueError, match="a_scale"):
        ql.qlinear_quantize_act(ql.BLOCK_FP8, x, torch.empty(M * K, dtype=torch.uint8),
                                torch.empty(M, dtype=torch.float32))
    with pytest.raises(ValueError, match="a_packed"):
        ql.qlinear_quantize_act_packed(ql.W8A8_INT8, x, torch.empty(M * K, dtype=torch.uint8),
                                       torch.empty(M, dtype=torch.float32))
    w = torch.empty(N, K, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="w_scale"):
        ql.qlinear_quantize_weight(ql.MXFP8, w, torch.empty(N, K, dtype=torch.uint8),
                                   torch.empty(N * K // 32 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="w_packed"):
        ql.qlinear_pack_weight(torch.empty(N, K, dtype=torch.int8), torch.empty(N * K, dtype=torch.int8))
    with pytest.raises(ValueError, match="packed"):
        ql.qlinear_pack_mx_scales(torch.empty(N, K // 32, dtype=torch.uint8), K, torch.empty(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="codes"):
        ql.qlinear_encode_e4m3(torch.empty(100), torch.empty(99, dtype=torch.uint8))
