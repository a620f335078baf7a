"""Host-side tests of the C ABI (CPU only: no kernel is launched here).

The library must load, export every function that include/qlinear.h
declares, and reject bad arguments on the host with the documented status
codes before touching the GPU.  Planning is host-only, so plans, the sweep
table and the QLINEAR_FORCE override are testable here too.
"""

import ctypes
import os
import re

import pytest
import torch

import quantized_gemm_decode_amd as ql
from quantized_gemm_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")

QL_OK, QL_E_INVALID, QL_E_UNSUPPORTED, QL_E_NO_TABLE_ENTRY, QL_E_HIP, QL_E_ALIGN, QL_E_TABLE = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:ql_status|int32_t|int64_t|void|const char\s*\*)\s*(qlinear_\w+)\s*\(", text, re.M))


def test_header_and_binding_agree():
    declared = _declared_functions()
    assert len(declared) >= 20
    assert declared == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = ql.lib()
    assert lib.qlinear_version() >= 100
    names = [lib.qlinear_status_string(i).decode() for i in range(7)]
    assert names == ["QL_OK", "QL_E_INVALID", "QL_E_UNSUPPORTED", "QL_E_NO_TABLE_ENTRY", "QL_E_HIP",
                     "QL_E_ALIGN", "QL_E_TABLE"]
    assert lib.qlinear_status_string(99).decode() == "QL_E_UNKNOWN"


def _plan_status(fmt, M, N, K, **cfg):
    h = ctypes.c_void_p()
    if cfg:
        c = ql.QLConfig(**ql.make_config(**cfg))
        st = ql.lib().qlinear_plan_with_config(fmt, M, N, K, ctypes.byref(c), ctypes.byref(h))
    else:
        st = ql.lib().qlinear_plan(fmt, M, N, K, ctypes.byref(h))
    if h.value:
        ql.lib().qlinear_plan_destroy(h)
    return st


def test_host_validation_status_codes():
    assert _plan_status(ql.W8A8_INT8, 8, 4096, 2048) == QL_OK
    assert _plan_status(7, 8, 4096, 2048) == QL_E_INVALID                 # unknown format
    assert _plan_status(ql.W8A8_INT8, 8, 4096, 2056) == QL_E_INVALID      # K % 16
    assert _plan_status(ql.BLOCK_FP8, 8, 4096, 2064) == QL_E_INVALID      # Block needs K % 128
    assert _plan_status(ql.FP8_DYNAMIC, -1, 4096, 2048) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 2 ** 20, 2048) == QL_E_UNSUPPORTED   # N*K > 2^30
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, split_k=3) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, split_k=512) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, waves_n=3, waves_k=1) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, rows_per_wave=48) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, prefetch=3) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, swap_ab=2) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, w_lds=2) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, w_layout=2) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, w_layout=1, w_lds=1) == QL_E_INVALID
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 2048, w_layout=1) == QL_OK
    # configurations that would spill registers are not instantiated
    assert _plan_status(ql.FP8_DYNAMIC, 32, 4096, 2048, rows_per_wave=32, prefetch=4) == QL_E_UNSUPPORTED
    # the LDS-staged activation chunk must fit the 64 KB budget
    assert _plan_status(ql.FP8_DYNAMIC, 32, 4096, 25600, split_k=1, a_mode=1) == QL_E_UNSUPPORTED
    assert _plan_status(ql.FP8_DYNAMIC, 32, 4096, 25600, split_k=1, a_mode=0) == QL_OK
    assert "LDS" in ql.lib().qlinear_last_error().decode() or True
    # a decode K chunk must hold fewer than 2^14 blocks of 128 (the kernel's packed launch word)
    assert _plan_status(ql.FP8_DYNAMIC, 1, 16, 2 ** 21, split_k=1, a_mode=0) == QL_E_UNSUPPORTED
    assert "2^14" in ql.lib().qlinear_last_error().decode()
    assert _plan_status(ql.FP8_DYNAMIC, 1, 16, 2 ** 21, split_k=2, a_mode=0) == QL_OK
    assert _plan_status(ql.FP8_DYNAMIC, 1, 16, 2 ** 21 - 128, split_k=1, a_mode=0) == QL_OK


def test_decode_row_tile_validation():
    """tile_n of a decode plan: a multiple of 8 in [8, 120] within the waves' rows, FP8_Dynamic /
    W8A8_INT8 / Block_FP8 with weights read directly; the workgroup count follows the tile."""
    packed = dict(waves_n=1, waves_k=4, rows_per_wave=32, w_layout=1, a_mode=2)
    assert _plan_status(ql.FP8_DYNAMIC, 8, 6144, 4096, tile_n=24, **packed) == QL_OK
    assert _plan_status(ql.W8A8_INT8, 8, 6144, 4096, tile_n=8, **packed) == QL_OK
    assert _plan_status(ql.FP8_DYNAMIC, 8, 6144, 4096, tile_n=12, **packed) == QL_E_INVALID    # not a multiple of 8
    assert _plan_status(ql.FP8_DYNAMIC, 8, 6144, 4096, tile_n=40, **packed) == QL_E_INVALID    # beyond 32 rows
    assert _plan_status(ql.FP8_DYNAMIC, 8, 6144, 4096, tile_n=128, waves_n=4, waves_k=1, rows_per_wave=32,
                        w_layout=1, a_mode=2) == QL_E_INVALID                                  # beyond 120
    assert _plan_status(ql.BLOCK_FP8, 8, 6144, 4096, tile_n=24, **packed) == QL_OK
    assert _plan_status(ql.MXFP8, 8, 6144, 4096, tile_n=24, **packed) == QL_E_UNSUPPORTED
    assert _plan_status(ql.FP8_DYNAMIC, 8, 6144, 4096, tile_n=24, waves_n=1, waves_k=4, rows_per_wave=32,
                        w_lds=1) == QL_E_UNSUPPORTED                                           # LDS transpose
    p = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 8, 6144, 4096, dict(tile_n=24, **packed))
    assert p.facts["workgroups"] == 256 and p.config["tile_n"] == 24
    p = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 8, 1000, 4096, dict(tile_n=24, split_k=2, **packed))
    assert p.facts["workgroups"] == 42 * 2


def test_quantizer_rejects_bad_arguments_on_host():
    lib = ql.lib()
    null = ctypes.c_void_p(0)
    assert lib.qlinear_quantize_act(ql.W8A8_INT8, null, 4, 100, null, null, null) == QL_E_INVALID  # K % 16
    assert lib.qlinear_quantize_act(ql.W8A8_INT8, null, 4, 128, null, null, null) == QL_E_INVALID  # NULL
    assert lib.qlinear_quantize_act(ql.W8A8_INT8, ctypes.c_void_p(8), 4, 128, ctypes.c_void_p(16),
                                    ctypes.c_void_p(16), null) == QL_E_ALIGN
    assert lib.qlinear_quantize_act(ql.W8A8_INT8, null, 0, 128, null, null, null) == QL_OK        # empty
    assert lib.qlinear_quantize_weight(ql.BLOCK_FP8, null, 4, 192, null, null, null) == QL_E_INVALID


def test_run_rejects_bad_arguments_on_host():
    p = ql.qlinear_plan_with_config(ql.W8A8_INT8, 8, 4096, 2048, dict(split_k=4))
    lib = ql.lib()
    v = ctypes.c_void_p
    good = v(1 << 20)
    assert lib.qlinear_run(p.handle, good, good, good, good, good, v(0), v(0)) == QL_E_INVALID   # no workspace
    assert lib.qlinear_run(p.handle, v(0), good, good, good, good, good, v(0)) == QL_E_INVALID
    assert lib.qlinear_run(p.handle, v(3), good, good, good, good, good, v(0)) == QL_E_ALIGN
    assert lib.qlinear_run(v(0), good, good, good, good, good, good, v(0)) == QL_E_INVALID
    assert lib.qlinear_run_debug_acc(p.handle, good, good, good, good, good, good, v(0), v(0)) == QL_E_INVALID
    assert lib.qlinear_graph_begin(v(0)) == QL_E_INVALID      # default stream cannot be captured


def test_plan_facts_and_workspace_sizes():
    p = ql.qlinear_plan_with_config(ql.W8A8_INT8, 8, 4096, 2048,
                                    dict(split_k=4, waves_n=2, waves_k=2, rows_per_wave=32))
    cfg, facts = p.info()
    assert facts["source"] == "custom"
    assert facts["chunks"] == 4 and facts["chunk_k"] == 512
    assert facts["workgroups"] == (4096 // 64) * 4 and facts["threads"] == 256
    assert p.workspace_bytes == 8 * 4096 * 4 + (4096 // 64) * 4
    assert ql.qlinear_plan_with_config(ql.W8A8_INT8, 8, 4096, 2048, dict(split_k=1)).workspace_bytes == 0
    # split clamps to the number of 128-wide K blocks and to balanced chunks
    q = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 4, 512, 640, dict(split_k=256, a_mode=0))
    assert q.config["split_k"] == 5 and q.facts["chunk_k"] == 128
    r = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 4, 512, 5120, dict(split_k=16))
    assert r.facts["chunks"] == 14 and r.facts["chunk_k"] == 384        # ceil(40/16)=3 blocks per chunk


def test_table_lookup_buckets_and_force(tmp_path):
    t = tmp_path / "t.txt"
    t.write_text("# fmt M N K algo swap split wn wk rows pf amode wlds wlayout tm tn us\n"
                 "0 8 4096 4096 0 1 4 4 1 16 2 1 0 0 0 0 3.1\n"
                 "0 32 4096 4096 0 0 4 2 2 32 2 1 1 0 0 0 3.3\n"
                 "0 8 4096 4096 0 0 2 1 4 16 2 0 0 1 0 0 2.2\n"
                 "\n")
    assert ql.qlinear_table_load(str(t)) == 3
    try:
        p = ql.qlinear_plan(ql.FP8_DYNAMIC, 5, 4096, 4096)           # bucket 8
        assert p.facts["source"] == "table" and p.config["swap_ab"] == 1 and p.config["split_k"] == 4
        p = ql.qlinear_plan(ql.FP8_DYNAMIC, 17, 4096, 4096)          # bucket 24 -> nearest tuned >= : 32
        assert p.config["waves_k"] == 2 and p.config["w_lds"] == 1
        p = ql.qlinear_plan(ql.FP8_DYNAMIC, 8, 4096, 2048)           # other K: heuristic
        assert p.facts["source"] == "heuristic"
        p = ql.qlinear_plan_packed(ql.FP8_DYNAMIC, 3, 4096, 4096)    # packed-layout entry
        assert p.facts["source"] == "table" and p.config["w_layout"] == 1 and p.config["waves_k"] == 4
        p = ql.qlinear_plan_packed(ql.FP8_DYNAMIC, 32, 4096, 4096)   # no packed entry at/above 32
        assert p.facts["source"] == "heuristic" and p.config["w_layout"] == 1
        with pytest.raises(ql.QLinearError) as e:
            ql.qlinear_plan_from_table(ql.W8A8_INT8, 8, 4096, 4096)
        assert e.value.status == QL_E_NO_TABLE_ENTRY
        os.environ["QLINEAR_FORCE"] = "0,0,2,1,4,16,4,0,1,0,0,0"
        try:
            p = ql.qlinear_plan(ql.FP8_DYNAMIC, 8, 4096, 4096)
            assert p.facts["source"] == "custom" and p.config["waves_k"] == 4 and p.config["w_lds"] == 1
        finally:
            del os.environ["QLINEAR_FORCE"]
    finally:
        ql.qlinear_table_clear()
    bad = tmp_path / "bad.txt"
    bad.write_text("0 8 4096\n")
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_table_load(str(bad))
    assert e.value.status == QL_E_TABLE
    with pytest.raises(ql.QLinearError):
        ql.qlinear_table_load(str(tmp_path / "missing.txt"))


def test_packed_weight_sizes():
    assert ql.qlinear_packed_weight_bytes(4096, 4096) == 4096 * 4096
    assert ql.qlinear_packed_weight_bytes(300, 1040) == 19 * 9 * 2048
    assert ql.qlinear_packed_weight_bytes(0, 128) == 0
    v = ctypes.c_void_p
    assert ql.lib().qlinear_pack_weight(v(16), 10, 100, v(16), v(0)) == QL_E_INVALID     # K % 16
    assert ql.lib().qlinear_pack_weight(v(8), 10, 128, v(16), v(0)) == QL_E_ALIGN


def test_heuristic_plans_cover_every_decode_workload():
    """Without a table every decode workload point still gets an instantiated
    plan for every operand layout, one K range per workgroup (split 1) and at
    least one workgroup per 64 weight rows."""
    from workloads import decode_points, decode_workloads
    ql.qlinear_table_clear()
    try:
        for cfg in decode_workloads(include_mx=True):
            layouts = [(1, 1), (1, 2)] if cfg.fmt in ql.MX_FORMATS else [(0, 0), (1, 0), (1, 1), (1, 2)]
            for (_, N, K, M) in decode_points(cfg):
                for lay in layouts:
                    p = ql.qlinear_plan_layouts(cfg.fmt, M, N, K, *lay)
                    assert p.config["split_k"] == 1, (cfg.name, N, K, M, lay, p.config)
                    assert p.facts["workgroups"] >= N // 64, (cfg.name, N, K, M, lay, p.config)
    finally:
        ql.load_default_table()


@pytest.mark.parametrize("N,K,small_m,large_m", [
    (2048, 2048, (1, 4, 16, 0), (1, 4, 16, 0)), (4096, 14336, (1, 4, 16, 0), (1, 4, 16, 0)),
    (5120, 5120, (2, 2, 16, 0), (2, 2, 16, 0)), (7168, 5120, (2, 2, 16, 0), (2, 2, 16, 0)),
    (5120, 17408, (1, 4, 32, 0), (1, 4, 32, 0)), (14336, 4096, (2, 2, 16, 0), (4, 1, 16, 1)),
    (34816, 5120, (1, 4, 32, 0), (1, 4, 32, 0))])
def test_heuristic_wave_shape_follows_the_row_groups(N, K, small_m, large_m):
    """Table-free decode plans: one 16-row group per 4-wave workgroup up to 256
    groups, 2 x 2 waves up to 1024 (4 x 1 with Swap-AB beyond 512 groups at
    M > 8), 32 rows a wave beyond 1024 groups or for a long K; split 1; a
    forward plan at M = 1 fuses the quantizer where the fused kernel fits.
    (waves_n, waves_k, rows_per_wave, swap_ab) for M <= 8 and for M > 8."""
    ql.qlinear_table_clear()
    try:
        for M in (1, 8, 16, 32):
            c = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, M, N, K, 1, 1).config
            want = small_m if M <= 8 else large_m
            assert (c["waves_n"], c["waves_k"], c["rows_per_wave"], c["swap_ab"]) == want, (M, c)
            assert c["split_k"] == 1 and c["a_mode"] == 2, (M, c)
        if (N, K) == (5120, 17408):   # the MX formats keep 2 x 2 waves on a long K up to 16 tokens
            for fmt in (ql.MXFP8, ql.MXFP4):
                c = ql.qlinear_plan_layouts(fmt, 16, N, K, 1, 1).config
                assert (c["waves_n"], c["waves_k"], c["rows_per_wave"]) == (2, 2, 16), c
                c = ql.qlinear_plan_layouts(fmt, 32, N, K, 1, 1).config
                assert (c["waves_n"], c["waves_k"], c["rows_per_wave"]) == (1, 4, 32), c
        f = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 1, N, K, 1, 2).config
        fits = K <= 16384 and K % 512 == 0
        assert (f["a_mode"] == 4) == fits, f
    finally:
        ql.load_default_table()


def test_heuristic_splits_only_few_row_groups_over_a_long_k():
    ql.qlinear_table_clear()
    try:
        assert ql.qlinear_plan_layouts(ql.W8A8_INT8, 8, 64, 65536, 1, 1).config["split_k"] == 8
        assert ql.qlinear_plan_layouts(ql.W8A8_INT8, 8, 64, 4096, 1, 1).config["split_k"] == 1
        assert ql.qlinear_plan_layouts(ql.W8A8_INT8, 8, 4096, 65536, 1, 1).config["split_k"] == 1
    finally:
        ql.load_default_table()


def test_fused_quantization_plans_are_validated_on_host():
    fused = dict(w_layout=1, a_mode=4, waves_n=1, waves_k=4)
    assert _plan_status(ql.FP8_DYNAMIC, 4, 4096, 4096, **fused) == QL_OK
    assert _plan_status(ql.W8A8_INT8, 1, 4096, 12288, **fused) == QL_OK
    assert _plan_status(ql.BLOCK_FP8, 1, 4096, 4096, **fused) == QL_OK
    assert _plan_status(ql.BLOCK_FP8, 16, 4096, 4096, **fused) == QL_E_UNSUPPORTED  # 16 x 4096 > 16384 ...
    assert _plan_status(ql.BLOCK_FP8, 16, 4096, 4096, split_k=4, **fused) == QL_OK  # ... a 1024-wide chunk fits
    assert _plan_status(ql.BLOCK_FP8, 17, 4096, 4096, split_k=8, **fused) == QL_E_UNSUPPORTED
    assert _plan_status(ql.FP8_DYNAMIC, 8, 4096, 4096, **fused) == QL_E_UNSUPPORTED  # M*K > 16384
    assert _plan_status(ql.FP8_DYNAMIC, 17, 4096, 512, **fused) == QL_E_UNSUPPORTED  # one token tile
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 4352, **fused) == QL_E_UNSUPPORTED  # K % 512
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 4096, a_mode=4) == QL_E_UNSUPPORTED  # needs packed weights
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 4096, a_mode=6, w_layout=1) == QL_E_INVALID
    # a fused plan quantizes X itself, so it only runs through qlinear_forward
    p = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 2, 1024, 4096, fused)
    assert p.facts["lds_bytes"] >= 512 + 2 * (4096 + 64)
    v = ctypes.c_void_p
    good = v(1 << 20)
    assert ql.lib().qlinear_run(p.handle, good, good, good, good, good, v(0), v(0)) == QL_E_INVALID
    assert "qlinear_forward" in ql.lib().qlinear_last_error().decode()
    assert ql.lib().qlinear_forward(p.handle, v(0), good, good, good, good, good, v(0), v(0)) == QL_E_INVALID
    assert ql.lib().qlinear_forward(p.handle, v(8), good, good, good, good, good, v(0), v(0)) == QL_E_ALIGN


def test_forward_table_entries(tmp_path):
    t = tmp_path / "t.txt"
    t.write_text("0 4 4096 4096 0 0 1 1 4 16 2 2 0 1 0 0 5.0\n"          # packed-A_q entry
                 "0 4 4096 4096 0 0 1 1 4 32 1 4 0 1 0 0 6.1 fwd\n"      # forward entry, fused
                 "0 8 4096 4096 0 1 1 1 4 16 2 3 0 1 0 0 8.2 fwd\n"      # forward entry, not fused
                 "0 16 4096 4096 0 0 2 1 4 16 2 2 0 1 0 0 6.0\n")
    assert ql.qlinear_table_load(str(t)) == 4
    try:
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 3, 4096, 4096, 1, 2)
        assert p.facts["source"] == "table" and p.config["a_mode"] == 4 and p.config["rows_per_wave"] == 32
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 3, 4096, 4096, 1, 1)   # the packed-A_q plan ignores fwd entries
        assert p.config["a_mode"] == 2 and p.config["rows_per_wave"] == 16
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 8, 4096, 4096, 1, 2)
        assert p.config["a_mode"] == 3 and p.config["swap_ab"] == 1
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 8, 4096, 4096, 1, 1)   # no packed-A_q entry at 8: next tuned
        assert p.config["a_mode"] == 2 and p.config["split_k"] == 2
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 12, 4096, 4096, 1, 2)  # no fwd entry at 16: packed-A_q entry
        assert p.facts["source"] == "table" and p.config["a_mode"] == 2 and p.config["split_k"] == 2
        with pytest.raises(ql.QLinearError):
            ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 4, 4096, 4096, 0, 2)   # forward plans need packed weights
    finally:
        ql.qlinear_table_clear()
    bad = tmp_path / "bad.txt"
    bad.write_text("0 4 4096 4096 0 0 1 1 4 16 2 2 0 1 0 0 5.0 xyz\n")
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_table_load(str(bad))
    assert e.value.status == QL_E_TABLE


def test_decode_plans_reach_64_tokens():
    cfg = dict(w_layout=1, a_mode=2, waves_n=1, waves_k=4, prefetch=1)
    assert _plan_status(ql.FP8_DYNAMIC, 64, 4096, 4096, **cfg) == QL_OK
    assert _plan_status(ql.W8A8_INT8, 33, 4096, 4096, **cfg) == QL_OK
    assert _plan_status(ql.FP8_DYNAMIC, 65, 4096, 4096, **cfg) == QL_E_UNSUPPORTED
    p = ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 50, 4096, 4096, cfg)
    assert p.config["algo"] == ql.ALGO_DECODE and p.facts["threads"] == 256
    # without a table entry M > 32 streams the weights while they are at most 512 row groups
    ql.qlinear_table_clear()
    try:
        assert ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 50, 4096, 4096, 1, 1).config["algo"] == ql.ALGO_DECODE
        assert ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 50, 16384, 4096, 1, 1).config["algo"] == ql.ALGO_TILED
    finally:
        ql.load_default_table()


def test_glu_plans_are_validated_on_host():
    def glu_status(fmt, M, N, K, **cfg):
        h = ctypes.c_void_p()
        c = ql.QLConfig(**ql.make_config(**cfg))
        st = ql.lib().qlinear_plan_glu_with_config(fmt, M, N, K, ctypes.byref(c), ctypes.byref(h))
        if h.value:
            ql.lib().qlinear_plan_destroy(h)
        return st
    good = dict(w_layout=1, a_mode=2, rows_per_wave=32, waves_n=1, waves_k=4, prefetch=1)
    assert glu_status(ql.FP8_DYNAMIC, 4, 1024, 512, **good) == QL_OK
    assert glu_status(ql.FP8_DYNAMIC, 4, 1040, 512, **good) == QL_E_INVALID                   # N % 32
    assert glu_status(ql.FP8_DYNAMIC, 4, 1024, 512, **dict(good, rows_per_wave=16)) == QL_E_UNSUPPORTED
    assert glu_status(ql.FP8_DYNAMIC, 4, 1024, 512, **dict(good, w_layout=0)) == QL_E_UNSUPPORTED
    assert glu_status(ql.FP8_DYNAMIC, 40, 1024, 512, **good) == QL_E_UNSUPPORTED              # decode only
    p = ql.qlinear_plan_glu_with_config(ql.W8A8_INT8, 4, 1024, 512, good)
    assert p.facts["epilogue"] == 1 and p.facts["workgroups"] == 512 // 16
    assert ql.qlinear_plan(ql.W8A8_INT8, 4, 1024, 512).facts["epilogue"] == 0
    v = ctypes.c_void_p
    good_ptr = v(1 << 20)
    assert ql.lib().qlinear_run_debug_acc(p.handle, good_ptr, good_ptr, good_ptr, good_ptr, good_ptr, v(0),
                                          good_ptr, v(0)) == QL_E_UNSUPPORTED
    q = ql.qlinear_plan_glu(ql.FP8_DYNAMIC, 2, 24576, 4096, 2)
    assert q.facts["epilogue"] == 1 and q.config["rows_per_wave"] == 32
    with pytest.raises(ql.QLinearError):
        ql.qlinear_plan_glu(ql.FP8_DYNAMIC, 2, 24576, 4096, 0)


def test_glu_table_entries(tmp_path):
    t = tmp_path / "t.txt"
    t.write_text("0 4 1024 512 0 1 2 2 2 32 2 2 0 1 0 0 5.0 glu\n"
                 "0 4 1024 512 0 0 1 1 4 16 2 2 0 1 0 0 4.0\n")
    assert ql.qlinear_table_load(str(t)) == 2
    try:
        p = ql.qlinear_plan_glu(ql.FP8_DYNAMIC, 3, 1024, 512, 1)
        assert p.facts["source"] == "table" and p.config["split_k"] == 2 and p.config["waves_n"] == 2
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 3, 1024, 512, 1, 1)     # the plain plan ignores glu entries
        assert p.config["rows_per_wave"] == 16 and p.facts["epilogue"] == 0
    finally:
        ql.qlinear_table_clear()


def test_mxfp8_plans_are_validated_on_host():
    good = dict(w_layout=1, a_mode=2, waves_n=4, waves_k=1, prefetch=2)
    assert _plan_status(ql.MXFP8, 8, 4096, 4096, **good) == QL_OK
    assert _plan_status(ql.MXFP8, 8, 4096, 4096, **dict(good, a_mode=3)) == QL_OK
    assert _plan_status(ql.MXFP8, 8, 4096, 4160, **good) == QL_E_INVALID             # K % 128
    assert _plan_status(ql.MXFP8, 8, 4096, 4096, **dict(good, w_layout=0, a_mode=0)) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP8, 8, 4096, 4096, **dict(good, a_mode=1)) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP8, 8, 4096, 4096, **dict(good, a_mode=4)) == QL_E_UNSUPPORTED   # no fused quantizer
    tiled = dict(good, algo=ql.ALGO_TILED, tile_m=128, tile_n=128)
    assert _plan_status(ql.MXFP8, 128, 4096, 4096, **tiled) == QL_OK                   # register ring
    assert _plan_status(ql.MXFP8, 128, 4096, 4096, **dict(tiled, w_lds=1)) == QL_E_UNSUPPORTED   # LDS-DMA ring
    assert _plan_status(ql.MXFP4, 128, 4096, 4096, **tiled) == QL_OK                   # E2M1 weights, register ring
    assert _plan_status(ql.MXFP4, 128, 4096, 4096, **dict(tiled, w_lds=1)) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP4, 128, 4096, 4096, **dict(tiled, w_layout=0, a_mode=0)) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP4, 65, 4096, 4096, **good) == QL_E_UNSUPPORTED          # decode: M <= 64
    assert _plan_status(ql.MXFP8, 65, 4096, 4096, **good) == QL_E_UNSUPPORTED
    # shapes whose registers would spill are not instantiated
    assert _plan_status(ql.MXFP8, 32, 4096, 4096, **dict(good, waves_n=2, waves_k=4, prefetch=2,
                                                         rows_per_wave=32)) == QL_E_UNSUPPORTED
    # the heuristic keeps MXFP8 on the decode kernel up to 64 tokens
    ql.qlinear_table_clear()
    try:
        for M in (1, 24, 50, 64):
            p = ql.qlinear_plan_layouts(ql.MXFP8, M, 4096, 4096, 1, 1)
            assert p.config["algo"] == ql.ALGO_DECODE and p.config["a_mode"] == 2, M
        with pytest.raises(ql.QLinearError):
            ql.qlinear_plan_layouts(ql.MXFP8, 8, 4096, 4096, 0, 0)     # row-major operands
    finally:
        ql.load_default_table()
    h = ctypes.c_void_p()
    c = ql.QLConfig(**ql.make_config(**dict(good, rows_per_wave=32)))
    assert ql.lib().qlinear_plan_glu_with_config(ql.MXFP8, 4, 1024, 512, ctypes.byref(c),
                                                 ctypes.byref(h)) == QL_E_UNSUPPORTED
    assert ql.act_scale_shape(ql.MXFP8, 5, 512) == (5, 16) and ql.weight_scale_shape(ql.MXFP8, 7, 256) == (7, 8)
    assert ql.scale_dtype(ql.MXFP8) == torch.uint8 and ql.scale_dtype(ql.BLOCK_FP8) == torch.float32
    null = ctypes.c_void_p(0)
    assert ql.lib().qlinear_quantize_act(ql.MXFP8, null, 4, 4160, null, null, null) == QL_E_INVALID


def test_mx_scale_layout_sizes():
    assert ql.qlinear_packed_mx_scale_bytes(1, 4096) == 32 * 64
    assert ql.qlinear_packed_mx_scale_bytes(17, 256) == 2 * 2 * 64
    assert ql.qlinear_packed_mx_scale_bytes(0, 256) == 0
    null = ctypes.c_void_p(0)
    assert ql.lib().qlinear_pack_mx_scales(null, 4, 4160, null, null) == QL_E_INVALID   # K % 128
    assert ql.lib().qlinear_pack_mx_scales(null, 4, 256, null, null) == QL_E_INVALID    # NULL
    assert ql.lib().qlinear_pack_mx_scales(null, 0, 256, null, null) == QL_OK          # empty


def test_mxfp4_plans_and_sizes():
    good = dict(w_layout=1, a_mode=2, waves_n=4, waves_k=1, prefetch=2)
    assert _plan_status(ql.MXFP4, 8, 4096, 4096, **good) == QL_OK
    assert _plan_status(ql.MXFP4, 8, 4096, 4160, **good) == QL_E_INVALID                # K % 128
    assert _plan_status(ql.MXFP4, 8, 4096, 4096, **dict(good, w_layout=0, a_mode=0)) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP4, 8, 4096, 4096, **dict(good, a_mode=4)) == QL_E_UNSUPPORTED
    assert ql.qlinear_packed_weight_bytes_fp4(17, 256) == 2 * 2 * 1024
    assert ql.weight_code_shape(ql.MXFP4, 10, 256) == (10, 128) and ql.weight_code_dtype(ql.MXFP4) == torch.uint8
    assert ql.code_dtype(ql.MXFP4) == torch.float8_e4m3fn          # activations stay E4M3
    null = ctypes.c_void_p(0)
    assert ql.lib().qlinear_pack_weight_fp4(null, 4, 4160, null, null) == QL_E_INVALID
    assert ql.lib().qlinear_quantize_weight(ql.MXFP4, null, 4, 4160, null, null, null) == QL_E_INVALID


@pytest.mark.parametrize("N,K,M,tile,split", [
    (4096, 4096, 96, (64, 128), 4), (4096, 4096, 256, (64, 128), 1), (4096, 4096, 1024, (128, 128), 1),
    (4096, 4096, 4096, (256, 256), 1), (14336, 4096, 64, (64, 128), 1), (14336, 4096, 256, (128, 128), 1),
    (14336, 4096, 1024, (256, 256), 1), (4096, 14336, 256, (64, 128), 2), (28672, 4096, 256, (128, 256), 1),
    (2048, 8192, 96, (64, 128), 4), (2048, 8192, 4096, (128, 256), 1)])
def test_tiled_heuristic_takes_the_largest_tile_that_fills_the_chip(N, K, M, tile, split):
    """Table-free tiled plans: the largest of 256 x 256, 128 x 256, 128 x 128
    and 64 x 128 that gives about 200 tiles, else 64 x 128 with split-K 4
    (<= 64 tiles) or 2 (<= 128 tiles over a K of 64 or more blocks).  Row-major
    operands cannot run the 256 x 256 ring and take the next tile; MXFP8 runs
    the register ring only."""
    ql.qlinear_table_clear()
    try:
        c = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, M, N, K, 1, 1).config
        assert c["algo"] == ql.ALGO_TILED and (c["tile_m"], c["tile_n"]) == tile and c["split_k"] == split, c
        assert c["w_lds"] == (1 if tile == (256, 256) else 0), c
        r = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, M, N, K, 0, 0).config
        assert r["algo"] == ql.ALGO_TILED and r["w_lds"] == 0, r
        if tile != (256, 256):
            assert (r["tile_m"], r["tile_n"]) == tile, r
        x = ql.qlinear_plan_layouts(ql.MXFP8, M, N, K, 1, 1).config
        if M > 64:
            assert x["algo"] == ql.ALGO_TILED and x["w_lds"] == 0 and (x["tile_m"], x["tile_n"]) != (256, 256), x
    finally:
        ql.load_default_table()


@pytest.mark.parametrize("N,K,M,cfg", [
    (4096, 4096, 64, (64, 128, 2, 0, 4)), (4096, 4096, 256, (64, 128, 2, 0, 2)), (4096, 4096, 1024, (64, 128, 1, 0, 1)),
    (4096, 4096, 4096, (128, 128, 1, 1, 1)), (4096, 14336, 256, (64, 128, 2, 0, 4)),
    (28672, 4096, 64, (64, 128, 2, 0, 1)), (14336, 4096, 1024, (128, 128, 1, 1, 1))])
def test_tiled_heuristic_block_fp8(N, K, M, cfg):
    """Block_FP8 table-free tiled plans (tile_m, tile_n, prefetch, swap_ab, split_k):
    128 x 128 with 1-block batches and Swap-AB from 400 such tiles, else 64 x 128."""
    ql.qlinear_table_clear()
    try:
        c = ql.qlinear_plan_layouts(ql.BLOCK_FP8, M, N, K, 1, 1).config
        assert (c["tile_m"], c["tile_n"], c["prefetch"], c["swap_ab"], c["split_k"]) == cfg, c
    finally:
        ql.load_default_table()


@pytest.mark.parametrize("N,K,waves", [(4096, 4096, (1, 4)), (2048, 8192, (1, 4)), (7168, 5120, (2, 2))])
def test_table_free_plans_up_to_64_tokens_stream_the_weights(N, K, waves):
    """32 < M <= 64 with packed weights and at most 512 row groups: the
    weight-streaming kernel with four token tiles; more rows, row-major
    weights or Block_FP8: the tiled kernel."""
    ql.qlinear_table_clear()
    try:
        for M in (33, 40, 64):
            for fmt in (ql.FP8_DYNAMIC, ql.W8A8_INT8):
                c = ql.qlinear_plan_layouts(fmt, M, N, K, 1, 1).config
                assert c["algo"] == ql.ALGO_DECODE and (c["waves_n"], c["waves_k"]) == waves, c
                assert ql.qlinear_plan_layouts(fmt, M, N, K, 0, 0).config["algo"] == ql.ALGO_TILED
            assert ql.qlinear_plan_layouts(ql.BLOCK_FP8, M, N, K, 1, 1).config["algo"] == ql.ALGO_TILED
        assert ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 64, 28672, 4096, 1, 1).config["algo"] == ql.ALGO_TILED
        assert ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 65, 4096, 4096, 1, 1).config["algo"] == ql.ALGO_TILED
    finally:
        ql.load_default_table()


def test_given_amax_plans_are_validated_on_host():
    """a_mode 5 (the per-token amax of X given): per-token formats, one token
    tile, whole 128-wide K blocks, M x chunk within the 16384 values a
    workgroup quantizes, packed weights."""
    m5 = dict(w_layout=1, a_mode=5, waves_n=1, waves_k=4)
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 12288, **m5) == QL_OK
    assert _plan_status(ql.W8A8_INT8, 16, 4096, 12288, split_k=16, **m5) == QL_OK   # 16 x 768 values
    assert _plan_status(ql.W8A8_INT8, 16, 4096, 12288, split_k=8, **m5) == QL_E_UNSUPPORTED   # 16 x 1536
    assert _plan_status(ql.FP8_DYNAMIC, 17, 4096, 512, **m5) == QL_E_UNSUPPORTED
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 4160, **m5) == QL_E_UNSUPPORTED     # K % 128
    assert _plan_status(ql.BLOCK_FP8, 1, 4096, 4096, **m5) == QL_E_UNSUPPORTED
    assert _plan_status(ql.MXFP8, 1, 4096, 4096, **m5) == QL_E_UNSUPPORTED
    assert _plan_status(ql.FP8_DYNAMIC, 1, 4096, 4096, a_mode=5) == QL_E_UNSUPPORTED  # needs packed weights


def test_given_amax_planning():
    """qlinear_plan_layouts(..., a_packed = 3): a_mode 5 up to 16 tokens over
    whole K blocks (split so that M x chunk fits), else the packed-A plan."""
    for M in (1, 4, 16):                      # an untabulated shape: the heuristic's plan
        p = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, M, 3072, 12288, 1, 3)
        assert p.config["a_mode"] == 5 and p.facts["source"] == "heuristic"
        assert M * p.facts["chunk_k"] <= 16384
    assert ql.qlinear_plan_layouts(ql.W8A8_INT8, 24, 3072, 12288, 1, 3).config["a_mode"] in (2, 3)
    assert ql.qlinear_plan_layouts(ql.W8A8_INT8, 4, 3072, 4160, 1, 3).config["a_mode"] in (2, 3)
    with pytest.raises(ql.QLinearError):
        ql.qlinear_plan_layouts(ql.BLOCK_FP8, 4, 4096, 4096, 1, 3)


def test_amax_buffer_layout_matches_the_header():
    """The amax buffer: 64 replica lines of 32 words, then 17 counter lines;
    the binding's size and layout constants are the header's (and the
    kernels', which index it with the same numbers)."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+QL_AMAX_BUFFER_BYTES\s+(\d+)", text)
    assert m and int(m.group(1)) == ql.AMAX_BUFFER_BYTES
    assert ql.AMAX_BUFFER_BYTES == (ql.AMAX_REPLICAS * ql.AMAX_LINE + 17 * ql.AMAX_LINE) * 4
    args = open(os.path.join(ROOT, "quantized_gemm_decode_amd", "csrc", "decode_args.hpp")).read()
    assert re.search(r"AMAX_REPLICAS\s*=\s*%d;" % ql.AMAX_REPLICAS, args)
    assert re.search(r"AMAX_LINE\s*=\s*%d;" % ql.AMAX_LINE, args)
    assert re.search(r"AMAX_GROUPS\s*=\s*16;", args)
    buf = ql.amax_buffer(device="cpu")
    assert buf.numel() * 4 == ql.AMAX_BUFFER_BYTES and not buf.any()
    words = buf.numpy().view("uint32")
    words[3 * ql.AMAX_LINE + 2] = 7
    words[40 * ql.AMAX_LINE + 2] = 9
    words[5] = 1
    assert list(ql.amax_of_buffer(buf, 3)) == [0, 0, 9]
