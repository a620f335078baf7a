"""Host logic of the offline sweep (CPU only): the tie-break that picks a
table entry, the table line it writes (read back through the C ABI), and the
candidate generators' limits."""

import pytest

import quantized_gemm_decode_amd as ql
from quantized_gemm_decode_amd import sweep


def _cfg(**kw):
    return ql.make_config(**kw)


def test_choose_prefers_the_simpler_variant_within_two_percent():
    std = (10.15, _cfg(swap_ab=0, split_k=1))
    swap = (10.05, _cfg(swap_ab=1, split_k=1))
    split2 = (10.0, _cfg(swap_ab=1, split_k=2))
    split8 = (10.1, _cfg(swap_ab=0, split_k=8))
    assert sweep.choose([split2, swap, std, split8]) is std            # all within 2 % of 10.0
    assert sweep.choose([split2, swap]) is swap
    assert sweep.choose([split8, split2]) is split2                     # same variant: smaller split


def test_choose_takes_the_fastest_beyond_two_percent():
    fast = (9.0, _cfg(swap_ab=1, split_k=4))
    std = (9.5, _cfg(swap_ab=0, split_k=1))                             # 5.6 % slower
    assert sweep.choose([std, fast]) is fast
    assert sweep.choose([std, fast], tie=0.1) is std


def test_table_line_round_trips_through_the_c_abi(tmp_path):
    cfg = dict(swap_ab=1, split_k=4, waves_n=2, waves_k=2, rows_per_wave=32, prefetch=1, a_mode=2, w_layout=1)
    line = sweep.table_line(ql.FP8_DYNAMIC, 8, 4096, 4096, cfg, 6.125)
    fields = line.split()
    assert len(fields) == 17 and fields[-1] == "6.125"
    fwd = sweep.table_line(ql.FP8_DYNAMIC, 2, 4096, 4096, dict(cfg, a_mode=4, split_k=1), 5.5, kind="fwd")
    assert fwd.endswith(" fwd")
    path = tmp_path / "t.txt"
    path.write_text("# test table\n" + line + "\n" + fwd + "\n")
    try:
        assert ql.qlinear_table_load(str(path)) == 2
        got = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 8, 4096, 4096, 1, 1)
        assert got.facts["source"] == "table"
        for k, v in cfg.items():
            assert got.config[k] == v, k
        f = ql.qlinear_plan_layouts(ql.FP8_DYNAMIC, 2, 4096, 4096, 1, 2)     # forward plan
        assert f.facts["source"] == "table" and f.config["a_mode"] == 4
    finally:
        ql.load_default_table()


def test_decode_candidates_plan_or_are_not_instantiated():
    """Every phase-1 decode candidate of a packed layout is a valid config:
    the planner accepts it or reports it as not instantiated (status 2)."""
    n_ok = 0
    for layout in (1, 2):
        for cfg in sweep.phase1_candidates(ql.FP8_DYNAMIC, 8, 4096, 4096, layout):
            try:
                ql.qlinear_plan_with_config(ql.FP8_DYNAMIC, 8, 4096, 4096, cfg)
                n_ok += 1
            except ql.QLinearError as e:
                assert e.status == 2, (cfg, e)
    assert n_ok > 50


def test_row_tile_candidates():
    """Row tiles are offered where N does not split evenly over 256 compute
    units in 16-row groups, for FP8_Dynamic / W8A8_INT8 only, and every
    candidate plans or is reported as not instantiated."""
    assert sweep.row_tiles(ql.FP8_DYNAMIC, 6144, 2) == [24]
    assert sweep.row_tiles(ql.W8A8_INT8, 10240, 2) == [40, 48]
    assert sweep.row_tiles(ql.FP8_DYNAMIC, 4096, 2) == [] and sweep.row_tiles(ql.FP8_DYNAMIC, 8192, 2) == []
    assert sweep.row_tiles(ql.BLOCK_FP8, 6144, 2) == [24] and sweep.row_tiles(ql.FP8_DYNAMIC, 6144, 4) == []
    assert sweep.row_tiles(ql.MXFP8, 6144, 2) == []
    assert sweep.row_tiles(ql.W8A8_INT8, 51200, 2) == [40]          # 1280 workgroups: 5 a compute unit
    assert sweep.row_tiles(ql.W8A8_INT8, 24576, 2) == []             # 768 x 32 rows: 3 a compute unit
    n_ok = 0
    for layout in (0, 1, 2, 3, 5):
        cands = list(sweep.row_tile_candidates(ql.W8A8_INT8, 8, 5120, 8192, layout))
        assert cands and all(c["tile_n"] == 24 and c["waves_n"] * c["rows_per_wave"] >= 24 for c in cands)
        for cfg in cands:
            try:
                ql.qlinear_plan_with_config(ql.W8A8_INT8, 8, 5120, 8192, cfg)
                n_ok += 1
            except ql.QLinearError as e:
                assert e.status == 2, (cfg, e)
    assert n_ok > 50
    assert all(c.get("tile_n", 0) == 0 for c in sweep.phase1_candidates(ql.FP8_DYNAMIC, 8, 4096, 4096, 2))


def test_fused_candidates_respect_the_fused_limits():
    assert sweep.fused_ok(ql.FP8_DYNAMIC, 4, 4096) and not sweep.fused_ok(ql.FP8_DYNAMIC, 8, 4096)
    assert not sweep.fused_ok(ql.W8A8_INT8, 1, 4160)                   # K % 512
    assert sweep.fused_ok(ql.BLOCK_FP8, 16, 12288) and not sweep.fused_ok(ql.BLOCK_FP8, 24, 4096)
    cands = list(sweep.phase1_candidates(ql.FP8_DYNAMIC, 2, 4096, 4096, 3))
    assert cands and all(c["a_mode"] == 4 and c["w_layout"] == 1 for c in cands)


def test_tiled_candidates_cover_the_tiles_and_rings():
    cands = list(sweep.tiled_candidates(1024, 4096, 4096, 2))
    tiles = {(c["tile_m"], c["tile_n"]) for c in cands}
    assert (256, 256) in tiles and (128, 256) in tiles and (64, 128) in tiles
    assert all(c["w_lds"] == 1 and c["prefetch"] == 2 for c in cands if (c["tile_m"], c["tile_n"]) == (256, 256))
    assert not [c for c in sweep.tiled_candidates(1024, 4096, 4096, 0) if c["w_lds"]]   # DMA ring: packed only
    small = list(sweep.tiled_candidates(40, 4096, 4096, 2))
    assert all(c["tile_m"] <= 80 or c["tile_m"] == 64 for c in small)


@pytest.mark.parametrize("M", [33, 64])
def test_decode_candidates_up_to_64_tokens(M):
    # the candidates read the activations in the layout the timer hands them:
    # packed (read per K block or staged in LDS) for layout 2, row-major for layout 1
    cands = list(sweep.decode_m64_candidates(M, 4096, 4096, 2))
    assert cands and all(c["w_layout"] == 1 and c["a_mode"] in (2, 3) for c in cands)
    assert {c["a_mode"] for c in cands} == {2, 3}
    cands = list(sweep.decode_m64_candidates(M, 4096, 4096, 1))
    assert cands and all(c["w_layout"] == 1 and c["a_mode"] == 0 for c in cands)


def test_merge_replaces_entries_of_the_same_key(tmp_path):
    """A partial re-sweep replaces exactly the entries the planner would look
    up by the same key (format, M, N, K, weight layout, activation class,
    kind) and keeps every other line."""
    base = tmp_path / "base.txt"
    upd = tmp_path / "upd.txt"
    base.write_text("# header\n"
                    "0 8 4096 12288 0 1 1 1 4 16 2 2 0 1 0 0 10.000\n"          # packed A: replaced
                    "0 8 4096 12288 0 1 1 1 4 16 2 0 0 1 0 0 11.000\n"          # row-major A: kept
                    "0 8 4096 12288 0 1 1 1 4 16 2 4 0 1 0 0 9.000 fwd\n"       # forward: replaced
                    "1 8 4096 12288 0 1 1 1 4 16 2 2 0 1 0 0 12.000\n"          # other format: kept
                    "# sweep wall time 5 s\n")
    upd.write_text("0 8 4096 12288 0 1 64 1 4 16 2 3 0 1 0 0 8.000\n"
                   "0 8 4096 12288 0 1 2 1 4 16 2 2 0 1 0 0 8.500 fwd\n"
                   "0 16 4096 12288 0 1 8 1 4 16 2 2 0 1 0 0 9.500\n")
    out = tmp_path / "out.txt"
    assert sweep.merge_tables(str(base), str(upd), str(out)) == 3
    lines = [l for l in out.read_text().splitlines() if l and not l.startswith("#")]
    assert lines == ["0 8 4096 12288 0 1 64 1 4 16 2 3 0 1 0 0 8.000",
                     "0 8 4096 12288 0 1 1 1 4 16 2 0 0 1 0 0 11.000",
                     "0 8 4096 12288 0 1 2 1 4 16 2 2 0 1 0 0 8.500 fwd",
                     "1 8 4096 12288 0 1 1 1 4 16 2 2 0 1 0 0 12.000",
                     "0 16 4096 12288 0 1 8 1 4 16 2 2 0 1 0 0 9.500"]
    assert out.read_text().rstrip().endswith("# sweep wall time 5 s")


def test_split_candidates_reach_256_clamped_to_the_k_blocks():
    cands = list(sweep.phase1_candidates(ql.FP8_DYNAMIC, 8, 4096, 32768, layout=2))
    chunks = {sweep._effective_chunks(32768, c["split_k"]) for c in cands}
    assert {64, 128, 256} <= chunks
    short = {sweep._effective_chunks(1024, c["split_k"])
             for c in sweep.phase1_candidates(ql.FP8_DYNAMIC, 8, 4096, 1024, layout=2)}
    assert max(short) == 8
