"""Offline per-shape sweep that writes the table qlinear_plan reads.

The pages tune each GEMM shape and token count ahead of time, with the
algorithmic switches (split_k over powers of two 1..256, swap_ab) searched
together with low-level kernel parameters, measured under graph replay
([Summary] "Put algorithm selection inside the search space" and "Hybrid
dispatch addresses runtime overhead"; [Noticias] "Autoajuste de los
kernels").  Here the space is small enough to search exhaustively in two
phases:

  1. swap_ab=1, prefetch=2 (1 where 2 is not instantiated); every
     (waves_n, waves_k), rows_per_wave, split_k (distinct effective chunk
     counts only), a_mode and w_lds -- for packed weights also 8- and 16-wave
     workgroups and 64 rows per wave;
  2. the best few of phase 1 again with swap_ab in {0, 1} x prefetch {1, 2, 4}.
For M > 32 (the tiled algorithm) the whole space -- tile, swap_ab, split_k,
ring depth -- is timed in one phase.  Operand layouts: row-major W and A,
packed W, packed W and A; each gets its own entries.  Layout 3 tunes
forward plans (packed W, quantize + GEMM timed together): every fused-
quantization configuration against the packed-A plan the table already
holds; the winner is written as a "fwd" entry (the Deep-dive page's fused
quantization, "Understanding Helion", as one more switch of the search
space).

Every candidate is timed as a hipGraph of back-to-back launches, each on its
own copy of the weights (>= 1 GiB of copies, so the Infinity Cache cannot
serve them), median of several replays.  Candidates must agree with each
other (INT8 bitwise; FP8 to 1e-2 normwise) or they are dropped.  Ties within
2 % go to Standard, then Swap-AB, then the smallest split.

  python -m quantized_gemm_decode_amd.sweep --workloads int8_linear_4096x2048,fp8_dynamic_8b,...

[Summary] = English summary of "Building a High-Performance and Portable
vLLM Linear Backend with Helion" (yuxiaoba.github.io); [Noticias] = "Helion
entra al backend lineal de vLLM y supera a CUTLASS en Hopper".
"""

import argparse
import datetime
import itertools
import os
import sys
import time

import torch

import quantized_gemm_decode_amd as ql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import config_by_name, decode_workloads, make_inputs  # noqa: E402

# split_k over the pages' powers of two 1..256 (clamped to the K blocks; only
# distinct chunk counts are timed)
SPLITS = (1, 2, 4, 8, 16, 32, 64, 128, 256)
WAVES = ((4, 1), (2, 2), (1, 4))
# packed weights also run 8- and 16-wave workgroups and 64 rows per wave
WAVES_PACKED = WAVES + ((1, 8), (2, 4), (1, 16))


def _effective_chunks(K, split):
    G = -(-K // 128)
    s = max(1, min(split, G))
    ck = -(-G // s)
    return -(-G // ck)


TILES = ((64, 128), (64, 256), (128, 128), (128, 256), (256, 128))


def tiled_candidates(M, N, K, layout):
    """Every tiled configuration for M > 32 (tile, orientation, split, register-ring depth,
    and with packed operands the LDS-DMA ring of 2 or 3 stages)."""
    rings = [(0, 1), (0, 2), (0, 4)] + ([(1, 2), (1, 3)] if layout == 2 else [])
    for (bm, bn), swap, split, (dma, pf) in itertools.product(TILES + ((256, 256),), (0, 1), (1, 2, 4, 8), rings):
        if bm > 64 and bm > 2 * M:
            continue
        if (bm, bn) == (256, 256) and (dma, pf) != (1, 2):
            continue                  # the 8-wave tile runs the 2-stage LDS-DMA ring only
        yield dict(algo=ql.ALGO_TILED, swap_ab=swap, split_k=split, tile_m=bm, tile_n=bn, prefetch=pf, w_lds=dma,
                   a_mode=2 if layout == 2 else 0, w_layout=1 if layout >= 1 else 0)


def fused_ok(fmt, M, K):
    """Shapes the fused-quantization decode kernel can serve (Block_FP8: with a
    large enough split; the planner rejects the candidates that do not fit)."""
    if fmt == ql.BLOCK_FP8:
        return M <= 16
    return M <= 16 and M * K <= 16384 and K % 512 == 0


def amax_mode_ok(fmt, M, K):
    """Shapes the given-amax prologue (a_mode 5) can serve."""
    return fmt in (ql.FP8_DYNAMIC, ql.W8A8_INT8) and M <= 16 and K % 128 == 0


def decode_m64_candidates(M, N, K, layout):
    """Weight-streaming configurations with four token tiles (32 < M <= 64,
    packed weights; packed activations read per K block or staged in LDS for
    layout 2, row-major ones for layout 1)."""
    seen = set()
    for (wn, wk), rows, split, amode in itertools.product(((4, 1), (2, 2), (1, 4), (2, 4), (1, 8)), (16, 32, 64),
                                                         SPLITS, (2, 3) if layout == 2 else (0,)):
        key = (wn, wk, rows, _effective_chunks(K, split), amode)
        if key in seen:
            continue
        seen.add(key)
        yield dict(swap_ab=1, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=2, a_mode=amode,
                   w_lds=0, w_layout=1)


def row_tiles(fmt, N, layout):
    """Decode row tiles (tile_n) that spread N over the 256 compute units
    more evenly than the waves' 16-row groups do (FP8_Dynamic, W8A8_INT8 and
    Block_FP8 linears; 16, 32 and 64 rows are what plain plans already
    cover): the smallest multiple of 8 rows that gives at most 256
    workgroups and the next one, and every multiple of 8 up to 120 that
    gives a whole number of workgroups per compute unit.  None where a plain
    plan already does that."""
    if fmt not in (ql.FP8_DYNAMIC, ql.W8A8_INT8, ql.BLOCK_FP8) or layout == 4:
        return []
    if any(N % (256 * r) == 0 for r in (16, 32, 64)):
        return []                         # plain plans already give every compute unit the same rows
    rt = -(-(-(-N // 256)) // 8) * 8
    even = [r for r in range(24, 121, 8) if (-(-N // r)) % 256 == 0]
    return sorted({r for r in [rt, rt + 8] + even if r not in (16, 32, 64) and r <= 120})


def row_tile_candidates(fmt, M, N, K, layout):
    """Decode configurations with a row tile: waves whose row groups cover
    the tile with less than 32 rows to spare, in the activation modes of the
    layout (phase 1 form: swap_ab 1, 2-block batches)."""
    amodes = {0: (0,), 1: (1, 0), 2: (3, 2), 3: (4,), 5: (5,)}[layout]
    seen = set()
    for rt in row_tiles(fmt, N, layout):
        for (wn, rows), wk, split, amode in itertools.product(((1, 16), (1, 32), (1, 64), (2, 16), (2, 32), (4, 16)),
                                                              (1, 2, 4, 8, 16), SPLITS, amodes):
            if not rt <= wn * rows < rt + 32 or wn * wk not in (4, 8, 16):
                continue
            if layout == 0 and (wn * wk != 4 or rows > 32):
                continue                  # row-major weights: 4-wave workgroups, up to 32 rows a wave
            key = (rt, wn, wk, rows, _effective_chunks(K, split), amode)
            if key in seen:
                continue
            seen.add(key)
            yield dict(swap_ab=1, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=2,
                       a_mode=amode, w_lds=0, w_layout=1 if layout >= 1 else 0, tile_n=rt)


def phase1_candidates(fmt, M, N, K, layout=0):
    if M <= 32:
        yield from row_tile_candidates(fmt, M, N, K, layout)
    if M > 32:
        yield from tiled_candidates(M, N, K, layout)
        if M <= 64 and layout >= 1:
            yield from decode_m64_candidates(M, N, K, layout)
        return
    if layout == 4:
        # SiLU-and-mul plans: 32 rows a wave (gate and up), packed or fused activations
        for swap, (wn, wk), pf, split, amode in itertools.product(
                (0, 1), ((1, 4), (2, 2), (4, 1), (1, 8), (2, 4)), (1, 2), SPLITS,
                (2, 4) if fused_ok(fmt, M, K) else (2,)):
            yield dict(swap_ab=swap, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=32, prefetch=pf,
                       a_mode=amode, w_lds=0, w_layout=1)
        return
    if layout == 5:
        # given-amax forward plans: each workgroup quantizes its own K chunk (M x chunk <= 16384 values)
        if not amax_mode_ok(fmt, M, K):
            return
        seen = set()
        for (wn, wk), rows, split in itertools.product(WAVES_PACKED, (16, 32, 64), SPLITS):
            ch = _effective_chunks(K, split)
            G = -(-K // 128)
            if M * -(-G // min(split, G)) * 128 > 16384:
                continue
            key = (wn, wk, rows, ch)
            if key in seen:
                continue
            seen.add(key)
            yield dict(swap_ab=1, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=2, a_mode=5,
                       w_lds=0, w_layout=1)
        return
    if layout == 3:
        seen = set()
        for (wn, wk), rows, split in itertools.product(WAVES_PACKED, (16, 32, 64), SPLITS):
            key = (wn, wk, rows, _effective_chunks(K, split))
            if key in seen:
                continue
            seen.add(key)
            yield dict(swap_ab=1, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=2, a_mode=4,
                       w_lds=0, w_layout=1)
        return
    seen = set()
    waves, rows_set = (WAVES, (16, 32)) if layout == 0 else (WAVES_PACKED, (16, 32, 64))
    amodes = (3, 2) if layout == 2 else (1, 0)
    for (wn, wk), rows, split, alds, wlds in itertools.product(waves, rows_set, SPLITS, amodes,
                                                              (1, 0) if layout == 0 else (0,)):
        ch = _effective_chunks(K, split)
        key = (wn, wk, rows, ch, alds, wlds)
        if key in seen:
            continue
        seen.add(key)
        yield dict(swap_ab=1, split_k=split, waves_n=wn, waves_k=wk, rows_per_wave=rows, prefetch=2, a_mode=alds,
                   w_lds=wlds, w_layout=1 if layout >= 1 else 0)


class Timer:
    """Times plans for one (format, N, K, operand layouts) on rotated weight copies.

    layout 0: row-major W_q and A_q; 1: packed W_q, row-major A_q; 2: packed W_q and A_q;
    3: packed W_q, whole forward (quantizer + GEMM, or the fused launch) timed;
    4: as 3 for SiLU-and-mul plans of a merged gate/up weight (output [M, N/2]);
    5: as 3 for an input whose per-token amax is given (qlinear_forward_amax)."""

    def __init__(self, fmt, N, K, x, w, stream, layout=0, max_copies=48):
        self.fmt, self.N, self.K, self.layout = fmt, N, K, layout
        w_q, w_s = ql.quantize_weight(fmt, w.cuda())
        if layout >= 1:
            w_q = ql.pack_weight_fp4(w_q) if fmt == ql.MXFP4 else ql.pack_weight(w_q)
            if fmt in ql.MX_FORMATS:
                w_s = ql.pack_mx_scales(w_s)      # MX plans read the scales in lane order
        self.copies = min(max_copies, max(2, -(-(1 << 30) // (N * K))))
        self.wq = torch.empty((self.copies,) + tuple(w_q.shape), dtype=w_q.dtype, device="cuda")
        self.ws = torch.empty((self.copies,) + tuple(w_s.shape), dtype=w_s.dtype, device="cuda")
        self.wq[:] = w_q
        self.ws[:] = w_s
        self.x = x.cuda()
        self.stream = stream

    def measure(self, plan, M, reps=5):
        """Median per-launch microseconds and the output of one launch."""
        fmt, s = self.fmt, self.stream
        xm = self.x[:M].contiguous()
        if self.layout >= 3:
            a_q = ql.act_buffer(plan)
            a_s = ql.act_scale_buffer(plan)
        elif self.layout == 2:
            a_q, a_s = ql.quantize_act_packed(fmt, xm)
        else:
            a_q, a_s = ql.quantize_act(fmt, xm)
        y = torch.empty(M, self.N // 2 if self.layout == 4 else self.N, dtype=torch.bfloat16, device="cuda")
        wsp = plan.new_workspace()
        R = self.copies
        if self.layout == 5:
            # one amax buffer per launch of the graph (each consumer clears its
            # own), refilled before every replay
            # (the maxima in replica 0; the consumer reads every replica)
            mag = (xm.view(torch.int16).to(torch.int32) & 0x7FFF) << 16
            words = torch.zeros(R, ql.AMAX_BUFFER_BYTES // 4, dtype=torch.int32, device="cuda")
            words[:, :M] = mag.max(dim=1).values
            amax0 = words.clone()

        def one(c, stream=None):
            if self.layout == 5:
                ql.qlinear_forward_amax(plan, xm, words[c], a_q, a_s, self.wq[c], self.ws[c], y, wsp, stream=stream)
            elif self.layout >= 3:
                ql.qlinear_forward(plan, xm, a_q, a_s, self.wq[c], self.ws[c], y, wsp, stream=stream)
            else:
                ql.qlinear_run(plan, a_q, a_s, self.wq[c], self.ws[c], y, wsp, stream=stream)
        # one eager launch first: a configuration that cannot launch fails here,
        # not later inside a captured graph
        one(0)
        torch.cuda.synchronize()
        if self.layout == 5:
            words.copy_(amax0)
        with torch.cuda.stream(s):
            ql.qlinear_graph_begin(s)
            for c in range(R):
                one(c, stream=s)
            g = ql.qlinear_graph_end(s)
        g.launch(s)
        s.synchronize()
        ts = []
        for _ in range(reps):
            if self.layout == 5:
                with torch.cuda.stream(s):
                    words.copy_(amax0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.launch(s)
            e1.record(s)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / R)
        ts.sort()
        return ts[len(ts) // 2], y.clone()


def _agrees(fmt, y, ref):
    if fmt == ql.W8A8_INT8:
        return torch.equal(y, ref)
    d = (y.float() - ref.float()).abs().max().item()
    m = ref.float().abs().max().item()
    return d <= 1e-2 * max(m, 1e-30)


def _variant_rank(cfg):
    """Standard (0) before Swap-AB (1) before Split-K (2)."""
    if cfg["split_k"] == 1:
        return 0 if cfg["swap_ab"] == 0 else 1
    return 2


def choose(results, tie=0.02):
    """Fastest candidate, except that anything within `tie` of it is ranked by
    variant (Standard > Swap-AB > Split-K) and then by smaller split."""
    best_us = min(u for u, _ in results)
    near = [r for r in results if r[0] <= best_us * (1 + tie)]
    near.sort(key=lambda r: (_variant_rank(r[1]), r[1]["split_k"], r[0]))
    return near[0]


def sweep_point(timer, fmt, M, N, K, log=print, top=6):
    results = []
    ref = None
    cands = list(phase1_candidates(fmt, M, N, K, timer.layout))
    if timer.layout in (3, 5):
        # the unfused contender: the packed-activation plan (table entry or heuristic)
        cands.insert(0, dict(ql.qlinear_plan_layouts(fmt, M, N, K, 1, 1).config))
    for cfg in cands:
        plan = None
        # decode shapes too large for 2-block batches are instantiated with 1-block ones
        for pf in ((cfg["prefetch"],) if cfg.get("algo") == ql.ALGO_TILED else (2, 1)):
            try:
                cfg = dict(cfg, prefetch=pf)
                plan = (ql.qlinear_plan_glu_with_config if timer.layout == 4 else ql.qlinear_plan_with_config)(
                    fmt, M, N, K, cfg)
                break
            except ql.QLinearError:
                continue
        if plan is None:
            continue
        cfg = dict(cfg, split_k=plan.config["split_k"])
        try:
            us, y = timer.measure(plan, M)
        except ql.QLinearError as e:
            log("  SKIP (does not launch: %s): %s" % (e, cfg))
            continue
        if ref is None:
            ref = y
        elif not _agrees(fmt, y, ref):
            log("  DROP (disagrees): %s" % cfg)
            continue
        results.append((us, cfg))
    results.sort(key=lambda t: t[0])
    seen = {tuple(sorted(c.items())) for _, c in results}
    # the tiled space is searched whole in phase 1; decode candidates get a second pass
    for _, base in [r for r in results if r[1].get("algo", ql.ALGO_DECODE) == ql.ALGO_DECODE][:top]:
        for swap, pf in itertools.product((0, 1), (1, 2, 4)):
            cfg = dict(base, swap_ab=swap, prefetch=pf)
            k = tuple(sorted(cfg.items()))
            if k in seen:
                continue
            seen.add(k)
            try:
                plan = (ql.qlinear_plan_glu_with_config if timer.layout == 4 else ql.qlinear_plan_with_config)(
                    fmt, M, N, K, cfg)
                us, y = timer.measure(plan, M)
            except ql.QLinearError:
                continue
            if not _agrees(fmt, y, ref):
                log("  DROP (disagrees): %s" % cfg)
                continue
            results.append((us, cfg))
    chosen = choose(results)
    results.sort(key=lambda t: t[0])
    return [chosen] + [r for r in results if r is not chosen]


def table_line(fmt, M, N, K, cfg, us, kind=""):
    c = ql.make_config(**cfg)
    return "%d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %.3f%s" % (
        fmt, M, N, K, c["algo"], c["swap_ab"], c["split_k"], c["waves_n"], c["waves_k"], c["rows_per_wave"],
        c["prefetch"], c["a_mode"], c["w_lds"], c["w_layout"], c["tile_m"], c["tile_n"], us,
        (" " + kind) if kind else "")


def _entry_key(line):
    """(format, M, N, K, weight layout, activation class, kind) of a table line:
    the key the planner looks entries up by."""
    f = line.split()
    a_mode = int(f[11])
    kind = f[17] if len(f) > 17 else ""
    return (f[0], f[1], f[2], f[3], f[13], "packed" if a_mode >= 2 else "rowmajor", kind)


def merge_tables(base, update, out):
    """Write `out`: the entries of `base`, each replaced by the entry of
    `update` with the same key where there is one, plus `update`'s new keys.
    Returns the number of entries taken from `update`."""
    def entries(path):
        return [l.rstrip("\n") for l in open(path) if l.strip() and not l.startswith("#")]
    new = {}
    for l in entries(update):
        new[_entry_key(l)] = l
    lines, used = [], set()
    for l in open(base):
        if l.strip() and not l.startswith("#"):
            k = _entry_key(l)
            if k in new:
                l = new[k] + "\n"
                used.add(k)
        lines.append(l if l.endswith("\n") else l + "\n")
    added = [new[k] + "\n" for k in new if k not in used]
    body = [l for l in lines if not l.startswith("# sweep wall time")]
    tail = [l for l in lines if l.startswith("# sweep wall time")]
    with open(out, "w") as f:
        f.writelines(body + added + ["# merged %d entries of a sweep (%s)\n" % (len(new), os.path.basename(update))]
                     + tail)
    return len(new)


def main(argv=None):
    ap = argparse.ArgumentParser(description="offline per-shape sweep")
    ap.add_argument("--workloads", default=",".join(c.name for c in decode_workloads()))
    ap.add_argument("--out", default=ql.DEFAULT_TABLE)
    ap.add_argument("--ms", default=None, help="comma list overriding the token counts")
    ap.add_argument("--shapes", default=None, help="comma list of shape labels to sweep (default: every shape)")
    ap.add_argument("--merge", default=None, metavar="TABLE",
                    help="after the sweep, write TABLE with this sweep's entries replacing its entries of the "
                         "same (format, M, N, K, operand layouts, kind)")
    ap.add_argument("--layouts", default="0,1,2,3,4,5",
                    help="operand layouts to tune: 0 row-major W and A, 1 packed W, 2 packed W and A, "
                         "3 forward plans (packed W; fused quantization or not), 4 SiLU-and-mul forward plans "
                         "of the gate_up shapes, 5 given-amax forward plans of the down shapes (the input is the "
                         "SiLU-and-mul output, whose per-token amax the gate_up epilogue folds)")
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    ql.load_default_table()     # forward tuning starts from the packed-activation entries
    t_start = time.time()
    hdr = ["# qlinear sweep table: fmt M N K algo swap_ab split_k waves_n waves_k rows_per_wave prefetch "
           "a_mode w_lds w_layout tile_m tile_n time_us",
           "# device: %s; hip %s; torch %s" % (torch.cuda.get_device_name(0), torch.version.hip, torch.__version__),
           "# written %s" % datetime.datetime.utcnow().strftime("%Y-%m-%d %H:%M UTC")]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    n = 0
    with open(args.out, "w") as f:
        f.write("\n".join(hdr) + "\n")
        for name in args.workloads.split(","):
            wl = config_by_name(name)
            ms = [int(m) for m in args.ms.split(",")] if args.ms else list(wl.ms)
            for (lab, N, K) in wl.shapes:
                if args.shapes and lab not in args.shapes.split(","):
                    continue
                x, w = make_inputs(K, N, max(ms), wl.sigma_w, seed=wl.seed)
                for layout in [int(v) for v in args.layouts.split(",")]:
                    lms = [m for m in ms if (layout != 3 or fused_ok(wl.fmt, m, K))
                           and (layout != 5 or amax_mode_ok(wl.fmt, m, K))]
                    if layout == 4 and (lab != "gate_up" or N % 32):
                        continue        # SiLU-and-mul plans: the merged gate/up projection only
                    if layout == 5 and lab != "down":
                        continue        # given-amax plans: the projection fed by the SiLU-and-mul output
                    if wl.fmt in ql.MX_FORMATS and layout != 2:
                        continue        # MX plans take packed weights and packed activations only
                    if not lms:
                        continue
                    timer = Timer(wl.fmt, N, K, x, w, stream, layout=layout)
                    for M in lms:
                        t0 = time.time()
                        res = sweep_point(timer, wl.fmt, M, N, K)
                        us, cfg = res[0]
                        f.write(table_line(wl.fmt, M, N, K, cfg, us,
                                           kind={3: "fwd", 4: "glu", 5: "amx"}.get(layout, ""))
                                + "\n")
                        f.flush()
                        n += 1
                        print("%-26s %-8s L%d M=%-3d best %.3f us (%s)  [%d cands, %.1fs]" % (
                            wl.name, lab, layout, M, us, cfg, len(res), time.time() - t0), flush=True)
                    del timer
                    torch.cuda.empty_cache()
        f.write("# sweep wall time %.0f s\n" % (time.time() - t_start))
    print("wrote %d entries to %s" % (n, args.out))
    if args.merge:
        k = merge_tables(args.merge, args.out, args.merge)
        print("merged: %d entries of %s replaced or added in %s" % (k, args.out, args.merge))


if __name__ == "__main__":
    main()
