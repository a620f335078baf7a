"""Decode quantized-linear benchmark on one MI355X.

Metric: µs per GEMM and achieved HBM GB/s (fraction of the 8 TB/s peak) at
decode token counts M = 1..32.  Workload (default): FP8_Dynamic (OCP E4M3,
per-token activation / per-channel weight scales) on the dense 8B-class
projections -- QKV 6144x4096, O 4096x4096, gate_up 24576x4096, down
4096x12288 -- at M in {1, 2, 4, 8, 16, 24, 32}: 28 linears per step.

One step = the whole hot path for every point: dynamic activation quantizer,
then the planned GEMM (standard / split-K / swap-AB from the sweep table),
captured once into hipGraphs and replayed.  By default the weights are packed
offline (qlinear_pack_weight) and each point runs its forward plan: where the
sweep found it faster, one launch that quantizes inside the GEMM (fused
quantization), else the quantizer writing packed activations and then the
GEMM -- either way every operand load of the GEMM is a contiguous kilobyte.
--layout selects the unfused packed or the row-major paths instead.  --workload fp8_dynamic_14b_large_m runs the
M = 64..4096 points through the tiled kernel and prices them against the
matrix-core peak instead of HBM.  Inputs are synthetic and resident
in HBM before timing.  Every GEMM of a step reads its own copy of the weights
(at least 1 GiB of copies per shape), so the 256 MB Infinity Cache cannot
serve them: the measured bandwidth is HBM bandwidth.

Output: one JSON line (see the keys below); per-point kernel timings ride
along under "per_point".
"""

import argparse
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense e4m3 (and int8) matrix-core peak
METRIC = "µs/GEMM & achieved HBM GB/s (fraction of peak), M=1–32, fp8/int8 decode shapes"


def algorithmic_bytes(fmt, M, N, K):
    """Bytes the method must move for one GEMM (weights, scales, activations, output)."""
    if fmt == 2:   # Block_FP8
        return N * K + 4 * (-(-N // 128)) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * N
    if fmt == 3:   # MXFP8: one E8M0 byte per 32 codes on both operands
        return N * K + N * (K // 32) + M * K + M * (K // 32) + 2 * M * N
    if fmt == 4:   # MXFP4 weights (half a byte a value), MXFP8 activations
        return N * K // 2 + N * (K // 32) + M * K + M * (K // 32) + 2 * M * N
    return N * K + 4 * N + M * K + 4 * M + 2 * M * N


def fused_kernel_bytes(fmt, M, N, K):
    """Bytes one fused-quantization GEMM launch must move: weights and their
    scales, bf16 X in, the codes and scales it hands back, and Y -- the
    unfused launch's bytes (codes and scales written instead of read) plus X."""
    return algorithmic_bytes(fmt, M, N, K) + 2 * M * K


def quantizer_bytes(fmt, M, K):
    if fmt in (3, 4):
        return 2 * M * K + M * K + M * (K // 32)
    return 2 * M * K + M * K + (4 * M * (K // 128) if fmt == 2 else 4 * M)


PKG = os.path.join(ROOT, "quantized_gemm_decode_amd")
LAYOUT_NAMES = {"fused": "packed weights, forward plans (quantization fused into the GEMM where faster)",
                "packed": "packed weights and activations", "packedw": "packed weights, row-major activations",
                "rowmajor": "row-major weights and activations"}
# (w_layout, a_packed) of qlinear_plan_layouts per --layout
LAYOUT_PLAN = {"fused": (1, 2), "packed": (1, 1), "packedw": (1, 0), "rowmajor": (0, 0)}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sources_digest():
    """sha256 over the HIP/C++ sources and the shipped sweep table: a recorded
    counter reading is valid only for the code (and plans) it was taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files.append(os.path.join(PKG, "tables", "decode_table.txt"))
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload, layout):
    return os.path.join(PROFILES, "decode_gemm_%s_%s_hbm_traffic.txt" % (workload, layout))


def recorded_traffic(workload, layout):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated) of one launch of every GEMM
    of the step, from the committed counter summary; None if absent or stale."""
    path = traffic_file(workload, layout)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    for line in open(path):
        f = line.split()
        if len(f) == 2 and not line.startswith("#"):
            kv[f[0]] = f[1]
    if kv.get("kernel_sources_sha256") != kernel_sources_digest():
        return None, "kernel sources changed since the counters were taken"
    return int(kv["traffic_bytes_per_step"]), "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, copy-calibrated"


def is_fused_instantiation(name):
    """A qgemm_decode_kernel<FMT, SWAP, MT, RG, NW, PF, AL, WM, GLU> name with AL = 4."""
    if "qgemm_decode_kernel<" not in name:
        return False
    args = name.split("qgemm_decode_kernel<", 1)[1].split(">", 1)[0].split(",")
    return len(args) == 9 and args[6].strip() == "4"


def pmc_summary(workload, layout, fetch_csv, write_csv):
    """Summarise two rocprofv3 --pmc runs of --profile-pass into the traffic record."""
    import csv
    from workloads import config_by_name, decode_points
    wl = config_by_name(workload)

    def load(path):
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows

    fr, wr = load(fetch_csv), load(write_csv)
    assert len(fr) == len(wr)
    cal = (256 << 20) / 1024.0                         # KiB read and written by each calibration copy
    fetch_copy = sum(float(r["Counter_Value"]) for r in fr[-3:]) / 3
    write_copy = sum(float(r["Counter_Value"]) for r in wr[-3:]) / 3
    kf, kw = cal / fetch_copy, cal / write_copy
    gem = [(float(a["Counter_Value"]), float(b["Counter_Value"]), a["Kernel_Name"].split("(")[0])
           for a, b in zip(fr, wr) if "qgemm" in a["Kernel_Name"]]
    pts = decode_points(wl)
    gem = gem[-3 * len(pts):]
    lines = ["# HBM traffic of the decode GEMM kernels, workload %s, %s" % (workload, LAYOUT_NAMES[layout]),
             "# commands (run from /tmp with TMPDIR=/tmp):",
             "#   rocprofv3 --pmc FETCH_SIZE -f csv -d <dir_f> -o fetch -- python3 <repo>/bench.py --workload %s "
             "--layout %s --profile-pass" % (workload, layout),
             "#   rocprofv3 --pmc WRITE_SIZE -f csv -d <dir_w> -o write -- python3 <repo>/bench.py --workload %s "
             "--layout %s --profile-pass" % (workload, layout),
             "#   python3 bench.py --workload %s --layout %s --pmc-summary <dir_f>/fetch_counter_collection.csv "
             "<dir_w>/write_counter_collection.csv" % (workload, layout),
             "# calibration: a 256 MiB device copy reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB per dispatch"
             % (fetch_copy, write_copy),
             "#   -> bytes = FETCH_SIZE * %.4f KiB, WRITE_SIZE * %.4f KiB" % (kf, kw),
             "# per GEMM: mean of 3 dispatches on distinct weight copies (a fused-quantization launch's",
             "# algorithmic bytes include bf16 X in and the codes and scales out)",
             "# shape    M    algorithmic_B   fetched_B  written_B  traffic/alg"]
    tot_a = tot_t = 0
    for i, (lab, N, K, M) in enumerate(pts):
        g = gem[3 * i:3 * i + 3]
        fb = sum(x[0] for x in g) / 3 * 1024 * kf
        wb = sum(x[1] for x in g) / 3 * 1024 * kw
        ab = (fused_kernel_bytes if is_fused_instantiation(g[0][2]) else algorithmic_bytes)(wl.fmt, M, N, K)
        tot_a += ab
        tot_t += fb + wb
        lines.append("# %-8s %-4d %13d %11.0f %10.0f  %.4f" % (lab, M, ab, fb, wb, (fb + wb) / ab))
    lines += ["kernel_sources_sha256 %s" % kernel_sources_digest(),
              "algorithmic_bytes_per_step %d" % tot_a,
              "traffic_bytes_per_step %d" % round(tot_t),
              "traffic_over_algorithmic %.4f" % (tot_t / tot_a)]
    return "\n".join(lines) + "\n"


def trace_summary(workload, layout, trace_csv, stats_csv, bench_json, ref_json=None):
    """Per-point kernel durations from a rocprofv3 --kernel-trace run of this script,
    next to the HIP-event per-launch times the same run printed."""
    import csv
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    bench = None
    for line in open(bench_json):
        if line.startswith("{"):
            bench = json.loads(line)
    pp = bench["per_point"]
    # The per-point timing phase ends the run: for each point a block of
    # (3 warm-up + kernel-reps timed) graph replays of R GEMM launches, in
    # point order (the unfused points' quantizer runs between blocks and is
    # skipped).  Slice the GEMM launches by those counts from the end.
    reps = bench.get("kernel_reps", 5)
    gemm = [r for r in rows if "qgemm" in r["Kernel_Name"]]
    sizes = [(3 + reps) * p["R"] for p in pp]
    tail = gemm[-sum(sizes):]
    runs, at = [], 0
    for n in sizes:
        runs.append((tail[at:at + n], n * reps // (3 + reps)))
        at += n
    lines = ["# rocprofv3 kernel trace of the GEMM kernels, workload %s, %s" % (workload, LAYOUT_NAMES[layout]),
             "# command (from /tmp with TMPDIR=/tmp):",
             "#   rocprofv3 --kernel-trace --stats -f csv -d <dir> -o bench -- python3 <repo>/bench.py --workload %s "
             "--layout %s --steps %d --warmup %d --kernel-reps %d --no-cpu-baseline"
             % (workload, layout, bench["steps"], bench["warmup"], bench.get("kernel_reps", 5)),
             "#   python3 bench.py --workload %s --layout %s --trace-summary <dir>/bench_kernel_trace.csv "
             "<dir>/bench_kernel_stats.csv <stdout of the command above> [--trace-ref <json of a plain run>]"
             % (workload, layout),
             "# per point: rocprof = mean kernel duration over the timed replays (last kernel-reps x R launches);",
             "# hip_events = the same run's HIP-event time per launch (median of replays / R)",
             "# shape    M    kernel_instantiation                                   rocprof_us  hip_events_us  ratio"]
    tot_r = tot_e = 0.0
    per_us = []
    for p, (run, n_timed) in zip(pp, runs):
        timed = run[-n_timed:]
        us = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed) / len(timed) / 1e3
        name = run[0]["Kernel_Name"].split("(")[0].replace("void ", "").replace("qlk::", "")
        tot_r += us
        tot_e += p["us"]
        per_us.append(us)
        lines.append("# %-8s %-4d %-54s %9.3f %13.3f  %.3f" % (p["shape"], p["M"], name, us, p["us"], p["us"] / us))
    lines.append("# sum over the %d points: rocprof %.2f us, hip events %.2f us (ratio %.3f)" % (len(pp), tot_r, tot_e,
                                                                                              tot_e / tot_r))
    rl = bench["roofline"]
    if rl["unit"] == "GB/s":
        ach = rl["algorithmic_bytes"] / (tot_r * 1e-6) / 1e9
        what = "algorithmic bytes of every point"
    else:
        big = [(p, us) for p, us in zip(pp, per_us) if p["M"] >= 1024]
        ach = sum(2.0 * p["M"] * p["N"] * p["K"] for p, _ in big) / (sum(us for _, us in big) * 1e-6) / 1e12
        what = "2*M*N*K of the M >= 1024 points"
    lines.append("# achieved (%s / rocprof durations): %.1f %s; bench roofline.achieved: %.1f %s"
                 % (what, ach, rl["unit"], rl["achieved"], rl["unit"]))
    if ref_json:
        ref = json.loads(open(ref_json).read().strip().splitlines()[-1])
        ref_pp = {(q["shape"], q["M"]): q["us"] for q in ref["per_point"]}
        tot_ref = sum(ref_pp.get((p["shape"], p["M"]), float("nan")) for p in pp)
        lines.append("# the same bench without the profiler (%s): roofline.achieved %.1f %s; its per-launch "
                     "times sum to %.2f us, %.3f x the rocprof kernel durations above"
                     % (os.path.basename(ref_json), ref["roofline"]["achieved"], ref["roofline"]["unit"], tot_ref,
                        tot_ref / tot_r))
    lines.append("# rocprofv3 --stats kernel summary (all launches of the run, every phase):")
    for line in open(stats_csv):
        lines.append("#   " + line.rstrip())
    return "\n".join(lines) + "\n"


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fp8_dynamic_8b")
    ap.add_argument("--layout", choices=("fused", "packed", "packedw", "rowmajor"), default="fused",
                    help="fused: packed weights (qlinear_pack_weight, offline) and each point's forward plan, "
                         "with the quantizer fused into the GEMM where the sweep found that faster; packed: "
                         "packed weights and activations (the quantizer writes them), two launches; packedw: "
                         "packed weights only; rowmajor: row-major both")
    ap.add_argument("--kernel-reps", type=int, default=30, help="graph replays per point for kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--table", default=None, help="sweep table path (default: the packaged table)")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic record from two rocprofv3 --pmc runs of --profile-pass, and exit")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_CSV", "STATS_CSV", "BENCH_STDOUT"),
                    help="print per-point rocprofv3 kernel durations next to the HIP-event times, and exit")
    ap.add_argument("--trace-ref", default=None, metavar="BENCH_JSON",
                    help="with --trace-summary: an unprofiled run's JSON line to set beside the trace")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for hardware-counter runs: launch each point's quantize+GEMM eagerly on 3 weight "
                         "copies, then a plain 256 MiB device copy 3 times (the counters' calibration), and exit")
    ap.add_argument("--glu", action="store_true",
                    help="time the workload's gate_up points two ways -- the forward plan writing Y [M, N], and "
                         "the SiLU-and-mul plan writing silu(gate)*up [M, N/2] -- print one JSON line, and exit")
    return ap.parse_args(argv)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only (--gpus %d requested); the linear shards "
              "column-wise across GPUs with no exchange, so per-GPU work is one GPU's share." % args.gpus,
              file=sys.stderr)
        return 2

    if args.trace_summary:
        sys.stdout.write(trace_summary(args.workload, args.layout, *args.trace_summary, ref_json=args.trace_ref))
        return 0
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(args.workload, args.layout, *args.pmc_summary))
        return 0

    import numpy as np
    import torch

    import quantized_gemm_decode_amd as ql
    from workloads import config_by_name, decode_points, make_inputs

    if not os.path.exists(os.path.join(ROOT, "quantized_gemm_decode_amd", "libqlinear.so")):
        from quantized_gemm_decode_amd import build as b
        b.build()
    torch.cuda.set_device(0)
    n_table = ql.qlinear_table_load(args.table) if args.table else ql.load_default_table()

    wl = config_by_name(args.workload)
    fmt = wl.fmt
    points = decode_points(wl)
    dev = "cuda"
    stream = torch.cuda.Stream()

    # ------------------------------------------------ inputs, weights, copies
    shapes = {}
    for (lab, N, K) in wl.shapes:
        x, w = make_inputs(K, N, max(wl.ms), wl.sigma_w, seed=wl.seed)
        wd = w.to(dev)
        w_q, w_s = ql.quantize_weight(fmt, wd)
        if args.layout != "rowmajor":           # offline, like the quantization itself
            w_q = ql.pack_weight_fp4(w_q) if fmt == ql.MXFP4 else ql.pack_weight(w_q)
            if fmt in ql.MX_FORMATS:
                w_s = ql.pack_mx_scales(w_s)   # MX plans read the scales in lane order
        del wd
        copies = max(2, -(-(1 << 30) // (N * K)))
        wq_all = torch.empty((copies,) + tuple(w_q.shape), dtype=w_q.dtype, device=dev)
        ws_all = torch.empty((copies,) + tuple(w_s.shape), dtype=w_s.dtype, device=dev)
        wq_all[:] = w_q
        ws_all[:] = w_s
        shapes[lab] = dict(N=N, K=K, x=x.to(dev), wq=wq_all, ws=ws_all, copies=copies)
    torch.cuda.synchronize()

    # ------------------------------------------------ per-point plans and buffers
    pts = []
    for (lab, N, K, M) in points:
        sh = shapes[lab]
        w_layout, a_packed = LAYOUT_PLAN[args.layout]
        plan = ql.qlinear_plan_layouts(fmt, M, N, K, w_layout, a_packed)
        cfg, facts = plan.info()
        fused = cfg["algo"] == ql.ALGO_DECODE and cfg["a_mode"] == 4
        pts.append(dict(lab=lab, N=N, K=K, M=M, plan=plan, cfg=cfg, facts=facts,
                        x=sh["x"][:M].contiguous(),
                        a_q=ql.act_buffer(plan, dev),
                        a_s=ql.act_scale_buffer(plan, dev),
                        y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                        wsp=plan.new_workspace(dev), fused=fused,
                        bytes=algorithmic_bytes(fmt, M, N, K), qbytes=quantizer_bytes(fmt, M, K),
                        kbytes=fused_kernel_bytes(fmt, M, N, K) if fused else algorithmic_bytes(fmt, M, N, K)))

    if args.profile_pass:
        return profile_pass(ql, fmt, pts, shapes, stream)
    if args.glu:
        return glu_pass(ql, wl, pts, shapes, stream, args)

    # ------------------------------------------------ step graphs (quantize + GEMM per point)
    n_graphs = 8
    graphs = []
    with torch.cuda.stream(stream):
        for gi in range(n_graphs):
            ql.qlinear_graph_begin(stream)
            for pi, p in enumerate(pts):
                sh = shapes[p["lab"]]
                c = (gi * len(pts) + pi) % sh["copies"]
                ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"],
                                   p["wsp"], stream=stream)
            graphs.append(ql.qlinear_graph_end(stream))
    stream.synchronize()

    for i in range(args.warmup):
        graphs[i % n_graphs].launch(stream)
    stream.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % n_graphs].launch(stream)
    t1.record(stream)
    stream.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / args.steps
    step_bytes = sum(p["bytes"] + p["qbytes"] for p in pts)
    value = step_bytes / (step_ms * 1e-3) / 1e9

    # ------------------------------------------------ per-point GEMM kernel timing (HIP events)
    # R back-to-back launches of the point's GEMM kernel: qlinear_run, or for a
    # fused plan qlinear_forward (which is that one kernel launch)
    reps = args.kernel_reps
    per_point = []
    tot_bytes = tot_us = tot_flops = 0.0
    for p in pts:
        sh = shapes[p["lab"]]
        R = min(sh["copies"], 64)
        with torch.cuda.stream(stream):
            ql.qlinear_graph_begin(stream)
            for c in range(R):
                if p["fused"]:
                    ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"],
                                       p["wsp"], stream=stream)
                else:
                    ql.qlinear_run(p["plan"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"], p["wsp"],
                                   stream=stream)
            g = ql.qlinear_graph_end(stream)
            if p["fused"]:
                pass
            elif p["cfg"]["a_mode"] >= 2:
                ql.qlinear_quantize_act_packed(fmt, p["x"], p["a_q"], p["a_s"], stream=stream)
            else:
                ql.qlinear_quantize_act(fmt, p["x"], p["a_q"], p["a_s"], stream=stream)
        for _ in range(3):
            g.launch(stream)
        stream.synchronize()
        samples = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.launch(stream)
            e1.record(stream)
            e1.synchronize()
            samples.append(e0.elapsed_time(e1) * 1e3 / R)
        us = float(np.median(samples))
        gbs = p["kbytes"] / (us * 1e-6) / 1e9
        flops = 2.0 * p["M"] * p["N"] * p["K"]
        tot_bytes += p["kbytes"]
        tot_flops += flops
        tot_us += us
        per_point.append(dict(shape=p["lab"], M=p["M"], N=p["N"], K=p["K"], us=round(us, 3),
                              us_p10=round(float(np.percentile(samples, 10)), 3),
                              us_p90=round(float(np.percentile(samples, 90)), 3),
                              GBs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                              TFLOPs=round(flops / (us * 1e-6) / 1e12, 1), algo=p["cfg"]["algo"],
                              variant=("split-k" if p["facts"]["chunks"] > 1 else
                                       ("swap-ab" if p["cfg"]["swap_ab"] else "standard")),
                              split=p["facts"]["chunks"], swap_ab=p["cfg"]["swap_ab"],
                              fused_quant=p["fused"], kernel_bytes=int(p["kbytes"]), R=R,
                              source=p["facts"]["source"]))
        del g
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    traffic, traffic_note = recorded_traffic(wl.name, args.layout)
    if max(wl.ms) <= 32:
        ceil_gbs = stream_ceiling(ql, per_point, stream, reps)
        roofline = {"kernel": "qgemm_decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": int(tot_bytes), "traffic_source": traffic_note,
                    "stream_ceiling": {"achieved": round(ceil_gbs, 1), "frac": round(ceil_gbs / HBM_PEAK_GBS, 4),
                                       "kernel_vs_ceiling": round(achieved / ceil_gbs, 4),
                                       "note": "a plain streaming read of each point's kernel bytes "
                                               "(qlinear_stream_read, best of 5 grids x 2 load depths), timed like the GEMMs; "
                                               "per point under ceiling_us"},
                    "note": "algorithmic bytes of one launch of each of the %d GEMM kernels (a fused-"
                            "quantization launch also reads bf16 X and writes the codes and scales) / sum of "
                            "their per-launch durations (HIP events around graph replays of back-to-back "
                            "launches); traffic is the HBM bytes those same %d launches moved"
                            % (len(pts), len(pts))}
    else:
        # token counts in the hundreds and thousands: the tiled kernel is matrix-core bound
        big = [q for q in per_point if q["M"] >= 1024]
        fl = sum(2.0 * q["M"] * q["N"] * q["K"] for q in big)
        t = sum(q["us"] for q in big) * 1e-6
        tflops = fl / t / 1e12
        roofline = {"kernel": "qgemm_tiled_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                    "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4),
                    "traffic": traffic, "traffic_source": traffic_note,
                    "note": "2*M*N*K of one launch of each M >= 1024 GEMM / sum of their per-launch durations; "
                            "the M = 64 and 256 points are HBM- or ridge-bound and are reported per point"}

    # ------------------------------------------------ CPU oracle baseline (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, shapes, args.cpu_budget_s)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "kernel_reps": args.kernel_reps,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "int8", 4: "fp8_e4m3 x fp4_e2m1"}.get(fmt, "fp8_e4m3"),
        "data": "synthetic (seeded N(0,1) activations with 1%% x20 outlier channels, N(0,%g) weights)" % wl.sigma_w,
        "config": {"workload": wl.name, "format": ql.FORMAT_NAMES[fmt],
                   "shapes": ["%s %dx%d" % s for s in wl.shapes], "token_counts": list(wl.ms),
                   "gemms_per_step": len(pts), "graph_replay": True, "table_entries": n_table,
                   "weight_layout": args.layout,
                   "fused_quant_points": sum(1 for p in pts if p["fused"]),
                   "us_per_gemm_step_avg": round(step_ms * 1e3 / len(pts), 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_point": per_point,
        "wall_s": round(wall, 3),
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")
    return 0


def stream_ceiling(ql, per_point, stream, reps):
    """The streaming-read ceiling of every point: the fastest plain read
    (qlinear_stream_read, best of 5 grids x 2 load depths) of the point's kernel bytes,
    timed as the GEMM is -- HIP events around graph replays of R back-to-back
    launches on distinct offsets of a 1 GiB buffer, so the Infinity Cache
    cannot serve it.  Sets per_point[i]["ceiling_us"]; returns the ceiling's
    GB/s over all points (their bytes / their ceiling times)."""
    import numpy as np
    import torch
    pool = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    best = {}
    for q in per_point:
        nb = q["kernel_bytes"] // 16 * 16
        if nb not in best:
            span = -(-nb // 4096) * 4096
            R = max(2, min(64, (1 << 30) // span))
            times = []
            for wg, lif in itertools.product((256, 512, 1024, 2048, 4096), (4, 8)):
                with torch.cuda.stream(stream):
                    ql.qlinear_graph_begin(stream)
                    for c in range(R):
                        ql.qlinear_stream_read(pool[c * span:], nb, wg, sink, loads_in_flight=lif, stream=stream)
                    g = ql.qlinear_graph_end(stream)
                for _ in range(3):
                    g.launch(stream)
                stream.synchronize()
                samples = []
                for _ in range(reps):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    g.launch(stream)
                    e1.record(stream)
                    e1.synchronize()
                    samples.append(e0.elapsed_time(e1) * 1e3 / R)
                times.append(float(np.median(samples)))
                del g
            best[nb] = min(times)
        q["ceiling_us"] = round(best[nb], 3)
    del pool
    tot_b = sum(q["kernel_bytes"] for q in per_point)
    tot_us = sum(best[q["kernel_bytes"] // 16 * 16] for q in per_point)
    return tot_b / (tot_us * 1e-6) / 1e9


def glu_pass(ql, wl, pts, shapes, stream, args):
    """Per-launch times of the gate_up points as a plain forward (Y [M, N]) and
    with the SiLU-and-mul epilogue (silu(gate)*up, [M, N/2]), HIP events around
    graph replays of R launches on distinct weight copies, as for the bench's
    per-point timing."""
    import numpy as np
    import torch
    fmt = wl.fmt
    out = []
    for p in pts:
        if p["lab"] != "gate_up":
            continue
        sh = shapes[p["lab"]]
        M, N, K = p["M"], p["N"], p["K"]
        R = min(sh["copies"], 64)
        res = {"M": M}
        for kind in ("plain", "glu"):
            plan = p["plan"] if kind == "plain" else ql.qlinear_plan_glu(fmt, M, N, K, 2)
            y = torch.empty(M, N if kind == "plain" else N // 2, dtype=torch.bfloat16, device="cuda")
            a_q = ql.act_buffer(plan)
            a_s = ql.act_scale_buffer(plan)
            wsp = plan.new_workspace()
            with torch.cuda.stream(stream):
                ql.qlinear_graph_begin(stream)
                for c in range(R):
                    ql.qlinear_forward(plan, p["x"], a_q, a_s, sh["wq"][c], sh["ws"][c], y, wsp, stream=stream)
                g = ql.qlinear_graph_end(stream)
            for _ in range(3):
                g.launch(stream)
            stream.synchronize()
            samples = []
            for _ in range(args.kernel_reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.launch(stream)
                e1.record(stream)
                e1.synchronize()
                samples.append(e0.elapsed_time(e1) * 1e3 / R)
            cfg = plan.config
            res[kind + "_us"] = round(float(np.median(samples)), 3)
            res[kind + "_fused_quant"] = cfg["a_mode"] == 4
            res[kind + "_config"] = "swap%d split%d waves%dx%d rows%d pf%d amode%d" % (
                cfg["swap_ab"], cfg["split_k"], cfg["waves_n"], cfg["waves_k"], cfg["rows_per_wave"],
                cfg["prefetch"], cfg["a_mode"])
            del g
        out.append(res)
    gu = [p for p in pts if p["lab"] == "gate_up"]
    print(json.dumps({"metric": "µs per gate_up forward: plain (Y [M, N]) vs SiLU-and-mul epilogue (silu(gate)*up, "
                                "[M, N/2])", "unit": "us", "workload": wl.name,
                      "shape": "gate_up %dx%d" % (gu[0]["N"], gu[0]["K"]) if gu else None,
                      "data": "synthetic", "kernel_reps": args.kernel_reps, "per_point": out}), flush=True)
    return 0


def profile_pass(ql, fmt, pts, shapes, stream):
    """Eager launches in a fixed order for per-dispatch hardware counters.

    Order: for every point, 3 x (quantize, GEMM) on weight copies 0, 1, 2;
    then 3 plain copies of 256 MiB (read 256 MiB, write 256 MiB), whose
    counter readings calibrate the byte counters."""
    import torch
    with torch.cuda.stream(stream):
        for p in pts:
            sh = shapes[p["lab"]]
            for c in range(3):
                ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"],
                                   p["wsp"], stream=stream)
            stream.synchronize()
            print("point %s M=%d N=%d K=%d bytes=%d" % (p["lab"], p["M"], p["N"], p["K"], p["bytes"]), flush=True)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        stream.synchronize()
        for _ in range(3):
            dst.copy_(src)
        stream.synchronize()
    print("copy bytes=%d" % (256 << 20), flush=True)
    return 0


def cpu_baseline(wl, shapes, budget_s):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle
    from workloads import bf16_bits, make_inputs

    n = len(os.sched_getaffinity(0))
    torch.set_num_threads(n)
    fmt = wl.fmt
    sample = []
    t_total = 0.0
    b_total = 0
    for (lab, N, K) in wl.shapes:
        x, w = make_inputs(K, N, max(wl.ms), wl.sigma_w, seed=wl.seed)
        if fmt == 4:
            w_q, s_w = oracle.mx4_quantize(bf16_bits(w))                # offline step: not timed
        elif fmt == 3:
            w_q, s_w = oracle.mx_quantize(bf16_bits(w))                 # offline step: not timed
        else:
            w_q, s_w = oracle.quantize_weight(fmt, bf16_bits(w))      # offline step: not timed
        for M in wl.ms:
            if 2.0 * M * N * K > 50e9:
                continue       # a single fp64 GEMM of minutes: outside the bounded sample
            xb = bf16_bits(x[:M])
            t0 = time.perf_counter()
            if fmt in (3, 4):
                a_q, s_a = oracle.mx_quantize(xb)
                y = (oracle.mx4_contract_exact if fmt == 4 else oracle.mx_contract_exact)(a_q, s_a, w_q, s_w)
                oracle.bf16_bits_from_f32(oracle.f32(y))
            else:
                a_q, s_a = oracle.quantize_act(fmt, xb)
                S = oracle.contract_exact(fmt, a_q, w_q)
                oracle.epilogue(fmt, S, s_a, s_w)
            dt = time.perf_counter() - t0
            t_total += dt
            b_total += algorithmic_bytes(fmt, M, N, K)
            sample.append("%s M=%d" % (lab, M))
            if t_total > budget_s:
                break
        if t_total > budget_s:
            break
    return {"value": round(b_total / t_total / 1e9, 3), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": "%s: activation quantizer + exact fp64 contraction + epilogue on %s (weights "
                      "pre-quantized, untimed); %.1f s of CPU time" % (wl.name, ", ".join(sample), t_total),
            "us_per_gemm": round(t_total / len(sample) * 1e6, 1)}


if __name__ == "__main__":
    sys.exit(main())
