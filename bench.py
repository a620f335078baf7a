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


def pmc_summary(wls, layout, fetch_csv, write_csv):
    """Summarise two rocprofv3 --pmc runs of --profile-pass into one traffic
    record per workload; returns {workload name: text}."""
    import csv
    from workloads import decode_points

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
    n_all = sum(3 * len(decode_points(wl)) for wl in wls)
    gem = gem[-n_all:]
    names = ",".join(wl.name for wl in wls) if len(wls) > 1 or wls[0].name not in DECODE_SET else wls[0].name
    if [wl.name for wl in wls] == list(DECODE_SET):
        names = "decode"
    out, at = {}, 0
    for wl in wls:
        pts = decode_points(wl)
        lines = ["# HBM traffic of the decode GEMM kernels, workload %s, %s" % (wl.name, LAYOUT_NAMES[layout]),
                 "# commands (run from /tmp with TMPDIR=/tmp):",
                 "#   rocprofv3 --pmc FETCH_SIZE -f csv -d <dir_f> -o fetch -- python3 <repo>/bench.py --workload %s "
                 "--layout %s --profile-pass" % (names, layout),
                 "#   rocprofv3 --pmc WRITE_SIZE -f csv -d <dir_w> -o write -- python3 <repo>/bench.py --workload %s "
                 "--layout %s --profile-pass" % (names, layout),
                 "#   python3 bench.py --workload %s --layout %s --pmc-summary <dir_f>/fetch_counter_collection.csv "
                 "<dir_w>/write_counter_collection.csv" % (names, layout),
                 "# calibration: a 256 MiB device copy reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB per "
                 "dispatch" % (fetch_copy, write_copy),
                 "#   -> bytes = FETCH_SIZE * %.4f KiB, WRITE_SIZE * %.4f KiB" % (kf, kw),
                 "# per GEMM: mean of 3 dispatches on distinct weight copies (a fused-quantization launch's",
                 "# algorithmic bytes include bf16 X in and the codes and scales out)",
                 "# shape    M    algorithmic_B   fetched_B  written_B  traffic/alg"]
        tot_a = tot_t = 0
        for (lab, N, K, M) in pts:
            g = gem[at:at + 3]
            at += 3
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
        out[wl.name] = "\n".join(lines) + "\n"
    return out


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
    blocks = bench["workloads"]
    pp = [dict(q, workload=b["workload"]) for b in blocks for q in b["per_point"]]
    # After the timed steps, each workload's per-point phase launches, for
    # each point, (3 warm-up + kernel-reps timed) graph replays of R GEMM
    # launches, in point order; quantizer and streaming-read timings follow
    # but launch no GEMM.  So the GEMM launches of the per-point phases are
    # the last ones of the run: slice them by those counts from the end.
    reps = bench.get("kernel_reps", 5)
    gemm = [r for r in rows if "qgemm" in r["Kernel_Name"]]
    sizes = [(3 + reps) * p["R"] for p in pp]
    tail = gemm[-sum(sizes):]
    runs, at = [], 0
    for n in sizes:
        runs.append((tail[at:at + n], n * reps // (3 + reps)))
        at += n
    lines = ["# rocprofv3 kernel trace of the GEMM kernels, workload %s, %s"
             % (bench["config"]["workload"], LAYOUT_NAMES[layout]),
             "# command (from /tmp with TMPDIR=/tmp):",
             "#   rocprofv3 --kernel-trace --stats -f csv -d <dir> -o bench -- python3 <repo>/bench.py --workload %s "
             "--layout %s --steps %d --warmup %d --kernel-reps %d --no-cpu-baseline --no-ceiling"
             % (workload, layout, bench["steps"], bench["warmup"], bench.get("kernel_reps", 5)),
             "#   python3 bench.py --workload %s --layout %s --trace-summary <dir>/bench_kernel_trace.csv "
             "<dir>/bench_kernel_stats.csv <stdout of the command above> [--trace-ref <json of a plain run>]"
             % (workload, layout),
             "# per point: rocprof = mean kernel duration over the timed replays (last kernel-reps x R launches);",
             "# hip_events = the same run's HIP-event time per launch (median of replays / R)",
             "# workload               shape    M    kernel_instantiation                                   "
             "rocprof_us  hip_events_us  ratio"]
    tot_r = tot_e = 0.0
    per_us = []
    for p, (run, n_timed) in zip(pp, runs):
        timed = run[-n_timed:]
        us = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed) / len(timed) / 1e3
        name = run[0]["Kernel_Name"].split("(")[0].replace("void ", "").replace("qlk::", "")
        tot_r += us
        tot_e += p["us"]
        per_us.append(us)
        lines.append("# %-22s %-8s %-4d %-54s %9.3f %13.3f  %.3f" % (p["workload"], p["shape"], p["M"], name, us,
                                                                   p["us"], p["us"] / us))
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
        ref_pp = {(b["workload"], q["shape"], q["M"]): q["us"] for b in ref["workloads"] for q in b["per_point"]}
        tot_ref = sum(ref_pp.get((p["workload"], p["shape"], p["M"]), float("nan")) for p in pp)
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
    ap.add_argument("--workload", default="decode",
                    help="'decode' (default): the INT8 4096x2048 linear, the FP8_Dynamic and Block_FP8 8B-class "
                         "sweeps and the W8A8_INT8 32B-class sweep, timed together; or one or more workload "
                         "names, comma-separated (e.g. fp8_dynamic_14b_large_m, mxfp8_8b)")
    ap.add_argument("--layout", choices=("fused", "packed", "packedw", "rowmajor"), default="fused",
                    help="fused: packed weights (qlinear_pack_weight, offline) and each point's forward plan, "
                         "with the quantizer fused into the GEMM where the sweep found that faster; packed: "
                         "packed weights and activations (the quantizer writes them), two launches; packedw: "
                         "packed weights only; rowmajor: row-major both")
    ap.add_argument("--kernel-reps", type=int, default=30, help="graph replays per point for kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling (for profiled runs: it launches thousands of kernels)")
    ap.add_argument("--cpu-budget-s", type=float, default=24.0, help="CPU oracle seconds, split over the workloads")
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
    ap.add_argument("--library-ref", action="store_true",
                    help="FP8_Dynamic workloads: time each point's GEMM kernel next to torch._scaled_mm "
                         "(the vendor library, rowwise scales: the same per-token x per-channel scaling) on the "
                         "same codes and weight copies; print one JSON line per workload, and exit")
    ap.add_argument("--glu", action="store_true",
                    help="time the workload's gate_up points two ways -- the forward plan writing Y [M, N], and "
                         "the SiLU-and-mul plan writing silu(gate)*up [M, N/2] -- and the gate_up -> down chain "
                         "two ways (down quantizing H in a pass of its own, or down quantizing its K chunk with the "
                         "per-token amax the SiLU-and-mul epilogue folded); print one JSON line, and exit")
    return ap.parse_args(argv)


# The decode workloads a default run measures together: the INT8 single
# linear (4096x2048 at M = 8), the FP8_Dynamic and Block_FP8 8B-class sweeps
# and the W8A8_INT8 32B-class sweep -- the fp8 / int8 decode shapes of the metric.
DECODE_SET = ("int8_linear_4096x2048", "fp8_dynamic_8b", "block_fp8_8b", "int8_32b")


def resolve_workloads(name):
    from workloads import config_by_name
    names = DECODE_SET if name == "decode" else tuple(name.split(","))
    return [config_by_name(n) for n in names]


def environment(ql, torch):
    """Versions of what the numbers were measured on."""
    import hashlib
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        prop = torch.cuda.get_device_properties(0)
        env["gpu"] = prop.name
        env["gcn_arch"] = getattr(prop, "gcnArchName", None)
        env["compute_units"] = prop.multi_processor_count
    except Exception as e:      # informational only
        env["gpu"] = "unknown (%s)" % e
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            env["rocm"] = open(path).read().strip()
            break
    env["library_version"] = int(ql.lib().qlinear_version())
    table = os.path.join(PKG, "tables", "decode_table.txt")
    if os.path.exists(table):
        env["table_sha256_16"] = hashlib.sha256(open(table, "rb").read()).hexdigest()[:16]
    env["kernel_sources_sha256_16"] = kernel_sources_digest()[:16]
    env["clocks"] = current_clocks()
    return env


def current_clocks():
    """The GPU's current clock levels as rocm-smi reports them (read-only;
    None where the tool is missing or refuses)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        data = json.loads(r.stdout[r.stdout.index("{"):]) if "{" in r.stdout else {}
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    card = next(iter(data.values()), {}) if isinstance(data, dict) else {}
    return {k.strip(" :"): v for k, v in card.items() if isinstance(v, str) and "clk" in k.lower()} or None


def prepare_workload(ql, torch, wl, layout, dev):
    """Weights (quantized on the GPU, packed offline, >= 1 GiB of copies per
    shape), activations and one plan + buffers per point."""
    from workloads import decode_points, make_inputs
    fmt = wl.fmt
    shapes = {}
    for (lab, N, K) in wl.shapes:
        x, w = make_inputs(K, N, max(wl.ms), wl.sigma_w, seed=wl.seed)
        wd = w.to(dev)
        w_q, w_s = ql.quantize_weight(fmt, wd)
        if layout != "rowmajor":              # offline, like the quantization itself
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
    pts = []
    for (lab, N, K, M) in decode_points(wl):
        sh = shapes[lab]
        w_layout, a_packed = LAYOUT_PLAN[layout]
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
    return dict(wl=wl, fmt=fmt, shapes=shapes, pts=pts)


def step_graphs(ql, W, stream, n_graphs=8):
    """hipGraphs of one step of a workload (every point's quantize + GEMM),
    each graph on its own weight copies."""
    graphs = []
    pts, shapes = W["pts"], W["shapes"]
    for gi in range(n_graphs):
        ql.qlinear_graph_begin(stream)
        for pi, p in enumerate(pts):
            sh = shapes[p["lab"]]
            c = (gi * len(pts) + pi) % sh["copies"]
            ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"],
                               p["wsp"], stream=stream)
        graphs.append(ql.qlinear_graph_end(stream))
    return graphs


def time_steps(torch, graph_sets, steps, stream):
    """HIP-event ms per step, a step replaying one graph of every workload."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    stream.synchronize()
    t0.record(stream)
    for i in range(steps):
        for gs in graph_sets:
            gs[i % len(gs)].launch(stream)
    t1.record(stream)
    stream.synchronize()
    return t0.elapsed_time(t1) / steps


def graph_us(torch, np, g, R, reps, stream):
    """Median / p10 / p90 per-launch µs of a graph of R launches (HIP events)."""
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
    return float(np.median(samples)), float(np.percentile(samples, 10)), float(np.percentile(samples, 90))


def point_timing(ql, torch, np, W, stream, reps):
    """Per point: a hipGraph of R back-to-back launches of the point's GEMM
    kernel (qlinear_run, or for a fused plan qlinear_forward, which is that one
    kernel) on distinct weight copies; then, for an unfused point, R launches
    of its activation quantizer alone."""
    fmt = W["fmt"]
    per_point = []
    for p in W["pts"]:
        sh = W["shapes"][p["lab"]]
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
            if not p["fused"]:        # the codes the GEMM reads
                quantize_into(ql, fmt, p, stream)
        us, p10, p90 = graph_us(torch, np, g, R, reps, stream)
        del g
        gbs = p["kbytes"] / (us * 1e-6) / 1e9
        flops = 2.0 * p["M"] * p["N"] * p["K"]
        rec = dict(shape=p["lab"], M=p["M"], N=p["N"], K=p["K"], us=round(us, 3), us_p10=round(p10, 3),
                   us_p90=round(p90, 3), GBs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                   TFLOPs=round(flops / (us * 1e-6) / 1e12, 1), algo=p["cfg"]["algo"],
                   variant=("split-k" if p["facts"]["chunks"] > 1 else
                            ("swap-ab" if p["cfg"]["swap_ab"] else "standard")),
                   split=p["facts"]["chunks"], swap_ab=p["cfg"]["swap_ab"],
                   fused_quant=p["fused"], kernel_bytes=int(p["kbytes"]), R=R, source=p["facts"]["source"])
        per_point.append(rec)
    # the separate quantizer launches (unfused points), after every GEMM timing
    for p, rec in zip(W["pts"], per_point):
        if p["fused"]:
            continue
        R = 64
        with torch.cuda.stream(stream):
            ql.qlinear_graph_begin(stream)
            for _ in range(R):
                quantize_into(ql, fmt, p, stream)
            g = ql.qlinear_graph_end(stream)
        rec["quant_us"] = round(graph_us(torch, np, g, R, reps, stream)[0], 3)
        del g
    return per_point


def quantize_into(ql, fmt, p, stream):
    if p["cfg"]["a_mode"] >= 2:
        ql.qlinear_quantize_act_packed(fmt, p["x"], p["a_q"], p["a_s"], stream=stream)
    else:
        ql.qlinear_quantize_act(fmt, p["x"], p["a_q"], p["a_s"], stream=stream)


def hbm_roofline(per_point, traffic, traffic_note, ceil_gbs, cu_gbs=None):
    tot_b = sum(q["kernel_bytes"] for q in per_point)
    tot_us = sum(q["us"] for q in per_point)
    achieved = tot_b / (tot_us * 1e-6) / 1e9
    r = {"kernel": "qgemm_decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
         "traffic": traffic, "algorithmic_bytes": int(tot_b), "traffic_source": traffic_note,
         "note": "algorithmic bytes of one launch of each of the %d GEMM kernels (a fused-quantization "
                 "launch also reads bf16 X and writes the codes and scales) / sum of their per-launch "
                 "durations (HIP events around graph replays of back-to-back launches); traffic is the HBM "
                 "bytes those same %d launches moved" % (len(per_point), len(per_point))}
    if ceil_gbs is not None:
        r["stream_ceiling"] = {"achieved": round(ceil_gbs, 1), "frac": round(ceil_gbs / HBM_PEAK_GBS, 4),
                               "kernel_vs_ceiling": round(achieved / ceil_gbs, 4),
                               "note": "a plain streaming read of each point's kernel bytes (qlinear_stream_read, "
                                       "best of 5 grids x 2 load depths), timed like the GEMMs; per point under "
                                       "ceiling_us"}
    if cu_gbs is not None:
        r["cu_ceiling"] = cu_ceiling_block(per_point, achieved, cu_gbs)
    return r


def cu_ceiling_block(per_point, achieved, cu_gbs):
    return {"achieved": round(cu_gbs, 1), "frac": round(cu_gbs / HBM_PEAK_GBS, 4),
            "kernel_vs_ceiling": round(achieved / cu_gbs, 4),
            "note": "one workgroup per compute unit reading its share of the weights from HBM and, "
                    "interleaved, every token's activations (bf16 X for a fused-quantization point) -- the "
                    "bytes each compute unit of an unsplit weight-streaming GEMM must load "
                    "(qlinear_stream_read_bcast, best of 2 thread counts x 2 load depths), timed like the "
                    "GEMMs; the point's algorithmic bytes over that time; per point under cu_ceiling_us"}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only (--gpus %d requested); the linear shards "
              "column-wise across GPUs with no exchange, so per-GPU work is one GPU's share." % args.gpus,
              file=sys.stderr)
        return 2

    wls = resolve_workloads(args.workload)
    if args.trace_summary:
        sys.stdout.write(trace_summary(args.workload, args.layout, *args.trace_summary, ref_json=args.trace_ref))
        return 0
    if args.pmc_summary:
        for name, text in pmc_summary(wls, args.layout, *args.pmc_summary).items():
            path = traffic_file(name, args.layout)
            with open(path, "w") as f:
                f.write(text)
            print("wrote", path)
        return 0

    import numpy as np
    import torch

    import quantized_gemm_decode_amd as ql

    if not os.path.exists(os.path.join(ROOT, "quantized_gemm_decode_amd", "libqlinear.so")):
        from quantized_gemm_decode_amd import build as b
        b.build()
    torch.cuda.set_device(0)
    n_table = ql.qlinear_table_load(args.table) if args.table else ql.load_default_table()
    dev = "cuda"
    stream = torch.cuda.Stream()

    Ws = [prepare_workload(ql, torch, wl, args.layout, dev) for wl in wls]
    if args.profile_pass:
        return profile_pass(ql, Ws, stream)
    if args.library_ref:
        for W in Ws:
            library_ref_pass(ql, torch, np, W, stream, args.kernel_reps)
        return 0
    if args.glu:
        # one JSON line per workload that has a gate_up projection
        for W in Ws:
            if any(p["lab"] == "gate_up" for p in W["pts"]):
                glu_pass(ql, W["wl"], W["pts"], W["shapes"], stream, args)
        return 0

    # ------------------------------------------------ the timed steps
    with torch.cuda.stream(stream):
        graph_sets = [step_graphs(ql, W, stream) for W in Ws]
    stream.synchronize()
    for i in range(args.warmup):
        for gs in graph_sets:
            gs[i % len(gs)].launch(stream)
    stream.synchronize()
    wall0 = time.perf_counter()
    step_ms = time_steps(torch, graph_sets, args.steps, stream)
    wall = time.perf_counter() - wall0
    step_bytes = sum(p["bytes"] + p["qbytes"] for W in Ws for p in W["pts"])
    value = step_bytes / (step_ms * 1e-3) / 1e9
    # the same K steps twice more (spread of repeated runs), then each workload alone
    repeats = [step_ms] + [time_steps(torch, graph_sets, args.steps, stream) for _ in range(2)]
    alone = [time_steps(torch, [gs], args.steps, stream) for gs in graph_sets]
    del graph_sets

    # ------------------------------------------------ per workload: kernels, ceiling, roofline, CPU oracle
    blocks = []
    all_pp = []
    traffic_sum, traffic_ok, notes = 0, True, set()
    cpu_budget = args.cpu_budget_s / len(Ws)
    for W, ms in zip(Ws, alone):
        wl = W["wl"]
        pp = point_timing(ql, torch, np, W, stream, args.kernel_reps)
        traffic, traffic_note = recorded_traffic(wl.name, args.layout)
        if traffic is None:
            traffic_ok = False
        else:
            traffic_sum += traffic
        notes.add(traffic_note)
        if max(wl.ms) <= 32:
            ceil_gbs = None if args.no_ceiling else stream_ceiling(ql, pp, stream, max(10, args.kernel_reps // 3))
            cu_gbs = None if args.no_ceiling else cu_ceiling(ql, pp, stream, max(10, args.kernel_reps // 3))
            roofline = hbm_roofline(pp, traffic, traffic_note, ceil_gbs, cu_gbs)
        else:
            # token counts in the hundreds and thousands: the tiled kernel is matrix-core bound
            big = [q for q in pp if q["M"] >= 1024]
            fl = sum(2.0 * q["M"] * q["N"] * q["K"] for q in big)
            t = sum(q["us"] for q in big) * 1e-6
            tflops = fl / t / 1e12
            roofline = {"kernel": "qgemm_tiled_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                        "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4),
                        "traffic": traffic, "traffic_source": traffic_note,
                        "note": "2*M*N*K of one launch of each M >= 1024 GEMM / sum of their per-launch durations; "
                                "the M = 64 and 256 points are HBM- or ridge-bound and are reported per point"}
        cpu = None if args.no_cpu_baseline else cpu_baseline(wl, cpu_budget)
        wbytes = sum(p["bytes"] + p["qbytes"] for p in W["pts"])
        qus = [q["quant_us"] for q in pp if "quant_us" in q]
        blocks.append({
            "workload": wl.name, "format": ql.FORMAT_NAMES[W["fmt"]],
            "shapes": ["%s %dx%d" % s for s in wl.shapes], "token_counts": list(wl.ms),
            "gemms_per_step": len(pp), "ms_per_step": round(ms, 4),
            "value": round(wbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "fused_quant_points": sum(1 for p in W["pts"] if p["fused"]),
            "quantizer_us_total": round(sum(qus), 3),
            "roofline": roofline, "cpu_baseline": cpu, "per_point": pp})
        all_pp += pp
        W.clear()
        torch.cuda.empty_cache()

    if all(max(b["token_counts"]) <= 32 for b in blocks):
        roofline = hbm_roofline(all_pp, traffic_sum if traffic_ok else None,
                                "; ".join(sorted(notes)), None)
        if not args.no_ceiling:
            ceil_b = sum(q["kernel_bytes"] for q in all_pp)
            ceil_us = sum(q["ceiling_us"] for q in all_pp)
            ceil_gbs = ceil_b / (ceil_us * 1e-6) / 1e9
            roofline["stream_ceiling"] = {"achieved": round(ceil_gbs, 1), "frac": round(ceil_gbs / HBM_PEAK_GBS, 4),
                                          "kernel_vs_ceiling": round(roofline["achieved"] / ceil_gbs, 4)}
            cu_us = sum(q["cu_ceiling_us"] for q in all_pp)
            roofline["cu_ceiling"] = cu_ceiling_block(all_pp, roofline["achieved"], ceil_b / (cu_us * 1e-6) / 1e9)
    else:
        roofline = blocks[0]["roofline"]
    cpu = None
    if not args.no_cpu_baseline:
        cb = [b["cpu_baseline"] for b in blocks]
        secs = sum(c["seconds"] for c in cb)
        cpu = {"value": round(sum(c["bytes"] for c in cb) / secs / 1e9, 3), "unit": "GB/s",
               "cores": cb[0]["cores"], "kind": "oracle",
               "sample": "; ".join(c["sample"] for c in cb)}
    fmts = sorted({b["format"] for b in blocks})
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "kernel_reps": args.kernel_reps,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_repeats": [round(r, 4) for r in repeats],
        "repeat_spread": round((max(repeats) - min(repeats)) / min(repeats), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(sorted({DTYPES.get(b["format"], "fp8_e4m3") for b in blocks})),
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outlier channels, N(0,0.02) weights "
                "(N(0,0.015) for the 32B-class shapes))",
        "config": {"workload": "+".join(b["workload"] for b in blocks), "formats": fmts,
                   "gemms_per_step": len(all_pp), "graph_replay": True, "table_entries": n_table,
                   "weight_layout": args.layout,
                   "fused_quant_points": sum(b["fused_quant_points"] for b in blocks),
                   "us_per_gemm_step_avg": round(step_ms * 1e3 / len(all_pp), 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "env": environment(ql, torch),
        "workloads": blocks,
        "wall_s": round(wall, 3),
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")
    return 0


DTYPES = {"W8A8_INT8": "int8", "MXFP4": "fp8_e4m3 x fp4_e2m1"}


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


def cu_ceiling(ql, per_point, stream, reps):
    """The per-compute-unit ceiling of every point: 256 workgroups (one per
    compute unit) each reading its share of the N x K weight codes from HBM and,
    interleaved, the whole activation block (M x K codes, or M x K bf16 X for a
    fused-quantization point) -- what each compute unit of a weight-streaming
    GEMM without a K split must load (qlinear_stream_read_bcast, best of 2
    thread counts x 2 load depths).  Timed as the GEMM is: HIP events around
    graph replays of R back-to-back launches on distinct weight offsets of a
    1 GiB buffer, one activation block shared by all of them.  Sets
    per_point[i]["cu_ceiling_us"]; returns the points' algorithmic bytes over
    the sum of these times (GB/s)."""
    import numpy as np
    import torch
    pool = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    best = {}
    for q in per_point:
        wb = q["N"] * q["K"] // 16 * 16
        ab = (2 if q["fused_quant"] else 1) * q["M"] * q["K"] // 16 * 16
        key = (wb, ab)
        if key not in best:
            act = torch.ones(max(ab, 16), dtype=torch.uint8, device="cuda")
            span = -(-wb // 4096) * 4096
            R = max(2, min(64, (1 << 30) // span))
            times = []
            for thr, lif in itertools.product((512, 1024), (2, 4)):
                with torch.cuda.stream(stream):
                    ql.qlinear_graph_begin(stream)
                    for c in range(R):
                        ql.qlinear_stream_read_bcast(pool[c * span:], wb, act, ab, sink, workgroups=256,
                                                     threads=thr, loads_in_flight=lif, stream=stream)
                    g = ql.qlinear_graph_end(stream)
                times.append(_graph_median_us(torch, np, stream, g, R, reps))
                del g
            best[key] = min(times)
            del act
        q["cu_ceiling_us"] = round(best[key], 3)
    del pool
    tot_b = sum(q["kernel_bytes"] for q in per_point)
    tot_us = sum(q["cu_ceiling_us"] for q in per_point)
    return tot_b / (tot_us * 1e-6) / 1e9


def _graph_median_us(torch, np, stream, g, R, reps, before=None):
    for _ in range(3):
        if before:
            before()
        g.launch(stream)
    stream.synchronize()
    samples = []
    for _ in range(reps):
        if before:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.launch(stream)
        e1.record(stream)
        e1.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3 / R)
    return round(float(np.median(samples)), 3)


def _cfg_str(cfg):
    return "swap%d split%d waves%dx%d rows%d pf%d amode%d" % (
        cfg["swap_ab"], cfg["split_k"], cfg["waves_n"], cfg["waves_k"], cfg["rows_per_wave"], cfg["prefetch"],
        cfg["a_mode"])


def _launches(cfg):
    """Kernel launches of one forward: one when the quantizer runs inside the GEMM."""
    return 1 if cfg["a_mode"] in (4, 5) else 2


def glu_pass(ql, wl, pts, shapes, stream, args):
    """The gated MLP's gate_up point, three ways, each timed as graph replays
    of R back-to-back forwards on distinct weight copies (HIP events):

      plain: the gate_up forward writing Y [M, N];
      glu:   the SiLU-and-mul plan writing H = silu(gate)*up [M, N/2];
      and the gate_up -> down chain, twice: 'chain_two_pass' = the SiLU-and-mul
      forward, then down's forward plan (its own quantizer launch, or the
      quantizer fused in where it fits the row); 'chain' = the SiLU-and-mul
      forward folding the per-token amax of H, then down's given-amax plan
      (each workgroup quantizes its K chunk of H in the GEMM launch)."""
    import numpy as np
    import torch
    fmt = wl.fmt
    per_token = fmt in (ql.FP8_DYNAMIC, ql.W8A8_INT8)
    downs = {p["M"]: p for p in pts if p["lab"] == "down"}
    out = []
    for p in pts:
        if p["lab"] != "gate_up":
            continue
        sh = shapes[p["lab"]]
        M, N, K = p["M"], p["N"], p["K"]
        R = min(sh["copies"], 64)
        res = {"M": M}
        glu_plan = ql.qlinear_plan_glu(fmt, M, N, K, 2)
        h = torch.empty(M, N // 2, dtype=torch.bfloat16, device="cuda")
        a_q, a_s = ql.act_buffer(glu_plan), ql.act_scale_buffer(glu_plan)
        wsp = glu_plan.new_workspace()
        for kind in ("plain", "glu"):
            plan = p["plan"] if kind == "plain" else glu_plan
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda") if kind == "plain" else h
            aq, as_ = (ql.act_buffer(plan), ql.act_scale_buffer(plan)) if kind == "plain" else (a_q, a_s)
            ws = plan.new_workspace() if kind == "plain" else wsp
            with torch.cuda.stream(stream):
                ql.qlinear_graph_begin(stream)
                for c in range(R):
                    ql.qlinear_forward(plan, p["x"], aq, as_, sh["wq"][c], sh["ws"][c], y, ws, stream=stream)
                g = ql.qlinear_graph_end(stream)
            res[kind + "_us"] = _graph_median_us(torch, np, stream, g, R, args.kernel_reps)
            res[kind + "_fused_quant"] = plan.config["a_mode"] == 4
            res[kind + "_config"] = _cfg_str(plan.config)
            del g
        d = downs.get(M)
        if d is not None and d["K"] == N // 2:
            dsh = shapes["down"]
            Rc = min(R, dsh["copies"])
            y2 = torch.empty(M, d["N"], dtype=torch.bfloat16, device="cuda")
            two = ql.qlinear_plan_layouts(fmt, M, d["N"], d["K"], 1, 2)
            chains = [("chain_two_pass", two)]
            if per_token:
                chains.append(("chain", ql.qlinear_plan_layouts(fmt, M, d["N"], d["K"], 1, 3)))
            amax = ql.amax_buffer(M)
            for kind, dplan in chains:
                da_q, da_s = ql.act_buffer(dplan), ql.act_scale_buffer(dplan)
                dws = dplan.new_workspace()
                with torch.cuda.stream(stream):
                    ql.qlinear_graph_begin(stream)
                    for c in range(Rc):
                        if kind == "chain":
                            ql.qlinear_forward_glu_amax(glu_plan, p["x"], a_q, a_s, sh["wq"][c], sh["ws"][c], h, amax,
                                                        wsp, stream=stream)
                            ql.qlinear_forward_amax(dplan, h, amax, da_q, da_s, dsh["wq"][c], dsh["ws"][c], y2, dws,
                                                    stream=stream)
                        else:
                            ql.qlinear_forward(glu_plan, p["x"], a_q, a_s, sh["wq"][c], sh["ws"][c], h, wsp,
                                               stream=stream)
                            ql.qlinear_forward(dplan, h, da_q, da_s, dsh["wq"][c], dsh["ws"][c], y2, dws,
                                               stream=stream)
                    g = ql.qlinear_graph_end(stream)
                res[kind + "_us"] = _graph_median_us(torch, np, stream, g, Rc, args.kernel_reps)
                res[kind + "_launches"] = _launches(glu_plan.config) + _launches(dplan.config)
                res[kind + "_down_config"] = _cfg_str(dplan.config)
                del g
        out.append(res)
    gu = [p for p in pts if p["lab"] == "gate_up"]
    print(json.dumps({"metric": "µs per gate_up forward: plain (Y [M, N]) vs SiLU-and-mul epilogue (silu(gate)*up, "
                                "[M, N/2]); µs per gate_up -> down chain: down quantizing H in its own pass vs "
                                "down quantizing its K chunk with the per-token amax the SiLU-and-mul epilogue "
                                "folded", "unit": "us", "workload": wl.name,
                      "shape": "gate_up %dx%d" % (gu[0]["N"], gu[0]["K"]) if gu else None,
                      "data": "synthetic", "kernel_reps": args.kernel_reps, "per_point": out}), flush=True)
    return 0


def library_ref_pass(ql, torch, np, W, stream, reps):
    """Per point: this library's GEMM kernel (as in point_timing) and
    torch._scaled_mm -- the vendor GEMM library, row-wise scales, bf16 out --
    on the same activation codes and the same number of distinct weight
    copies (row-major codes, as that library takes them), both timed as
    graphs of back-to-back launches with HIP events.  A reference for the
    compute-bound points, not part of the product path."""
    wl = W["wl"]
    if W["fmt"] != ql.FP8_DYNAMIC:
        print(json.dumps({"workload": wl.name, "skipped": "the reference takes FP8_Dynamic (row-wise) only"}))
        return
    from workloads import make_inputs
    ours = {(q["shape"], q["M"]): q for q in point_timing(ql, torch, np, W, stream, reps)}
    out = []
    rm = {}
    for p in W["pts"]:
        sh = W["shapes"][p["lab"]]
        M, N, K = p["M"], p["N"], p["K"]
        if p["lab"] not in rm:
            rm.clear()
            _, w = make_inputs(K, N, max(wl.ms), wl.sigma_w, seed=wl.seed)   # the weights prepare_workload made
            w_q, w_s = ql.quantize_weight(ql.FP8_DYNAMIC, w.to("cuda"))
            copies = sh["copies"]
            wq_all = torch.empty((copies,) + tuple(w_q.shape), dtype=w_q.dtype, device="cuda")
            wq_all[:] = w_q
            rm[p["lab"]] = (wq_all, w_s.view(1, N).contiguous(), copies)
        wq_all, sb, copies = rm[p["lab"]]
        a_q, a_s = ql.quantize_act(ql.FP8_DYNAMIC, p["x"])
        sa = a_s.view(M, 1).contiguous()
        torch.cuda.synchronize()
        R = min(copies, 64)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        def lib_mm(c):
            torch._scaled_mm(a_q, wq_all[c].t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16, out=y)
        try:
            with torch.cuda.stream(stream):
                y_ref = torch._scaled_mm(a_q, wq_all[0].t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
                lib_mm(0)
            stream.synchronize()
            # captured like this library's launches; trusted only if a replay reproduces the eager output
            y.zero_()
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                ql.qlinear_graph_begin(stream)
                for c in range(R):
                    lib_mm(c)
                g = ql.qlinear_graph_end(stream)
            g.launch(stream)
            stream.synchronize()
            captured = bool(torch.equal(y, y_ref))
        except RuntimeError as e:
            out.append(dict(shape=p["lab"], M=M, N=N, K=K, us=ours[(p["lab"], M)]["us"], library_error=str(e)[:160]))
            continue
        samples = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if captured:
                g.launch(stream)
            else:                 # eager launches (host launch overhead included)
                with torch.cuda.stream(stream):
                    for c in range(R):
                        lib_mm(c)
            e1.record(stream)
            e1.synchronize()
            samples.append(e0.elapsed_time(e1) * 1e3 / R)
        del g
        lib_us = float(np.median(samples))
        q = ours[(p["lab"], M)]
        flops = 2.0 * M * N * K
        # the two compute the same linear: largest difference relative to max |Y|
        with torch.cuda.stream(stream):
            ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][0], sh["ws"][0], y, p["wsp"],
                               stream=stream)
        stream.synchronize()
        rel = float((y.float() - y_ref.float()).abs().max() / y_ref.float().abs().max().clamp_min(1e-30))
        out.append(dict(shape=p["lab"], M=M, N=N, K=K, us=q["us"], TFLOPs=round(flops / (q["us"] * 1e-6) / 1e12, 1),
                        library_us=round(lib_us, 3), library_TFLOPs=round(flops / (lib_us * 1e-6) / 1e12, 1),
                        ratio=round(lib_us / q["us"], 3), algo=p["cfg"]["algo"], R=R, library_graph=captured,
                        max_rel_diff=round(rel, 5)))
    print(json.dumps({"metric": "µs per GEMM: this library's plan vs torch._scaled_mm (the vendor GEMM library, "
                                "row-wise scales) on the same codes; ratio = library / this", "workload": wl.name,
                      "data": "synthetic", "kernel_reps": reps, "per_point": out}), flush=True)


def profile_pass(ql, Ws, stream):
    """Eager launches in a fixed order for per-dispatch hardware counters.

    Order: for every workload, for every point, 3 x (quantize, GEMM) on weight
    copies 0, 1, 2; then 3 plain copies of 256 MiB (read 256 MiB, write
    256 MiB), whose counter readings calibrate the byte counters."""
    import torch
    with torch.cuda.stream(stream):
        for W in Ws:
            for p in W["pts"]:
                sh = W["shapes"][p["lab"]]
                for c in range(3):
                    ql.qlinear_forward(p["plan"], p["x"], p["a_q"], p["a_s"], sh["wq"][c], sh["ws"][c], p["y"],
                                       p["wsp"], stream=stream)
                stream.synchronize()
                print("point %s %s M=%d N=%d K=%d bytes=%d" % (W["wl"].name, p["lab"], p["M"], p["N"], p["K"],
                                                              p["bytes"]), flush=True)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        stream.synchronize()
        for _ in range(3):
            dst.copy_(src)
        stream.synchronize()
    print("copy bytes=%d" % (256 << 20), flush=True)
    return 0


def cpu_baseline(wl, budget_s):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload."""
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
        for M in (wl.ms if len(wl.ms) < 3 else (wl.ms[0], wl.ms[-1])):
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
            "us_per_gemm": round(t_total / len(sample) * 1e6, 1), "seconds": round(t_total, 3),
            "bytes": int(b_total)}


if __name__ == "__main__":
    sys.exit(main())
