import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# FP8 acceptance statistics of every parity check, per test: with
# QL_PARITY_REPORT_DIR set, the session writes a summary there at its end.
_RECORDS = []


@pytest.fixture(autouse=True)
def _parity_statistics(request):
    import oracle
    n0 = len(oracle.parity_statistics())
    yield
    new = oracle.parity_statistics()[n0:]
    if new:
        _RECORDS.append((request.node.nodeid, new))


def _summary(records):
    by_file = {}
    for nodeid, stats in records:
        by_file.setdefault(nodeid.split("::")[0], []).append((nodeid, stats))
    lines = ["# command: QL_PARITY_REPORT_DIR=<dir> python -m pytest %s" % " ".join(sys.argv[1:]),
             "# FP8 / Block_FP8 / MXFP8 / MXFP4 parity statistics of one pytest session",
             "# element rule: within 1 bf16 ulp of y_ref, or within half an ulp plus the bound B of y_true",
             "# per file: checks, elements, lowest and element-weighted fraction within 1 ulp, elements that",
             "# needed the bound clause, largest normwise error max|y - y_ref| / max|y_ref|",
             "# file                                   checks   elements  min_frac_1ulp  frac_1ulp  needed_B  "
             "max_normwise"]
    tot_n = tot_in = tot_b = tot_c = 0
    worst = []
    for f in sorted(by_file):
        sts = [s for _, ss in by_file[f] for s in ss]
        n = sum(s["n"] for s in sts)
        inside = sum(s["frac_within_ulp"] * s["n"] for s in sts)
        nb = sum(s["n_needed_bound"] for s in sts)
        lines.append("%-42s %6d %10d  %13.6f  %9.6f  %8d  %12.3e" % (
            f, len(sts), n, min(s["frac_within_ulp"] for s in sts), inside / max(n, 1), nb,
            max(s["normwise"] for s in sts)))
        tot_n, tot_in, tot_b, tot_c = tot_n + n, tot_in + inside, tot_b + nb, tot_c + len(sts)
        worst += [(s["frac_within_ulp"], s["n"], nodeid) for nodeid, ss in by_file[f] for s in ss]
    lines.append("%-42s %6d %10d  %13.6f  %9.6f  %8d" % ("all", tot_c, tot_n, min(w[0] for w in worst),
                                                         tot_in / max(tot_n, 1), tot_b))
    lines.append("# the ten checks with the lowest fraction within 1 ulp (fraction, elements, test):")
    for fr, n, nodeid in sorted(worst)[:10]:
        lines.append("#   %.6f %7d  %s" % (fr, n, nodeid))
    return "\n".join(lines) + "\n"


def pytest_sessionfinish(session, exitstatus):
    d = os.environ.get("QL_PARITY_REPORT_DIR")
    if d and _RECORDS:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "fp8_parity_statistics.txt"), "w") as f:
            f.write(_summary(_RECORDS))
