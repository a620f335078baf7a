"""Which kernel configurations the instantiation tests run.

Each GPU instantiation test enumerates a product of configuration fields
(waves, rows per wave, batch, operand modes, tiles, ...).  Not every point of
such a product is instantiated: shapes that would spill registers or exceed
the LDS are left out of the kernel tables, and the planner (host-only, no
GPU needed) rejects them with QL_E_UNSUPPORTED.  The tests run exactly the
points the planner accepts, listed at collection time by ``cases``, and
``tests/test_instantiation_manifest.py`` (CPU) holds those lists to the
committed ``tests/instantiated_cases.txt``: an instantiation that disappears
fails that test instead of turning into one more skip.

    python -m tests.instantiations --write     # regenerate the manifest
"""

import os
import sys

import quantized_gemm_decode_amd as ql

MANIFEST = os.path.join(os.path.dirname(os.path.abspath(__file__)), "instantiated_cases.txt")
_FAMILIES = {}


def accepted(plan_fn, *args):
    """True when the planner builds the plan; False when it reports the
    configuration as not instantiated (QL_E_UNSUPPORTED); other errors raise."""
    try:
        plan_fn(*args)
        return True
    except ql.QLinearError as e:
        if e.status != 2:
            raise
        return False


def cases(family, candidates, plan_args, plan_fn=None):
    """The candidates whose plan the planner accepts.  plan_args(*case) gives
    (fmt, M, N, K, cfg) for plan_fn (default qlinear_plan_with_config)."""
    fn = plan_fn or ql.qlinear_plan_with_config
    out = [c for c in candidates if accepted(fn, *plan_args(*c))]
    _FAMILIES[family] = out
    return out


FAMILY_MODULES = ("tests.test_gpu_gemm", "tests.test_gpu_fused", "tests.test_gpu_glu", "tests.test_gpu_mx",
                  "tests.test_gpu_tiled")


def all_families():
    """family -> list of cases, from every instantiation test module."""
    import importlib
    for m in FAMILY_MODULES:
        importlib.import_module(m)
    return dict(sorted(_FAMILIES.items()))


def manifest_lines(families):
    lines = ["# instantiation-test cases the planner accepts: family, then the case tuple",
             "# regenerate: python -m tests.instantiations --write"]
    for fam, cs in families.items():
        lines += ["%s %s" % (fam, " ".join(str(v) for v in c)) for c in cs]
    return lines


def read_manifest():
    with open(MANIFEST) as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


if __name__ == "__main__":
    if "--write" in sys.argv:
        # the test modules register their families with the importable module, not with __main__
        from tests import instantiations as mod
        with open(MANIFEST, "w") as f:
            f.write("\n".join(mod.manifest_lines(mod.all_families())) + "\n")
        print("wrote", MANIFEST)
