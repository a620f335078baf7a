"""The instantiation tests run exactly the configurations the planner accepts;
this CPU test holds those lists to the committed manifest, so a kernel
instantiation that disappears (a dispatch-table edit, a new register spill)
fails here instead of shrinking the GPU tests silently."""

from tests import instantiations


def test_instantiated_cases_match_the_manifest():
    got = instantiations.manifest_lines(instantiations.all_families())
    want = instantiations.read_manifest()
    got = [l for l in got if not l.startswith("#")]
    missing = sorted(set(want) - set(got))
    extra = sorted(set(got) - set(want))
    assert not missing, ("instantiations no longer accepted by the planner", missing[:20], len(missing))
    assert not extra, ("new instantiations: regenerate the manifest (python -m tests.instantiations --write)",
                       extra[:20], len(extra))
