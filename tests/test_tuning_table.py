"""The automatic tile choice checked against the tuning table
(profiles/tuning_fp32.json: per shape, the measured time per call of
every lean variant and of the automatic choice, taken on MI355X; per
variant, resources and the cfg_valid filter).  CPU only: the table holds
the measurements, the library's variant choice makes no HIP call.
"""
import json
import os

import pytest

from fp32_sgemm_tuning_amd import build, capi, tuning

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "profiles", "tuning_fp32.json")
AL = 0x10000          # a 16-byte aligned fake address (only inspected for alignment)


@pytest.fixture(scope="module")
def table():
    return json.load(open(TABLE))


def _shape(s):
    return tuple(int(x) for x in s.split("x"))


def test_table_was_taken_on_the_current_dispatch(table):
    """Every recorded automatic choice is the one the library makes now (a
    change of the dispatch rules needs a new table)."""
    capi.load()
    for shape, e in table["shapes"].items():
        M, N, K = _shape(shape)
        v = capi.sgemm_select_variant(M, N, K, AL, K, AL, N, 0.0, AL, N)
        assert capi.sgemm_variant_name(v) == e["auto_variant"], shape


def test_auto_choice_within_spread_of_the_best(table):
    """On every recorded shape the automatic plan (timed under both its
    names in the sweep, the mean taken) runs within the table's stated
    measurement spread of the fastest valid variant: 7%, or 15% for
    problems under 50 us, from the spread of identical plans timed in
    sweeps on different boxes."""
    worse = {}
    for shape, e in table["shapes"].items():
        spread = table["spread_short"] if e["best_us"] < table["short_us"] else table["spread"]
        if e["auto_plan_us"] > e["best_us"] * (1.0 + spread):
            worse[shape] = (e["auto_variant"], e["auto_plan_us"], e["best_variant"], e["best_us"])
    assert not worse, worse
    # and the plan is the fastest measured, or within 2%, on most shapes of
    # at least 50 us (below that the sweep's event times hold the host's
    # launch latency, which the choice of kernel does not set; the split
    # of small grids is checked on kernel-trace times in test_splitk_fit)
    long = {s: e for s, e in table["shapes"].items() if e["best_us"] >= table["short_us"]}
    close = [s for s, e in long.items() if e["auto_plan_us"] <= e["best_us"] * 1.02]
    assert len(long) >= 10
    assert len(close) >= 0.7 * len(long), sorted(set(long) - set(close))


def test_dispatch_uses_only_valid_configurations(table):
    """Every variant the automatic choice picks on the recorded shapes passes
    cfg_valid: it fits the LDS of a compute unit and spills nothing."""
    for shape, e in table["shapes"].items():
        v = table["variants"][e["auto_variant"]]
        assert v["cfg_valid"], (shape, e["auto_variant"], v)
        assert v["lds_bytes"] <= tuning.LDS_LIMIT and v["max_scratch_bytes_per_lane"] == 0


def test_cfg_valid_filter():
    ok = {"lds": 65536, "scratch": 0}
    assert tuning.cfg_valid([ok, ok])
    assert not tuning.cfg_valid([ok, {"lds": 160 * 1024 + 16, "scratch": 0}])
    assert not tuning.cfg_valid([ok, {"lds": 1024, "scratch": 8}])
    assert not tuning.cfg_valid([])


def test_table_resources_match_the_build(table):
    """The table's resource figures are those of the library as built (the
    build writes the compiler's resource report)."""
    path = os.path.join(build.BUILD_DIR, "resource_usage.txt")
    if not os.path.exists(path):
        pytest.skip("no resource report: the library was not built here")
    res = tuning.parse_resource_usage(open(path).read())
    for name, v in table["variants"].items():
        inst = tuning.variant_resources(name, res)
        assert tuning.cfg_valid(inst) == v["cfg_valid"], name
        assert max(r.get("vgpr", 0) for r in inst) == v["max_vgpr"], name
        assert max(r.get("lds", 0) for r in inst) == v["lds_bytes"], name


def test_variant_names_parse():
    assert tuning.variant_tile("lean_dw_64x64x64_w4x1_splitk") == (64, 64, 64, 4, 1, True)
    assert tuning.variant_tile("lean_128x128x32_w2x2") == (128, 128, 32, 2, 2, False)
    assert tuning.variant_tile("db_128x128x32_w2x2_vec") is None
    args = tuning.lean_template_args("_ZN12sgemm_mi355x17sgemm_lean_kernelILi128ELi128ELi32ELi2ELi2ELb1ELb0ELb0E"
                                     "Lb0ELb0ELb0EEEvNS_4ArgsE")
    assert args == (128, 128, 32, 2, 2, True, False, False, False, False, False)
