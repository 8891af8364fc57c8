"""The 16-bit automatic choice against its recorded measurements
(profiles/tuning_lowp_bf16.json: BF16 products on MI355X, the automatic
choice and every fast variant forced, each with its own split factor).
CPU only: the choice is made on the host without a HIP call."""
import json
import os
import statistics

import pytest

from fp32_sgemm_tuning_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "profiles", "tuning_lowp_bf16.json")


@pytest.fixture(scope="module")
def table():
    return json.load(open(TABLE))


def _shape(s):
    return tuple(int(x) for x in s.split("x"))


def test_recorded_choice_is_the_current_rule(table):
    """Every recorded run of the automatic choice ran the variant the
    library chooses now (a change of the rule needs new runs); the packed
    operands the sweep used are 16-byte aligned, which null pointers stand
    for here."""
    capi.load()
    names = {v: capi.sgemm_lowp_variant_name(v) for v in capi.lowp_variants()}
    for shape, e in table["shapes"].items():
        M, N, K = _shape(shape)
        v = capi.sgemm_lowp_select_variant(M, N, K, 0, K, 0, N)
        assert names[v] == e["auto_variant"], (shape, names[v], e["auto_variant"])


def test_choice_against_the_fastest_variant(table):
    """On the recorded shapes the automatic choice runs within 2% of the
    fastest forced variant on average and within 20% at worst (the worst,
    768x1024x16384, takes the two-stage kernel's split where the
    alternating kernel's ran faster; the prediction puts the two within
    1%)."""
    over = [e["auto_us"] / e["best_us"] for e in table["shapes"].values()]
    assert len(over) >= 30
    assert statistics.mean(over) <= 1.02, statistics.mean(over)
    assert max(over) <= 1.20, max(over)
