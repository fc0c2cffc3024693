"""The prefill planner's cost model against measured timings (no GPU).

tests/data/prefill_tilings_gfx950.json holds the time of every prefill tiling
(and of the 8-row decode plan at m <= 16) on 54 shapes, measured on gfx950
with block_wise_int4_matmulnbits_amd.plan_tune.  mnb_plan_default prices
those candidates with a fitted table and takes the cheapest; these tests
check its choice against the measured times and against a fresh fit of the
same data, so a stale table or a wrong formula in the C++ fails here."""
import json
import os

import pytest

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import plan_tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DATA = json.load(open(os.path.join(ROOT, "tests", "data", "prefill_tilings_gfx950.json")))
SHAPES = sorted((tuple(map(int, k.split(","))), row) for k, row in DATA["shapes"].items())


def planner_pick(m, K, N):
    p = mnb.mnb_plan_default(m, K, N, DATA["cus"], 0)
    if p.engine != 2:
        assert p.as_dict() == mnb.mnb_plan_default(8, K, N, DATA["cus"], 0).as_dict()
        return "decode"
    return "%d,%d,%d" % (p.row_tiles, p.cols_per_tile, p.waves_per_wg)


def test_planner_choice_is_near_the_measured_fastest():
    regrets = []
    for (m, K, N), row in SHAPES:
        pick = planner_pick(m, K, N)
        assert pick in row, (m, K, N, pick)
        best = min(v["us"] for v in row.values())
        regrets.append(row[pick]["us"] / best - 1)
        assert regrets[-1] <= 0.045, ((m, K, N), pick, row[pick]["us"], best)
    assert sum(regrets) / len(regrets) <= 0.005


def test_planner_table_is_the_fit_of_the_measurements():
    pytest.importorskip("scipy")
    table, dec = plan_tune.fit_model(DATA)
    for (m, K, N), row in SHAPES:
        assert planner_pick(m, K, N) == plan_tune.model_pick(table, dec, m, K, N, DATA["cus"], row), (m, K, N)


def test_every_candidate_the_model_can_pick_was_measured():
    # The sweep times each tiling that mnb_plan_check accepts; the planner
    # considers the same set, so a measured row lists all of them.
    for (m, K, N), row in SHAPES:
        for t in plan_tune.TILINGS:
            q = mnb.mnb_plan(engine=2, row_tiles=t[0], cols_per_tile=t[1], waves_per_wg=t[2], workgroups=1)
            assert (mnb.mnb_plan_check(m, K, N, q) == 0) == (plan_tune.key_of(t) in row), (m, K, N, t)
        assert ("decode" in row) == (m <= 16)
