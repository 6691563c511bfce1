"""The planner's predictions against measured step times (CPU only: the
measurements are the committed profiles/planner_profiles.json, recorded on an
MI355X by persistent_megakernel_latency_amd.planner_profile).

The two machine constants are fixed at batch 1; the other 23 predictions are
out of sample.  The bars below are the accuracy the model reached when the
profiles were recorded, so a change to the simulation that makes its
predictions worse fails here."""
import json
import os

import pytest

from persistent_megakernel_latency_amd.planner import DESIGNS, Planner, markdown

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def evaluation():
    with open(os.path.join(ROOT, "profiles", "planner_profiles.json")) as f:
        prof = json.load(f)
    pl = Planner(prof)
    ev = pl.evaluate()
    pl.close()
    return ev


def test_calibration_meets_batch_one(evaluation):
    r = evaluation["rows"][0]
    assert r["batch"] == 1
    assert abs(r["error"]["tile_edges"]) < 1e-3
    assert abs(r["error"]["conventional"]) < 2e-3
    assert 0.0 < evaluation["load_latency_us"] < 20.0 and 0.0 < evaluation["launch_gap_us"] < 20.0


def test_predictions_within_a_third(evaluation):
    for r in evaluation["rows"]:
        for d in DESIGNS:
            assert abs(r["error"][d]) < 0.35, (r["batch"], d, r["error"][d])


def test_ranking_agreement(evaluation):
    # ties (barrier edges predicted equal to tile edges) count as disagreements
    assert evaluation["pairwise_agreement"] >= 0.75
    assert evaluation["best_design_correct"] >= 3
    assert evaluation["max_regret"] <= 0.12


def test_markdown_lists_every_case(evaluation):
    text = markdown(evaluation)
    assert text.count("\n| ") == len(evaluation["rows"]) * len(DESIGNS)
