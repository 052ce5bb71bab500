"""Regression: the oracle still reproduces its frozen tiny-config output."""
import json
import os

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_tiny_output():
    with open(os.path.join(HERE, "golden", "tiny_fp32_seed0.json")) as f:
        frozen = json.load(f)
    assert json.loads(json.dumps(compute())) == frozen
