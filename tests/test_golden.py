"""The oracle reproduces its stored regression values bit for bit
(tests/golden/oracle_small.json, written by tests/golden/make_golden.py
from oracle/ only)."""
import json
import os

from tests.golden.make_golden import OUT, compute


def test_oracle_matches_stored_regression_values(orc):
    with open(OUT) as f:
        stored = json.load(f)
    assert compute() == stored
