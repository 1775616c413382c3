"""The oracle still reproduces the stored digests written by tests/golden/make_golden.py
(which calls only oracle/). Guards against unintended changes of the oracle's arithmetic."""

import json
import os

from tests.golden import make_golden


def test_tiny_oracle_digests_unchanged():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    with open(path) as f:
        stored = json.load(f)
    assert make_golden.compute() == stored
