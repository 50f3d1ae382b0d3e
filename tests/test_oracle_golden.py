"""The oracle still produces the recorded tiny-block outputs (regression record
written by tests/golden/make_golden.py, which calls only the oracle)."""

import json
import os

from tests.golden.make_golden import record

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_block_matches_record():
    with open(os.path.join(HERE, "golden", "tiny_block.json")) as f:
        want = json.load(f)
    assert json.loads(json.dumps(record(), sort_keys=True)) == want
