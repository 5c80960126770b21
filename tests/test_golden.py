"""The oracle still reproduces the stored expected values of tests/golden/ (written by make_golden.py from the
oracle alone): a regression pin on its chains, roots, key generation, key-switch and transform."""
import json
import os

from tests.golden import make_golden

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_golden.json")


def _stored() -> dict:
    with open(GOLDEN) as f:
        return json.load(f)


def test_chains_and_roots_reproduce():
    assert make_golden.chains() == _stored()["chains"]


def test_workload1_keyswitch_reproduces():
    want = _stored()["workload1"]
    got = make_golden.workload1()
    for k in want:
        assert got[k] == want[k], k
