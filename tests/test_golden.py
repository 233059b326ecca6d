"""The oracle still reproduces the digests stored by tests/golden/make_golden.py."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_tiny_oracle_digests():
    stored = {}
    with open(os.path.join(HERE, "golden", "tiny_oracle.txt")) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            key, val = ln.rstrip("\n").split(" ", 1)
            stored[key] = val
    now = make_golden.tiny_records()
    assert set(stored) == set(now)
    for k in stored:
        assert stored[k] == str(now[k]), k
