"""Regression guard: the oracle reproduces the digests stored by tests/golden/make_golden.py."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))


def test_oracle_digests_unchanged(orc):
    import make_golden
    stored = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "oracle_digests.txt")):
        if line.startswith("#"):
            continue
        t = line.split()
        stored[t[0]] = t[1:]
    for row in make_golden.digest_rows():
        assert [str(v) for v in row[1:]] == stored[row[0]], row[0]
