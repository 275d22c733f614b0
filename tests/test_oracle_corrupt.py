"""The oracle's decoder on seeded corrupt streams: every case ends in OK or CORRUPT.

Damage to the magic or version, truncation and a wrong value count must be CORRUPT; damage the
format cannot see (the fixed plane's remainder bits, alignment padding, trailing bytes) decodes; the
rest may go either way (the format has no checksum).  Run under the
sanitizer build (tests/test_oracle_sanitizers.py), an access outside the stream aborts the run.
"""
import numpy as np

from stream_mutations import cases


def test_every_corrupt_case_is_ok_or_corrupt(orc):
    seen = {"ok": 0, "corrupt": 0}
    for name, s, n in cases(orc):
        rc = orc.decode_status(s, n)
        assert rc in (orc.OK, orc.ERR_CORRUPT), (name, rc)
        seen["ok" if rc == orc.OK else "corrupt"] += 1
        kind = name.split(":")[1]
        # the header has free fields (seed, the informational bit totals, reserved bytes) and a
        # step that may stay in range, so a random header flip can decode; these never can
        if kind in ("magic",) or kind.startswith("n+"):
            assert rc == orc.ERR_CORRUPT, name
        if kind.startswith("truncate"):
            # a stream cut short of its total size cannot pass the header check
            assert rc == orc.ERR_CORRUPT, name
        if kind in ("intact", "trailing") or name.endswith(":pad"):
            assert rc == orc.OK, name
    assert seen["ok"] > 50 and seen["corrupt"] > 100, seen


def test_fixed_plane_damage_changes_values_not_verdict(orc):
    """A flipped remainder bit is invisible to the format: the stream decodes, to other values."""
    for name, s, n in cases(orc, per_base=16, seed=1):
        if not name.endswith(":fixed") or ":flip1:" not in name:
            continue
        base = [c for c in cases(orc, per_base=0) if c[0].split(":")[0] == name.split(":")[0]][0]
        assert orc.decode_status(s, n) == orc.OK
        y, y0 = orc.decode(s, n), orc.decode(base[1], n)
        assert y.shape == y0.shape
