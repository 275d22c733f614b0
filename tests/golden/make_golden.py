"""Writes tests/golden/oracle_digests.txt from the CPU oracle alone (no GPU code is imported).

The digests guard the oracle against unintended changes: a change of its arithmetic changes them,
and regenerating them is a deliberate step whose commit names the reason.  Run from the repository
root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = [
    # name, input, lattice, target bps, seed, dither
    ("tiny_e8_4bps", "tiny", "e8", 4.0, 0, False),
    ("tiny_d4_4bps", "tiny", "d4", 4.0, 0, False),
    ("tiny_z_4bps", "tiny", "z", 4.0, 0, False),
    ("tiny_e8_2bps_dither", "tiny", "e8", 2.0, 5, True),
    ("tiny_a2_4bps", "tiny", "a2", 4.0, 0, False),
    ("tiny_a2_3bps_dither", "tiny", "a2", 3.0, 5, True),
    ("weight16x4096_e8_3bps", "weight16", "e8", 3.0, 0, False),
    ("tiny_e8_4bps_tile64", "tiny", "e8", 4.0, 0, False, 64),
    ("tiny_e8_3bps_dither_tile256", "tiny", "e8", 3.0, 5, True, 256),
    # dither flags 7: 24-bit draw from 7-round Philox calls
    ("tiny_e8_2bps_dither_flags7", "tiny", "e8", 2.0, 5, 7),
]


def make_input(name):
    if name == "tiny":
        return synth.tiny()
    if name == "weight16":
        return synth.weight(rows=16)
    raise KeyError(name)


def digest_rows():
    rows = []
    for name, inp, lat, tb, seed, dither, *tile in CASES:
        x = make_input(inp)
        s, info = oracle.encode(x, oracle.LATTICES[lat], tb, seed=seed, dither=dither, tile=(tile or [128])[0])
        y = oracle.decode(s, x.size)
        rows.append((name, info["step_bits"], info["k"], info["payload_bits"], s.size,
                     hashlib.sha256(s.tobytes()).hexdigest(), hashlib.sha256(y.tobytes()).hexdigest()))
    return rows


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.txt")
    with open(out, "w") as f:
        f.write("# Written by tests/golden/make_golden.py from the CPU oracle only.\n")
        f.write("# name step_bits k payload_bits stream_bytes sha256(stream) sha256(decoded fp32)\n")
        for r in digest_rows():
            f.write(" ".join(str(v) for v in r) + "\n")
    print(out)
