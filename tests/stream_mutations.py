"""Seeded corrupt-stream cases for the decoders (test helper, no step of the method).

Base streams come from the oracle's encoder.  Each case is a copy of one with a mutation: single or
multiple bit flips placed in a chosen section (header, chunk index, fixed plane, unary plane, the
alignment padding), a truncation, trailing bytes, or a wrong value count.  A decoder given any case
must return OK or CORRUPT, never touch memory outside the buffers it was given, and (when two
decoders are compared) agree on the verdict and, for accepted streams, on every decoded value.
"""
from __future__ import annotations

import numpy as np

LATS = {"z": 0, "d4": 1, "e8": 2, "a2": 3}

# (lattice, tile, dither flags, tiles, step, rice k): ragged chunks, every lattice and tile length
BASES = [
    ("e8", 128, 0, 200, 0.30, 2),
    ("e8", 128, 1, 131, 1.20, 0),
    ("e8", 256, 0, 70, 0.15, 3),
    ("d4", 64, 1, 300, 0.40, 1),
    ("a2", 128, 0, 90, 0.25, 2),
    ("z", 128, 0, 65, 0.05, 5),
    ("e8", 64, 5, 129, 0.60, 1),
]


def base_streams(orc):
    out = []
    for i, (lat, tl, df, T, step, k) in enumerate(BASES):
        rng = np.random.default_rng(1000 + i)
        x = (rng.standard_normal((T, tl)) * 10.0 ** rng.uniform(-2, 2, (T, 1))).astype(np.float32)
        s, _ = orc.encode(x, LATS[lat], 0.0, seed=7 + i, dither=df, step=step, rice_k=k, tile=tl)
        out.append((f"{lat}/tl{tl}/d{df}/T{T}", s, x.size, tl))
    return out


def _section_ranges(s: np.ndarray, tl: int):
    """Byte ranges of the stream's sections, from its own header (base streams are valid)."""
    h = s[:128].view(np.uint32)
    chunks = int(h[10])
    fixed_off = int(h[12]) | (int(h[13]) << 32)
    unary_off = int(h[14]) | (int(h[15]) << 32)
    total = int(h[22]) | (int(h[23]) << 32)
    idx_end = 128 + 4 * (chunks + 1)
    return {"header": (0, 128), "index": (128, idx_end), "pad": (idx_end, fixed_off),
            "fixed": (fixed_off, unary_off), "unary": (unary_off, total)}


def cases(orc, per_base: int = 60, seed: int = 0):
    """[(name, stream bytes, n)]: mutations of every base stream (seeded)."""
    rng = np.random.default_rng(seed)
    out = []
    for name, s, n, tl in base_streams(orc):
        secs = _section_ranges(s, tl)
        out.append((name + ":intact", s.copy(), n))
        for j in range(per_base):
            m = s.copy()
            kind = j % 8
            if kind < 5:
                sec = ("header", "index", "fixed", "unary", "unary")[kind]
                a, b = secs[sec]
                if b <= a:
                    continue
                flips = 1 if j % 3 else int(rng.integers(2, 9))
                for _ in range(flips):
                    pos = int(rng.integers(a * 8, b * 8))
                    m[pos >> 3] ^= np.uint8(1 << (pos & 7))
                out.append((f"{name}:flip{flips}:{sec}", m, n))
            elif kind == 5:
                cut = int(rng.integers(0, s.size))
                out.append((f"{name}:truncate{cut}", m[:cut].copy(), n))
            elif kind == 6:
                extra = rng.integers(0, 256, int(rng.integers(1, 300)), dtype=np.uint8)
                out.append((f"{name}:trailing", np.concatenate([m, extra]), n))
            else:
                out.append((f"{name}:n+{tl}", m, n + tl))
                g = s.copy()
                pos = int(rng.integers(0, 6 * 8))  # magic and version: never valid when changed
                g[pos >> 3] ^= np.uint8(1 << (pos & 7))
                out.append((f"{name}:magic", g, n))
                a, b = secs["pad"]
                if b > a:
                    p = m.copy()
                    p[int(rng.integers(a, b))] ^= np.uint8(1 << int(rng.integers(0, 8)))
                    out.append((f"{name}:flip1:pad", p, n))
    return out
