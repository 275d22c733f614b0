"""Pins of the oracle's nearest-point decoders (E8, D4, A2, Z) and of bit-stripping.

HyperQuant summary (gist.science/ko/paper/2606.23406), Methodology component 2: the rotated tile is
quantised to E8, D4, A2 or Z; these lattices have a lower normalised second moment G than Z; E8 has
a constant-time closed-form decoder.  Component 3: bits fixed by lattice membership are stripped
losslessly.  Pinned by brute-force search over all lattice points near v (fp64), the minimal-vector
counts, G by Monte Carlo against its textbook values, and strip/unstrip round trips.
"""
import itertools

import numpy as np
import pytest

OFFS8 = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.float64)   # 6561 x 8
OFFS4 = np.array(list(itertools.product((-1, 0, 1), repeat=4)), dtype=np.float64)


def brute_e8(v):
    """All E8 points within distance 1.5 of v per coordinate (covering radius is 1): D8 points
    around round(v) and D8+1/2 points around floor(v)+1/2.  Returns (best point, gap to the
    second-best distinct point) in fp64."""
    v = np.asarray(v, dtype=np.float64)
    ci = np.round(v) + OFFS8
    ci = ci[(ci.sum(axis=1) % 2) == 0]
    ch = np.floor(v) + 0.5 + OFFS8
    ch = ch[((ch - 0.5).sum(axis=1) % 2) == 0]
    c = np.vstack([ci, ch])
    d = ((c - v) ** 2).sum(axis=1)
    o = np.argsort(d, kind="stable")
    return c[o[0]], d[o[1]] - d[o[0]]


def brute_d4(v):
    v = np.asarray(v, dtype=np.float64)
    c = np.round(v) + OFFS4
    c = c[(c.sum(axis=1) % 2) == 0]
    d = ((c - v) ** 2).sum(axis=1)
    o = np.argsort(d, kind="stable")
    return c[o[0]], d[o[1]] - d[o[0]]


SQRT3 = np.sqrt(3.0)
OFFS2 = np.array(list(itertools.product(range(-2, 3), repeat=2)), dtype=np.float64)


def brute_a2(w):
    """Nearest point of the hexagonal lattice A2 = (Z x sqrt3 Z) u ((Z+1/2) x (sqrt3 Z + sqrt3/2))
    to the data-space point (w0, w1 sqrt 3), by search over both cosets around it, in fp64.
    Returns (best point in data space, gap to the second-best distinct point)."""
    v = np.array([float(w[0]), float(w[1]) * SQRT3])
    pts = []
    for p in (0.0, 0.5):
        base = np.array([np.floor(v[0]), np.floor(v[1] / SQRT3)]) + p
        c = base + OFFS2
        pts.append(np.stack([c[:, 0], c[:, 1] * SQRT3], axis=1))
    c = np.vstack(pts)
    d = ((c - v) ** 2).sum(axis=1)
    o = np.argsort(d, kind="stable")
    return c[o[0]], d[o[1]] - d[o[0]]


def a2_points(z):
    """Data-space points of A2 codes z (pairs in stretched coordinates, the point is z/2)."""
    z = np.asarray(z, dtype=np.float64).reshape(-1, 2)
    return np.stack([z[:, 0] / 2, z[:, 1] / 2 * SQRT3], axis=1)


def _test_vectors(rng, n):
    vs = [rng.uniform(-4, 4, (n, 8)), rng.standard_normal((n, 8)) * 3, rng.uniform(-1, 1, (n, 8)),
          rng.standard_normal((n // 4, 8)) * 40]
    return np.vstack(vs).astype(np.float32)


def test_e8_matches_brute_force(orc):
    rng = np.random.default_rng(0)
    V = _test_vectors(rng, 1500)
    codes = orc.nearest(orc.LAT_E8, V)
    skipped = 0
    for v, z in zip(V, codes):
        best, gap = brute_e8(v)
        if gap < 1e-5:
            skipped += 1
            continue
        assert np.array_equal(z.astype(np.float64) / 2, best), (v, z, best)
    assert skipped < 5


def test_d4_and_z_match_brute_force(orc):
    rng = np.random.default_rng(1)
    V = _test_vectors(rng, 1500)
    cd = orc.nearest(orc.LAT_D4, V)
    cz = orc.nearest(orc.LAT_Z, V)
    for v, x, z in zip(V, cd, cz):
        for h in (0, 4):
            best, gap = brute_d4(v[h:h + 4])
            if gap >= 1e-5:
                assert np.array_equal(x[h:h + 4].astype(np.float64), best)
        assert np.array_equal(z, np.rint(v).astype(np.int32))


def test_a2_matches_brute_force(orc):
    """A2's closed rule (round both cosets of the rectangular sublattice, keep the nearer under the
    metric diag(1, 3) of the stretched coordinates) equals the nearest data-space lattice point."""
    rng = np.random.default_rng(3)
    V = _test_vectors(rng, 1500)
    codes = orc.nearest(orc.LAT_A2, V)
    skipped = 0
    for v, z in zip(V, codes):
        got = a2_points(z)
        for j in range(4):
            best, gap = brute_a2(v[2 * j:2 * j + 2])
            if gap < 1e-5:
                skipped += 1
                continue
            assert np.allclose(got[j], best, rtol=0, atol=1e-9), (v[2 * j:2 * j + 2], z[2 * j:2 * j + 2], best)
    assert skipped < 10


def test_a2_codes_lattice_and_covering_radius(orc):
    """Both coordinates of a pair share their parity (z/2 in Z^2 or (Z+1/2)^2), and every input lies
    within A2's covering radius 1/sqrt 3 of its code (minimal distance 1)."""
    rng = np.random.default_rng(4)
    V = _test_vectors(rng, 4000)
    z = orc.nearest(orc.LAT_A2, V).astype(np.int64).reshape(-1, 2)
    assert np.all((z[:, 0] & 1) == (z[:, 1] & 1))
    v = V.astype(np.float64).reshape(-1, 2)
    d = np.sqrt(((a2_points(z) - np.stack([v[:, 0], v[:, 1] * SQRT3], axis=1)) ** 2).sum(axis=1))
    assert d.max() <= 1 / SQRT3 + 1e-6


def test_codes_are_lattice_points_and_within_covering_radius(orc):
    rng = np.random.default_rng(2)
    V = _test_vectors(rng, 4000)
    z = orc.nearest(orc.LAT_E8, V).astype(np.int64)
    par = z & 1
    assert np.all(par == par[:, :1])                       # one parity per octet
    assert np.all(z.sum(axis=1) % 4 == 0)                  # sum = 0 mod 4  <=>  z/2 in E8
    d = np.sqrt(((z / 2.0 - V) ** 2).sum(axis=1))
    assert d.max() <= 1.0 + 1e-6                           # covering radius of E8 is 1
    x = orc.nearest(orc.LAT_D4, V).astype(np.int64)
    assert np.all(x[:, :4].sum(axis=1) % 2 == 0) and np.all(x[:, 4:].sum(axis=1) % 2 == 0)


def _e8_min_vectors():
    pts = []
    for c in itertools.product((-1, 0, 1), repeat=8):
        if sum(abs(t) for t in c) == 2 and sum(c) % 2 == 0:
            pts.append(c)
    for s in itertools.product((-0.5, 0.5), repeat=8):
        if sum(1 for t in s if t < 0) % 2 == 0:
            pts.append(s)
    return np.array(pts, dtype=np.float64)


def test_e8_minimal_vectors(orc):
    P = _e8_min_vectors()
    assert P.shape == (CONST["e8"][3], 8)
    assert np.allclose((P ** 2).sum(axis=1), 2.0)
    z = orc.nearest(orc.LAT_E8, (0.9 * P).astype(np.float32))
    assert np.array_equal(z / 2.0, P)
    z0 = orc.nearest(orc.LAT_E8, (0.4 * P).astype(np.float32))
    assert np.all(z0 == 0)


def test_d4_minimal_vectors(orc):
    P = np.array([c for c in itertools.product((-1, 0, 1), repeat=4) if sum(abs(t) for t in c) == 2],
                 dtype=np.float64)
    assert P.shape == (24, 4)
    V = np.hstack([0.9 * P, 0.9 * P[::-1]]).astype(np.float32)
    x = orc.nearest(orc.LAT_D4, V)
    assert np.array_equal(x[:, :4], P.astype(np.int32)) and np.array_equal(x[:, 4:], P[::-1].astype(np.int32))


def test_a2_minimal_vectors(orc):
    """The 6 minimal vectors of A2, (+-1, 0) and (+-1/2, +-sqrt3/2), in stretched coordinates
    (+-1, 0) and (+-1/2, +-1/2): 0.9 c quantises to c, 0.4 c to 0."""
    P = np.array([(1, 0), (-1, 0), (0.5, 0.5), (0.5, -0.5), (-0.5, 0.5), (-0.5, -0.5)], dtype=np.float64)
    assert P.shape[0] == CONST["a2"][3]
    assert np.allclose(P[:, 0] ** 2 + 3 * P[:, 1] ** 2, 1.0)
    V = np.hstack([0.9 * P, 0.9 * P[::-1], 0.9 * P, 0.9 * P[::-1]]).astype(np.float32)
    z = orc.nearest(orc.LAT_A2, V)
    assert np.array_equal(z[:, :2] / 2.0, P) and np.array_equal(z[:, 2:4] / 2.0, P[::-1])
    z0 = orc.nearest(orc.LAT_A2, np.hstack([0.4 * P] * 4).astype(np.float32))
    assert np.all(z0 == 0)


def _constants():
    import os
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "lattice_constants.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, dim, vol, g, nmin, norm = line.split()
        rows[name.lower()] = (int(dim), float(vol), float(g), int(nmin), float(norm))
    return rows


CONST = _constants()


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_normalised_second_moment(orc, lattice):
    dim, vol, G = CONST[lattice][:3]
    """G = E|v - Q(v)|^2 / (d V^(2/d)) for v uniform over many cells; cell volume per d dims (A2:
    uniform in stretched coordinates is uniform in data space; the error is measured there)."""
    rng = np.random.default_rng(10)
    N = 400_000
    V = rng.uniform(-8, 8, (N, 8)).astype(np.float32)
    z = orc.nearest(orc.LATTICES[lattice], V).astype(np.float64)
    pts = z / 2.0 if lattice in ("e8", "a2") else z
    w = np.ones(8) if lattice != "a2" else np.tile([1.0, 3.0], 4)   # the metric in data space
    err2 = (w * (V.astype(np.float64) - pts) ** 2).reshape(N, 8 // dim, dim).sum(axis=2).ravel()
    g = err2 / (dim * vol ** (2.0 / dim))
    se = g.std() / np.sqrt(g.size)
    assert abs(g.mean() - G) < 5 * se, (g.mean(), G, se)


def test_g_ordering(orc):
    """E8 < D4 < A2 < Z in normalised second moment (the quantiser gain the pages rely on)."""
    rng = np.random.default_rng(11)
    V = rng.uniform(-8, 8, (200_000, 8)).astype(np.float32)
    ge8 = ((V - orc.nearest(orc.LAT_E8, V) / 2.0) ** 2).sum(axis=1).mean() / 8
    gd4 = ((V - orc.nearest(orc.LAT_D4, V)) ** 2).sum(axis=1).mean() / 8 / 2 ** 0.5
    ea2 = (np.tile([1.0, 3.0], 4) * (V - orc.nearest(orc.LAT_A2, V) / 2.0) ** 2).sum(axis=1).mean()
    ga2 = ea2 / 8 / (3 ** 0.5 / 2)
    gz = ((V - orc.nearest(orc.LAT_Z, V)) ** 2).sum(axis=1).mean() / 8
    assert ge8 < gd4 < ga2 < gz


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_strip_roundtrip_and_stripped_bits(orc, lattice):
    L = orc.LATTICES[lattice]
    rng = np.random.default_rng(12)
    V = (rng.standard_normal((3000, 8)) * rng.uniform(0.1, 50, (3000, 1))).astype(np.float32)
    codes = orc.nearest(L, V)
    for c in codes:
        sym, cos = orc.strip_octet(L, c)
        assert np.array_equal(orc.unstrip_octet(L, sym, cos), c)
    # the map is a bijection onto all symbol tuples: random symbols (and coset bits) unstrip to a
    # lattice point that strips back to the same symbols
    for _ in range(2000):
        sym = rng.integers(0, 200, size=8).astype(np.uint32)
        cos = int(rng.integers(0, 2)) if lattice == "e8" else int(rng.integers(0, 16)) if lattice == "a2" else 0
        c = orc.unstrip_octet(L, sym, cos).astype(np.int64)
        if lattice == "e8":
            assert np.all((c & 1) == cos) and c.sum() % 4 == 0
        if lattice == "a2":
            assert all((c[2 * j] & 1) == (c[2 * j + 1] & 1) == ((cos >> j) & 1) for j in range(4))
        if lattice == "d4":
            assert c[:4].sum() % 2 == 0 and c[4:].sum() % 2 == 0
        s2, cos2 = orc.strip_octet(L, c.astype(np.int32))
        assert np.array_equal(s2, sym) and cos2 == cos
    # fixed record per tile: 16 scale bits + coset bits (E8: 16, A2: 64) + the remainder widths, k
    # for full slots and k-1 for the halved ones (1 per E8 octet, 1 per D4 block, 1 per A2 pair).
    halved = {"e8": 1, "d4": 2, "a2": 4, "z": 0}[lattice]
    coset_bits = {"e8": 16, "a2": 64}.get(lattice, 0)
    for k in range(1, 16):
        F = orc.tile_fixed_bits(L, k)
        assert F == 16 + coset_bits + 16 * (8 * k - halved)


def test_e8_symbols_are_halved_for_slot7(orc):
    """The parity-fixed coordinate's symbol is half the magnitude of the others (it carries one
    bit less), which is why its Rice width is k-1."""
    rng = np.random.default_rng(13)
    V = (rng.standard_normal((20000, 8)) * 20).astype(np.float32)
    syms = np.array([orc.strip_octet(orc.LAT_E8, c)[0] for c in orc.nearest(orc.LAT_E8, V)], dtype=np.float64)
    r = syms[:, 7].mean() / syms[:, :7].mean()
    assert 0.45 < r < 0.55


def test_a2_stretched_slots_are_smaller(orc):
    """A2's odd slots hold the coordinate divided by sqrt 3, so their symbols average 1/sqrt 3 of
    the even slots' (which is why they take Rice width k-1)."""
    rng = np.random.default_rng(14)
    V = (rng.standard_normal((20000, 8)) * 20).astype(np.float32)
    V[:, 1::2] /= np.float32(SQRT3)   # data-space Gaussian pairs in stretched coordinates
    syms = np.array([orc.strip_octet(orc.LAT_A2, c)[0] for c in orc.nearest(orc.LAT_A2, V)], dtype=np.float64)
    r = syms[:, 1::2].mean() / syms[:, 0::2].mean()
    assert abs(r - 1 / SQRT3) < 0.02
