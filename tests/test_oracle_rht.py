"""Pins of the oracle's randomized Hadamard transform and tile scale.

HyperQuant summary (gist.science/ko/paper/2606.23406), Methodology component 1: RHT_n(x) = H_n D x
with a Walsh-Hadamard H_n and a random sign diagonal D; the transform is orthogonal and keeps l2
errors.  Pinned against scipy's dense Hadamard matrix, H H = 128 I, norm preservation and the exact
inverse, and the tile scale against an exact rational computation.
"""
from fractions import Fraction

import numpy as np
import scipy.linalg

H = scipy.linalg.hadamard(128).astype(np.int64)


def test_fwht_columns_are_sylvester_hadamard(orc):
    for i in range(128):
        e = np.zeros(128, dtype=np.float32)
        e[i] = 1.0
        assert np.array_equal(orc.fwht128(e), H[:, i].astype(np.float32))


def test_fwht_exact_on_integers_and_involution(orc):
    rng = np.random.default_rng(0)
    for _ in range(50):
        x = rng.integers(-2**15, 2**15, size=128)
        y = orc.fwht128(x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), H @ x)          # exact: |Hx| < 2^23
        z = orc.fwht128(y)
        assert np.array_equal(z.astype(np.int64), 128 * x)        # H H = 128 I


def test_fwht_float_accuracy_and_norm(orc):
    rng = np.random.default_rng(1)
    for scale in (1e-30, 1e-3, 1.0, 1e20):
        x = (rng.standard_normal(128) * scale).astype(np.float32)
        y = orc.fwht128(x).astype(np.float64)
        ref = H @ x.astype(np.float64)
        assert np.max(np.abs(y - ref)) <= 1e-6 * np.linalg.norm(ref)
        assert abs(np.sum(y * y) / (128 * np.sum(x.astype(np.float64) ** 2)) - 1) < 1e-6


def test_rht_inverse(orc):
    rng = np.random.default_rng(2)
    for seed in (0, 5, 2**33 + 1):
        d = orc.signs(seed)
        x = rng.standard_normal(128).astype(np.float32)
        y = orc.fwht128(d * x)
        back = d * (orc.fwht128(y) * np.float32(2.0 ** -7))
        assert np.max(np.abs(back - x)) <= 2.0 ** -19 * np.linalg.norm(x)


def test_sumsq_pairwise_accuracy(orc):
    rng = np.random.default_rng(3)
    for _ in range(100):
        y = (rng.standard_normal(128) * 10.0 ** rng.uniform(-5, 5)).astype(np.float32)
        ref = float(np.sum(y.astype(np.float64) ** 2))
        assert abs(orc.sumsq128(y) / ref - 1) < 8 * 2.0 ** -24
        yi = rng.integers(-300, 300, size=128).astype(np.float32)   # sum < 2^24: exact in binary32
        assert orc.sumsq128(yi) == float(np.sum(yi.astype(np.int64) ** 2))


def _bf16_values_near(r: float):
    """All positive bfloat16 values within a few ulps of r, as exact Fractions with their bits."""
    b = int(np.array([r], dtype=np.float32).view(np.uint32)[0]) >> 16
    out = []
    for c in range(max(b - 3, 1), b + 4):
        v = np.array([c << 16], dtype=np.uint32).view(np.float32)[0]
        out.append((Fraction(float(v)), c))
    return out


def test_scale_is_exact_rne_of_sqrt(orc):
    """s = the bfloat16 nearest to sqrt(S/128) (ties to even), decided in exact rational arithmetic."""
    rng = np.random.default_rng(4)
    Ss = list((10.0 ** rng.uniform(-40, 38, 3000)).astype(np.float32))
    # exact ties and near-ties: S = 128 m^2 for bfloat16 midpoints m, and one ulp either side
    for _ in range(300):
        c = int(rng.integers(0x3000, 0x5000))
        lo = np.array([c << 16], dtype=np.uint32).view(np.float32)[0]
        hi = np.array([(c + 1) << 16], dtype=np.uint32).view(np.float32)[0]
        m = (np.float64(lo) + np.float64(hi)) / 2
        S = np.float32(128.0 * m * m)
        Ss += [S, np.nextafter(S, np.float32(np.inf)), np.nextafter(S, np.float32(0))]
    for S in Ss:
        S = np.float32(S)
        if not np.isfinite(S) or S <= 0:
            continue
        X = Fraction(float(S)) / 128
        cands = _bf16_values_near(float(np.sqrt(np.float64(S) / 128)))
        cands.sort()
        # nearest candidate to sqrt(X): s1 < s2 neighbours, sqrt(X) < (s1+s2)/2  <=>  X < ((s1+s2)/2)^2
        best = None
        for (a, ca), (b, cb) in zip(cands, cands[1:]):
            mid2 = ((a + b) / 2) ** 2
            if a * a <= X <= b * b:
                if X < mid2:
                    best = ca
                elif X > mid2:
                    best = cb
                else:
                    best = ca if ca % 2 == 0 else cb
                break
        assert best is not None
        assert orc.scale_bits(float(S)) == best, S
    assert orc.scale_bits(0.0) == 0


# ---- tiles of 64 and 256 values (the summary gives 128 as an example tile size) ----------------

import pytest  # noqa: E402


@pytest.mark.parametrize("n", [64, 256])
def test_fwht_other_tile_lengths(orc, n):
    """H_n e_i is column i of scipy's Sylvester matrix; exact on integers; H_n H_n = n I."""
    Hn = scipy.linalg.hadamard(n).astype(np.int64)
    for i in range(n):
        e = np.zeros(n, dtype=np.float32)
        e[i] = 1.0
        assert np.array_equal(orc.fwht(e), Hn[:, i].astype(np.float32))
    rng = np.random.default_rng(n)
    for _ in range(20):
        x = rng.integers(-2**14, 2**14, size=n)
        y = orc.fwht(x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), Hn @ x)
        assert np.array_equal(orc.fwht(y).astype(np.int64), n * x)
    x = rng.standard_normal(n).astype(np.float32)
    y = orc.fwht(x).astype(np.float64)
    assert abs(np.sum(y * y) / (n * np.sum(x.astype(np.float64) ** 2)) - 1) < 1e-6
    # the 128-value transform is the same routine
    x = rng.standard_normal(128).astype(np.float32)
    assert np.array_equal(orc.fwht(x), orc.fwht128(x))


@pytest.mark.parametrize("n", [64, 256])
def test_sumsq_and_scale_other_lengths(orc, n):
    rng = np.random.default_rng(n + 1)
    for _ in range(50):
        y = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 5)).astype(np.float32)
        ref = float(np.sum(y.astype(np.float64) ** 2))
        assert abs(orc.sumsq(y) / ref - 1) < 9 * 2.0 ** -24
        yi = rng.integers(-200, 200, size=n).astype(np.float32)
        assert orc.sumsq(yi) == float(np.sum(yi.astype(np.int64) ** 2))
    # the scale is sqrt(S / n) rounded to bfloat16: S = n m^2 for an exact bfloat16 m gives m
    for c in (0x3F80, 0x4049, 0x3A12, 0x4611):
        m = np.array([c << 16], dtype=np.uint32).view(np.float32)[0]
        S = np.float32(np.float64(m) * np.float64(m) * n)
        assert orc.scale_bits(float(S), n) == c


def test_signs_of_other_lengths_extend_the_128_diagonal(orc):
    """Tiles of 64 use the first 64 signs of the 128-value diagonal; tiles of 256 append the 128
    signs of the next Philox counter (1, 0, 0, 0), bit i mod 32 of word i/32 as before."""
    for seed in (0, 7, 2**40 + 3):
        d128 = orc.signs(seed)
        assert np.array_equal(orc.signs(seed, 64), d128[:64])
        d256 = orc.signs(seed, 256)
        assert np.array_equal(d256[:128], d128)
        w = orc.philox4x32_10([1, 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        bits = np.array([(int(w[i >> 5]) >> (i & 31)) & 1 for i in range(128)])
        assert np.array_equal(d256[128:], np.where(bits == 1, -1.0, 1.0).astype(np.float32))
        assert 40 < np.sum(d256 < 0) < 216


@pytest.mark.parametrize("n", [64, 256])
def test_rht_inverse_other_lengths(orc, n):
    rng = np.random.default_rng(n + 2)
    d = orc.signs(3, n)
    x = rng.standard_normal(n).astype(np.float32)
    back = d * (orc.fwht(orc.fwht(d * x)) * np.float32(1.0 / n))
    assert np.max(np.abs(back - x)) <= 2.0 ** -19 * np.linalg.norm(x)
