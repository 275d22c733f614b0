"""Pins of the oracle's dither format options (HyperQuant summary, Methodology component 4: a fresh
U ~ Unif(V(L)) added before quantising and subtracted after).  The pages fix neither the generator's
round count nor the draw's resolution; the dither flags choose them (bit 0 on, bit 1 Philox with 7
rounds, bit 2 a 24-bit draw).  Every option must keep U on the Voronoi cell, uniform (the dithered
error's closed form), and the reconstruction unbiased; the draws must differ between options and
decode exactly."""
import numpy as np
import pytest

import synth

FLAGS = (1, 3, 5, 7)
G = {"e8": (929.0 / 12960.0, 8, 1.0), "d4": (0.0766032346, 4, 2.0), "z": (1.0 / 12.0, 1, 1.0),
     "a2": (5.0 / (36.0 * 3.0 ** 0.5), 2, 3.0 ** 0.5 / 2.0)}


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_dither_lies_in_the_voronoi_cell(orc, flags, lattice):
    """U = b - Q(b): its nearest lattice point is the origin, for every option."""
    L = orc.LATTICES[lattice]
    u = np.stack([orc.dither_octet(11, t, o, L, flags) for t in range(40) for o in range(16)])
    assert np.all(orc.nearest(L, u) == 0)


def test_dither_resolution(orc):
    """b = U + Q(b) sits on the draw's grid: 2^-15 for the 16-bit draw, 2^-23 for the 24-bit one
    (and not on the coarser grid)."""
    L = orc.LAT_Z   # Q(b) is an integer vector: b = U + rint(b) exactly
    for flags, grid, coarser in ((1, 2.0 ** 15, None), (5, 2.0 ** 23, 2.0 ** 15)):
        u = np.stack([orc.dither_octet(2, t, o, L, flags) for t in range(64) for o in range(16)]).astype(np.float64)
        b = np.mod(u, 1.0)
        assert np.all(b * grid == np.round(b * grid))
        if coarser:
            assert np.mean(b * coarser != np.round(b * coarser)) > 0.9


def test_options_draw_different_streams(orc):
    us = {f: np.stack([orc.dither_octet(4, t, o, orc.LAT_E8, f) for t in range(8) for o in range(16)])
          for f in FLAGS}
    for a in FLAGS:
        for b in FLAGS:
            if a < b:
                assert np.mean(us[a] != us[b]) > 0.99, (a, b)


@pytest.mark.parametrize("flags", (3, 5, 7))
@pytest.mark.parametrize("lattice", ["e8", "a2"])
def test_dithered_mse_closed_form_options(orc, flags, lattice):
    """Uniform U on V(L) makes the per-tile error |xhat - x|^2 / s^2 = G V^(2/d) step^2."""
    g, d, vol = G[lattice]
    L = orc.LATTICES[lattice]
    x = synth.gaussian(128 * 3000, seed=23).reshape(-1, 128)
    step = 0.5
    codes, scales = orc.quantize(x, L, step, seed=3, dither=flags)
    y = orc.dequantize(codes, scales, L, step, seed=3, dither=flags).reshape(x.shape)
    s = synth.bf16_to_f32(scales).astype(np.float64)
    r = ((y - x).astype(np.float64) ** 2).sum(axis=1) / (s * s)
    want = g * vol ** (2.0 / d) * step ** 2
    se = r.std() / np.sqrt(r.size)
    assert abs(r.mean() - want) < 5 * se, (r.mean(), want, se)


def test_unbiased_with_7_rounds_and_24_bits(orc):
    """One tile repeated M times, flags 7: the mean reconstruction converges to x."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(128).astype(np.float32)
    q = rng.standard_normal(128)
    M = 20000
    X = np.tile(x, (M, 1))
    c, sc = orc.quantize(X, orc.LAT_E8, 1.0, seed=13, dither=7)
    Y = orc.dequantize(c, sc, orc.LAT_E8, 1.0, seed=13, dither=7).reshape(M, 128).astype(np.float64)
    ip = Y @ q - float(x.astype(np.float64) @ q)
    assert abs(ip.mean()) < 4 * ip.std() / np.sqrt(M)
    assert np.all(np.abs(Y.mean(axis=0) - x) < 5 * Y.std(axis=0) / np.sqrt(M))


@pytest.mark.parametrize("flags", (3, 5, 7))
def test_stream_roundtrip_with_options(orc, flags):
    """The stream records the flags (header byte 7) and decodes to the dequantised codes."""
    x = synth.tiny()
    s, info = orc.encode(x, orc.LAT_E8, 2.0, seed=5, dither=flags)
    assert int(s[7]) == flags
    assert abs(info["payload_bps"] - 2.0) <= 0.01
    c, sc = orc.quantize(x, orc.LAT_E8, info["step"], seed=5, dither=flags)
    want = orc.dequantize(c, sc, orc.LAT_E8, info["step"], seed=5, dither=flags)
    assert np.array_equal(orc.decode(s, x.size).view(np.uint32), want.view(np.uint32))


def test_invalid_flags_rejected(orc):
    x = synth.tiny(tiles=4)
    for bad in (2, 4, 6, 8, 9):
        with pytest.raises(orc.OracleError) as e:
            orc.encode(x, orc.LAT_E8, 2.0, dither=bad)
        assert e.value.code == orc.ERR_INVALID_ARG
    s, _ = orc.encode(x, orc.LAT_E8, 2.0, dither=1)
    for bad in (2, 4, 6, 8):
        t = s.copy()
        t[7] = bad
        with pytest.raises(orc.OracleError) as e:
            orc.decode(t, x.size)
        assert e.value.code == orc.ERR_CORRUPT
