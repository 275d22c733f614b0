"""Statistical pins of the oracle (HyperQuant summary, gist.science/ko/paper/2606.23406):

* Methodology component 3 / contributions: the realised rate lands within ~0.01 bps of the target;
* component 4: subtractive dither gives strict per-vector inner-product unbiasedness;
* component 2: lattice gain (E8 < D4 < Z, and A2 < Z, distortion at equal rate); and the Shannon bound
  D >= 2^(-2R) for Gaussian sources as a sanity floor;
* dithered distortion equals the closed form G(L) V^(2/d) step^2 (relative to the tile energy).
"""
import numpy as np
import pytest

import synth

G = {"e8": (929.0 / 12960.0, 8, 1.0), "d4": (0.0766032346, 4, 2.0), "z": (1.0 / 12.0, 1, 1.0),
     "a2": (5.0 / (36.0 * 3.0 ** 0.5), 2, 3.0 ** 0.5 / 2.0)}


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("target", [2.0, 3.0, 4.0, 5.0])
def test_rate_within_0p01_tiny(orc, lattice, target):
    x = synth.tiny()
    s, info = orc.encode(x, orc.LATTICES[lattice], target)
    assert abs(info["payload_bps"] - target) <= 0.01


@pytest.mark.parametrize("target", [3.0, 4.0, 5.0])
def test_rate_within_0p01_weight_slice(orc, target):
    """A 2048 x 4096 slice of the weight workload: 65,536 tiles, so rate control samples 1/8."""
    w = synth.weight(rows=2048)
    s, info = orc.encode(w, orc.LAT_E8, target)
    assert abs(info["payload_bps"] - target) <= 0.01


@pytest.mark.parametrize("target", [2.0, 3.0])
def test_rate_within_0p01_kv_slice_dithered(orc, target):
    k = synth.kv(layer=3, is_v=0, heads=2, tokens=8192)
    s, info = orc.encode(k, orc.LAT_E8, target, seed=synth.kv_seed(3, 0), dither=True)
    assert abs(info["payload_bps"] - target) <= 0.01


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_dithered_mse_closed_form(orc, lattice):
    """With dither the error in lattice units is uniform on the Voronoi cell, so per tile
    E|xhat - x|^2 / |x|^2 = G V^(2/d) step^2 (up to the bf16 rounding of the scale)."""
    g, d, vol = G[lattice]
    L = orc.LATTICES[lattice]
    x = synth.gaussian(128 * 4000, seed=21).reshape(-1, 128)
    step = 0.5
    codes, scales = orc.quantize(x, L, step, seed=3, dither=True)
    y = orc.dequantize(codes, scales, L, step, seed=3, dither=True).reshape(x.shape)
    s = synth.bf16_to_f32(scales).astype(np.float64)
    r = ((y - x).astype(np.float64) ** 2).sum(axis=1) / (s * s)
    want = g * vol ** (2.0 / d) * step ** 2
    se = r.std() / np.sqrt(r.size)
    assert abs(r.mean() - want) < 5 * se, (r.mean(), want, se)


@pytest.mark.parametrize("lattice", ["e8", "a2", "z"])
def test_dither_per_vector_unbiased(orc, lattice):
    """One fixed tile x, repeated M times: every copy gets its own dither draw (the dither counter
    holds the tile index) and the same D.  The mean reconstruction converges to x, so
    <q, xhat> is unbiased for every q; without dither the error is systematic."""
    L = orc.LATTICES[lattice]
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128).astype(np.float32)
    q = rng.standard_normal(128)
    M = 20000
    X = np.tile(x, (M, 1))
    step = 1.0
    c, sc = orc.quantize(X, L, step, seed=11, dither=True)
    Y = orc.dequantize(c, sc, L, step, seed=11, dither=True).reshape(M, 128).astype(np.float64)
    ip = Y @ q - float(x.astype(np.float64) @ q)
    assert abs(ip.mean()) < 4 * ip.std() / np.sqrt(M)
    assert np.all(np.abs(Y.mean(axis=0) - x) < 5 * Y.std(axis=0) / np.sqrt(M))
    # control: no dither -> deterministic reconstruction, biased by many standard errors
    c0, sc0 = orc.quantize(X[:1], L, step, seed=11, dither=False)
    y0 = orc.dequantize(c0, sc0, L, step, seed=11, dither=False).astype(np.float64)
    assert abs(y0 @ q - float(x.astype(np.float64) @ q)) > 10 * ip.std() / np.sqrt(M)


def test_shannon_floor_and_lattice_ordering(orc):
    x = synth.gaussian(128 * 2048, seed=31)
    mse = {}
    for lat in ("e8", "d4", "a2", "z"):
        s, info = orc.encode(x, orc.LATTICES[lat], 4.0)
        y = orc.decode(s, x.size)
        mse[lat] = float(np.mean((y.astype(np.float64) - x) ** 2) / np.mean(x.astype(np.float64) ** 2))
        assert mse[lat] >= 2.0 ** (-2 * info["payload_bps"])
    assert mse["e8"] < mse["d4"] < mse["z"]
    assert mse["a2"] < mse["z"]


def test_sample_tiles_cover_each_stratum(orc):
    T, N = 458752, 8192
    ts = [orc.sample_tile(i, T, N) for i in range(N)]
    for i in range(0, N, 97):
        lo, hi = (i * T) // N, ((i + 1) * T) // N
        assert lo <= ts[i] < hi
    # positions within a 32-tile row are spread over all residues (no aliasing with row length)
    assert len(set(t % 32 for t in ts)) == 32
    assert [orc.sample_tile(i, 100, 100) for i in range(100)] == list(range(100))


@pytest.mark.parametrize("tile", [64, 256])
@pytest.mark.parametrize("target", [2.0, 4.0])
def test_rate_within_0p01_other_tiles(orc, tile, target):
    x = synth.tiny()
    for lat in ("e8", "d4"):
        s, info = orc.encode(x, orc.LATTICES[lat], target, tile=tile)
        assert abs(info["payload_bps"] - target) <= 0.01


@pytest.mark.parametrize("tile", [64, 256])
def test_dithered_mse_closed_form_other_tiles(orc, tile):
    """The per-tile dithered error |xhat - x|^2 / s^2 = G V^(2/d) step^2 holds at every tile length
    (x - xhat = D H (y - yhat) / n and |H z|^2 = n |z|^2)."""
    g, d, vol = G["e8"]
    x = synth.gaussian(tile * 3000, seed=22).reshape(-1, tile)
    step = 0.5
    codes, scales = orc.quantize(x, orc.LAT_E8, step, seed=3, dither=True, tile=tile)
    y = orc.dequantize(codes, scales, orc.LAT_E8, step, seed=3, dither=True, tile=tile).reshape(x.shape)
    s = synth.bf16_to_f32(scales).astype(np.float64)
    r = ((y - x).astype(np.float64) ** 2).sum(axis=1) / (s * s)
    want = g * vol ** (2.0 / d) * step ** 2
    se = r.std() / np.sqrt(r.size)
    assert abs(r.mean() - want) < 5 * se, (r.mean(), want, se)
