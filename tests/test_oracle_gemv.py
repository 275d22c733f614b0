"""Pins of the oracle's product with the decoded matrix (test infrastructure of the fused
decode + matrix-vector product): the coordinate decoder against the oracle's own binary32 decode,
the Hadamard construction against scipy, and the reference product against a plain product with
the decoded matrix."""
import numpy as np
import pytest
import scipy.linalg

import synth

U = 2.0 ** -24


def test_hadamard128_is_sylvester(orc):
    assert np.array_equal(orc.hadamard128(), scipy.linalg.hadamard(128).astype(np.float64))


@pytest.mark.parametrize("lattice,dither,target", [("e8", False, 4.0), ("e8", True, 2.0), ("d4", False, 3.0),
                                                    ("a2", True, 3.0), ("z", False, 5.0)])
def test_decode_coords_reconstruct_the_decode(orc, lattice, dither, target):
    """D H yhat / 128 in binary64 equals the oracle's binary32 decode up to the seven butterfly
    roundings: |difference| <= 8 u ||yhat_tile||_1 / 128 per value."""
    x = synth.tiny(seed=3, tiles=64)
    s, _ = orc.encode(x, orc.LATTICES[lattice], target, seed=11, dither=dither)
    n = x.size
    yh = orc.decode_coords(s, n).reshape(-1, 128)
    d = orc.signs(11).astype(np.float64)
    exact = (yh @ scipy.linalg.hadamard(128).astype(np.float64)) * d / 128.0
    got = orc.decode(s, n).reshape(-1, 128).astype(np.float64)
    tol = 8 * U * np.abs(yh).sum(axis=1, keepdims=True) / 128.0
    assert np.all(np.abs(got - exact) <= tol + 1e-300)
    # and the coordinates are the lattice values times the tile factor: not all zero, finite
    assert np.isfinite(yh).all() and np.abs(yh).sum() > 0


def test_gemv_reference_is_the_product_with_the_decoded_matrix(orc):
    """gemv_reference equals W_hat @ x with W_hat the oracle's binary32 decode, within the decode's
    rounding (8 u ||yhat||_1 / 128 per value, times |x|)."""
    rows, cols = 24, 512
    g = np.random.Generator(np.random.PCG64(5))
    w = g.standard_normal((rows, cols)).astype(np.float32)
    x = g.standard_normal(cols)
    s, _ = orc.encode(w, orc.LAT_E8, 4.0, seed=7)
    y, bound = orc.gemv_reference(s, rows, cols, x, seed=7)
    wh = orc.decode(s, rows * cols).reshape(rows, cols).astype(np.float64)
    plain = wh @ x
    yh = orc.decode_coords(s, rows * cols).reshape(rows, cols // 128, 128)
    # per value |W_exact - W_hat| <= 8 u ||yhat_tile||_1 / 128, so per row the products differ by
    # at most the sum over tiles of that times ||x_tile||_1
    tol = (8 * U / 128.0) * np.einsum("rj,j->r", np.abs(yh).sum(axis=2), np.abs(x.reshape(-1, 128)).sum(axis=1))
    assert np.all(np.abs(y - plain) <= tol + 1e-12)
    assert np.all(bound >= 0) and bound.shape == (rows,)


def test_gemv_reference_tracks_the_original_matrix(orc):
    """At 6 bits per value the decoded matrix is close to the original: the product's error is
    the quantisation error, far below the product itself."""
    rows, cols = 16, 1024
    g = np.random.Generator(np.random.PCG64(9))
    w = (0.02 * g.standard_normal((rows, cols))).astype(np.float32)
    x = g.standard_normal(cols)
    s, _ = orc.encode(w, orc.LAT_E8, 6.0, seed=1)
    y, _ = orc.gemv_reference(s, rows, cols, x, seed=1)
    exact = w.astype(np.float64) @ x
    assert np.linalg.norm(y - exact) <= 0.05 * np.linalg.norm(exact)


@pytest.mark.parametrize("tile", [64, 256])
def test_decode_coords_other_tiles(orc, tile):
    """D H_n yhat / n reconstructs the oracle's binary32 decode at tiles of 64 and 256 values."""
    x = synth.tiny(seed=4, tiles=64)
    s, _ = orc.encode(x, orc.LAT_E8, 3.0, seed=2, dither=True, tile=tile)
    n = x.size
    yh = orc.decode_coords(s, n).reshape(-1, tile)
    exact = (yh @ scipy.linalg.hadamard(tile).astype(np.float64)) * orc.signs(2, tile).astype(np.float64) / tile
    got = orc.decode(s, n).reshape(-1, tile).astype(np.float64)
    tol = 9 * U * np.abs(yh).sum(axis=1, keepdims=True) / tile
    assert np.all(np.abs(got - exact) <= tol + 1e-300)
