"""hq_encode_bound (host only, from the C-ABI library) against the oracle's streams of adversarial tiles.

The bound is derived in include/hq.h: the tile scale normalises each tile's energy (component 2 of
"Methodology: the HyperQuant pipeline"), so by Cauchy-Schwarz the sum of the lattice inputs'
magnitudes is at most TL K / step, and a Rice code (component 3, no overload region) spends
u / 2^k + 1 unary bits on a symbol of magnitude u.  Impulse tiles reach the Cauchy-Schwarz bound
with equality (a one-hot tile transforms into equal magnitudes), so they are the hardest inputs.
Every stream here is the oracle's; nothing comes from the GPU path.
"""
import numpy as np
import pytest

import kv_quantization_tile_amd as hq

LATS = {"z": 0, "d4": 1, "e8": 2, "a2": 3}


def _tiles(kind: str, T: int, tl: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = np.zeros((T, tl), dtype=np.float32)
    if kind == "impulse":            # one nonzero per tile: equal magnitudes after the transform
        x[np.arange(T), rng.integers(0, tl, T)] = rng.choice([-1.0, 1.0], T) * 10.0 ** rng.uniform(-3, 3, T)
    elif kind == "huge":             # one huge coordinate over small noise
        x[:] = rng.standard_normal((T, tl)) * 1e-3
        x[np.arange(T), rng.integers(0, tl, T)] = 1e6
    elif kind == "gauss":
        x[:] = rng.standard_normal((T, tl)) * 10.0 ** rng.uniform(-2, 2, (T, 1))
    elif kind == "flat":             # every value the same magnitude
        x[:] = rng.choice([-1.0, 1.0], (T, tl))
    elif kind == "edge":             # the precondition's edge: largest magnitude exactly 2^-60
        x[:] = rng.uniform(-1, 1, (T, tl)) * 2.0 ** -60
        x[np.arange(T), rng.integers(0, tl, T)] = 2.0 ** -60
    elif kind == "mixed":            # zero tiles, impulses and Gaussians side by side
        x[1::3, 0] = 3.0
        x[2::3] = rng.standard_normal((len(range(2, T, 3)), tl))
    return x.astype(np.float32)


def _bound(n, lat, step, k, dither, tl):
    return hq.hq_encode_bound(n, lat, step, k, dither, tl)


@pytest.mark.parametrize("lat", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("tl", [64, 128, 256])
@pytest.mark.parametrize("kind", ["impulse", "huge", "gauss", "flat", "edge", "mixed"])
def test_oracle_streams_within_bound(orc, lat, tl, kind):
    x = _tiles(kind, 9, tl, seed=tl + len(kind))
    for dither in (0, 1, 7):
        for step, k in ((2.0 ** -12, 0), (2.0 ** -12, 15), (0.05, 0), (0.3, 2), (1.0, 1), (2.0 ** 12, 0),
                        (0.3, 15), (3.7, 4)):
            s, _ = orc.encode(x, LATS[lat], 0.0, seed=5, dither=dither, step=step, rice_k=k, tile=tl)
            b = _bound(x.size, lat, step, k, dither, tl)
            assert s.size <= b, (lat, tl, kind, dither, step, k, s.size, b)
            # automatic k and rate control bound every fixed choice
            assert b <= _bound(x.size, lat, step, -1, dither, tl) <= _bound(x.size, lat, 0.0, -1, dither, tl)


@pytest.mark.parametrize("lat", ["e8", "d4", "a2", "z"])
def test_impulse_tiles_come_close_to_the_bound(orc, lat):
    """The bound is not vacuous: on impulse tiles the unary plane reaches a large part of it."""
    x = np.zeros((64, 128), dtype=np.float32)
    x[np.arange(64), np.arange(64) * 2] = 1.0
    for step, k in ((2.0 ** -12, 0), (2.0 ** -6, 2)):
        s, info = orc.encode(x, LATS[lat], 0.0, step=step, rice_k=k)
        fixed = hq.hq_stream_fixed_bytes(x.size, lat, k, 128)
        b = _bound(x.size, lat, step, k, 0, 128)
        assert s.size <= b
        assert (s.size - fixed) >= 0.7 * (b - fixed), (lat, step, k, s.size, b, fixed)


def test_rate_controlled_streams_within_bound_at_their_point(orc):
    """With rate control the stream stays under the bound taken at the point rate control picked."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((300, 128)) * 0.02).astype(np.float32)
    for lat in LATS:
        for tb in (2.0, 4.0, 6.0):
            s, info = orc.encode(x, LATS[lat], tb)
            assert s.size <= _bound(x.size, lat, info["step"], info["k"], 0, 128)


def test_below_the_stated_precondition_the_bound_can_fail(orc):
    """The bound's stated limit is real: a tile whose values all lie below 2^-60 can have its energy
    rounded down in binary32 (squares below 2^-150 vanish), a scale that is too small, and a stream
    longer than the bound.  Tiles of that kind are outside what include/hq.h promises."""
    y = np.full(128, 2.0 ** -75 * (1 - 2.0 ** -10))
    y[0] = 1.5 * 2.0 ** -75
    y *= np.where(np.arange(128) % 3 == 0, -1.0, 1.0)
    d = orc.signs(0)
    x = (d * (orc.hadamard(128) @ y) / 128.0).astype(np.float32)[None, :]
    assert np.abs(x).max() < 2.0 ** -60
    s, _ = orc.encode(x, orc.LAT_E8, 0.0, seed=0, step=1.0, rice_k=0)
    assert s.size > _bound(x.size, "e8", 1.0, 0, 0, 128)


def test_bound_rejects_bad_arguments():
    import ctypes
    out = ctypes.c_uint64(0)
    L = hq.lib()
    for kw, code in ((dict(tile=32), hq.HQ_ERR_UNSUPPORTED), (dict(lattice=7), hq.HQ_ERR_INVALID_ARG),
                     (dict(step=-3.0), hq.HQ_ERR_INVALID_ARG), (dict(step=1e-9), hq.HQ_ERR_INVALID_ARG),
                     (dict(rice_k=16), hq.HQ_ERR_INVALID_ARG), (dict(dither=2), hq.HQ_ERR_INVALID_ARG)):
        base = dict(lattice="e8", target_bps=4.0)
        base.update(kw)
        tile = base.pop("tile", 128)
        p = hq.make_params(**base, tile=tile)
        assert L.hq_encode_bound(1024, ctypes.byref(p), ctypes.byref(out)) == code, kw
    p = hq.make_params("e8", 4.0)
    assert L.hq_encode_bound(1000, ctypes.byref(p), ctypes.byref(out)) == hq.HQ_ERR_INVALID_ARG  # n % 128
    assert L.hq_encode_bound(1024, None, ctypes.byref(out)) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_encode_bound(0, ctypes.byref(p), ctypes.byref(out)) == hq.HQ_OK
    assert out.value == hq.hq_stream_fixed_bytes(0, "e8", 0)
