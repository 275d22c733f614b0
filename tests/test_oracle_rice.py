"""Pins of the oracle's Rice coder and bitstream (HyperQuant summary, gist.science/ko/paper/2606.23406,
Methodology component 3: remaining symbols are Rice-coded; the coding is lossless).

Exhaustive Rice round trips on a small domain, the code-length formula, whole-stream round trips
(decode(encode(x)) equals the direct dequantisation of the quantiser's codes), and corrupt-stream
rejection.
"""
import numpy as np
import pytest

import synth


def test_rice_exhaustive_roundtrip_and_length(orc):
    vals = np.arange(4096, dtype=np.uint32)
    for k in range(16):
        out, ulen = orc.rice_roundtrip(vals, k)
        assert np.array_equal(out, vals)
        assert ulen == int(np.sum(vals >> k)) + vals.size     # unary part: q zeros + a one


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("dither", [False, True])
def test_stream_roundtrip_equals_dequantisation(orc, lattice, dither):
    L = orc.LATTICES[lattice]
    x = synth.tiny(seed=3, tiles=130)          # two full chunks + a ragged one
    s, info = orc.encode(x, L, 3.0, seed=7, dither=dither)
    y = orc.decode(s, x.size)
    codes, scales = orc.quantize(x, L, info["step"], seed=7, dither=dither)
    ref = orc.dequantize(codes, scales, L, info["step"], seed=7, dither=dither)
    assert np.array_equal(y, ref)
    # bf16 output is the round-to-nearest-even of the fp32 output
    yb = orc.decode(s, x.size, out_dtype="bf16")
    assert np.array_equal(yb, synth.bf16_bits(ref))
    # stream size bookkeeping
    assert info["bytes"] == s.size
    fo, uo, F = orc.layout(x.size, L, info["k"])
    assert info["payload_bits"] == 130 * (F - 16) + info["unary_bits"]


def test_bf16_input_and_empty(orc):
    w = synth.weight(rows=16, cols=512)
    s, info = orc.encode(w, orc.LAT_E8, 4.0)
    y = orc.decode(s, w.size)
    codes, scales = orc.quantize(w, orc.LAT_E8, info["step"])
    assert np.array_equal(y, orc.dequantize(codes, scales, orc.LAT_E8, info["step"]))
    e = np.zeros(0, dtype=np.float32)
    s0, info0 = orc.encode(e, orc.LAT_E8, 4.0)
    assert s0.size == info0["bytes"] and orc.decode(s0, 0).size == 0


def test_fixed_step_and_k(orc):
    x = synth.tiny(seed=4)
    s, info = orc.encode(x, orc.LAT_E8, 0.0, step=0.3, rice_k=5)
    assert info["k"] == 5 and abs(info["step"] - 0.3) < 1e-7
    codes, scales = orc.quantize(x, orc.LAT_E8, info["step"])
    assert np.array_equal(orc.decode(s, x.size), orc.dequantize(codes, scales, orc.LAT_E8, info["step"]))


def test_corrupt_streams_rejected(orc):
    x = synth.tiny(seed=5)
    s, info = orc.encode(x, orc.LAT_E8, 4.0)
    assert orc.decode_status(s, x.size) == orc.OK
    bad = s.copy(); bad[0] ^= 1
    assert orc.decode_status(bad, x.size) == orc.ERR_CORRUPT           # magic
    assert orc.decode_status(s, x.size + 128) == orc.ERR_CORRUPT       # wrong n
    assert orc.decode_status(s[:-8], x.size) == orc.ERR_CORRUPT        # truncated
    bad = s.copy(); bad[128 + 4] ^= 0xFF                                # chunk index end entry
    assert orc.decode_status(bad, x.size) == orc.ERR_CORRUPT
    bad = s.copy(); bad[-8:] = 0                                         # lose terminators
    assert orc.decode_status(bad, x.size) == orc.ERR_CORRUPT


def test_nonfinite_input(orc):
    x = synth.tiny(seed=6).copy()
    x[3, 7] = np.inf
    with pytest.raises(orc.OracleError) as e:
        orc.encode(x, orc.LAT_E8, 4.0, step=0.3, rice_k=2)
    assert e.value.code == orc.ERR_NONFINITE


@pytest.mark.parametrize("tile", [64, 256])
@pytest.mark.parametrize("lattice", ["e8", "a2", "z"])
def test_stream_roundtrip_other_tiles(orc, tile, lattice):
    """Tiles of 64 and 256 values: decode(encode(x)) equals the direct dequantisation, a chunk holds
    8192 / tile tiles, and the tile record has 16 scale bits, the lattice's coset bits and the
    remainders of tile / 8 octets."""
    L = orc.LATTICES[lattice]
    x = synth.tiny(seed=5, tiles=130).reshape(-1)        # 16640 values: ragged last chunk
    for dither in (False, True):
        s, info = orc.encode(x, L, 3.0, seed=4, dither=dither, tile=tile)
        y = orc.decode(s, x.size)
        codes, scales = orc.quantize(x, L, info["step"], seed=4, dither=dither, tile=tile)
        assert np.array_equal(y, orc.dequantize(codes, scales, L, info["step"], seed=4, dither=dither, tile=tile))
        h = s[:128]
        assert int(h[8]) | (int(h[9]) << 8) == tile and int(h[11]) == {64: 7, 256: 5}[tile]
        fo, uo, F = orc.layout(x.size, L, info["k"], tile)
        oct_bits = {"e8": 8 * info["k"] - (1 if info["k"] else 0), "a2": 8 * info["k"] - (4 if info["k"] else 0),
                    "z": 8 * info["k"]}[lattice]
        coset = {"e8": tile // 8, "a2": tile // 2, "z": 0}[lattice]
        assert F == 16 + coset + (tile // 8) * oct_bits
        assert info["payload_bits"] == (x.size // tile) * (F - 16) + info["unary_bits"]
        # a stream is decoded only at its own tile size: another n or a damaged tile field fails
        bad = s.copy()
        bad[8] ^= 0xC0
        with pytest.raises(orc.OracleError):
            orc.decode(bad, x.size)


@pytest.mark.parametrize("case", ["weight_4bps", "kv_dither_2bps"])
def test_per_tile_rice_k_would_not_pay(orc, case):
    """Why the Rice parameter is one per stream, not one per tile: after the per-tile RMS scale,
    every tile's symbols follow nearly the same law, so the per-tile best k saves far less than
    the 4 bits per tile (1/32 bit per value) it would cost to store.  Measured on the oracle's own
    stripped symbols at the rate-controlled operating point."""
    if case == "weight_4bps":
        x, tb, seed, dither = synth.weight(rows=64), 4.0, 0, False
    else:
        x, tb, seed, dither = synth.kv(1, 0, heads=1, tokens=2048), 2.0, synth.kv_seed(1, 0), True
    step, _, k_glob = orc.rate(x, orc.LAT_E8, tb, seed=seed, dither=dither)
    codes, _ = orc.quantize(x, orc.LAT_E8, step, seed=seed, dither=dither)
    tiles = codes.reshape(-1, 128)
    ks = np.arange(0, 12)
    bits = np.zeros((tiles.shape[0], ks.size), dtype=np.int64)
    for t in range(tiles.shape[0]):
        syms = np.stack([orc.strip_octet(orc.LAT_E8, tiles[t, 8 * o:8 * o + 8])[0] for o in range(16)])
        for j, k in enumerate(ks):
            w = np.array([k] * 7 + [max(k - 1, 0)], dtype=np.int64)
            bits[t, j] = ((syms.astype(np.int64) >> w) + 1 + w).sum()
    glob = bits.sum(axis=0)
    assert int(np.argmin(glob)) == k_glob
    saving_per_value = (glob.min() - bits.min(axis=1).sum()) / codes.size
    assert saving_per_value < 0.25 * (4.0 / 128.0), saving_per_value
