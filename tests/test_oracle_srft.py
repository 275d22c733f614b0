"""Pins of the oracle's SRFT fixed-rate KV codec ("When quantization is free" summary, Methodology 1-3:
SRFT(x) = pack(F diag(s) x) with F the unitary DFT, radix-2 Stockham FFT, Hermitian unpack,
per-channel lambda, per-group absmax, signed int4 / int8, nibble packing).

Independent references: numpy's FFT in binary64 (the transform and its packing), closed forms (an
impulse, orthogonality, the transpose as inverse), numpy's binary16 conversion (the group scales), and
the quantiser's own invariants (code range, the group maximum at +-L, error at most half a step)."""
import numpy as np
import pytest


def packed_reference(x, seed, orc, lam=None):
    """SRFT(x) / lambda in binary64 from numpy's FFT: y_0 = X_0, y_1 = X_64, y_2k + i y_2k+1 =
    sqrt(2) X_k for the unitary DFT X of s * x."""
    s = np.zeros(128, dtype=np.float32)
    orc.lib().hqo_signs(seed, orc._p(s))
    X = np.fft.fft(s.astype(np.float64) * np.asarray(x, dtype=np.float64)) / np.sqrt(128.0)
    y = np.zeros(128)
    y[0], y[1] = X[0].real, X[64].real
    y[2::2] = np.sqrt(2.0) * X[1:64].real
    y[3::2] = np.sqrt(2.0) * X[1:64].imag
    return y / (1.0 if lam is None else np.asarray(lam, dtype=np.float64))


def test_twiddles(orc):
    for n in (64, 128):
        for k in range(n):
            c, s = orc.srft_twiddle(n, k)
            rc, rs = np.float32(np.cos(2 * np.pi * k / n)), np.float32(np.sin(2 * np.pi * k / n))
            assert abs(c - rc) <= 6e-8 and abs(s - rs) <= 6e-8, (n, k)
        for k in range(n // 4 + 1):  # first quadrant: cos(pi/2 - a) = sin(a), bit for bit
            c, s = orc.srft_twiddle(n, k)
            c2, s2 = orc.srft_twiddle(n, n // 4 - k)
            assert (c, s) == (s2, c2), (n, k)
        for k, want in ((0, (1.0, 0.0)), (n // 4, (0.0, 1.0)), (n // 2, (-1.0, 0.0)), (3 * n // 4, (0.0, -1.0))):
            c, s = orc.srft_twiddle(n, k)
            assert (c, s) == want
            assert np.signbit(np.float32(c)) == np.signbit(np.float32(want[0]))


@pytest.mark.parametrize("seed", [0, 7, 123456789])
def test_forward_matches_numpy_dft(orc, seed):
    g = np.random.default_rng(seed)
    for scale in (1.0, 30.0):
        x = (g.standard_normal(128) * scale).astype(np.float32)
        v = orc.srft_forward(x, seed)
        ref = packed_reference(x, seed, orc)
        assert np.abs(v - ref).max() <= 2e-6 * np.linalg.norm(x)
    lam = (0.5 + g.random(128)).astype(np.float32)
    v = orc.srft_forward(x, seed, lam)
    ref = packed_reference(x, seed, orc, lam)
    assert np.abs(v - ref).max() <= 4e-6 * np.linalg.norm(x)


def test_impulse_closed_form(orc):
    seed = 9
    s = np.zeros(128, dtype=np.float32)
    orc.lib().hqo_signs(seed, orc._p(s))
    for j in (0, 1, 77):
        x = np.zeros(128, dtype=np.float32)
        x[j] = 1.0
        v = orc.srft_forward(x, seed).astype(np.float64)
        k = np.arange(1, 64)
        want = np.zeros(128)
        want[0] = s[j] / np.sqrt(128.0)
        want[1] = s[j] * (-1.0) ** j / np.sqrt(128.0)
        want[2::2] = s[j] * np.cos(2 * np.pi * k * j / 128) / 8.0
        want[3::2] = -s[j] * np.sin(2 * np.pi * k * j / 128) / 8.0
        assert np.abs(v - want).max() < 2e-7, j


def test_orthogonal_and_inverse_is_transpose(orc):
    g = np.random.default_rng(3)
    for seed in (1, 2):
        x = g.standard_normal(128).astype(np.float32)
        v = orc.srft_forward(x, seed)
        assert abs(np.linalg.norm(v.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) < 1e-6 * np.linalg.norm(x)
        assert np.abs(orc.srft_inverse(v, seed) - x).max() < 2e-6 * np.linalg.norm(x)
    # the inverse applied to a packed basis vector is the matching row of the forward map
    seed = 4
    fwd = np.stack([orc.srft_forward(np.eye(128, dtype=np.float32)[i], seed) for i in range(128)]).astype(np.float64)
    for c in (0, 1, 2, 3, 64, 127):
        e = np.zeros(128, dtype=np.float32)
        e[c] = 1.0
        assert np.abs(orc.srft_inverse(e, seed) - fwd[:, c]).max() < 2e-7, c


@pytest.mark.parametrize("bits", [4, 8])
def test_quantiser_invariants(orc, bits):
    L = 7 if bits == 4 else 127
    g = np.random.default_rng(11 + bits)
    nv = 64
    x = (g.standard_normal((nv, 128)) * g.uniform(0.01, 50.0, (nv, 1))).astype(np.float32)
    codes, scales = orc.srft_encode(x, 5, bits)
    assert codes.shape == (nv, 64 if bits == 4 else 128) and scales.shape == (nv, 16)
    for t in range(nv):
        v = orc.srft_forward(x[t], 5)
        if bits == 4:
            lo = (codes[t] & 15).astype(np.int32)
            hi = (codes[t] >> 4).astype(np.int32)
            q = np.empty(128, dtype=np.int32)
            q[0::2], q[1::2] = lo, hi
            q[q >= 8] -= 16
        else:
            q = codes[t].view(np.int8).astype(np.int32)
        for gi in range(16):
            vg = v[8 * gi: 8 * gi + 8]
            a = np.float32(np.abs(vg).max())
            want = np.float16(a / np.float32(L)).view(np.uint16)  # numpy's binary16 rounding
            assert scales[t, gi] == want
            qg = q[8 * gi: 8 * gi + 8]
            assert np.abs(qg).max() == L and np.abs(qg).max() <= L
            delta = np.float64(np.uint16(scales[t, gi]).view(np.float16))
            assert np.all(np.abs(qg * delta - vg) <= 0.5 * delta * (1 + 1e-6) + 1e-30)


def test_zero_nan_and_saturation(orc):
    x = np.zeros((3, 128), dtype=np.float32)
    x[1, 5] = np.nan
    x[2] = 1e7
    codes, scales = orc.srft_encode(x, 0, 4)
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0)
    assert np.all(codes[1] == 0) and np.all(scales[1] == 0x7E00)
    assert scales[2, 0] == 0x7BFF  # absmax / 7 beyond 65504 saturates
    y = orc.srft_decode(codes, scales, x.size, 0, 4, out_dtype="f32").reshape(3, 128)
    assert np.all(y[0] == 0) and not np.any(np.signbit(y[0]))
    assert np.all(np.isnan(y[1]))


@pytest.mark.parametrize("bits", [4, 8])
def test_round_trip_error_is_the_transform_domain_error(orc, bits):
    """Orthogonality: the decode error equals the quantisation error of the packed coordinates,
    and is within the half-step bound; lambda = 2 (exact) leaves codes and decode unchanged."""
    g = np.random.default_rng(21)
    nv = 32
    x = g.standard_normal((nv, 128)).astype(np.float32)
    codes, scales = orc.srft_encode(x, 3, bits)
    y = orc.srft_decode(codes, scales, x.size, 3, bits, out_dtype="f32").reshape(nv, 128)
    for t in range(nv):
        v = orc.srft_forward(x[t], 3).astype(np.float64)
        delta = np.repeat(scales[t].view(np.float16).astype(np.float64), 8)
        if bits == 4:
            q = np.empty(128, dtype=np.int32)
            q[0::2], q[1::2] = codes[t] & 15, codes[t] >> 4
            q[q >= 8] -= 16
        else:
            q = codes[t].view(np.int8).astype(np.int32)
        e_dom = np.linalg.norm(q * delta - v)
        e_out = np.linalg.norm(y[t].astype(np.float64) - x[t])
        assert abs(e_out - e_dom) <= 1e-5 * np.linalg.norm(x[t]) + 1e-6
    nmse = float(((y - x) ** 2).sum() / (x ** 2).sum())
    assert nmse < (0.02 if bits == 4 else 1e-4)
    lam = np.full(128, 2.0, dtype=np.float32)
    c2, s2 = orc.srft_encode(x, 3, bits, lam)
    assert np.array_equal(c2, codes)
    y2 = orc.srft_decode(c2, s2, x.size, 3, bits, lam, out_dtype="f32").reshape(nv, 128)
    assert np.array_equal(y2, y)


def test_decode_of_one_code_is_a_signed_constant(orc):
    """A record with code 1 at packed coordinate 0 and scale 1.0 decodes to x_i = s_i / sqrt(128)."""
    seed = 6
    s = np.zeros(128, dtype=np.float32)
    orc.lib().hqo_signs(seed, orc._p(s))
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 0] = 1
    scales = np.zeros((1, 16), dtype=np.uint16)
    scales[0, 0] = np.float16(1.0).view(np.uint16)
    y = orc.srft_decode(codes, scales, 128, seed, 4, out_dtype="f32")
    assert np.abs(y - s / np.sqrt(128.0)).max() < 1e-7
