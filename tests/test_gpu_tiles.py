"""GPU parity at the other tile lengths (64 and 256 values; the HyperQuant summary's component 1
gives 128 as an example size): the gfx950 codec through the C ABI against the CPU oracle.

Same bar as at 128 values: identical streams and decoded values (fp32 and bf16), identical tile
scales, lattice codes identical up to Voronoi-boundary ties, the same rate-control operating point,
and the fused matrix-vector product within its rounding bound.  A chunk is 8192 values at every
tile length, so the cases span several chunks and end in a ragged one.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

LAT = {"z": 0, "d4": 1, "e8": 2, "a2": 3}
U = 2.0 ** -24
TILES = (64, 256)


def dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()


def host_bytes(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def bf16_host(t) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def say(msg):
    print(msg, flush=True)


def same_stream(gpu_bytes, orc_bytes, what=""):
    if gpu_bytes.size == orc_bytes.size and np.array_equal(gpu_bytes, orc_bytes):
        return
    n = min(gpu_bytes.size, orc_bytes.size)
    diff = np.nonzero(gpu_bytes[:n] != orc_bytes[:n])[0]
    h = hq.header_fields(orc_bytes)
    first = int(diff[0]) if diff.size else n
    raise AssertionError(f"{what}: sizes {gpu_bytes.size} vs {orc_bytes.size}, {diff.size} differing bytes, "
                         f"first at {first} (fixed_off {h['fixed_off']}, unary_off {h['unary_off']})")


def scaled_gaussian_tiles(T, tile, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, tile)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("dither", [False, True])
def test_stream_parity_fixed_point_tiles(orc, tile, lattice, dither):
    per_chunk = 8192 // tile
    for T in (1, per_chunk + 1, 3 * per_chunk + 7):
        say(f"case: tile {tile} fixed point {lattice} dither={dither} T={T}")
        x = scaled_gaussian_tiles(T, tile, seed=T + tile)
        for step, k in ((0.3, 2), (1.1, 0), (0.05, 5)):
            s_orc, _ = orc.encode(x, LAT[lattice], 0.0, seed=9, dither=dither, step=step, rice_k=k, tile=tile)
            s_gpu, _ = hq.hq_encode(dev(x), lattice, 0.0, seed=9, dither=dither, step=step, rice_k=k, tile=tile)
            same_stream(host_bytes(s_gpu), s_orc, f"step {step} k {k}")
            assert hq.header_fields(host_bytes(s_gpu))["tile"] == tile
            y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.decode(s_orc, x.size).view(np.uint32))
            yb = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
            assert np.array_equal(bf16_host(yb), orc.decode(s_orc, x.size, out_dtype="bf16"))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("lattice,dither", [("e8", False), ("e8", True), ("a2", True), ("d4", False)])
def test_codes_parity_weight_slice_tiles(orc, tile, lattice, dither):
    say(f"case: tile {tile} codes {lattice} dither={dither} weight 256x4096")
    w = synth.weight(rows=256)
    for step in (0.12, 0.6):
        c_orc, s_orc = orc.quantize(w, LAT[lattice], step, seed=3, dither=dither, tile=tile)
        c_gpu, s_gpu = hq.hq_codes(dev(w), step, lattice, seed=3, dither=dither, tile=tile)
        assert np.array_equal(s_gpu.cpu().numpy().view(np.uint16), s_orc)
        cg = c_gpu.cpu().numpy()
        bad = np.nonzero((cg.reshape(-1, 8) != c_orc.reshape(-1, 8)).any(axis=1))[0]
        if bad.size:   # only Voronoi-boundary ties may differ
            v = orc.lattice_inputs(w, LAT[lattice], step, 3, dither, tile=tile).reshape(-1, 8).astype(np.float64)
            half = 0.5 if lattice in ("e8", "a2") else 1.0
            wm = np.tile([1.0, 3.0], 4) if lattice == "a2" else np.ones(8)
            for i in bad:
                a, b = cg.reshape(-1, 8)[i] * half, c_orc.reshape(-1, 8)[i] * half
                gap = abs((wm * (v[i] - a) ** 2).sum() - (wm * (v[i] - b) ** 2).sum())
                assert gap / (2 * np.sqrt((wm * (a - b) ** 2).sum())) <= 1e-5
            assert bad.size <= max(1, int(1e-6 * c_orc.size / 8))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("case", ["tiny_e8", "tiny_a2", "weight2048", "kv_dither"])
def test_rate_control_parity_tiles(orc, tile, case):
    say(f"case: tile {tile} rate control {case}")
    if case == "tiny_e8":
        x, lat, tb, seed, dither = synth.tiny(), "e8", 3.0, 0, False
    elif case == "tiny_a2":
        x, lat, tb, seed, dither = synth.tiny(), "a2", 3.0, 0, False
    elif case == "weight2048":
        x, lat, tb, seed, dither = synth.weight(rows=2048), "e8", 4.0, 0, False
    else:
        x, lat, tb, seed, dither = synth.kv(1, 0, heads=2, tokens=8192), "e8", 2.0, synth.kv_seed(1, 0), True
    st, sb, k = orc.rate(x, LAT[lat], tb, seed=seed, dither=dither, tile=tile)
    info = hq.hq_rate(dev(x), lat, tb, seed=seed, dither=dither, tile=tile)
    got = np.array([info["step"]], dtype=np.float32).view(np.uint32)[0]
    assert int(got) == sb and info["rice_k"] == k


@pytest.mark.parametrize("tile", TILES)
def test_weight_full_size_tiles(orc, tile):
    """The 14336 x 4096 bf16 MLP weight, E8 at 4 bps: full stream and decode parity."""
    say(f"case: tile {tile} weight 14336x4096 E8 4 bps")
    w = synth.weight()
    s_orc, info_orc = orc.encode(w, orc.LAT_E8, 4.0, tile=tile)
    s_gpu, info = hq.hq_encode(dev(w), "e8", 4.0, tile=tile)
    assert info["step"] == info_orc["step"] and info["rice_k"] == info_orc["k"]
    same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - 4.0) <= 0.01
    y = hq.hq_decode(s_gpu, w.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, w.size, out_dtype="bf16"))


@pytest.mark.parametrize("tile", TILES)
def test_empty_and_single_tile_tiles(orc, tile):
    say(f"case: tile {tile} empty and single tile")
    e = np.zeros(0, dtype=np.float32)
    s_orc, _ = orc.encode(e, orc.LAT_E8, 4.0, tile=tile)
    s_gpu, _ = hq.hq_encode(torch.zeros(0, device="cuda"), "e8", 4.0, tile=tile)
    same_stream(host_bytes(s_gpu), s_orc)
    x = scaled_gaussian_tiles(1, tile, seed=1)
    s_orc, _ = orc.encode(x, orc.LAT_E8, 4.0, tile=tile)
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 4.0, tile=tile)
    same_stream(host_bytes(s_gpu), s_orc)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("lattice,dither,target", [("e8", False, 4.0), ("a2", True, 3.0)])
def test_gemv_tiles(orc, tile, lattice, dither, target):
    """Fused decode + matrix-vector product on a 97 x 1280 matrix (a ragged last chunk) against the
    oracle's binary64 product; bound (column tiles + 32) 2^-24 B_r / tile per row."""
    rows, cols = 97, 1280
    say(f"case: tile {tile} gemv {rows}x{cols} {lattice} dither={dither}")
    g = np.random.Generator(np.random.PCG64(23))
    w = synth.bf16_bits(0.02 * g.standard_normal((rows, cols)).astype(np.float32))
    x = g.standard_normal(cols).astype(np.float32)
    s_gpu, _ = hq.hq_encode(dev(w), lattice, target, seed=5, dither=dither, tile=tile)
    y = hq.hq_gemv(s_gpu, rows, cols, dev(x)).cpu().numpy().astype(np.float64)
    y_ref, bound = orc.gemv_reference(s_gpu.cpu().numpy(), rows, cols, x.astype(np.float64), seed=5, tile=tile)
    tol = (cols // tile + 32) * U * bound / tile
    assert np.all(np.abs(y - y_ref) <= tol), float(np.max(np.abs(y - y_ref) / tol))
    assert np.linalg.norm(y - y_ref) <= 1e-5 * np.linalg.norm(y_ref)


def test_gemv_rejects_cols_not_multiple_of_tile():
    """A stream of 256-value tiles cannot be read as rows of 384 values: the header check reports
    a corrupt stream and no kernel reads past the activation."""
    say("case: gemv with cols not a multiple of the stream's tile")
    rows, cols = 2, 384
    w = scaled_gaussian_tiles(3, 256, seed=4)
    s_gpu, _ = hq.hq_encode(dev(w), "e8", 4.0, tile=256)
    with pytest.raises(hq.HqError) as e:
        hq.hq_gemv(s_gpu, rows, cols, torch.ones(cols, device="cuda"))
    assert e.value.code == hq.HQ_ERR_CORRUPT


def test_decode_rejects_n_not_multiple_of_stream_tile():
    say("case: decode with n not a multiple of the stream's tile")
    x = scaled_gaussian_tiles(5, 256, seed=6)
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 4.0, tile=256)
    with pytest.raises(hq.HqError) as e:
        hq.hq_decode(s_gpu, x.size - 128, out_dtype=torch.float32)
    assert e.value.code == hq.HQ_ERR_CORRUPT
