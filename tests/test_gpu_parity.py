"""GPU parity: the gfx950 codec (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar (integer, byte and index work is bit-exact):
* integer lattice codes and tile scales: identical; any mismatch must lie within 1e-5 (lattice
  units) of a Voronoi boundary and affect at most 1e-6 of the octets;
* bitstreams: byte-identical, at fixed operating points and after rate control;
* rate control: the same step bit pattern and Rice parameter;
* decoded values: identical (fp32 and bf16), which is stricter than the 1e-6 relative bound;
* payload rate within 0.01 bits per value of the target.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

LAT = {"z": 0, "d4": 1, "e8": 2, "a2": 3}


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


def assert_same_stream(gpu_bytes: np.ndarray, orc_bytes: np.ndarray, what=""):
    """Byte equality, reporting the section of the first difference."""
    if gpu_bytes.size == orc_bytes.size and np.array_equal(gpu_bytes, orc_bytes):
        return
    n = min(gpu_bytes.size, orc_bytes.size)
    diff = np.nonzero(gpu_bytes[:n] != orc_bytes[:n])[0]
    h = hq.header_fields(orc_bytes)
    first = int(diff[0]) if diff.size else n
    sect = ("header" if first < 128 else "index/pad" if first < h["fixed_off"] else
            "fixed/pad" if first < h["unary_off"] else "unary")
    raise AssertionError(f"{what}: sizes {gpu_bytes.size} vs {orc_bytes.size}, {diff.size} differing bytes, "
                         f"first at {first} ({sect}; fixed_off {h['fixed_off']}, unary_off {h['unary_off']})")


def boundary_check(orc, x, lattice, step, seed, dither, codes_gpu, codes_orc):
    """Every mismatching octet must be within 1e-5 of the Voronoi boundary between the two points,
    and mismatches must be at most 1e-6 of all octets (rounded down: none on inputs below a
    million octets)."""
    bad = np.nonzero((codes_gpu.reshape(-1, 8) != codes_orc.reshape(-1, 8)).any(axis=1))[0]
    if bad.size == 0:
        return 0
    v = orc.lattice_inputs(x, LAT[lattice], step, seed, dither).reshape(-1, 8).astype(np.float64)
    half = 0.5 if lattice in ("e8", "a2") else 1.0
    # squared-distance weights: A2 is quantised in stretched coordinates (odd slots / sqrt 3)
    wm = np.tile([1.0, 3.0], 4) if lattice == "a2" else np.ones(8)
    for i in bad:
        cg = codes_gpu.reshape(-1, 8)[i] * half
        co = codes_orc.reshape(-1, 8)[i] * half
        dg, do = (wm * (v[i] - cg) ** 2).sum(), (wm * (v[i] - co) ** 2).sum()
        dist = abs(dg - do) / (2 * np.sqrt((wm * (cg - co) ** 2).sum()))
        assert dist <= 1e-5, (i, dist)
    assert bad.size <= int(1e-6 * codes_orc.size / 8), bad.size
    return bad.size


# ---------------------------------------------------------------------------------------------

def test_tiny_roundtrip_bitexact(orc):
    say("case: tiny E8 4 bps, rate-controlled")
    x = synth.tiny()
    s_orc, info_orc = orc.encode(x, orc.LAT_E8, 4.0)
    s_gpu, info = hq.hq_encode(dev(x), "e8", 4.0)
    assert info["step"] == info_orc["step"] and info["rice_k"] == info_orc["k"]
    assert_same_stream(host_bytes(s_gpu), s_orc)
    y_orc = orc.decode(s_orc, x.size)
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
    assert np.array_equal(y.cpu().numpy(), y_orc)
    yb = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(yb), orc.decode(s_orc, x.size, out_dtype="bf16"))
    assert abs(info["payload_bps"] - 4.0) <= 0.01
    assert info["payload_bits"] == info_orc["payload_bits"] and info["bytes"] == info_orc["bytes"]


def _scaled_gaussian_tiles(T, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, 128)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("dither", [False, True])
@pytest.mark.parametrize("T", [1, 65, 130, 1000])
def test_stream_parity_fixed_point(orc, lattice, dither, T):
    say(f"case: fixed point {lattice} dither={dither} T={T}")
    x = _scaled_gaussian_tiles(T, seed=T)
    for step, k in ((0.3, 2), (1.1, 0), (0.05, 5)):
        s_orc, _ = orc.encode(x, LAT[lattice], 0.0, seed=9, dither=dither, step=step, rice_k=k)
        s_gpu, info = hq.hq_encode(dev(x), lattice, 0.0, seed=9, dither=dither, step=step, rice_k=k)
        assert_same_stream(host_bytes(s_gpu), s_orc, f"step {step} k {k}")
        y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.decode(s_orc, x.size).view(np.uint32))


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
@pytest.mark.parametrize("dither", [False, True])
def test_codes_parity_weight_slice(orc, lattice, dither):
    say(f"case: codes {lattice} dither={dither} weight 512x4096")
    w = synth.weight(rows=512)
    for step in (0.12, 0.27, 0.6):
        c_orc, s_orc = orc.quantize(w, LAT[lattice], step, seed=3, dither=dither)
        c_gpu, s_gpu = hq.hq_codes(dev(w), step, lattice, seed=3, dither=dither)
        assert np.array_equal(s_gpu.cpu().numpy().view(np.uint16), s_orc)
        boundary_check(orc, w, lattice, step, 3, dither, c_gpu.cpu().numpy(), c_orc)


@pytest.mark.parametrize("case", ["tiny", "weight2048", "kv_dither", "tiny_a2", "kv_dither_a2"])
def test_rate_control_parity(orc, case):
    say(f"case: rate control {case}")
    if case == "tiny":
        x, lat, tb, seed, dither = synth.tiny(), "e8", 3.0, 0, False
    elif case == "weight2048":
        x, lat, tb, seed, dither = synth.weight(rows=2048), "e8", 4.0, 0, False
    elif case == "tiny_a2":
        x, lat, tb, seed, dither = synth.tiny(), "a2", 3.0, 0, False
    elif case == "kv_dither_a2":
        x, lat, tb, seed, dither = synth.kv(1, 0, heads=2, tokens=8192), "a2", 2.5, synth.kv_seed(1, 0), True
    else:
        x, lat, tb, seed, dither = synth.kv(1, 0, heads=2, tokens=8192), "e8", 2.0, synth.kv_seed(1, 0), True
    st, sb, k = orc.rate(x, LAT[lat], tb, seed=seed, dither=dither)
    info = hq.hq_rate(dev(x), lat, tb, seed=seed, dither=dither)
    got = np.array([info["step"]], dtype=np.float32).view(np.uint32)[0]
    assert int(got) == sb and info["rice_k"] == k


@pytest.mark.parametrize("target", [3.0, 4.0, 5.0])
def test_weight_full_size(orc, target):
    """The 14336 x 4096 bf16 MLP weight, E8, no dither: full stream and decode parity."""
    say(f"case: weight 14336x4096 E8 {target} bps")
    w = synth.weight()
    s_orc, info_orc = orc.encode(w, orc.LAT_E8, target)
    s_gpu, info = hq.hq_encode(dev(w), "e8", target)
    assert info["step"] == info_orc["step"] and info["rice_k"] == info_orc["k"]
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - target) <= 0.01
    y = hq.hq_decode(s_gpu, w.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, w.size, out_dtype="bf16"))


@pytest.mark.parametrize("layer,is_v,target", [(0, 0, 2.0), (31, 1, 3.0)])
def test_kv_call_full_size(orc, layer, is_v, target):
    """One (layer, K|V) call of the KV workload: [8][32768][128] bf16, E8 with dither."""
    say(f"case: kv layer {layer} {'V' if is_v else 'K'} {target} bps")
    x = synth.kv(layer, is_v)
    seed = synth.kv_seed(layer, is_v)
    s_orc, info_orc = orc.encode(x, orc.LAT_E8, target, seed=seed, dither=True)
    s_gpu, info = hq.hq_encode(dev(x), "e8", target, seed=seed, dither=True)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - target) <= 0.01
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, x.size, out_dtype="bf16"))


@pytest.mark.parametrize("lattice", ["z", "d4", "a2"])
def test_lattice_sweep_weight(orc, lattice):
    """Lattice sweep on the 14336 x 4096 weight at 4 bps (Z, D4, A2; E8 is covered above): the same
    step and Rice parameter as the oracle, identical stream and decode, rate within 0.01."""
    say(f"case: weight 14336x4096 {lattice} 4 bps")
    w = synth.weight()
    s_orc, info_orc = orc.encode(w, orc.LATTICES[lattice], 4.0)
    s_gpu, info = hq.hq_encode(dev(w), lattice, 4.0)
    assert info["step"] == info_orc["step"] and info["rice_k"] == info_orc["k"]
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - 4.0) <= 0.01
    y = hq.hq_decode(s_gpu, w.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, w.size, out_dtype="bf16"))


def test_lattice_sweep_distortion_order():
    """At an equal payload rate the lattice with the smaller normalized second moment gives the
    smaller error: E8 < D4 < Z, and A2 < Z, in normalized MSE on the weight at 4 bps."""
    say("case: lattice sweep distortion order")
    x = dev(synth.weight())
    xf = x.float()
    nmse = {}
    for lat in ("z", "d4", "a2", "e8"):
        s, info = hq.hq_encode(x, lat, 4.0)
        assert abs(info["payload_bps"] - 4.0) <= 0.01
        y = hq.hq_decode(s, x.numel(), out_dtype=torch.float32)
        nmse[lat] = float(((y - xf) ** 2).sum() / (xf ** 2).sum())
    say(f"nmse {nmse}")
    assert nmse["e8"] < nmse["d4"] < nmse["z"]
    assert nmse["a2"] < nmse["z"]


@pytest.mark.parametrize("index", [0, 1, 6])
def test_model_tensor_full_size(orc, index):
    """Linear weights of the 8B-shaped decoder (q [4096,4096], k [1024,4096], down [4096,14336]),
    E8 at 4 bps: identical stream and decode."""
    name, shape = synth.model_shapes()[index]
    say(f"case: model tensor {index} {name} {shape}")
    w = synth.model_tensor(index, shape)
    s_orc, info_orc = orc.encode(w, orc.LAT_E8, 4.0, seed=index)
    s_gpu, info = hq.hq_encode(dev(w), "e8", 4.0, seed=index)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - 4.0) <= 0.01
    y = hq.hq_decode(s_gpu, w.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, w.size, out_dtype="bf16"))


# ---- edge cases and error paths ---------------------------------------------------------------

def test_empty_and_single_tile(orc):
    say("case: empty and single tile")
    e = np.zeros(0, dtype=np.float32)
    s_orc, _ = orc.encode(e, orc.LAT_E8, 4.0)
    s_gpu, info = hq.hq_encode(torch.zeros(0, device="cuda"), "e8", 4.0)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert hq.hq_decode(s_gpu, 0, out_dtype=torch.float32).numel() == 0
    x = synth.tiny(tiles=1)
    s_orc, _ = orc.encode(x, orc.LAT_E8, 4.0)
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 4.0)
    assert_same_stream(host_bytes(s_gpu), s_orc)


def test_zero_tiles_and_tiny_values(orc):
    say("case: zero and denormal tiles")
    x = synth.tiny(tiles=70).copy()
    x[3] = 0.0
    x[10] = np.float32(1e-30) * x[10]
    x[11] = np.float32(1e-42)
    x[20] = np.float32(1e15) * x[20]
    for lat in ("e8", "d4", "a2", "z"):
        for dither in (False, True):
            s_orc, _ = orc.encode(x, LAT[lat], 0.0, seed=1, dither=dither, step=0.25, rice_k=3)
            s_gpu, _ = hq.hq_encode(dev(x), lat, 0.0, seed=1, dither=dither, step=0.25, rice_k=3)
            assert_same_stream(host_bytes(s_gpu), s_orc, f"{lat} dither={dither}")
            y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.decode(s_orc, x.size).view(np.uint32))
            yb = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)   # incl. bf16 denormal outputs
            assert np.array_equal(bf16_host(yb), orc.decode(s_orc, x.size, out_dtype="bf16"))


def test_long_unary_segments(orc):
    """k = 0 at a small step: ~35 unary bits per value, so a chunk's unary segment spans several
    staging windows of the encoder, and the decoder takes its long-segment path (positions beyond
    16 bits: the table holds half the chunk's at a time); the last chunk is short (1024 values)
    and takes the common path."""
    say("case: long unary segments")
    x = synth.gaussian(128 * 200, seed=4).reshape(200, 128)
    s_orc, info_orc = orc.encode(x, orc.LAT_Z, 0.0, step=0.05, rice_k=0)
    assert info_orc["unary_bits"] / x.size > 20
    s_gpu, _ = hq.hq_encode(dev(x), "z", 0.0, step=0.05, rice_k=0)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
    assert np.array_equal(y.cpu().numpy(), orc.decode(s_orc, x.size))


def _segment_words(s: np.ndarray):
    h = s[:128].view(np.uint32)
    chunks = int(h[10])
    idx = s[128:128 + 4 * (chunks + 1)].view(np.uint32).astype(np.int64)
    return 2 * np.diff(idx)  # 32-bit words per chunk


@pytest.mark.parametrize("lattice,tile,dither,step,tiles", [
    ("e8", 128, 1, 0.03, 148),    # E8 at k = 0 (the compile-time k path), dither; last chunk 2560 values
    ("e8", 256, 0, 0.02, 70),     # tiles of 256; last chunk 1536 values
    ("a2", 64, 0, 0.03, 300),     # tiles of 64; last chunk 2816 values
    ("d4", 128, 1, 0.05, 128),    # whole chunks only
])
def test_long_segments_every_lattice(orc, lattice, tile, dither, step, tiles):
    """The decoder's long-segment path (a chunk's unary segment above 2048 words) on every lattice,
    tile length and both outputs, including a short last chunk whose second half has no valid tile,
    against the oracle bit for bit."""
    say(f"case: long segments {lattice} tile {tile} dither {dither} step {step} tiles {tiles}")
    x = synth.gaussian(tile * tiles, seed=11).reshape(tiles, tile)
    s_orc, _ = orc.encode(x, LAT[lattice], 0.0, seed=9, dither=dither, step=step, rice_k=0, tile=tile)
    words = _segment_words(s_orc)
    assert (words > 2048).all(), words  # every chunk, the last one too, takes the long path
    s_gpu, _ = hq.hq_encode(dev(x), lattice, 0.0, seed=9, dither=dither, step=step, rice_k=0, tile=tile)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
    assert np.array_equal(y.cpu().numpy(), orc.decode(s_orc, x.size))
    yb = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(yb), orc.decode(s_orc, x.size, out_dtype="bf16"))


def test_mixed_segment_lengths(orc):
    """Chunks of both kinds in one stream: all-zero chunks (every symbol 0: short segments, 16-bit
    positions) alternate with noise chunks at a small step (long segments)."""
    say("case: mixed segment lengths")
    g = np.random.Generator(np.random.PCG64(31))
    T = 64 * 6 + 40
    x = g.standard_normal((T, 128)).astype(np.float32)
    for c in range(0, 7, 2):
        x[64 * c: 64 * c + 64] = 0.0
    s_orc, _ = orc.encode(x, orc.LAT_E8, 0.0, step=0.03, rice_k=1)
    words = _segment_words(s_orc)
    assert (words > 2048).any() and (words <= 2048).any(), words
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 0.0, step=0.03, rice_k=1)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    yb = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(yb), orc.decode(s_orc, x.size, out_dtype="bf16"))


def test_nonfinite_reported():
    say("case: non-finite input")
    x = synth.tiny().copy()
    x[5, 3] = np.nan
    with pytest.raises(hq.HqError) as e:
        hq.hq_encode(dev(x), "e8", 0.0, step=0.3, rice_k=2)
    assert e.value.code == hq.HQ_ERR_NONFINITE


def test_capacity_reported_and_retry(orc):
    say("case: capacity")
    x = synth.tiny(tiles=300)
    s_orc, _ = orc.encode(x, orc.LAT_E8, 4.0)
    xd = dev(x)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    ws = hq.workspace(x.size)
    import ctypes
    p = hq.make_params("e8", 4.0)
    nb = ctypes.c_uint64(0)
    rc = hq.lib().hq_encode(ctypes.c_void_p(xd.data_ptr()), 0, x.size, ctypes.byref(p),
                            ctypes.c_void_p(small.data_ptr()), small.numel(), ctypes.byref(nb), None,
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert rc == hq.HQ_ERR_CAPACITY and nb.value == s_orc.size
    s_gpu, _ = hq.hq_encode(xd, "e8", 4.0, out=small)   # the binding grows the buffer and retries
    assert_same_stream(host_bytes(s_gpu), s_orc)


def test_corrupt_streams_reported(orc):
    say("case: corrupt streams")
    x = synth.tiny(tiles=130)
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 4.0)
    good = s_gpu.clone()
    for mutate in ("magic", "n", "index", "terminators"):
        s = good.clone()
        n = x.size
        if mutate == "magic":
            s[0] ^= 1
        elif mutate == "n":
            n = x.size + 128
        elif mutate == "index":
            s[128 + 4] = 0xFF
        else:
            s[-16:] = 0
        with pytest.raises(hq.HqError) as e:
            hq.hq_decode(s, n, out_dtype=torch.float32)
        assert e.value.code == hq.HQ_ERR_CORRUPT, mutate
    y = hq.hq_decode(good, x.size, out_dtype=torch.float32)   # and the good one still decodes
    assert torch.isfinite(y).all()


def test_async_rate_then_encode_equals_one_call(orc):
    """hq_rate (asynchronous) + hq_encode(step=-1) on the same workspace = hq_encode with rate control."""
    say("case: rate then encode")
    w = synth.weight(rows=1024)
    xd = dev(w)
    a, _ = hq.hq_encode(xd, "e8", 3.5)
    ws = hq.workspace(w.size)
    hq.hq_rate(xd, "e8", 3.5, ws=ws, blocking=False)
    b, _ = hq.hq_encode(xd, "e8", 3.5, step=-1.0, ws=ws)
    assert torch.equal(a, b)
    s_orc, _ = orc.encode(w, orc.LAT_E8, 3.5)
    assert_same_stream(host_bytes(b), s_orc)


def test_async_rate_then_encode_with_capacity_retry(orc):
    """An encode at the workspace's operating point (step=-1) into too small a buffer reports
    CAPACITY with the size needed; the retry at the same point, on the same workspace, succeeds
    (every encode call resets the workspace's status and offset flags first)."""
    say("case: rate then encode(step=-1) with a capacity retry")
    import ctypes
    w = synth.weight(rows=256)
    xd = dev(w)
    s_orc, _ = orc.encode(w, orc.LAT_E8, 3.0)
    ws = hq.workspace(w.size)
    hq.hq_rate(xd, "e8", 3.0, ws=ws, blocking=False)
    small = torch.empty(4096, dtype=torch.uint8, device="cuda")
    p = hq.make_params("e8", 3.0, step=-1.0)
    nb = ctypes.c_uint64(0)
    assert xd.dtype == torch.bfloat16 and xd.numel() == w.size
    rc = hq.lib().hq_encode(ctypes.c_void_p(xd.data_ptr()), hq.HQ_BF16, w.size, ctypes.byref(p),
                            ctypes.c_void_p(small.data_ptr()), small.numel(), ctypes.byref(nb), None,
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert rc == hq.HQ_ERR_CAPACITY and nb.value == s_orc.size
    s_gpu, _ = hq.hq_encode(xd, "e8", 3.0, step=-1.0, ws=ws, out=small)  # the binding retries
    assert_same_stream(host_bytes(s_gpu), s_orc)


def test_repeated_encodes_at_the_workspace_point(orc):
    """KV-append pattern: the operating point is chosen once (rate control on the first block), then
    further blocks of different data and sizes are encoded at that point with step=-1 on the same
    workspace; each stream equals the oracle's at that fixed point."""
    say("case: repeated step=-1 encodes on one workspace")
    blocks = [synth.kv(3, 0, heads=1, tokens=t) for t in (4096, 1000, 2500)]
    seed = synth.kv_seed(3, 0)
    ws = hq.workspace(max(b.size for b in blocks))
    first, info = hq.hq_encode(dev(blocks[0]), "e8", 2.0, seed=seed, dither=True, ws=ws)
    s_orc, info_orc = orc.encode(blocks[0], orc.LAT_E8, 2.0, seed=seed, dither=True)
    assert_same_stream(host_bytes(first), s_orc)
    for b in blocks[1:] + blocks[:1]:
        s_gpu, inf = hq.hq_encode(dev(b), "e8", 2.0, seed=seed, dither=True, step=-1.0, ws=ws)
        assert inf["step"] == info["step"] and inf["rice_k"] == info["rice_k"]
        s_o, _ = orc.encode(b, orc.LAT_E8, 0.0, seed=seed, dither=True, step=info["step"], rice_k=info["rice_k"])
        assert_same_stream(host_bytes(s_gpu), s_o, f"block of {b.size} values")


def test_encode_at_workspace_point_without_one_is_rejected():
    say("case: step=-1 on a workspace with no operating point")
    x = synth.tiny()
    ws = torch.zeros(hq.hq_workspace_size(x.size), dtype=torch.uint8, device="cuda")
    with pytest.raises(hq.HqError) as e:
        hq.hq_encode(dev(x), "e8", 4.0, step=-1.0, ws=ws)
    assert e.value.code == hq.HQ_ERR_INVALID_ARG
    # a decode on that workspace sets no operating point either
    ok, _ = hq.hq_encode(dev(x), "e8", 4.0)
    hq.hq_decode(ok, x.size, ws=ws)
    with pytest.raises(hq.HqError) as e:
        hq.hq_encode(dev(x), "e8", 4.0, step=-1.0, ws=ws)
    assert e.value.code == hq.HQ_ERR_INVALID_ARG


@pytest.mark.parametrize("lattice,dither,step,k", [("e8", False, 0.27, 2), ("e8", True, 1.3, 0),
                                                   ("d4", True, 0.4, 1), ("a2", False, 0.2, 3),
                                                   ("z", False, 2.0 ** -6, 6)])
def test_async_encode_into_exactly_the_bound(orc, lattice, dither, step, k):
    """An asynchronous encode at a fixed point into a buffer of exactly hq_encode_bound bytes
    succeeds, and its stream equals the oracle's."""
    say(f"case: async encode into the bound {lattice} dither={dither}")
    w = synth.weight(rows=128)
    cap = hq.hq_encode_bound(w.size, lattice, step, k, dither)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    ws = hq.workspace(w.size)
    hq.hq_encode(dev(w), lattice, 0.0, seed=2, dither=dither, step=step, rice_k=k, out=out, ws=ws, blocking=False)
    assert hq.hq_status(ws) == hq.HQ_OK
    size = hq.header_fields(host_bytes(out[:128]))["total_bytes"]
    s_orc, _ = orc.encode(w, LAT[lattice], 0.0, seed=2, dither=dither, step=step, rice_k=k)
    assert size == s_orc.size <= cap
    assert_same_stream(host_bytes(out[:size]), s_orc)


def test_async_encode_sized_by_the_binding(orc):
    """The binding's asynchronous encode with rate control and no buffer: a blocking rate pass,
    a buffer of the bound at that point, then the asynchronous encode at the workspace's point."""
    say("case: async encode sized by the binding")
    w = synth.weight(rows=300)
    out, _ = hq.hq_encode(dev(w), "e8", 4.0, blocking=False)
    torch.cuda.synchronize()
    size = hq.header_fields(host_bytes(out[:128]))["total_bytes"]
    s_orc, _ = orc.encode(w, orc.LAT_E8, 4.0)
    assert_same_stream(host_bytes(out[:size]), s_orc)


@pytest.mark.parametrize("case", ["weight_full", "kv_dither", "tiles64", "tiles256"])
def test_wait_fallbacks_give_the_same_streams(orc, monkeypatch, case):
    """Forward progress does not rest on the order workgroups start in: a look-back wait that
    outlasts its spin budget computes the missing predecessor's aggregate from its input, and a
    pass-B wavefront that does not see pass A's solve published solves it itself.  A budget of 0
    (set from the host) makes every wait that finds its value missing take that path at once; the
    streams must be unchanged."""
    say(f"case: wait fallbacks forced ({case})")
    monkeypatch.setenv("HQ_SPIN_BUDGET", "0")
    if case == "weight_full":
        x, lat, tb, seed, dither, tile = synth.weight(), "e8", 4.0, 0, False, 128
    elif case == "kv_dither":
        x, lat, tb, seed, dither, tile = synth.kv(2, 1, heads=2), "e8", 2.0, synth.kv_seed(2, 1), True, 128
    elif case == "tiles64":
        x, lat, tb, seed, dither, tile = synth.weight(rows=700), "d4", 3.0, 1, True, 64
    else:
        x, lat, tb, seed, dither, tile = synth.weight(rows=700), "a2", 3.0, 1, False, 256
    ws = hq.workspace(x.size)
    s_gpu, info = hq.hq_encode(dev(x), lat, tb, seed=seed, dither=dither, tile=tile, ws=ws)
    fb = hq.hq_fallbacks(ws)
    s_orc, info_orc = orc.encode(x, LAT[lat], tb, seed=seed, dither=dither, tile=tile)
    assert info["step"] == info_orc["step"] and info["rice_k"] == info_orc["k"]
    assert_same_stream(host_bytes(s_gpu), s_orc, case)
    # the fallbacks did run: every pass-B workgroup starts before workgroup 0 can have published
    # pass A's solve, so with no budget each solves pass A itself; and among the weight's 7168
    # chunks some look-back finds a predecessor not yet published
    assert fb & hq.FALLBACK_CENTRE, fb
    if case == "weight_full":
        assert fb & hq.FALLBACK_LOOKBACK, fb
    monkeypatch.delenv("HQ_SPIN_BUDGET")
    s_again, _ = hq.hq_encode(dev(x), lat, tb, seed=seed, dither=dither, tile=tile, ws=ws)
    assert torch.equal(s_again, s_gpu)
    assert hq.hq_fallbacks(ws) == 0  # with the normal budget no wait runs out


def test_deterministic_repeat():
    say("case: determinism")
    w = synth.weight(rows=1024)
    xd = dev(w)
    a, _ = hq.hq_encode(xd, "e8", 4.0)
    b, _ = hq.hq_encode(xd, "e8", 4.0)
    assert torch.equal(a, b)


def test_overflowing_energy_is_nonfinite(orc):
    """A finite input whose transformed energy overflows binary32 is reported like NaN input."""
    say("case: energy overflow")
    x = synth.tiny().copy()
    x[7] *= np.float32(1e30)
    with pytest.raises(orc.OracleError) as eo:
        orc.encode(x, orc.LAT_E8, 0.0, step=0.3, rice_k=2)
    assert eo.value.code == orc.ERR_NONFINITE
    with pytest.raises(hq.HqError) as e:
        hq.hq_encode(dev(x), "e8", 0.0, step=0.3, rice_k=2)
    assert e.value.code == hq.HQ_ERR_NONFINITE


# ---- dither format options (flags: + 2 Philox with 7 rounds, + 4 a 24-bit draw) -------------------

@pytest.mark.parametrize("flags", [3, 5, 7])
@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_dither_options_fixed_point(orc, flags, lattice):
    say(f"case: dither flags {flags} fixed point {lattice}")
    for T in (1, 65, 300):
        x = _scaled_gaussian_tiles(T, seed=T + flags)
        for step, k in ((0.3, 2), (1.1, 0)):
            s_orc, _ = orc.encode(x, LAT[lattice], 0.0, seed=9, dither=flags, step=step, rice_k=k)
            s_gpu, _ = hq.hq_encode(dev(x), lattice, 0.0, seed=9, dither=flags, step=step, rice_k=k)
            assert_same_stream(host_bytes(s_gpu), s_orc, f"T {T} step {step} k {k}")
            assert hq.header_fields(host_bytes(s_gpu))["dither"] == flags
            y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.decode(s_orc, x.size).view(np.uint32))


@pytest.mark.parametrize("flags", [3, 5, 7])
def test_dither_options_codes_and_rate(orc, flags):
    say(f"case: dither flags {flags} codes and rate control")
    w = synth.weight(rows=256)
    c_orc, s_orc = orc.quantize(w, orc.LAT_E8, 0.27, seed=3, dither=flags)
    c_gpu, s_gpu = hq.hq_codes(dev(w), 0.27, "e8", seed=3, dither=flags)
    assert np.array_equal(s_gpu.cpu().numpy().view(np.uint16), s_orc)
    boundary_check(orc, w, "e8", 0.27, 3, flags, c_gpu.cpu().numpy(), c_orc)
    x = synth.kv(1, 0, heads=2, tokens=8192)
    st, sb, k = orc.rate(x, orc.LAT_E8, 2.0, seed=synth.kv_seed(1, 0), dither=flags)
    info = hq.hq_rate(dev(x), "e8", 2.0, seed=synth.kv_seed(1, 0), dither=flags)
    assert int(np.array([info["step"]], dtype=np.float32).view(np.uint32)[0]) == sb and info["rice_k"] == k


@pytest.mark.parametrize("flags", [3, 7])
def test_dither_options_kv_call_full_size(orc, flags):
    """One (layer, K|V) call of the KV workload, [8][32768][128] bf16, E8 at 3 bps with the option."""
    say(f"case: kv layer 5 K 3 bps dither flags {flags}")
    x = synth.kv(5, 0)
    seed = synth.kv_seed(5, 0)
    s_orc, info_orc = orc.encode(x, orc.LAT_E8, 3.0, seed=seed, dither=flags)
    s_gpu, info = hq.hq_encode(dev(x), "e8", 3.0, seed=seed, dither=flags)
    assert_same_stream(host_bytes(s_gpu), s_orc)
    assert abs(info["payload_bps"] - 3.0) <= 0.01
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_host(y), orc.decode(s_orc, x.size, out_dtype="bf16"))


def test_corrupt_dither_flags_reported():
    say("case: corrupt dither flags")
    x = synth.tiny(tiles=8)
    s_gpu, _ = hq.hq_encode(dev(x), "e8", 3.0, dither=True)
    for bad in (2, 4, 6, 8):
        s = s_gpu.clone()
        s[7] = bad
        with pytest.raises(hq.HqError) as e:
            hq.hq_decode(s, x.size, out_dtype=torch.float32)
        assert e.value.code == hq.HQ_ERR_CORRUPT


def test_tensor_beyond_4_gib(orc):
    """n = 2^31 + 3 * 8192 + 5 * 128 bf16 values (4.3 GB of input, byte offsets past 2^32 in the
    input, the decoded output and the stream's planes), E8 at 4 bps with rate control.  The oracle
    checks the rate-control point on the whole tensor (it reads only the sampled tiles), then each
    sampled chunk's fixed record, unary segment and decoded values against its own encoding of
    those chunks at the same point (without dither a chunk's bytes depend only on its tiles)."""
    n = (1 << 31) + 3 * 8192 + 5 * 128
    say(f"case: {n} values, E8 4 bps")
    x = synth.device_normal_bf16(n, seed=77)
    x_host = x.view(torch.int16).cpu().numpy().view(np.uint16)
    st, sb, k = orc.rate(x_host, orc.LAT_E8, 4.0)
    s_gpu, info = hq.hq_encode(x, "e8", 4.0)
    assert int(np.array([info["step"]], dtype=np.float32).view(np.uint32)[0]) == sb and info["rice_k"] == k
    assert abs(info["payload_bps"] - 4.0) <= 0.01
    y = hq.hq_decode(s_gpu, n, out_dtype=torch.bfloat16)
    s = host_bytes(s_gpu)
    h = hq.header_fields(s)
    chunks = h["chunks"]
    assert chunks == (n + 8191) // 8192 and h["tiles"] == n // 128
    idx = s[128:128 + 4 * (chunks + 1)].view(np.uint32).astype(np.int64)
    rec = 64 * h["F"] // 8
    for c in (0, 1, (1 << 31) // 8192 - 1, (1 << 31) // 8192, chunks // 3, chunks - 2, chunks - 1):
        lo, hi = 8192 * c, min(8192 * (c + 1), n)
        sub, _ = orc.encode(x_host[lo:hi], orc.LAT_E8, 0.0, step=st, rice_k=k)
        hs = hq.header_fields(sub)
        assert hs["F"] == h["F"]
        f_gpu = s[h["fixed_off"] + c * rec: h["fixed_off"] + (c + 1) * rec]
        assert np.array_equal(f_gpu, sub[hs["fixed_off"]: hs["fixed_off"] + rec]), c
        u_gpu = s[h["unary_off"] + 8 * idx[c]: h["unary_off"] + 8 * idx[c + 1]]
        assert np.array_equal(u_gpu, sub[hs["unary_off"]: hs["unary_off"] + 8 * hs["unary_words"]]), c
        yb = bf16_host(y[lo:hi])
        assert np.array_equal(yb, orc.decode(sub, hi - lo, out_dtype="bf16")), c


@pytest.mark.parametrize("lattice", ["e8", "d4", "a2", "z"])
def test_fixed_step_automatic_k_and_fixed_k_rate_control(orc, lattice):
    """The two mixed operating modes: a fixed step with the Rice parameter chosen by one sample pass,
    and rate control on the step with the Rice parameter fixed."""
    say(f"case: fixed step / auto k and rate control / fixed k, {lattice}")
    w = synth.weight(rows=512)
    for dither in (False, True):
        s_orc, info_orc = orc.encode(w, LAT[lattice], 0.0, seed=4, dither=dither, step=0.3, rice_k=-1)
        s_gpu, info = hq.hq_encode(dev(w), lattice, 0.0, seed=4, dither=dither, step=0.3, rice_k=-1)
        assert info["rice_k"] == info_orc["k"]
        assert_same_stream(host_bytes(s_gpu), s_orc, f"fixed step, dither={dither}")
        s_orc, info_orc = orc.encode(w, LAT[lattice], 3.0, seed=4, dither=dither, rice_k=1)
        s_gpu, info = hq.hq_encode(dev(w), lattice, 3.0, seed=4, dither=dither, rice_k=1)
        assert info["rice_k"] == 1 and info["step"] == info_orc["step"]
        assert_same_stream(host_bytes(s_gpu), s_orc, f"fixed k, dither={dither}")


def test_concurrent_calls_on_separate_streams(orc):
    """Calls in flight together on three streams, each with its own workspaces and buffers (the
    streamed series of the benchmark): every stream and decode equals the oracle's."""
    say("case: concurrent calls on three streams")
    xs = [synth.weight(rows=rows, seed=s) for rows, s in ((256, 3), (512, 4), (128, 5))]
    streams = [torch.cuda.Stream() for _ in xs]
    outs = []
    for x, st in zip(xs, streams):
        n = x.size
        xd = dev(x)
        cap = hq.capacity_estimate(n, "e8", 4.0)
        out = torch.empty(cap, dtype=torch.uint8, device="cuda")
        y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        ws, wsd = hq.workspace(n), hq.workspace(0)
        torch.cuda.synchronize()
        outs.append((xd, out, y, ws, wsd, st))
    for _ in range(3):   # several rounds of the three calls in flight together
        for (xd, out, y, ws, wsd, st), x in zip(outs, xs):
            hq.hq_encode(xd, "e8", 4.0, out=out, ws=ws, blocking=False, stream=st)
            hq.hq_decode(out, x.size, out=y, ws=wsd, check=False, stream=st)
    torch.cuda.synchronize()
    for (xd, out, y, ws, wsd, st), x in zip(outs, xs):
        assert hq.hq_status(ws, st) == 0 and hq.hq_status(wsd, st) == 0
        s_orc, _ = orc.encode(x, orc.LAT_E8, 4.0)
        assert_same_stream(host_bytes(out)[: s_orc.size], s_orc)
        assert np.array_equal(bf16_host(y), orc.decode(s_orc, x.size, out_dtype="bf16"))
