"""GPU: the per-layer Haar-uniform rotation (hq_rotate, MFMA) against the oracle's binary64
product, and the KV path with the full rotation end to end.

Bar for the rotation: per value |y - Q x| <= 2^-8 |Q x| + 3e-5 ||x_v||_2: half a bf16 ulp of the
output (at most 2^-8 relative) plus the binary32 result's own error, at most about 1.8e-5 ||x_v||_2
(the two-part bf16 split of Q leaves 2^-17 of each entry, binary32 accumulation over 128 terms
128 x 2^-24, and the library's binary32 Q against the oracle's binary64 Q 2e-7 per entry).  The codec after the rotation is held to its usual bar: byte-identical stream and
decode, given the rotated bf16 tensor."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()


def host_f64(t) -> np.ndarray:
    return synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def say(msg):
    print(msg, flush=True)


def check_rotation(y, ref, x64):
    xn = np.linalg.norm(x64.reshape(-1, 128), axis=1).repeat(128)
    err = np.abs(y - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 3e-5 * xn
    worst = float(np.max(err / tol))
    say(f"worst err/tol {worst:.3g}")
    assert np.all(err <= tol), worst


@pytest.mark.parametrize("nvec,transpose", [(100, False), (4096, False), (4096, True), (1, True), (40037, False),
                                             (40037, True)])
def test_rotate_matches_reference(orc, nvec, transpose):
    say(f"case: rotate {nvec} vectors transpose={transpose}")
    g = np.random.Generator(np.random.PCG64(41))
    x = synth.bf16_bits(g.standard_normal(nvec * 128).astype(np.float32) * 3.0)
    seed = 17
    q = torch.from_numpy(hq.hq_haar_matrix(seed)).cuda()
    y = host_f64(hq.hq_rotate(dev(x), q, transpose=transpose))
    x64 = synth.bf16_to_f32(x).astype(np.float64)
    ref = orc.rotate_reference(x64, orc.haar_matrix(seed), transpose=transpose)
    check_rotation(y, ref, x64)


@pytest.mark.parametrize("transpose", [False, True])
def test_rotate_full_kv_layer_sampled(orc, transpose):
    """The bench's launch: one KV layer's [8][32768][128] bf16 tensor (262144 vectors, several groups
    per workgroup), checked on 3000 sampled vectors plus the last 64 against the oracle."""
    nvec = 8 * 32768
    say(f"case: rotate full layer {nvec} vectors transpose={transpose}")
    x = synth.kv(2, 1)
    assert x.size == nvec * 128
    seed = 2
    q = torch.from_numpy(hq.hq_haar_matrix(seed)).cuda()
    y = hq.hq_rotate(dev(x), q, transpose=transpose)
    g = np.random.Generator(np.random.PCG64(43))
    pick = np.unique(np.concatenate([g.integers(0, nvec, 3000), np.arange(nvec - 64, nvec)]))
    yv = y.view(torch.int16).view(nvec, 128)[torch.from_numpy(pick).cuda()]
    ys = synth.bf16_to_f32(yv.cpu().numpy().view(np.uint16)).astype(np.float64)
    x64 = synth.bf16_to_f32(x.reshape(nvec, 128)[pick]).astype(np.float64)
    ref = orc.rotate_reference(x64.reshape(-1), orc.haar_matrix(seed), transpose=transpose)
    check_rotation(ys.reshape(-1), ref, x64.reshape(-1))


def test_rotate_round_trip_and_empty():
    say("case: rotate round trip")
    g = np.random.Generator(np.random.PCG64(42))
    x = synth.bf16_bits(g.standard_normal(512 * 128).astype(np.float32))
    q = torch.from_numpy(hq.hq_haar_matrix(5)).cuda()
    xd = dev(x)
    back = host_f64(hq.hq_rotate(hq.hq_rotate(xd, q), q, transpose=True))
    x64 = synth.bf16_to_f32(x).astype(np.float64)
    assert np.abs(back - x64).max() <= 2.0 ** -7 * np.abs(x64).max()
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    assert hq.hq_rotate(e, q).numel() == 0


def test_kv_call_with_haar_rotation(orc):
    """One KV call with the full per-layer rotation: rotate (MFMA), encode with dither at 2 bps,
    decode, rotate back.  Stream and bf16 decode identical to the oracle's on the rotated tensor;
    the rotated-back values within the rotation bar of the oracle's binary64 inverse rotation."""
    say("case: kv layer 3 K with Haar rotation, 2 bps")
    layer, is_v = 3, 0
    x = synth.kv(layer, is_v, tokens=4096)
    seed = synth.kv_seed(layer, is_v)
    q = torch.from_numpy(hq.hq_haar_matrix(1000 + layer)).cuda()
    xr = hq.hq_rotate(dev(x), q)
    xr_host = xr.view(torch.int16).cpu().numpy().view(np.uint16)
    s_gpu, info = hq.hq_encode(xr, "e8", 2.0, seed=seed, dither=True)
    s_orc, _ = orc.encode(xr_host, orc.LAT_E8, 2.0, seed=seed, dither=True)
    g = s_gpu.cpu().numpy().view(np.uint8)
    assert g.size == s_orc.size and np.array_equal(g, s_orc)
    assert abs(info["payload_bps"] - 2.0) <= 0.01
    yd = hq.hq_decode(s_gpu, x.size, out_dtype=torch.bfloat16)
    y_orc = orc.decode(s_orc, x.size, out_dtype="bf16")
    assert np.array_equal(yd.view(torch.int16).cpu().numpy().view(np.uint16), y_orc)
    back = host_f64(hq.hq_rotate(yd, q, transpose=True))
    yd64 = synth.bf16_to_f32(y_orc).astype(np.float64)
    ref = orc.rotate_reference(yd64, orc.haar_matrix(1000 + layer), transpose=True)
    check_rotation(back, ref, yd64)
