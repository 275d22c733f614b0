"""GPU parity over a seeded sweep of small configurations: lattice, tile length, dither flags,
input type, tile count (ragged chunks included), value scale, and the operating mode (rate
control, fixed step with fixed or automatic Rice parameter).  Each case compares the stream byte
for byte and the fp32 decode bit for bit with the oracle's."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

LAT = {"z": 0, "d4": 1, "e8": 2, "a2": 3}


def cases(count=120, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        tile = int(rng.choice([64, 128, 256]))
        lat = str(rng.choice(list(LAT)))
        dither = int(rng.choice([0, 1, 3, 5, 7]))
        dtype = str(rng.choice(["f32", "bf16"]))
        tiles = int(rng.choice([1, 2, 7, 8192 // tile - 1, 8192 // tile, 8192 // tile + 1, 3 * 8192 // tile + 5]))
        scale = float(10.0 ** rng.uniform(-4, 4))
        mode = str(rng.choice(["rate", "fixed", "fixed_auto_k"]))
        target = float(rng.choice([1.75, 2.5, 3.0, 4.0, 5.5]))
        if lat == "e8":
            target = max(target, 1.25)
        if lat == "a2":
            target = max(target, 1.75)
        step = float(10.0 ** rng.uniform(-1.5, 0.5))
        k = int(rng.integers(0, 9))
        out.append((i, tile, lat, dither, dtype, tiles, scale, mode, target, step, k, int(rng.integers(0, 2 ** 32))))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"c{c[0]}")
def test_sweep_case(orc, case):
    i, tile, lat, dither, dtype, tiles, scale, mode, target, step, k, seed = case
    print(f"case {i}: tile {tile} {lat} dither {dither} {dtype} tiles {tiles} scale {scale:.3g} {mode}", flush=True)
    x = synth.gaussian(tiles * tile, seed=seed % 100000, std=scale).astype(np.float32)
    if dtype == "bf16":
        x = synth.bf16_bits(x)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xd = torch.from_numpy(x).cuda()
    if mode == "rate":
        kw = dict(target_bps=target)
    elif mode == "fixed":
        kw = dict(target_bps=0.0, step=step, rice_k=k)
    else:
        kw = dict(target_bps=0.0, step=step, rice_k=-1)
    tb = kw.pop("target_bps")
    s_orc, info_orc = orc.encode(x, LAT[lat], tb, seed=seed, dither=dither, tile=tile, **kw)
    s_gpu, info = hq.hq_encode(xd, lat, tb, seed=seed, dither=dither, tile=tile, **kw)
    g = s_gpu.cpu().numpy()
    assert g.size == s_orc.size and np.array_equal(g, s_orc), (g.size, s_orc.size)
    if mode == "rate":
        assert abs(info["payload_bps"] - target) <= 0.01 or tiles * tile < 4096
    y = hq.hq_decode(s_gpu, x.size, out_dtype=torch.float32)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.decode(s_orc, x.size).view(np.uint32))
