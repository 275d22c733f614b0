"""GPU: the SRFT fixed-rate KV codec (hq_srft_encode / hq_srft_decode) against the oracle, bit for bit.

Codes and scales are integers decided in binary32 by the same operations on both sides, so they must be
identical; the decoded values are binary32 (or their bf16 rounding) computed by the same operations, so
they must be identical too (NaN outputs compared as NaN, zeros are +0 on both sides)."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def to_dev(a: np.ndarray):
    a = np.ascontiguousarray(a).reshape(-1)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


def gpu_encode(x, seed, bits, lam=None):
    c, s = hq.hq_srft_encode(to_dev(x), seed=seed, bits=bits, lam=lam)
    return c.cpu().numpy(), s.cpu().numpy().view(np.uint16)


def same_floats(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a)
    b = np.asarray(b)
    if a.dtype == np.uint16:
        fa, fb = synth.bf16_to_f32(a), synth.bf16_to_f32(b)
    else:
        fa, fb = a, b
    na, nb = np.isnan(fa), np.isnan(fb)
    return bool(np.array_equal(na, nb) and np.array_equal(a.view(np.uint8)[~np.repeat(na, a.itemsize)],
                                                           b.view(np.uint8)[~np.repeat(nb, b.itemsize)]))


def check(x, seed, bits, lam=None, out_dtypes=("bf16", "f32")):
    n = np.asarray(x).size
    cg, sg = gpu_encode(x, seed, bits, lam)
    co, so = synth_oracle.srft_encode(x, seed, bits, lam)
    assert np.array_equal(sg, so), "scales differ"
    assert np.array_equal(cg, co), "codes differ"
    for od in out_dtypes:
        yg = hq.hq_srft_decode(torch.from_numpy(cg).cuda(), torch.from_numpy(sg.view(np.int16)).cuda(), n, seed=seed,
                               bits=bits, lam=lam, out_dtype=torch.bfloat16 if od == "bf16" else torch.float32)
        yg = yg.view(torch.int16).cpu().numpy().view(np.uint16) if od == "bf16" else yg.cpu().numpy()
        yo = synth_oracle.srft_decode(co, so, n, seed, bits, lam, out_dtype=od)
        assert same_floats(yg, yo), f"decode ({od}) differs"
    return cg, sg


synth_oracle = None


@pytest.fixture(autouse=True)
def _orc(orc):
    global synth_oracle
    synth_oracle = orc


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("nvec", [1, 300, 4096])
def test_kv_vectors_bit_exact(bits, nvec):
    say(f"case: srft kv layer 1 K, {nvec} vectors, bits={bits}")
    x = synth.kv(1, 0, tokens=(nvec + 7) // 8).reshape(-1)[: 128 * nvec]
    check(x, synth.kv_seed(1, 0), bits)


def test_float32_input_and_lambda():
    say("case: srft float32 input, random lambda")
    g = np.random.default_rng(5)
    x = (g.standard_normal(128 * 777) * g.uniform(0.01, 100.0)).astype(np.float32)
    lam = g.uniform(0.25, 4.0, 128).astype(np.float32)
    for bits in (4, 8):
        check(x, 123, bits, lam)
    xb = synth.kv(4, 0, tokens=64).reshape(-1)
    check(xb, 9, 4, lam)


def test_edge_vectors():
    say("case: srft zero / NaN / inf / huge / tiny vectors")
    g = np.random.default_rng(8)
    rows = [np.zeros(128, dtype=np.float32)]
    r = g.standard_normal(128).astype(np.float32); r[17] = np.nan; rows.append(r)
    r = g.standard_normal(128).astype(np.float32); r[0] = np.inf; rows.append(r)
    rows.append(np.full(128, 3.0e36, dtype=np.float32))              # sums overflow binary32
    rows.append((g.standard_normal(128) * 1e6).astype(np.float32))   # scales saturate at 65504
    rows.append((g.standard_normal(128) * 1e-38).astype(np.float32))  # subnormal scales / zero codes
    rows.append((g.standard_normal(128) * 1e-6).astype(np.float32))
    e = np.zeros(128, dtype=np.float32); e[5] = 1.0; rows.append(e)
    x = np.concatenate(rows)
    for bits in (4, 8):
        cg, sg = check(x, 77, bits)
    xb = synth.bf16_bits(x)
    check(xb, 77, 4)
    empty = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    c, s = hq.hq_srft_encode(empty)
    assert c.numel() == 0 and s.numel() == 0


@pytest.mark.parametrize("bits", [4, 8])
def test_full_kv_layer_sampled(bits):
    """The bench's launch: one KV layer [8][32768][128] bf16 (262144 vectors); 2000 sampled vectors
    and the last 64 against the oracle (vectors are independent)."""
    say(f"case: srft full layer, bits={bits}")
    x = synth.kv(0, 0)
    nv = x.size // 128
    seed = synth.kv_seed(0, 0)
    xd = to_dev(x)
    cg, sg = hq.hq_srft_encode(xd, seed=seed, bits=bits)
    yg = hq.hq_srft_decode(cg, sg, x.size, seed=seed, bits=bits)
    g = np.random.default_rng(44)
    pick = np.unique(np.concatenate([g.integers(0, nv, 2000), np.arange(nv - 64, nv)]))
    xs = x.reshape(nv, 128)[pick]
    co, so = synth_oracle.srft_encode(xs, seed, bits)
    ig = torch.from_numpy(pick).cuda()
    assert np.array_equal(sg[ig].cpu().numpy().view(np.uint16), so)
    assert np.array_equal(cg[ig].cpu().numpy(), co)
    yo = synth_oracle.srft_decode(co, so, xs.size, seed, bits).reshape(-1, 128)
    ys = yg.view(torch.int16).view(nv, 128)[ig].cpu().numpy().view(np.uint16)
    assert np.array_equal(ys, yo)
    xf = torch.from_numpy(x.reshape(-1).view(np.int16)).view(torch.bfloat16).cuda().float()
    nmse = float(((yg.float() - xf) ** 2).sum() / (xf ** 2).sum())
    say(f"nmse {nmse:.5f}")
    assert nmse < (0.02 if bits == 4 else 1e-4)
