"""GPU: the fused decode + matrix-vector product (hq_gemv) against the oracle's binary64 product
with the decoded matrix.

Bar: per row, |y_gpu - y_ref| <= (column tiles + 32) * 2^-24 * B_r / 128, where B_r is the sum over
the row's tiles of ||yhat_tile||_1 * ||x_tile||_1 (the rounding scale of rotating the activation in
binary32, the tile's products and tree sum, and the row's sum in column order); and the relative
error of the whole vector is far below that bound."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()


def say(msg):
    print(msg, flush=True)


def check_rows(orc, s_gpu, rows, cols, x_host, x_dev, seed):
    y = hq.hq_gemv(s_gpu, rows, cols, x_dev).cpu().numpy().astype(np.float64)
    s_host = s_gpu.cpu().numpy()
    xr = x_host.astype(np.float64) if x_host.dtype != np.uint16 else synth.bf16_to_f32(x_host).astype(np.float64)
    y_ref, bound = orc.gemv_reference(s_host, rows, cols, xr, seed=seed)
    tol = (cols // 128 + 32) * U * bound / 128.0
    err = np.abs(y - y_ref)
    worst = float(np.max(err / np.maximum(tol, 1e-300)))
    say(f"rows {rows} cols {cols}: worst err/tol {worst:.3g}, rel {np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref):.3g}")
    assert np.all(err <= tol), worst
    assert np.linalg.norm(y - y_ref) <= 1e-5 * np.linalg.norm(y_ref)
    return y


@pytest.mark.parametrize("lattice,dither,target", [("e8", False, 4.0), ("e8", True, 2.0), ("d4", False, 4.0),
                                                    ("a2", True, 3.0), ("e8", 7, 2.0),
                                                    ("z", False, 3.0)])
def test_gemv_small_matrix(orc, lattice, dither, target):
    say(f"case: gemv 96x1024 {lattice} dither={dither} {target} bps")
    rows, cols = 96, 1024
    g = np.random.Generator(np.random.PCG64(21))
    w = synth.bf16_bits(0.02 * g.standard_normal((rows, cols)).astype(np.float32))
    x = g.standard_normal(cols).astype(np.float32)
    s_gpu, _ = hq.hq_encode(dev(w), lattice, target, seed=5, dither=dither)
    check_rows(orc, s_gpu, rows, cols, x, dev(x), seed=5)


def test_gemv_long_segments(orc):
    """The decoder's long-segment path (k = 0 at a small step: every chunk's unary segment above
    2048 words) under the fused product."""
    say("case: gemv 64x1024 e8 long segments")
    rows, cols = 64, 1024
    g = np.random.Generator(np.random.PCG64(23))
    w = synth.bf16_bits(0.02 * g.standard_normal((rows, cols)).astype(np.float32))
    x = g.standard_normal(cols).astype(np.float32)
    s_gpu, _ = hq.hq_encode(dev(w), "e8", 0.0, seed=5, step=0.03, rice_k=0)
    s_host = s_gpu.cpu().numpy()
    h = s_host[:128].view(np.uint32)
    idx = s_host[128:128 + 4 * (int(h[10]) + 1)].view(np.uint32).astype(np.int64)
    assert (2 * np.diff(idx) > 2048).all()
    check_rows(orc, s_gpu, rows, cols, x, dev(x), seed=5)


def test_gemv_bf16_activation_and_ragged_chunk(orc):
    """bf16 activation; 3 x 1024 is 24 tiles, one partly filled chunk."""
    say("case: gemv 3x1024 bf16 x")
    rows, cols = 3, 1024
    g = np.random.Generator(np.random.PCG64(22))
    w = synth.bf16_bits(g.standard_normal((rows, cols)).astype(np.float32))
    xb = synth.bf16_bits(g.standard_normal(cols).astype(np.float32))
    s_gpu, _ = hq.hq_encode(dev(w), "e8", 4.0, seed=2)
    check_rows(orc, s_gpu, rows, cols, xb, dev(xb), seed=2)


def test_gemv_rows_across_chunks(orc):
    """The down projection's shape: 112 column tiles per row, so rows straddle 64-tile chunks."""
    say("case: gemv 40x14336")
    rows, cols = 40, 14336
    g = np.random.Generator(np.random.PCG64(23))
    w = synth.bf16_bits(0.02 * g.standard_normal((rows, cols)).astype(np.float32))
    x = g.standard_normal(cols).astype(np.float32)
    s_gpu, _ = hq.hq_encode(dev(w), "e8", 4.0, seed=6)
    check_rows(orc, s_gpu, rows, cols, x, dev(x), seed=6)


def test_gemv_full_weight(orc):
    """The 14336 x 4096 MLP weight at 4 bps with a N(0,1) activation: every row within the bound."""
    say("case: gemv full weight 14336x4096")
    w = synth.weight()
    x = synth.gaussian(4096, seed=31)
    s_gpu, _ = hq.hq_encode(dev(w), "e8", 4.0)
    check_rows(orc, s_gpu, 14336, 4096, x, dev(x), seed=0)


def test_gemv_rejects_mismatched_shape():
    """A stream of n values read as a matrix of another size is corrupt (header n check)."""
    say("case: gemv shape mismatch")
    w = dev(synth.bf16_bits(np.ones((8, 1024), dtype=np.float32)))
    s_gpu, _ = hq.hq_encode(w, "e8", 4.0)
    x = torch.ones(1024, device="cuda")
    with pytest.raises(hq.HqError) as e:
        hq.hq_gemv(s_gpu, 16, 1024, x)
    assert e.value.code == hq.HQ_ERR_CORRUPT


def test_gemv_empty_matrix():
    """rows = 0: only the stream is checked (the activation may then be empty)."""
    say("case: gemv on an empty matrix")
    s_gpu, _ = hq.hq_encode(torch.zeros(0, device="cuda"), "e8", 4.0)
    y = hq.hq_gemv(s_gpu, 0, 1024, torch.zeros(1024, device="cuda"))
    assert y.numel() == 0
    bad = s_gpu.clone()
    bad[0] ^= 1
    with pytest.raises(hq.HqError) as e:
        hq.hq_gemv(bad, 0, 1024, torch.zeros(1024, device="cuda"))
    assert e.value.code == hq.HQ_ERR_CORRUPT
