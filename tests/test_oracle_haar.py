"""Pins of the per-layer Haar-uniform rotation (HyperQuant summary, Methodology component 4: the full
Haar-uniform matrix alternative to the +-1 sign diagonal), and agreement of the library's host
construction (Householder) with the oracle's (Gram-Schmidt)."""
import numpy as np
import pytest

import kv_quantization_tile_amd as hq


def test_gaussians_look_standard_normal(orc):
    g = np.concatenate([orc.haar_gaussians(s).ravel() for s in range(8)])
    assert abs(g.mean()) < 0.01 and abs(g.std() - 1.0) < 0.01
    # fourth moment of N(0,1) is 3
    assert abs((g ** 4).mean() - 3.0) < 0.06


def test_gaussians_pass_normality_and_independence(orc):
    """Kolmogorov-Smirnov against N(0,1) over 4 seeds (65 536 draws), and no correlation between the
    two members of a Box-Muller pair or between neighbouring pairs."""
    from scipy import stats
    g = np.stack([orc.haar_gaussians(s).ravel() for s in (3, 4, 5, 6)])
    assert stats.kstest(g.ravel(), "norm").pvalue > 1e-3
    pairs = g.reshape(-1, 2)
    assert abs(np.corrcoef(pairs[:, 0], pairs[:, 1])[0, 1]) < 0.02
    quads = g.reshape(-1, 4)
    assert abs(np.corrcoef(quads[:, 0], quads[:, 2])[0, 1]) < 0.02
    assert not np.allclose(orc.haar_gaussians(3), orc.haar_gaussians(4))


def test_rotate_reference_closed_forms(orc):
    """Q e_j is column j of Q and Q^T e_j is row j; the rotation keeps every vector's norm and Q^T
    undoes Q."""
    q = orc.haar_matrix(11)
    e = np.eye(128)
    assert np.array_equal(orc.rotate_reference(e.ravel(), q).reshape(128, 128), q.T)
    assert np.array_equal(orc.rotate_reference(e.ravel(), q, transpose=True).reshape(128, 128), q)
    x = np.random.Generator(np.random.PCG64(5)).standard_normal(64 * 128)
    y = orc.rotate_reference(x, q)
    assert np.allclose(np.linalg.norm(y.reshape(-1, 128), axis=1), np.linalg.norm(x.reshape(-1, 128), axis=1),
                       rtol=1e-13)
    assert np.abs(orc.rotate_reference(y, q, transpose=True) - x).max() < 1e-10


@pytest.mark.parametrize("seed", [0, 1, 12345, (7 << 1) | 1])
def test_haar_is_the_orthogonal_factor_with_positive_r(orc, seed):
    """Q is orthogonal and R = Q^T G is upper triangular with a positive diagonal: Q is the Q of
    G's QR decomposition normalised to diag(R) > 0, which makes it Haar-distributed."""
    g = orc.haar_gaussians(seed)
    q = orc.haar_matrix(seed)
    assert np.abs(q.T @ q - np.eye(128)).max() < 1e-12
    r = q.T @ g
    assert np.abs(np.tril(r, -1)).max() < 1e-10
    assert np.all(np.diag(r) > 0)


def test_haar_statistics(orc):
    """Over seeds, entries of a Haar matrix have mean 0 and variance 1/128, and the trace has mean 0
    and variance 1."""
    qs = np.stack([orc.haar_matrix(s) for s in range(200)])
    assert abs(qs.mean()) < 2e-3
    assert abs(qs.var() - 1.0 / 128) < 2e-4
    tr = np.trace(qs, axis1=1, axis2=2)
    assert abs(tr.mean()) < 0.25 and abs(tr.var() - 1.0) < 0.35


@pytest.mark.parametrize("seed", [0, 3, 999])
def test_library_matrix_matches_oracle(orc, seed):
    """hq_haar_matrix (host code of the library, Householder) equals the oracle's Gram-Schmidt
    construction of the same definition, to binary32 rounding."""
    q_lib = hq.hq_haar_matrix(seed).astype(np.float64)
    q_orc = orc.haar_matrix(seed)
    assert np.abs(q_lib - q_orc).max() < 2e-7
