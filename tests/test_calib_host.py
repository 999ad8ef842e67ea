"""The library's host-side basis solver (sjsa_calib_basis, no GPU work) against the
oracle's closed form and numpy's symmetric eigensolver."""
import numpy as np
import pytest

import token_level_sparse_kv_amd as sj
from oracle import calib


def _sums(rng, H, d, n, aniso):
    q = rng.standard_normal((H, n, d)) * aniso
    k = rng.standard_normal((H, n, d)) * aniso[::-1] * 7.0
    SQ = np.einsum("hni,hnj->hij", q, q)
    SK = np.einsum("hni,hnj->hij", k, k)
    return SQ, SK


@pytest.mark.parametrize("d,r", [(16, 4), (128, 32), (128, 16)])
def test_host_basis_matches_closed_form(d, r):
    rng = np.random.default_rng(d + r)
    aniso = np.exp(-np.arange(d) / (d / 6))
    SQ, SK = _sums(rng, 3, d, 4 * d, aniso)
    M, w = sj.calib_basis(SQ, SK, r)
    for h in range(3):
        Mo, wo = calib.basis_from_sums(SQ[h], SK[h], r)
        ref = np.linalg.eigvalsh(calib.trace_normalize(SQ[h]) + calib.trace_normalize(SK[h]))[::-1]
        assert np.allclose(w[h], ref, rtol=1e-10, atol=1e-13)
        assert np.allclose(w[h], wo, rtol=1e-10, atol=1e-13)
        gap = wo[r - 1] - wo[r]
        assert gap > 1e-6
        assert calib.subspace_overlap(M[h].astype(np.float64), Mo) > 1 - 1e-6
        G = M[h].astype(np.float64) @ M[h].astype(np.float64).T
        assert np.max(np.abs(G - np.eye(r))) < 1e-6
        # sign convention: each row's largest-magnitude component is positive
        assert np.all(M[h][np.arange(r), np.argmax(np.abs(M[h]), axis=1)] > 0)


def test_host_basis_of_a_diagonal_problem():
    # diagonal moments: the eigenvectors are unit vectors, in descending diagonal order
    d, r = 8, 3
    SQ = np.diag(np.arange(1.0, d + 1))[None]
    SK = np.diag(np.arange(d, 0, -1.0) ** 2)[None]
    M, w = sj.calib_basis(SQ, SK, r)
    a = np.arange(1.0, d + 1) / np.arange(1.0, d + 1).sum() + np.arange(d, 0, -1.0) ** 2 / (
        np.arange(d, 0, -1.0) ** 2).sum()
    order = np.argsort(-a, kind="stable")
    assert np.allclose(w[0], a[order], rtol=1e-12)
    assert np.array_equal(np.abs(M[0]), np.eye(d, dtype=np.float32)[order[:r]])


def test_host_basis_rejects_bad_arguments():
    SQ = np.eye(4)[None]
    with pytest.raises(sj.SjsaError):
        sj.calib_basis(SQ, SQ, 0)
    with pytest.raises(sj.SjsaError):
        sj.calib_basis(SQ, SQ, 5)
    with pytest.raises(sj.SjsaError):
        sj.calib_basis(np.zeros((1, 4, 4)), SQ, 2)          # no samples: zero trace
