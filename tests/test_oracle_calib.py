"""Pins for the calibration oracle (closed-form basis, losses, bound).

Checks: orthonormal rows; Ky Fan optimality of the closed form for L_marg (its
minimum over rank-r projectors is the sum of the trailing eigenvalues, and random
projectors never beat it); the bound L_sel <= L_marg^2 / 4 from the JSSA article's
section "精确目标与它的上界"; the product-marginal factorization (section
"乘积边缘分布") brute-forced over every (query, key) sample pair; and agreement
with an independent solver (SVD of the stacked, trace-scaled samples)."""
import numpy as np
import pytest

from oracle import calib
import workloads


def _samples(seed=0, N=512, d=64, G=4):
    rng = np.random.default_rng(seed)
    scale = np.ones(d)
    scale[rng.choice(d, 4, replace=False)] = 8.0
    q_heads = rng.standard_normal((N, G, d)) * np.linspace(0.5, 2.0, d)
    keys = rng.standard_normal((N, d)) * scale + 0.3
    return q_heads, keys


def _random_projector(d, r, rng):
    Q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return Q @ Q.T


@pytest.mark.parametrize("r", [4, 16, 32])
def test_closed_form_is_orthonormal_and_ky_fan_optimal(r):
    q_heads, keys = _samples()
    GQ, GK = calib.second_moments(calib.group_mean_queries(q_heads), keys)
    GQn, GKn = calib.trace_normalize(GQ), calib.trace_normalize(GK)
    assert abs(np.trace(GQn) - 1) < 1e-12 and abs(np.trace(GKn) - 1) < 1e-12
    M, w = calib.closed_form_basis(GQn, GKn, r)
    assert M.shape == (r, GQ.shape[0])
    assert np.max(np.abs(M @ M.T - np.eye(r))) < 1e-12
    P = calib.projector(M)
    lm = calib.marginal_loss(P, GQn, GKn)
    assert abs(lm - w[r:].sum()) <= 1e-12 * max(1.0, w.sum())
    rng = np.random.default_rng(1)
    for _ in range(100):
        Pr = _random_projector(GQ.shape[0], r, rng)
        assert calib.marginal_loss(Pr, GQn, GKn) >= lm - 1e-12
        # the bound holds for every orthogonal projector
        assert calib.selection_loss(Pr, GQn, GKn) <= 0.25 * calib.marginal_loss(Pr, GQn, GKn) ** 2 + 1e-15
    assert calib.selection_loss(P, GQn, GKn) <= 0.25 * lm ** 2 + 1e-15


def test_product_marginal_identity_brute_force():
    q_heads, keys = _samples(seed=2, N=512, d=32)
    qb = calib.group_mean_queries(q_heads)
    GQ, GK = calib.second_moments(qb, keys)
    rng = np.random.default_rng(3)
    P = _random_projector(32, 8, rng)
    R = np.eye(32) - P
    # E over independent (q_bar_a, k_b) pairs of the squared projection error
    errs = (qb @ R) @ keys.T                      # [N, N]: q_bar_a^T (I-P) k_b for all pairs
    lhs = np.mean(errs ** 2)
    rhs = np.trace(R @ GQ @ R @ GK)
    assert abs(lhs - rhs) <= 1e-10 * abs(rhs)
    # normalized form is L_sel
    rhs_n = calib.selection_loss(P, calib.trace_normalize(GQ), calib.trace_normalize(GK))
    assert abs(lhs / (np.trace(GQ) * np.trace(GK)) - rhs_n) <= 1e-10 * abs(rhs_n)


def test_independent_svd_solver_spans_the_same_subspace():
    q_heads, keys = _samples(seed=4)
    N = keys.shape[0]
    qb = q_heads.mean(axis=1)
    tq = np.sum(qb * qb) / N
    tk = np.sum(keys * keys) / N
    A = np.vstack([qb / np.sqrt(N * tq), keys / np.sqrt(N * tk)])      # A^T A = G_hatQ + G_hatK
    _, sv, Vt = np.linalg.svd(A, full_matrices=False)
    r = 16
    assert sv[r - 1] ** 2 - sv[r] ** 2 > 1e-6                      # eigengap at r
    M = calib.calibrate(q_heads, keys, r)
    assert calib.subspace_overlap(M, Vt[:r]) > 1 - 1e-10
    # and a basis from the wrong (un-normalized) target is measurably different
    GQ, GK = calib.second_moments(qb, keys)
    Mu, _ = calib.closed_form_basis(GQ, GK, r)
    assert calib.subspace_overlap(M, Mu) < 0.999


def test_tiny_single_head_calibration():
    wl = workloads.tiny_single_head()
    M = calib.calibrate(wl.calib_q.numpy(), wl.calib_k.numpy(), wl.rank)
    assert M.shape == (16, 128)
    assert np.max(np.abs(M @ M.T - np.eye(16))) < 1e-12
    # the 4 scaled key channels carry most of the key energy; each lies almost
    # entirely inside the calibrated subspace
    P = calib.projector(M)
    for c in wl.extra["outlier_channels"].tolist():
        assert P[c, c] > 0.95


def test_accumulated_sums_brute_force_and_invariants():
    # the sums equal an explicit loop of outer products of the decode step's mean
    # queries (pinned in the step tests) and of the keys; they are symmetric PSD with
    # trace = sum of squared norms; splitting the samples adds the sums
    from oracle import jssa
    from oracle.numerics import bf16_to_f32, round_to_bf16
    rng = np.random.default_rng(9)
    qh = round_to_bf16(rng.standard_normal((40, 4, 16)))
    ks = round_to_bf16(rng.standard_normal((40, 16)))
    SQ, SK = calib.accumulate_moments(qh, ks)
    bq = np.zeros((16, 16))
    bk = np.zeros((16, 16))
    for i in range(40):
        qb = jssa.mean_query(qh[i]).astype(np.float64)
        kv = bf16_to_f32(ks[i]).astype(np.float64)
        for a in range(16):
            for b in range(16):
                bq[a, b] += qb[a] * qb[b]
                bk[a, b] += kv[a] * kv[b]
    assert np.allclose(SQ, bq, rtol=1e-13, atol=1e-13) and np.allclose(SK, bk, rtol=1e-13, atol=1e-13)
    assert np.array_equal(SQ, SQ.T) and np.min(np.linalg.eigvalsh(SK)) > -1e-9
    assert abs(np.trace(SK) - (bf16_to_f32(ks).astype(np.float64) ** 2).sum()) < 1e-9
    a = calib.accumulate_moments(qh[:13], ks[:13])
    b = calib.accumulate_moments(qh[13:], ks[13:])
    assert np.allclose(a[0] + b[0], SQ, rtol=1e-13) and np.allclose(a[1] + b[1], SK, rtol=1e-13)
    # the basis from sums equals the basis from means (the normalization cancels N)
    M1, w1 = calib.basis_from_sums(SQ, SK, 5)
    GQ, GK = calib.second_moments(np.stack([jssa.mean_query(qh[i]) for i in range(40)]),
                                  bf16_to_f32(ks).astype(np.float64))
    M2, w2 = calib.closed_form_basis(calib.trace_normalize(GQ), calib.trace_normalize(GK), 5)
    assert np.allclose(w1, w2, atol=1e-12) and calib.subspace_overlap(M1, M2) > 1 - 1e-10
