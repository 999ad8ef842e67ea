"""GPU parity of the calibration accumulation (sjsa_calib_accumulate) against the
oracle's sums, and the basis the host solver derives from them."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
from oracle import calib
from oracle.numerics import bf16_to_f32
from tests.gpu_helpers import bits, say

pytestmark = pytest.mark.gpu


def _prefill(B, Hkv, G, T, seed, aniso=True):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    scale = torch.exp(-torch.arange(128, device="cuda") / 20.0) if aniso else torch.ones(128, device="cuda")
    q = (torch.randn(B, Hkv * G, T, 128, generator=g, device="cuda") * scale).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, T, 128, generator=g, device="cuda") * scale.flip(0) * 5).to(torch.bfloat16)
    return q, k


def _oracle_sums(q, k, h, G):
    qb, kb = bits(q), bits(k)               # [B, Hq, T, d], [B, Hkv, T, d]
    B, _, T, d = qb.shape
    qh = qb[:, h * G:(h + 1) * G].transpose(0, 2, 1, 3).reshape(B * T, G, d)
    ks = kb[:, h].reshape(B * T, d)
    return calib.accumulate_moments(qh, ks), qh, ks


def _bound(qh, ks):
    """Elementwise bound of the fp32 summation error: 256 positions per fp32 run."""
    from oracle import jssa
    qbar = np.stack([jssa.mean_query(qh[i]) for i in range(qh.shape[0])]).astype(np.float64)
    kf = bf16_to_f32(ks).astype(np.float64)
    return (np.abs(qbar).T @ np.abs(qbar)) * 256 * 2.0 ** -24 + 1e-30, \
        (np.abs(kf).T @ np.abs(kf)) * 256 * 2.0 ** -24 + 1e-30


@pytest.mark.parametrize("G,B,T", [(4, 2, 3000), (1, 1, 1), (8, 3, 517), (2, 1, 4096)])
def test_calib_sums_match_oracle(G, B, T):
    say(f"calibration sums G={G} B={B} T={T}")
    Hkv = 2
    q, k = _prefill(B, Hkv, G, T, seed=90 + G)
    SQ = torch.zeros(Hkv, 128, 128, dtype=torch.float64, device="cuda")
    SK = torch.zeros_like(SQ)
    sj.calib_accumulate(q, k, SQ, SK)
    torch.cuda.synchronize()
    for h in range(Hkv):
        (rq, rk), qh, ks = _oracle_sums(q, k, h, G)
        bq, bk = _bound(qh, ks)
        assert np.all(np.abs(SQ[h].cpu().numpy() - rq) <= bq), h
        assert np.all(np.abs(SK[h].cpu().numpy() - rk) <= bk), h


def test_calib_accumulates_across_calls_and_is_deterministic():
    say("calibration: two prefills add up; repeat runs are bit-identical")
    q1, k1 = _prefill(1, 2, 4, 2000, seed=95)
    q2, k2 = _prefill(1, 2, 4, 1500, seed=96)
    runs = []
    for _ in range(2):
        SQ = torch.zeros(2, 128, 128, dtype=torch.float64, device="cuda")
        SK = torch.zeros_like(SQ)
        sj.calib_accumulate(q1, k1, SQ, SK)
        sj.calib_accumulate(q2, k2, SQ, SK)
        torch.cuda.synchronize()
        runs.append((SQ.cpu().numpy(), SK.cpu().numpy()))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    for h in range(2):
        (a, b), qa, ka = _oracle_sums(q1, k1, h, 4)
        (c, e), qc, kc = _oracle_sums(q2, k2, h, 4)
        bq1, bk1 = _bound(qa, ka)
        bq2, bk2 = _bound(qc, kc)
        assert np.all(np.abs(runs[0][0][h] - (a + c)) <= bq1 + bq2)
        assert np.all(np.abs(runs[0][1][h] - (b + e)) <= bk1 + bk2)


def test_calibrated_basis_matches_oracle_basis():
    say("calibration: basis from GPU sums vs the oracle's closed form")
    q, k = _prefill(2, 2, 4, 4096, seed=97)
    SQ = torch.zeros(2, 128, 128, dtype=torch.float64, device="cuda")
    SK = torch.zeros_like(SQ)
    sj.calib_accumulate(q, k, SQ, SK)
    torch.cuda.synchronize()
    M, w = sj.calib_basis(SQ, SK, 32)
    for h in range(2):
        (rq, rk), _, _ = _oracle_sums(q, k, h, 4)
        Mo, wo = calib.basis_from_sums(rq, rk, 32)
        assert np.allclose(w[h], wo, rtol=1e-6, atol=1e-9)
        assert wo[31] - wo[32] > 1e-4
        assert calib.subspace_overlap(M[h].astype(np.float64), Mo) > 1 - 1e-5
