"""Calibration of the JSSA scoring basis, as a CPU oracle (fp64, NumPy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the benchmark's
cpu_baseline leg may import anything under oracle/.

Source: the JSSA article ("JSSA 完全拆解…"), sections "乘积边缘分布", "迹归一化",
"精确目标与它的上界" and "闭式谱解" (paper §3.2, App. B.1-B.3), plus
"校准:一次前向 + 一次特征分解" (App. A.4).

  * second moments of the group-mean query and of the keys, uncentered:
        G_Q = E[q_bar q_bar^T],  G_K = E[k k^T]
  * each normalized to unit trace:  G_hat = G / tr(G)
  * exact selection objective for an orthogonal projector P (rank r):
        L_sel(P)  = tr((I-P) G_hatQ (I-P) G_hatK)
  * its tractable surrogate, an upper bound L_sel <= L_marg^2 / 4:
        L_marg(P) = tr((I-P) (G_hatQ + G_hatK))
  * closed-form minimizer of L_marg: M* = (top-r eigenvectors of G_hatQ + G_hatK),
    one eigenvector per row, so M* is r x d with M* M*^T = I_r and P = M*^T M*.

Readings: the hats lost in the page's extraction are restored on all three
formulas; the bound constant is 1/4 (the AM-GM step); TopEig_r yields d x r
columns and M* is their transpose. Eigenvector signs are arbitrary, so bases are
compared through subspace overlap (mean squared cosine of the principal angles,
section "直接优化精确目标:为什么没必要").
"""
from __future__ import annotations

import numpy as np


def group_mean_queries(q_heads: np.ndarray) -> np.ndarray:
    """[N, G, d] query heads -> [N, d] group-mean queries (fp64)."""
    return np.asarray(q_heads, dtype=np.float64).mean(axis=1)


def second_moments(q_bar: np.ndarray, keys: np.ndarray):
    """Uncentered second moments G_Q = (1/N) sum q_bar q_bar^T and G_K likewise."""
    qb = np.asarray(q_bar, dtype=np.float64)
    kk = np.asarray(keys, dtype=np.float64)
    return qb.T @ qb / qb.shape[0], kk.T @ kk / kk.shape[0]


def trace_normalize(G: np.ndarray) -> np.ndarray:
    return G / np.trace(G)


def closed_form_basis(GQn: np.ndarray, GKn: np.ndarray, r: int):
    """M* (r x d, rows = eigenvectors of GQn + GKn for the r largest eigenvalues,
    in descending eigenvalue order) and all eigenvalues in descending order."""
    A = GQn + GKn
    A = 0.5 * (A + A.T)
    w, U = np.linalg.eigh(A)                 # ascending
    order = np.argsort(w)[::-1]
    w = w[order]
    U = U[:, order]
    return U[:, :r].T.copy(), w


def calibrate(q_heads: np.ndarray, keys: np.ndarray, r: int) -> np.ndarray:
    """Basis from calibration samples: q_heads [N, G, d], keys [N, d] -> M [r, d] fp64."""
    GQ, GK = second_moments(group_mean_queries(q_heads), keys)
    M, _ = closed_form_basis(trace_normalize(GQ), trace_normalize(GK), r)
    return M


def projector(M: np.ndarray) -> np.ndarray:
    """P = M^T M, the rank-r orthogonal projector of an orthonormal r x d basis."""
    Md = np.asarray(M, dtype=np.float64)
    return Md.T @ Md


def selection_loss(P: np.ndarray, GQn: np.ndarray, GKn: np.ndarray) -> float:
    """L_sel(P) = tr((I-P) G_hatQ (I-P) G_hatK)."""
    R = np.eye(P.shape[0]) - P
    return float(np.trace(R @ GQn @ R @ GKn))


def marginal_loss(P: np.ndarray, GQn: np.ndarray, GKn: np.ndarray) -> float:
    """L_marg(P) = tr((I-P)(G_hatQ + G_hatK))."""
    R = np.eye(P.shape[0]) - P
    return float(np.trace(R @ (GQn + GKn)))


def subspace_overlap(Ma: np.ndarray, Mb: np.ndarray) -> float:
    """Mean squared cosine of the principal angles between the row spaces of two
    orthonormal r x d bases: ||Ma Mb^T||_F^2 / r (1 when the subspaces coincide)."""
    C = np.asarray(Ma, dtype=np.float64) @ np.asarray(Mb, dtype=np.float64).T
    return float((C * C).sum() / Ma.shape[0])


def accumulate_moments(q_heads_bits: np.ndarray, keys_bits: np.ndarray):
    """Sums of outer products over calibration positions, the quantities a prefill
    accumulates (section "校准:一次前向 + 一次特征分解": one dense prefill per
    calibration sequence accumulates the second moments of the group-mean query and
    of the key, per layer and KV head):
        S_Q = sum_n q_bar_n q_bar_n^T,   S_K = sum_n k_n k_n^T   (fp64, exact sums of
    the fp32 / bf16 values). q_bar_n is the decode step's group-mean query: the fp32
    sum of the G bf16 heads in head order divided by G in fp32. Dividing by the
    sample count gives G_Q and G_K; the trace normalization cancels it.
    q_heads_bits [N, G, d], keys_bits [N, d] bf16 bits."""
    from .jssa import mean_query
    from .numerics import bf16_to_f32
    qh = np.asarray(q_heads_bits)
    qbar = np.zeros((qh.shape[0], qh.shape[2]))
    for i in range(qh.shape[0]):
        qbar[i] = mean_query(qh[i])
    k = bf16_to_f32(keys_bits).astype(np.float64)
    return qbar.T @ qbar, k.T @ k


def basis_from_sums(SQ: np.ndarray, SK: np.ndarray, r: int):
    """M* and the descending eigenvalues of G_hatQ + G_hatK from accumulated sums."""
    return closed_form_basis(trace_normalize(SQ), trace_normalize(SK), r)
