"""CPU oracle for one decode step of JSSA token-level sparse attention.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the benchmark's
cpu_baseline leg may import anything under oracle/. Nothing here is shared with
the HIP path: no kernels, headers, helpers or tables.

Source: the JSSA article, "JSSA 完全拆解:联合 query-key 子空间打分与 gather-free
内核,训练无关的 token 级稀疏解码" (pinghaoyang.com.cn). Section names below are
that page's headings.

What one step computes, per sequence b and KV head h (section "JSSA 的整体结构",
Fig. 1 of the paper):
  1. the mean query of the G query heads that share KV head h,
  2. its projection onto the orthonormal scoring basis M_h (r x d, M M^T = I_r),
  3. a score for every cached position j < n_b against the projected key cache
     Kproj = K M^T (section "打分误差的定义": s_hat = qbar^T M^T M k = (M qbar).(M k)),
  4. the top-k positions, one index set per KV head, shared by its G query heads,
  5. exact softmax attention of each of the G full-dimension queries over the
     selected positions, reading the original K and V (the scoring cache is used
     for selection only; section "JSSA 的整体结构" and "原理详解(二)").

Readings taken where the pages are silent (each is also listed in the design notes):
  * precision: "plain fp32 scoring" - q_bar, q_hat and every score are fp32 values.
    Each is the fp32 rounding of its value computed from the fp32/bf16 inputs
    (q_bar: fp32 sum in head order, then division by G in fp32; q_hat and s: fp64
    dot products rounded once to fp32). Identical Kproj rows therefore always get
    bit-identical scores.
  * ties: lower position wins; -0 and +0 are equal; NaN ranks below every number.
  * k > n_b: all n_b positions are selected; idx is padded with -1.
  * idx lists the selected positions in ascending order (the set is what matters).
  * query head h_q belongs to KV head h_q // G.
  * softmax scale: 1/sqrt(d) unless the caller gives one; scoring is scale free.
  * n_b = 0: nothing is selected and the output is zero.
  * the attention itself is exact: fp64 logits, fp64 softmax, fp64 weighted sum
    of the bf16 V rows.
  * scoring-cache format: bf16 by default; "fp8" is OCP E4M3 (the page keeps the
    cache in FP8 without naming a variant), written unscaled and saturating at
    +-448, rounded once from the fp64 dot.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import bf16_to_f32, fp8e4m3_to_f32, round_to_bf16, round_to_fp8e4m3


# --------------------------------------------------------------------------- prep
def mean_query(q_heads_bits: np.ndarray) -> np.ndarray:
    """q_bar = (1/G) * sum_g q_g for the G query heads of one KV head
    (section "打分误差的定义"). Input [G, d] bf16 bits; fp32 result: the sum is
    accumulated in fp32 in head order, then divided by G in fp32."""
    qf = bf16_to_f32(q_heads_bits)
    acc = np.zeros(qf.shape[-1], dtype=np.float32)
    for g in range(qf.shape[0]):
        acc = (acc + qf[g]).astype(np.float32)
    return (acc / np.float32(qf.shape[0])).astype(np.float32)


def project_query(q_bar: np.ndarray, M: np.ndarray) -> np.ndarray:
    """q_hat = M q_bar (r values), the query side of s_hat = (M q_bar).(M k)."""
    Md = np.asarray(M, dtype=np.float32).astype(np.float64)
    qd = np.asarray(q_bar, dtype=np.float32).astype(np.float64)
    return (Md * qd[None, :]).sum(axis=1).astype(np.float32)


KPROJ_FORMATS = ("bf16", "fp8")   # fp8: OCP E4M3, unscaled, saturating


def project_keys(k_bits: np.ndarray, M: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Projected scoring-cache rows Kproj = K M^T, rounded to the cache format.

    k_bits [..., d] bf16 bits, M [r, d] fp32 -> [..., r] bits (uint16 for bf16, uint8
    for fp8). The dot products are taken in fp64 and rounded once, ties to even (section
    "投影打分缓存与校准成本": the scoring cache holds every key projected onto the
    basis; the page keeps it in FP8, which is the "fp8" format here)."""
    kf = bf16_to_f32(k_bits).astype(np.float64)
    Md = np.asarray(M, dtype=np.float32).astype(np.float64)
    prod = kf[..., None, :] * Md            # [..., r, d]
    dots = prod.sum(axis=-1)
    if fmt == "fp8":
        return round_to_fp8e4m3(dots)
    assert fmt == "bf16", fmt
    return round_to_bf16(dots)


def decode_kproj(kproj_bits: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Stored scoring-cache values as fp32 (exact)."""
    if fmt == "fp8":
        return fp8e4m3_to_f32(kproj_bits)
    assert fmt == "bf16", fmt
    return bf16_to_f32(kproj_bits)


# ------------------------------------------------------------------------ scoring
def score_positions(q_hat: np.ndarray, kproj_bits: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """s_j = q_hat . Kproj_j for every row j of the stored projected cache.

    kproj_bits [n, r] (bf16 or fp8 bits) -> fp32 [n]. The products of an fp32 and a
    stored value are exact in fp64; the r-term sum is done row by row in the same
    order for every row and rounded once to fp32."""
    kp = decode_kproj(kproj_bits, fmt).astype(np.float64)
    qd = np.asarray(q_hat, dtype=np.float32).astype(np.float64)
    return (kp * qd[None, :]).sum(axis=1).astype(np.float32)


# ------------------------------------------------------------------------- top-k
def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ascending, padded with -1 to length k.

    Ranking: larger score first; equal scores by lower position; NaN last.
    np.argsort on the negated scores with a stable sort gives exactly that order:
    -0 and +0 compare equal, NaN sorts to the end."""
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[0]
    kk = min(int(k), n)
    out = np.full(int(k), -1, dtype=np.int32)
    if kk > 0:
        order = np.argsort(-s, kind="stable")
        out[:kk] = np.sort(order[:kk]).astype(np.int32)
    return out


# --------------------------------------------------------------------- attention
def attend(q_heads_bits: np.ndarray, K_bits: np.ndarray, V_bits: np.ndarray,
           idx: np.ndarray, sm_scale: float) -> np.ndarray:
    """Exact softmax attention of each query head over the selected positions.

    o_g = sum_{j in S} softmax_j(sm_scale * q_g . k_j) v_j, S = {idx >= 0}
    (the neighbour-set attention of the sparse-attention knowledge base page, with
    N(i) = S). q_heads [G, d], K/V [n, d] bf16 bits. Returns fp64 [G, d]."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    G, d = q_heads_bits.shape
    if sel.size == 0:
        return np.zeros((G, d), dtype=np.float64)
    qd = bf16_to_f32(q_heads_bits).astype(np.float64)
    Kd = bf16_to_f32(K_bits[sel]).astype(np.float64)
    Vd = bf16_to_f32(V_bits[sel]).astype(np.float64)
    scale = float(np.float32(sm_scale))
    out = np.empty((G, d), dtype=np.float64)
    for g in range(G):
        z = (Kd @ qd[g]) * scale
        z = z - z.max()
        p = np.exp(z)
        p = p / p.sum()
        out[g] = p @ Vd
    return out


def default_sm_scale(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


# ------------------------------------------------------------------ one full step
def decode_unit(q_heads_bits, K_bits, V_bits, kproj_bits, M, n, k, sm_scale, fmt="bf16"):
    """One (sequence, KV head) unit of the step. Arrays are that unit's slices:
    q_heads [G, d], K/V [cap, d] (bf16 bits), kproj [cap, r] (bits of `fmt`), M [r, d]
    fp32. Returns (out fp64 [G, d], idx int32 [k], scores fp32 [n])."""
    q_bar = mean_query(q_heads_bits)
    q_hat = project_query(q_bar, M)
    s = score_positions(q_hat, kproj_bits[:n], fmt)
    idx = select_topk(s, k)
    out = attend(q_heads_bits, K_bits[:n], V_bits[:n], idx, sm_scale)
    return out, idx, s


def decode_step(q_bits, K_bits, V_bits, kproj_bits, M, seq_len, k, sm_scale=0.0, units=None, fmt="bf16"):
    """The whole step over a batch.

    q [B, H_q, d], K/V [B, H_kv, cap, d], kproj [B, H_kv, cap, r] (bf16 bits),
    M [H_kv, r, d] fp32, seq_len [B]. Returns out fp64 [B, H_q, d] and
    idx int32 [B, H_kv, k]. With `units` (a list of (b, h)), only those units are
    computed and the rest of out/idx is left at zero/-1."""
    B, Hq, d = q_bits.shape
    Hkv = K_bits.shape[1]
    cap = K_bits.shape[2]
    G = Hq // Hkv
    scale = sm_scale if sm_scale != 0.0 else default_sm_scale(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    idx = np.full((B, Hkv, int(k)), -1, dtype=np.int32)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        n = int(min(max(int(seq_len[b]), 0), cap))
        o, ix, _ = decode_unit(q_bits[b, h * G:(h + 1) * G], K_bits[b, h], V_bits[b, h],
                               kproj_bits[b, h], M[h], n, k, scale, fmt)
        out[b, h * G:(h + 1) * G] = o
        idx[b, h] = ix
    return out, idx


def append_rows(k_new_bits, v_new_bits, M, pos, K_bits, V_bits, kproj_bits, fmt="bf16"):
    """Append T new tokens per (b, h) at positions pos[b] .. pos[b]+T-1 (in place):
    K and V get the rows as given, Kproj gets project_keys of the new keys.
    Rows that would land outside [0, cap) are dropped."""
    B, Hkv, T, _ = k_new_bits.shape
    cap = K_bits.shape[2]
    for b in range(B):
        for h in range(Hkv):
            rows = project_keys(k_new_bits[b, h], M[h], fmt)
            for t in range(T):
                p = int(pos[b]) + t
                if 0 <= p < cap:
                    K_bits[b, h, p] = k_new_bits[b, h, t]
                    V_bits[b, h, p] = v_new_bits[b, h, t]
                    kproj_bits[b, h, p] = rows[t]
