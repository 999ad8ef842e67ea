"""CPU oracle for the gated-logit sparse decode step (SAS).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the benchmark's
cpu_baseline leg may import anything under oracle/. Nothing here is shared with
the HIP path.

Source: the SAS article, "SAS：用门控稀疏注意力把上下文排序端到端对齐 LM 损失"
(papers.ananclaw.com explainer of arXiv 2609.13141). Section names below are that
page's headings.

What one decode step computes, per sequence b and KV head h, with the cached
tokens grouped into context units of `unit_size` consecutive positions:
  1. normalized softmax gates over the sequence's units: g = softmax(u), u being the
     selector's score per unit (section 2.2 (b));
  2. the decode-time selection: the units with the largest gates (argtop_k over g),
     the current unit always kept (sections 2.3 and 2.2 (b));
  3. attention of every query head over the tokens of the selected units, with the
     gate injected in log form into each logit: logit_j = q.k_j + lambda*log g_i for
     the unit i holding token j (section 2.1), then softmax and the weighted sum of V.

Readings taken where the page is silent (each is also listed in the design notes):
  * a unit is unit_size consecutive positions; unit i covers [i*unit_size,
    (i+1)*unit_size); a sequence of n tokens has ceil(n/unit_size) units, the last one
    possibly partial, and that last one (holding position n-1) is the current unit;
  * the budget k_units counts the current unit: the current unit plus the
    k_units - 1 other units with the largest gates (ties: lower unit index), or every
    unit when there are at most k_units;
  * the gates are normalized over the sequence's units (all of them, the current one
    included), and every selected unit, the current one included, gets its gate bias;
  * the dot product is scaled by sm_scale (1/sqrt(d) by default) as in the rest of the
    path, and the gate term is added after scaling: logit = sm_scale*q.k + lambda*ln g;
  * the selected tokens are listed in ascending position, padded with -1 to
    k_units*unit_size entries; n = 0 selects nothing and gives a zero output;
  * the gate scores u are fp32 values, finite or -inf; a score of -inf gives its unit
    the gate softmax assigns it, exactly 0, so its tokens get zero weight (ln g = -inf);
    each non-empty sequence has at least one finite score. lambda = 0 drops the gate
    term (lambda * ln g is taken as 0 even where g = 0). When every selected token of a
    query head has zero weight the output is zero, as for an empty selection.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32


def n_units(n: int, unit_size: int) -> int:
    """Units of a sequence of n tokens (the last one may be partial)."""
    return (int(n) + unit_size - 1) // unit_size


def log_gates(u_valid: np.ndarray) -> np.ndarray:
    """log g for g = softmax(u) over the sequence's units, in fp64 (section 2.2 (b))."""
    u = np.asarray(u_valid, dtype=np.float32).astype(np.float64)
    m = u.max()
    return (u - m) - np.log(np.exp(u - m).sum())


def select_units(u: np.ndarray, n: int, unit_size: int, k_units: int) -> np.ndarray:
    """Selected unit indices, ascending: the current unit plus the k_units - 1 others
    with the largest gates (section 2.3: argtop_k over g; 2.2 (b): the current unit is
    always kept). g = softmax(u) is strictly increasing in u, so ranking the fp32 u
    gives exactly the gates' order (ranking rounded fp64 gates could merge two
    distinct ones). Equal scores go to the lower unit index."""
    U = n_units(n, unit_size)
    if U == 0:
        return np.zeros(0, dtype=np.int64)
    if U <= k_units:
        return np.arange(U, dtype=np.int64)
    cur = U - 1
    others = np.asarray(u[:cur], dtype=np.float32)
    order = np.argsort(-others, kind="stable")          # stable: lower index first on ties
    chosen = np.concatenate([order[:k_units - 1], [cur]])
    return np.sort(chosen).astype(np.int64)


def unit_tokens(units: np.ndarray, n: int, unit_size: int, k_units: int) -> np.ndarray:
    """Token positions of the selected units, ascending, padded with -1 to
    k_units * unit_size entries; positions >= n (the partial current unit) are left out."""
    out = np.full(k_units * unit_size, -1, dtype=np.int32)
    toks = [np.arange(i * unit_size, min((i + 1) * unit_size, n)) for i in units]
    if toks:
        t = np.concatenate(toks)
        out[:t.size] = t
    return out


def attend_gated(q_heads_bits, K_bits, V_bits, idx, bias, sm_scale) -> np.ndarray:
    """Softmax attention of each query head over the selected tokens with an additive
    logit term per token (section 2.1): z_j = sm_scale * q_g.k_j + bias_j, all fp64.
    q_heads [G, d], K/V [n, d] bf16 bits, idx / bias per entry (-1 entries ignored)."""
    idx = np.asarray(idx)
    keep = idx >= 0
    sel = idx[keep]
    G, d = q_heads_bits.shape
    if sel.size == 0:
        return np.zeros((G, d), dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)[keep]
    qd = bf16_to_f32(q_heads_bits).astype(np.float64)
    Kd = bf16_to_f32(K_bits[sel]).astype(np.float64)
    Vd = bf16_to_f32(V_bits[sel]).astype(np.float64)
    scale = float(np.float32(sm_scale))
    out = np.empty((G, d), dtype=np.float64)
    for g in range(G):
        z = (Kd @ qd[g]) * scale + b
        if not np.isfinite(z.max()):              # every weight is zero (all gates 0)
            out[g] = 0.0
            continue
        z = z - z.max()
        p = np.exp(z)
        out[g] = (p / p.sum()) @ Vd
    return out


def gated_decode_unit(q_heads_bits, K_bits, V_bits, u, n, unit_size, k_units, lam, sm_scale):
    """One (sequence, KV head) of the gated step. u [>= ceil(n/unit_size)] fp32 gate
    scores. Returns (out fp64 [G, d], idx int32 [k_units*unit_size], selected units)."""
    U = n_units(n, unit_size)
    units = select_units(u, n, unit_size, k_units)
    idx = unit_tokens(units, n, unit_size, k_units)
    if U == 0:
        return np.zeros((q_heads_bits.shape[0], q_heads_bits.shape[1])), idx, units
    lg = log_gates(np.asarray(u[:U], dtype=np.float32))
    bias = np.zeros(idx.size, dtype=np.float64)
    valid = idx >= 0
    if float(np.float32(lam)) != 0.0:
        bias[valid] = float(np.float32(lam)) * lg[idx[valid] // unit_size]
    out = attend_gated(q_heads_bits, K_bits[:n], V_bits[:n], idx, bias, sm_scale)
    return out, idx, units
