"""Pins for the oracle's exact attention over a selected set.

With the full set selected the step reduces to dense softmax attention, checked
against torch's scaled_dot_product_attention in fp64; the other cases have closed
forms (one row, constant rows, equal logits)."""
import numpy as np
import torch

from oracle import jssa
from oracle.numerics import bf16_to_f32, round_to_bf16


def _bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float64))


def test_full_set_equals_dense_sdpa():
    rng = np.random.default_rng(0)
    G, d, n = 4, 128, 700
    qh, K, V = _bf16(rng.standard_normal((G, d))), _bf16(rng.standard_normal((n, d))), _bf16(rng.standard_normal((n, d)))
    scale = jssa.default_sm_scale(d)
    out = jssa.attend(qh, K, V, np.arange(n), scale)
    q = torch.from_numpy(bf16_to_f32(qh).astype(np.float64))[None, :, None, :]       # [1, G, 1, d]
    k = torch.from_numpy(bf16_to_f32(K).astype(np.float64))[None, None].expand(1, G, n, d)
    v = torch.from_numpy(bf16_to_f32(V).astype(np.float64))[None, None].expand(1, G, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_single_row_constant_rows_equal_logits():
    rng = np.random.default_rng(1)
    G, d, n = 4, 128, 64
    qh, K, V = _bf16(rng.standard_normal((G, d))), _bf16(rng.standard_normal((n, d))), _bf16(rng.standard_normal((n, d)))
    out = jssa.attend(qh, K, V, np.array([17, -1, -1]), 0.1)
    assert np.array_equal(out, np.tile(bf16_to_f32(V[17]).astype(np.float64), (G, 1)))
    Vc = np.tile(V[3], (n, 1))
    out = jssa.attend(qh, K, Vc, np.arange(0, n, 3), 0.1)
    assert np.max(np.abs(out - bf16_to_f32(V[3]))) < 1e-12
    zq = _bf16(np.zeros((G, d)))
    sel = np.array([2, 9, 33, 60])
    out = jssa.attend(zq, K, V, sel, 0.1)
    assert np.max(np.abs(out - bf16_to_f32(V[sel]).astype(np.float64).mean(axis=0))) < 1e-12


def test_set_semantics_and_empty_set():
    rng = np.random.default_rng(2)
    G, d, n = 2, 128, 50
    qh, K, V = _bf16(rng.standard_normal((G, d))), _bf16(rng.standard_normal((n, d))), _bf16(rng.standard_normal((n, d)))
    a = jssa.attend(qh, K, V, np.array([4, 8, 15, 16, 23, 42]), 0.2)
    b = jssa.attend(qh, K, V, np.array([42, -1, 23, 16, 15, 8, 4, -1]), 0.2)
    assert np.max(np.abs(a - b)) < 1e-14
    assert np.array_equal(jssa.attend(qh, K, V, np.array([-1, -1]), 0.2), np.zeros((G, d)))
