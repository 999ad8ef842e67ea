"""Pins of the gated-logit (SAS) oracle against closed forms, an independent
library softmax and brute force."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import jssa, sas
from oracle.numerics import bf16_to_f32, round_to_bf16


def _bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float64))


def _rand_unit(rng, n, G=4, d=16):
    q = _bf16(rng.standard_normal((G, d)))
    K = _bf16(rng.standard_normal((n, d)))
    V = _bf16(rng.standard_normal((n, d)))
    return q, K, V


def test_log_gates_are_the_log_of_scipy_softmax():
    rng = np.random.default_rng(0)
    u = (rng.integers(-256, 256, size=37) / 64.0).astype(np.float32)     # u + 1000 stays exact in fp32
    lg = sas.log_gates(u)
    ref = scipy.special.softmax(u.astype(np.float64))
    assert np.allclose(np.exp(lg), ref, rtol=1e-13, atol=0)
    assert abs(np.exp(lg).sum() - 1.0) < 1e-13
    # large scores do not overflow
    lg2 = sas.log_gates(u + np.float32(1000.0))
    assert np.allclose(lg2, lg, atol=1e-12)


def _brute_units(u, U, k_units):
    """Among the subsets of size k_units - 1 of the non-current units, the one with
    the largest gate sum; ties broken by the lexicographically smallest index tuple."""
    g = scipy.special.softmax(np.asarray(u[:U], dtype=np.float64))
    best, best_key = None, None
    for c in itertools.combinations(range(U - 1), k_units - 1):
        key = (-sum(sorted(g[list(c)])), c)     # sum in a fixed order: equal sets tie exactly
        if best_key is None or key < best_key:
            best, best_key = c, key
    return sorted(list(best) + [U - 1])


@pytest.mark.parametrize("seed", range(6))
def test_unit_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    unit = 4
    for U in range(1, 9):
        n = (U - 1) * unit + int(rng.integers(1, unit + 1))
        u = rng.integers(-2, 3, size=U).astype(np.float32)      # many exact ties
        for k_units in range(1, 10):
            got = sas.select_units(u, n, unit, k_units)
            if U <= k_units:
                assert list(got) == list(range(U))
            else:
                assert list(got) == _brute_units(u, U, k_units), (U, k_units, u)


def test_current_unit_is_kept_with_the_smallest_gate():
    u = np.array([5, 4, 3, 2, 1, -50], dtype=np.float32)
    got = sas.select_units(u, 6 * 8 - 3, 8, 3)
    assert list(got) == [0, 1, 5]


def test_gate_shift_leaves_selection_and_output_unchanged():
    rng = np.random.default_rng(1)
    n, unit = 200, 16
    q, K, V = _rand_unit(rng, n)
    u = (rng.integers(-256, 256, size=sas.n_units(n, unit)) / 64.0).astype(np.float32)   # exact shift
    a = sas.gated_decode_unit(q, K, V, u, n, unit, 5, 1.0, 0.25)
    b = sas.gated_decode_unit(q, K, V, u + np.float32(3.0), n, unit, 5, 1.0, 0.25)
    assert np.array_equal(a[1], b[1])
    assert np.max(np.abs(a[0] - b[0])) < 1e-12


def test_token_expansion_and_partial_current_unit():
    units = np.array([0, 3, 6])
    idx = sas.unit_tokens(units, 6 * 10 + 4, 10, 4)
    assert list(idx[:10]) == list(range(10))
    assert list(idx[10:20]) == list(range(30, 40))
    assert list(idx[20:24]) == [60, 61, 62, 63]
    assert np.all(idx[24:] == -1) and idx.size == 40


def test_lambda_zero_is_plain_attention_over_the_units():
    rng = np.random.default_rng(2)
    n, unit = 300, 32
    q, K, V = _rand_unit(rng, n)
    u = rng.standard_normal(sas.n_units(n, unit)).astype(np.float32)
    out, idx, units = sas.gated_decode_unit(q, K, V, u, n, unit, 4, 0.0, 0.3)
    ref = jssa.attend(q, K, V, idx, 0.3)
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("lam", [1.0, 2.0, 0.5])
def test_log_gate_equals_multiplicative_gate(lam):
    # softmax(z + lam*ln g) = g^lam e^z / sum g^lam e^z: the product form, written without logs
    rng = np.random.default_rng(3)
    n, unit = 257, 16
    q, K, V = _rand_unit(rng, n)
    U = sas.n_units(n, unit)
    u = rng.standard_normal(U).astype(np.float32)
    out, idx, units = sas.gated_decode_unit(q, K, V, u, n, unit, 6, lam, 0.2)
    g = scipy.special.softmax(u.astype(np.float64))
    sel = idx[idx >= 0]
    w_gate = g[sel // unit] ** lam
    qf = bf16_to_f32(q).astype(np.float64)
    Kf = bf16_to_f32(K[sel]).astype(np.float64)
    Vf = bf16_to_f32(V[sel]).astype(np.float64)
    for h in range(q.shape[0]):
        e = np.exp((Kf @ qf[h]) * float(np.float32(0.2)))
        w = w_gate * e
        ref = (w[:, None] * Vf).sum(0) / w.sum()
        assert np.max(np.abs(out[h] - ref)) < 1e-12


def test_zero_keys_weight_units_by_their_gates():
    # q.k = 0 everywhere: each token of unit i weighs g_i^lam
    rng = np.random.default_rng(4)
    n, unit, lam = 100, 10, 1.5
    q, _, V = _rand_unit(rng, n)
    K = np.zeros_like(V)
    u = rng.standard_normal(10).astype(np.float32)
    out, idx, units = sas.gated_decode_unit(q, K, V, u, n, unit, 4, lam, 0.1)
    g = scipy.special.softmax(u.astype(np.float64))
    Vf = bf16_to_f32(V).astype(np.float64)
    num = sum(g[i] ** lam * Vf[i * unit:(i + 1) * unit].sum(0) for i in units)
    den = sum(g[i] ** lam * unit for i in units)
    for h in range(q.shape[0]):
        assert np.max(np.abs(out[h] - num / den)) < 1e-12


def test_empty_and_short_sequences():
    rng = np.random.default_rng(5)
    q, K, V = _rand_unit(rng, 64)
    u = rng.standard_normal(8).astype(np.float32)
    out, idx, units = sas.gated_decode_unit(q, K, V, u, 0, 8, 3, 1.0, 0.25)
    assert units.size == 0 and np.all(idx == -1) and np.all(out == 0)
    out, idx, units = sas.gated_decode_unit(q, K, V, u, 13, 8, 3, 1.0, 0.25)   # 2 units <= budget
    assert list(units) == [0, 1] and list(idx[:13]) == list(range(13)) and np.all(idx[13:] == -1)
    # a single token: the output is its V row
    out, idx, units = sas.gated_decode_unit(q, K, V, u, 1, 8, 3, 1.0, 0.25)
    assert np.max(np.abs(out - bf16_to_f32(V[0]).astype(np.float64)[None])) < 1e-15


def test_minus_inf_score_is_a_zero_gate():
    # softmax gives a score of -inf the gate 0, so that unit's tokens carry no weight:
    # the output equals the attention over the other selected units' tokens alone (with
    # lambda = 1 their log gates differ from renormalized ones by one common constant,
    # which the softmax cancels). The current unit is kept even with a zero gate.
    rng = np.random.default_rng(7)
    n, unit, k_units = 200, 16, 5
    q, K, V = _rand_unit(rng, n)
    U = sas.n_units(n, unit)
    u = rng.standard_normal(U).astype(np.float32)
    u[[0, 3, U - 1]] = -np.inf                      # a kept unit, a dropped one, the current one
    u[1] = np.float32(5.0)                          # unit 1 is surely kept
    out, idx, units = sas.gated_decode_unit(q, K, V, u, n, unit, k_units, 1.0, 0.25)
    assert U - 1 in units and 1 in units and 3 not in units
    live = [int(i) for i in units if np.isfinite(u[i])]
    toks = np.concatenate([np.arange(i * unit, min((i + 1) * unit, n)) for i in live])
    lg = np.log(scipy.special.softmax(u[live].astype(np.float64)))
    bias = np.repeat(lg, [min((i + 1) * unit, n) - i * unit for i in live])
    ref = sas.attend_gated(q, K, V, toks, bias, 0.25)
    assert np.all(np.isfinite(out)) and np.max(np.abs(out - ref)) < 1e-12
    # lambda = 0 drops the gate term: plain attention over every selected token
    out0, idx0, _ = sas.gated_decode_unit(q, K, V, u, n, unit, k_units, 0.0, 0.25)
    assert np.max(np.abs(out0 - jssa.attend(q, K, V, idx0, 0.25))) < 1e-12
    # every selected unit with gate 0 (only the current unit kept): zero output
    u2 = np.full(U, -np.inf, dtype=np.float32)
    u2[0] = 1.0
    out2, idx2, units2 = sas.gated_decode_unit(q, K, V, u2, n, unit, 1, 1.0, 0.25)
    assert list(units2) == [U - 1] and np.all(out2 == 0.0)
