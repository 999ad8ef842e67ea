"""End-to-end pins for the oracle's decode step and append."""
import numpy as np
import torch

import workloads
from oracle import jssa
from oracle.numerics import bf16_to_f32, round_to_bf16
from tests import golden_toy
from tests.util import bits


def test_golden_toy_hand_worked():
    g = golden_toy.load()
    qh = round_to_bf16(np.array(g["q_heads"], dtype=np.float64))
    K = round_to_bf16(np.array(g["K"], dtype=np.float64))
    V = round_to_bf16(np.array(g["V"], dtype=np.float64))
    M = np.array(g["M"], dtype=np.float32)
    kproj = jssa.project_keys(K, M)
    assert np.array_equal(bf16_to_f32(kproj), np.array(g["kproj"], dtype=np.float32))
    q_hat = jssa.project_query(jssa.mean_query(qh), M)
    s = jssa.score_positions(q_hat, kproj)
    assert np.array_equal(s, np.array(g["scores"], dtype=np.float32))
    for c in g["cases"]:
        out, idx, _ = jssa.decode_unit(qh, K, V, kproj, M, 5, c["k"], g["sm_scale"])
        assert list(idx) == c["idx"]
        if c["out"] is not None:
            assert np.max(np.abs(out - c["out"])) < 1e-15


def test_golden_toy_padded_to_d128():
    g = golden_toy.load()
    q, K, V, M = golden_toy.padded(g)
    kproj = jssa.project_keys(K, M)
    for c in g["cases"]:
        out, idx, _ = jssa.decode_unit(q, K, V, kproj, M, 5, c["k"], g["sm_scale"])
        assert list(idx) == c["idx"]
        if c["out"] is not None:
            assert np.max(np.abs(out[:, :4] - c["out"])) < 1e-15
            assert np.all(out[:, 4:] == 0)


def _dense(q_heads, K, V, scale):
    G, d = q_heads.shape
    n = K.shape[0]
    q = torch.from_numpy(bf16_to_f32(q_heads).astype(np.float64))[None, :, None, :]
    k = torch.from_numpy(bf16_to_f32(K).astype(np.float64))[None, None].expand(1, G, n, d)
    v = torch.from_numpy(bf16_to_f32(V).astype(np.float64))[None, None].expand(1, G, n, d)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0].numpy()


def test_budget_covering_context_is_dense_attention():
    wl = workloads.gaussian(2, 2, 4, 128, 16, 300, 300, seed=11, seq_len=[300, 123])
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.numpy()
    kproj = np.stack([np.stack([jssa.project_keys(K[b, h], M[h]) for h in range(2)]) for b in range(2)])
    for k in (300, 1000):
        out, idx = jssa.decode_step(q, K, V, kproj, M, wl.seq_len.numpy(), k)
        for b, n in ((0, 300), (1, 123)):
            for h in range(2):
                assert list(idx[b, h, :n]) == list(range(n)) and np.all(idx[b, h, n:] == -1)
                ref = _dense(q[b, 4 * h:4 * h + 4], K[b, h, :n], V[b, h, :n], jssa.default_sm_scale(128))
                assert np.max(np.abs(out[b, 4 * h:4 * h + 4] - ref)) < 1e-12


def test_full_rank_identity_basis_selects_exact_mean_query_topk():
    wl = workloads.gaussian(1, 2, 4, 128, 128, 2000, 100, seed=12, with_basis=False)
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = np.stack([np.eye(128, dtype=np.float32)] * 2)
    kproj = np.stack([np.stack([jssa.project_keys(K[0, h], M[h]) for h in range(2)])])
    _, idx = jssa.decode_step(q, K, V, kproj, M, [2000], 100)
    for h in range(2):
        qb = bf16_to_f32(q[0, 4 * h:4 * h + 4]).astype(np.float64).mean(axis=0)
        s = bf16_to_f32(K[0, h]).astype(np.float64) @ qb
        want = np.sort(np.argsort(-s, kind="stable")[:100])
        assert np.array_equal(idx[0, h], want)


def test_empty_sequence_gives_zero_output():
    wl = workloads.gaussian(2, 1, 4, 128, 16, 64, 8, seed=13, seq_len=[0, 64])
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.numpy()
    kproj = np.stack([np.stack([jssa.project_keys(K[b, 0], M[0])]) for b in range(2)])
    out, idx = jssa.decode_step(q, K, V, kproj, M, wl.seq_len.numpy(), 8)
    assert np.all(idx[0] == -1) and np.all(out[0] == 0)
    assert np.all(idx[1] >= 0)


def test_append_rows():
    wl = workloads.gaussian(2, 2, 4, 128, 32, 10, 4, seed=14, capacity=16)
    K, V = bits(wl.K).copy(), bits(wl.V).copy()
    kproj = np.zeros((2, 2, 16, 32), dtype=np.uint16)
    k_new, v_new = workloads.new_token(wl, seed=15, T=3)
    kn, vn = bits(k_new), bits(v_new)
    M = wl.M.numpy()
    jssa.append_rows(kn, vn, M, [10, 14], K, V, kproj)
    for h in range(2):
        assert np.array_equal(K[0, h, 10:13], kn[0, h]) and np.array_equal(V[0, h, 10:13], vn[0, h])
        assert np.array_equal(kproj[0, h, 10:13], jssa.project_keys(kn[0, h], M[h]))
        assert np.array_equal(K[1, h, 14:16], kn[1, h, :2])       # third row falls off the end
        assert np.all(kproj[1, h, :14] == 0)
