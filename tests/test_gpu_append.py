"""GPU parity of sjsa_append_kv against the oracle's key projection."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from oracle.numerics import bf16_to_f32
from tests.gpu_helpers import bits, kproj_close, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("r", [16, 32, 64])
def test_append_rows_and_projection(r):
    say(f"append r={r}")
    B, H, cap, T = 2, 3, 300, 130
    wl = workloads.gaussian(B, H, 1, 128, r, 10, 4, seed=100 + r, capacity=cap, device="cuda")
    K = torch.full((B, H, cap, 128), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    V = K.clone()
    Kp = torch.full((B, H, cap, r), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    k_new, v_new = workloads.new_token(wl, seed=5, T=T)
    pos = torch.tensor([5, 250], dtype=torch.int32, device="cuda")     # second one runs past cap
    sj.append_kv(k_new, v_new, wl.M, pos, K, V, Kp)
    torch.cuda.synchronize()
    Kb, Vb, Pb = bits(K), bits(V), bits(Kp)
    kn, vn = bits(k_new), bits(v_new)
    M = wl.M.cpu().numpy()
    exp_K = np.full_like(Kb, 7)
    exp_V = np.full_like(Vb, 7)
    exp_P = np.full_like(Pb, 7)
    jssa.append_rows(kn, vn, M, [5, 250], exp_K, exp_V, exp_P)
    assert np.array_equal(Kb, exp_K) and np.array_equal(Vb, exp_V)
    # projected rows: fp32 dot on the GPU vs one rounding of the fp64 dot in the oracle
    written = np.zeros_like(Pb, dtype=bool)
    written[0, :, 5:5 + T] = True
    written[1, :, 250:cap] = True
    assert np.all(Pb[~written] == 7)
    for b, (lo, hi) in ((0, (5, 5 + T)), (1, (250, cap))):
        for h in range(H):
            ok, exact = kproj_close(Pb[b, h, lo:hi], exp_P[b, h, lo:hi], Kb[b, h, lo:hi], M[h])
            assert ok and exact >= 0.999, (b, h, exact)
    # a value-level check: the projected values are the dot products
    pv = bf16_to_f32(Pb[0, 0, 5:5 + T]).astype(np.float64)
    ref = bf16_to_f32(kn[0, 0]).astype(np.float64) @ M[0].astype(np.float64).T
    assert np.max(np.abs(pv - ref) / (np.abs(ref) + 1e-3)) < 2 ** -7


def test_single_token_append_bulk_equivalence():
    say("append single vs bulk")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 64, 8, seed=7, capacity=64, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=8, T=16)
    outs = []
    for mode in ("bulk", "single"):
        K = torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
        V = torch.zeros_like(K)
        Kp = torch.zeros(2, 2, 64, 32, dtype=torch.bfloat16, device="cuda")
        if mode == "bulk":
            sj.append_kv(k_new, v_new, wl.M, torch.tensor([3, 40], dtype=torch.int32, device="cuda"), K, V, Kp)
        else:
            for t in range(16):
                sj.append_kv(k_new[:, :, t:t + 1].contiguous(), v_new[:, :, t:t + 1].contiguous(), wl.M,
                             torch.tensor([3 + t, 40 + t], dtype=torch.int32, device="cuda"), K, V, Kp)
        torch.cuda.synchronize()
        outs.append((bits(K), bits(V), bits(Kp)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
