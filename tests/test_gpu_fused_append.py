"""sjsa_decode_step_append (the prep kernel appends the new token) against
sjsa_append_kv followed by sjsa_decode_step: identical caches and results, bit
for bit, and oracle parity of the fused step itself."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_F32, bits, check_unit, say

pytestmark = pytest.mark.gpu


def _fill_kproj(wl):
    Kp = torch.zeros(wl.batch, wl.n_kv_heads, wl.capacity, wl.rank, dtype=torch.bfloat16, device="cuda")
    pos0 = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    sj.append_kv(wl.K, wl.V, wl.M, pos0, wl.K.clone(), wl.V.clone(), Kp)   # projection of every slot
    return Kp


@pytest.mark.parametrize("r,G,seq", [(32, 4, [3000, 1777]), (16, 1, [1500, 40]), (64, 8, [20000, 2048])])
def test_fused_equals_append_then_step(r, G, seq):
    say(f"fused append r={r} G={G} seq={seq}")
    cap = max(seq) + 8
    wl = workloads.gaussian(2, 2, G, 128, r, max(seq), 256, seed=40 + r + G, capacity=cap, device="cuda",
                            seq_len=seq)
    Kp = _fill_kproj(wl)
    k_new, v_new = workloads.new_token(wl, seed=41, T=1)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    pos = seq_len - 1                       # the new token is the last of each sequence
    results = []
    for fused in (False, True):
        K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
        if fused:
            out, idx = sj.decode_step_append(k_new, v_new, pos, wl.q, K, V, P, wl.M, seq_len, 256, out_f32=True)
        else:
            sj.append_kv(k_new, v_new, wl.M, pos, K, V, P)
            out, idx = sj.decode_step(wl.q, K, V, P, wl.M, seq_len, 256, out_f32=True)
        torch.cuda.synchronize()
        results.append([bits(K), bits(V), bits(P), out.cpu().numpy(), idx.cpu().numpy()])
    for a, b in zip(*results):
        assert np.array_equal(a, b)
    # and the fused step itself against the oracle
    K, V, P, out, idx = results[1]
    q = bits(wl.q)
    M = wl.M.cpu().numpy()
    for b in range(2):
        for h in range(2):
            check_unit(out[b, h * G:(h + 1) * G], idx[b, h], q, K, V, P, M, b, h, G, seq[b], 256,
                       jssa.default_sm_scale(128), OUT_TOL_F32, "fused")


def test_fused_slot_outside_capacity_writes_nothing():
    say("fused append, slot past capacity")
    wl = workloads.gaussian(2, 1, 4, 128, 32, 500, 64, seed=45, capacity=500, device="cuda")
    Kp = _fill_kproj(wl)
    k_new, v_new = workloads.new_token(wl, seed=46, T=1)
    pos = torch.tensor([500, -1], dtype=torch.int32, device="cuda")
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    seq_len = torch.tensor([500, 500], dtype=torch.int32, device="cuda")
    out, idx = sj.decode_step_append(k_new, v_new, pos, wl.q, K, V, P, wl.M, seq_len, 64)
    ref_out, ref_idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, seq_len, 64)
    torch.cuda.synchronize()
    assert np.array_equal(bits(K), bits(wl.K)) and np.array_equal(bits(V), bits(wl.V))
    assert np.array_equal(bits(P), bits(Kp))
    assert np.array_equal(idx.cpu().numpy(), ref_idx.cpu().numpy())
    assert np.array_equal(bits(out), bits(ref_out))
