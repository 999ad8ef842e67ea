"""The allocation-free decode step (sjsa_decode_step_append_noalloc, the library's
static scratch array in place of a workspace) against sjsa_decode_step_append with a
caller workspace: identical index lists, outputs and appended caches, over two calls
in a row (the second with a smaller shape, so it runs on what the first left in the
array), then the first shape again; one unit of each call against the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_BF16, OUT_TOL_F32, bits, check_unit, say

pytestmark = pytest.mark.gpu


def _case(B, Hkv, G, r, cap, seq, k, seed, out_f32):
    wl = workloads.gaussian(B, Hkv, G, 128, r, max(seq), k, seed=seed, capacity=cap, device="cuda", seq_len=seq)
    Kp = torch.zeros(B, Hkv, cap, r, dtype=torch.bfloat16, device="cuda")
    sj.append_kv(wl.K, wl.V, wl.M, torch.zeros(B, dtype=torch.int32, device="cuda"), wl.K.clone(), wl.V.clone(), Kp)
    k_new, v_new = workloads.new_token(wl, seed=seed + 1, T=1)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    pos = seq_len - 1
    return wl, Kp, k_new, v_new, pos, seq_len


def _run(case, k, out_f32, noalloc):
    wl, Kp, k_new, v_new, pos, seq_len = case
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    out = torch.empty(wl.q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    idx = torch.empty(wl.batch, wl.n_kv_heads, k, dtype=torch.int32, device="cuda")
    if noalloc:
        sj.decode_step_append_noalloc(k_new, v_new, pos, wl.q, K, V, P, wl.M, seq_len, k, out, idx, out_f32=out_f32)
    else:
        sj.decode_step_append(k_new, v_new, pos, wl.q, K, V, P, wl.M, seq_len, k, out=out, idx=idx, out_f32=out_f32)
    torch.cuda.synchronize()
    return K, V, P, idx, out


def _same(a, b, tag):
    for name, x, y in zip(("K", "V", "Kproj", "idx", "out"), a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y), f"{tag}: {name} differs"


def _oracle_unit(case, res, k, seq, out_f32, b, h, tag):
    wl = case[0]
    K, V, P, idx, out = res
    G = wl.group
    check_unit(out.float().cpu().numpy()[b, h * G:(h + 1) * G], idx.cpu().numpy()[b, h], bits(wl.q), bits(K),
               bits(V), bits(P), wl.M.cpu().numpy(), b, h, G, seq[b], k, jssa.default_sm_scale(128),
               OUT_TOL_F32 if out_f32 else OUT_TOL_BF16, tag)


def test_noalloc_step_equals_workspace_step_on_two_calls():
    big = dict(B=2, Hkv=4, G=4, r=32, cap=32768, seq=[32768, 20001], k=1024, seed=140, out_f32=False)
    small = dict(B=1, Hkv=2, G=2, r=16, cap=9000, seq=[8999], k=300, seed=150, out_f32=True)
    cases = {}
    for name, c in (("big", big), ("small", small), ("big again", big)):
        tag = f"noalloc {name}"
        say(tag, {kk: v for kk, v in c.items() if kk != "seq"})
        if name not in cases:
            cases[name] = _case(c["B"], c["Hkv"], c["G"], c["r"], c["cap"], c["seq"], c["k"], c["seed"],
                                c["out_f32"])
        case = cases[name if name in cases else "big"]
        got = _run(case, c["k"], c["out_f32"], True)
        ref = _run(case, c["k"], c["out_f32"], False)
        _same(ref, got, tag)
        _oracle_unit(case, got, c["k"], c["seq"], c["out_f32"], c["B"] - 1, c["Hkv"] - 1, tag)
        ix = got[3].cpu().numpy()
        assert np.all((ix >= -1) & (ix < c["cap"]))
