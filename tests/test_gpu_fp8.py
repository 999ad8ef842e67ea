"""GPU parity of the FP8 (E4M3, one byte per element) scoring cache: the append
kernel's projected bytes against the oracle's projection in that format, and the
decode step over an FP8 cache against the oracle's decode in that format."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from oracle.numerics import fp8e4m3_to_f32, round_to_fp8e4m3
from tests.gpu_helpers import OUT_TOL_BF16, OUT_TOL_F32, bits, check_unit, kproj_close_fp8, kproj_oracle, say

pytestmark = pytest.mark.gpu


def _kp_cuda(kp_bytes: np.ndarray, as_float8: bool = False) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(kp_bytes)).cuda()
    return t.view(torch.float8_e4m3fn) if as_float8 else t


def _check_step(wl, kp, k, out_f32=True, tag="", as_float8=False):
    out, idx = sj.decode_step(wl.q, wl.K, wl.V, _kp_cuda(kp, as_float8), wl.M, wl.seq_len, k, out_f32=out_f32)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ix = idx.cpu().numpy()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.cpu().numpy()
    G = wl.group
    for b in range(wl.batch):
        n = min(max(int(wl.seq_len[b]), 0), wl.capacity)
        for h in range(wl.n_kv_heads):
            check_unit(o[b, h * G:(h + 1) * G], ix[b, h], q, K, V, kp, M, b, h, G, n, k,
                       jssa.default_sm_scale(128), OUT_TOL_F32 if out_f32 else OUT_TOL_BF16, tag, fmt="fp8")
    return o, ix


@pytest.mark.parametrize("r", [16, 32, 64])
def test_fp8_append_projection(r):
    say(f"fp8 append r={r}")
    B, H, cap, T = 2, 3, 300, 130
    wl = workloads.gaussian(B, H, 1, 128, r, 10, 4, seed=300 + r, capacity=cap, device="cuda")
    K = torch.zeros(B, H, cap, 128, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    Kp = torch.full((B, H, cap, r), 0x55, dtype=torch.uint8, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=6, T=T)
    pos = torch.tensor([5, 250], dtype=torch.int32, device="cuda")     # second one runs past cap
    sj.append_kv(k_new, v_new, wl.M, pos, K, V, Kp)
    torch.cuda.synchronize()
    Pb = Kp.cpu().numpy()
    kn = bits(k_new)
    M = wl.M.cpu().numpy()
    written = np.zeros_like(Pb, dtype=bool)
    written[0, :, 5:5 + T] = True
    written[1, :, 250:cap] = True
    assert np.all(Pb[~written] == 0x55)
    for b, (lo, hi) in ((0, (5, 5 + T)), (1, (250, cap))):
        for h in range(H):
            ref = jssa.project_keys(kn[b, h, :hi - lo], M[h], "fp8")
            ok, exact = kproj_close_fp8(Pb[b, h, lo:hi], ref, kn[b, h, :hi - lo], M[h])
            assert ok and exact >= 0.999, (b, h, exact)


def test_fp8_append_saturates_like_the_oracle():
    say("fp8 append saturation")
    B, H, cap, T = 1, 2, 128, 128
    wl = workloads.gaussian(B, H, 1, 128, 32, 10, 4, seed=310, capacity=cap, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=7, T=T)
    k_new = (k_new.float() * 300.0).to(torch.bfloat16)    # many projections exceed 448
    K = torch.zeros(B, H, cap, 128, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    Kp = torch.zeros(B, H, cap, 32, dtype=torch.float8_e4m3fn, device="cuda")
    sj.append_kv(k_new, v_new, wl.M, torch.zeros(1, dtype=torch.int32, device="cuda"), K, V, Kp)
    torch.cuda.synchronize()
    Pb = Kp.view(torch.uint8).cpu().numpy()
    kn = bits(k_new)
    M = wl.M.cpu().numpy()
    for h in range(H):
        ref = jssa.project_keys(kn[0, h], M[h], "fp8")
        sat = np.abs(fp8e4m3_to_f32(ref)) == 448.0
        assert sat.mean() > 0.05
        ok, exact = kproj_close_fp8(Pb[0, h], ref, kn[0, h], M[h])
        assert ok and exact >= 0.999
        assert not np.any((Pb[0, h] & 0x7F) == 0x7F)                  # never a NaN code
        assert np.mean(Pb[0, h][sat] == ref[sat]) >= 0.999


def test_fp8_single_token_equals_bulk_append():
    say("fp8 append single vs bulk")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 64, 8, seed=311, capacity=64, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=8, T=16)
    outs = []
    for mode in ("bulk", "single"):
        K = torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
        V = torch.zeros_like(K)
        Kp = torch.zeros(2, 2, 64, 32, dtype=torch.uint8, device="cuda")
        if mode == "bulk":
            sj.append_kv(k_new, v_new, wl.M, torch.tensor([3, 40], dtype=torch.int32, device="cuda"), K, V, Kp)
        else:
            for t in range(16):
                sj.append_kv(k_new[:, :, t:t + 1].contiguous(), v_new[:, :, t:t + 1].contiguous(), wl.M,
                             torch.tensor([3 + t, 40 + t], dtype=torch.int32, device="cuda"), K, V, Kp)
        torch.cuda.synchronize()
        outs.append(Kp.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("r,G", [(16, 1), (32, 4), (64, 8)])
def test_fp8_step_ragged(r, G):
    say(f"fp8 step ragged r={r} G={G}")
    seq = [7000, 1, 0, 4099, 6999]
    wl = workloads.gaussian(5, 2, G, 128, r, 7000, 300, seed=320 + r + G, device="cuda", seq_len=seq,
                            capacity=7003)
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy(), "fp8")
    for k in (300, 1, 7000):
        _check_step(wl, kp, k, tag=f"fp8 ragged r{r} G{G} k{k}", as_float8=(k == 1))


def test_fp8_sequence_past_one_gather_chunk():
    # 150,001 rows: more 4096-row scan tiles per unit than the selection gathers in one
    # round trip (32), so its second chunk runs
    say("fp8 step: sequences past one selection gather chunk")
    seq = [150001, 140000]
    wl = workloads.gaussian(2, 1, 4, 128, 32, 150001, 1024, seed=333, device="cuda", seq_len=seq, capacity=150001)
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy(), "fp8")
    _check_step(wl, kp, 1024, tag="fp8 two gather chunks")


def test_fp8_step_llama8b_layer():
    say("fp8 step llama8b-shaped layer n=32768 k=2048")
    wl = workloads.llama8b_layer(device="cuda")
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy(), "fp8")
    _check_step(wl, kp, wl.k, out_f32=False, tag="fp8 llama8b")


def _ties_check_fp8(wl, kp, k, tag):
    o, ix = _check_step(wl, kp, k, tag=tag)
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.cpu().numpy()
    G = wl.group
    for b in range(wl.batch):
        n = int(wl.seq_len[b])
        for h in range(wl.n_kv_heads):
            _, ref_idx, _ = jssa.decode_unit(q[b, G * h:G * h + G], K[b, h], V[b, h], kp[b, h], M[h], n, k,
                                             jssa.default_sm_scale(128), "fp8")
            assert np.array_equal(ix[b, h], ref_idx), (tag, b, h)


def test_fp8_candidate_overflow_falls_back_exactly():
    # identical projected rows: every score ties, 40000 candidates, dense fallback
    say("fp8 step candidate overflow -> exact fallback")
    wl = workloads.gaussian(1, 2, 4, 128, 16, 40000, 1500, seed=330, device="cuda")
    kp = kproj_oracle(bits(wl.K[:, :, :1].contiguous()), wl.M.cpu().numpy(), "fp8")
    kp = np.ascontiguousarray(np.repeat(kp, 40000, axis=2))
    _ties_check_fp8(wl, kp, 1500, "fp8 overflow")


def test_fp8_scan_stage_overflow_falls_back_exactly():
    # one scan tile of high rows, the rest low (see the bf16 test of the same name)
    say("fp8 step scan stage overflow -> exact fallback")
    n, k = 40000, 1500
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, k, seed=331, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    low = jssa.project_keys(bits(wl.K[0, 0, :1].contiguous()), M[0], "fp8")[0]
    high = round_to_fp8e4m3(np.sign(qhat) * 4.0)
    kp = np.tile(low, (1, 1, n, 1)).astype(np.uint8)
    kp[0, 0, :4096] = high
    _ties_check_fp8(wl, kp, k, "fp8 stage overflow")


def test_fp8_fused_equals_append_then_step():
    say("fp8 fused append")
    seq = [3000, 1777]
    cap = max(seq) + 8
    wl = workloads.gaussian(2, 2, 4, 128, 32, max(seq), 256, seed=340, capacity=cap, device="cuda", seq_len=seq)
    M = wl.M.cpu().numpy()
    Kp = _kp_cuda(kproj_oracle(bits(wl.K), M, "fp8"))
    k_new, v_new = workloads.new_token(wl, seed=341, T=1)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    pos = seq_len - 1
    results = []
    for fused in (False, True):
        K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
        if fused:
            out, idx = sj.decode_step_append(k_new, v_new, pos, wl.q, K, V, P, wl.M, seq_len, 256, out_f32=True)
        else:
            sj.append_kv(k_new, v_new, wl.M, pos, K, V, P)
            out, idx = sj.decode_step(wl.q, K, V, P, wl.M, seq_len, 256, out_f32=True)
        torch.cuda.synchronize()
        results.append([bits(K), bits(V), P.cpu().numpy(), out.cpu().numpy(), idx.cpu().numpy()])
    for a, b in zip(*results):
        assert np.array_equal(a, b)
    K, V, P, out, idx = results[1]
    q = bits(wl.q)
    for b in range(2):
        for h in range(2):
            check_unit(out[b, h * 4:(h + 1) * 4], idx[b, h], q, K, V, P, M, b, h, 4, seq[b], 256,
                       jssa.default_sm_scale(128), OUT_TOL_F32, "fp8 fused", fmt="fp8")


def test_fp8_kproj_dtype_must_match_flags():
    say("fp8 dtype/flag mismatch rejected")
    wl = workloads.gaussian(1, 1, 4, 128, 32, 100, 8, seed=350, device="cuda")
    shape = sj.shape_of(wl.q, wl.K, wl.M)                  # bf16 flags
    ws = sj.alloc_workspace(shape, 8)
    Kp8 = torch.zeros(1, 1, wl.capacity, 32, dtype=torch.uint8, device="cuda")
    with pytest.raises(TypeError):
        sj.select(shape, Kp8, wl.seq_len, 8, ws)
