"""GPU gather-free attention (sjsa_attend) against the oracle's exact attention over
the same index sets: every group size, split counts from 1 to many, -1 padding,
out-of-range and duplicate entries, bf16 and fp32 outputs."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_BF16, OUT_TOL_F32, bits, say

pytestmark = pytest.mark.gpu


def _ref(q, K, V, idx, seq_len, G, scale):
    B, Hq, d = q.shape
    H = K.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = min(max(int(seq_len[b]), 0), K.shape[2])
        for h in range(H):
            sel = idx[b, h]
            sel = sel[(sel >= 0) & (sel < n)]
            out[b, h * G:(h + 1) * G] = jssa.attend(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], sel, scale)
    return out


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [1, 63, 64, 65, 1000, 4096])
def test_attend_matches_oracle(G, k):
    say(f"attend G={G} k={k}")
    B, H, n = 2, 2, 5000
    wl = workloads.gaussian(B, H, G, 128, 16, n, k, seed=G * 1000 + k, device="cuda", seq_len=[n, 4321])
    rng = np.random.default_rng(k)
    idx = np.stack([np.stack([np.sort(rng.choice(n, size=min(k, n), replace=False)) for _ in range(H)])
                    for _ in range(B)]).astype(np.int32)
    idx_t = torch.from_numpy(idx).cuda()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    scale = jssa.default_sm_scale(128)
    ref = _ref(q, K, V, idx, wl.seq_len.cpu().numpy(), G, scale)
    for out_f32, tol in ((True, OUT_TOL_F32), (False, OUT_TOL_BF16)):
        out = sj.attend(wl.q, wl.K, wl.V, idx_t, wl.seq_len, out_f32=out_f32)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        err = np.max(np.abs(got - ref))
        assert err <= tol, (out_f32, err)


def test_attend_padding_duplicates_out_of_range_and_scale():
    say("attend padding/duplicates")
    B, H, G, n = 2, 1, 4, 300
    wl = workloads.gaussian(B, H, G, 128, 16, n, 64, seed=9, device="cuda", seq_len=[300, 0])
    idx = np.full((B, H, 200), -1, dtype=np.int32)
    idx[0, 0, :50] = np.arange(0, 100, 2)
    idx[0, 0, 50:60] = 10                     # duplicates count as often as they appear
    idx[0, 0, 60:70] = 5000                   # beyond n: skipped
    idx[1, 0, :20] = np.arange(20)            # sequence 1 is empty: everything skipped
    idx_t = torch.from_numpy(idx).cuda()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    for scale in (0.0, 0.37):
        s = scale if scale else jssa.default_sm_scale(128)
        ref = _ref(q, K, V, idx, [300, 0], G, s)
        out = sj.attend(wl.q, wl.K, wl.V, idx_t, wl.seq_len, sm_scale=scale, out_f32=True)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.max(np.abs(got - ref)) <= OUT_TOL_F32
        assert np.all(got[1] == 0)


def test_single_selected_row_reproduces_v():
    say("attend k=1 -> V row")
    wl = workloads.gaussian(1, 2, 4, 128, 16, 100, 1, seed=10, device="cuda")
    idx_t = torch.tensor([[[17], [93]]], dtype=torch.int32, device="cuda")
    out = sj.attend(wl.q, wl.K, wl.V, idx_t, wl.seq_len)
    torch.cuda.synchronize()
    o = bits(out)
    V = bits(wl.V)
    for g in range(4):
        assert np.array_equal(o[0, g], V[0, 0, 17])
        assert np.array_equal(o[0, 4 + g], V[0, 1, 93])


@pytest.mark.parametrize("G", [2, 4])
def test_attend_interleaved_invalid_entries_and_growing_logits(G):
    # invalid entries (-1, other negatives, positions at or past n) sit between valid
    # ones inside every batch of rows, and the query is scaled up so that later rows
    # raise the softmax reference again and again (the rescale path)
    say(f"attend interleaved invalid entries G={G}")
    B, H, n, k = 1, 2, 3000, 700
    wl = workloads.gaussian(B, H, G, 128, 16, n, k, seed=31, device="cuda")
    rng = np.random.default_rng(32)
    idx = rng.integers(0, n, size=(B, H, k)).astype(np.int32)
    idx[..., 1::3] = -1
    idx[..., 2::7] = -7
    idx[..., 5::11] = n + rng.integers(0, 50)
    idx[0, 0, :] = np.sort(idx[0, 0, :])            # ascending, as the selection writes them
    q = wl.q.float() * 2.0
    wl.q.copy_(q.to(torch.bfloat16))
    # unit (0, 0): the K rows grow with the position, so its logits keep rising along
    # the (ascending) list; unit (0, 1) walks its rows in random order
    Kf = wl.K.float()
    Kf[0, 0] *= torch.linspace(0.5, 4.0, n, device="cuda")[:, None]
    wl.K.copy_(Kf.to(torch.bfloat16))
    idx_t = torch.from_numpy(idx).cuda()
    qb, Kb, Vb = bits(wl.q), bits(wl.K), bits(wl.V)
    s = jssa.default_sm_scale(128)
    ref = _ref(qb, Kb, Vb, idx, [n], G, s)
    out = sj.attend(wl.q, wl.K, wl.V, idx_t, wl.seq_len, out_f32=True)
    torch.cuda.synchronize()
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= OUT_TOL_F32


@pytest.mark.parametrize("G,k", [(4, 4096), (2, 20000)])
def test_split_attention_on_an_uninitialised_workspace(G, k):
    # the workspace needs no initialisation: one of random bytes, used by several calls
    # in a row, gives the oracle's output every time (the splits' partials and their
    # merge go through it), and the calls agree bit for bit
    say(f"attend on a random workspace G={G} k={k}")
    B, H, n = 2, 2, 30000
    wl = workloads.gaussian(B, H, G, 128, 16, n, k, seed=G + k, device="cuda", seq_len=[n, 25001])
    rng = np.random.default_rng(G + k)
    idx = np.stack([np.stack([np.sort(rng.choice(n, size=k, replace=False)) for _ in range(H)])
                    for _ in range(B)]).astype(np.int32)
    idx_t = torch.from_numpy(idx).cuda()
    shape = sj.make_shape(B, H, G, 128, 16, n)
    ws = sj.alloc_workspace(shape, k)
    ws.copy_(torch.from_numpy(rng.integers(0, 256, ws.numel(), dtype=np.uint8)).cuda())
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    ref = _ref(q, K, V, idx, wl.seq_len.cpu().numpy(), G, jssa.default_sm_scale(128))
    first = None
    for call in range(3):
        out = sj.attend(wl.q, wl.K, wl.V, idx_t, wl.seq_len, out_f32=True, workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - ref)) <= OUT_TOL_F32, call
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out, first), call
