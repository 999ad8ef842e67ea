"""Parity at the full 128K batch-16 size, in the launch configuration the benchmark
times (B=16, 8 KV heads, G=4, n=131072, r=32, k=4096): the oracle checks every one
of the 128 (sequence, KV head) units (a thread pool over units), and every index list
is checked for the properties it must have."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_BF16, bits, check_unit, kproj_torch, say

pytestmark = pytest.mark.gpu


def _check_all_units(tag, out, idx, q, K, V, Kp, M, n, k, fmt="bf16", G=4):
    """check_unit on every unit; K, V, Kp host bit arrays [B, H, n, .]."""
    o = out.float().cpu().numpy()
    ix = idx.cpu().numpy()
    assert np.all(ix >= 0) and np.all(ix < n) and np.all(np.diff(ix, axis=-1) > 0)
    assert np.all(np.isfinite(o))
    B, H = ix.shape[:2]
    scale = jssa.default_sm_scale(128)

    def one(u):
        b, h = divmod(u, H)
        check_unit(o[b, h * G:(h + 1) * G], ix[b, h], q[b:b + 1, h * G:(h + 1) * G], K[b, h][None, None],
                   V[b, h][None, None], Kp[b, h][None, None], M[h:h + 1], 0, 0, G, n, k, scale, OUT_TOL_BF16,
                   tag=f"{tag} unit ({b},{h})", fmt=fmt)
        return u

    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        for i, _ in enumerate(ex.map(one, range(B * H))):
            if i % 32 == 31:
                say(f"{tag}: {i + 1} of {B * H} units match the oracle")


def test_long_batched_full_size():
    say("full size: generating B=16 n=131072 on the GPU")
    wl = workloads.long_batched(device="cuda")
    Kp = kproj_torch(wl.K, wl.M)
    say("full size: decode step")
    out, idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, wl.k)
    torch.cuda.synchronize()
    say("full size: copying the inputs to the host")
    q, K, V, P, M = bits(wl.q), bits(wl.K), bits(wl.V), bits(Kp), wl.M.cpu().numpy()
    _check_all_units("full size", out, idx, q, K, V, P, M, wl.capacity, wl.k)
    # every unit through the exact path (no scan workgroup takes what its prep
    # publishes): the four-workgroup recompute and dense selection give the same result
    say("full size: every unit on the exact path")
    shape = sj.make_shape(16, 8, 4, 128, 32, wl.capacity, fused_wait_us=-1)
    ws = sj.alloc_workspace(shape, wl.k)
    idx2 = torch.empty_like(idx)
    sj.prep_scan(shape, wl.q, wl.M, Kp, wl.seq_len, wl.k, ws)
    sj.select(shape, Kp, wl.seq_len, wl.k, ws, idx=idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx), "exact path differs from the candidate path"


def _cache_by_library_append(wl, fp8):
    """The projected cache built the way the benchmark builds it: the library's own
    append over every cached token (in chunks of 8192)."""
    B, H, n, r = wl.batch, wl.n_kv_heads, wl.capacity, wl.rank
    Kp = torch.empty(B, H, n, r, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    for t0 in range(0, n, 8192):
        pos = torch.full((B,), t0, dtype=torch.int32, device="cuda")
        sj.append_kv(wl.K[:, :, t0:t0 + 8192].contiguous(), wl.V[:, :, t0:t0 + 8192].contiguous(), wl.M, pos,
                     wl.K, wl.V, Kp)
    return Kp


@pytest.mark.parametrize("fp8", [False, True])
def test_long_batched_full_size_as_benchmarked(fp8):
    # the benchmark's step: the decode step whose first kernel appends the new token
    # (slot n-1), then scan, select, attend and merge, at B=16, n=131072, k=4096
    say(f"full size as benchmarked (fp8 cache: {fp8}): building the cache with the library's append")
    wl = workloads.long_batched(device="cuda")
    Kp = _cache_by_library_append(wl, fp8)
    k_new, v_new = workloads.new_token(wl, seed=99)
    n, k = wl.capacity, wl.k
    pos = torch.full((wl.batch,), n - 1, dtype=torch.int32, device="cuda")
    say("full size as benchmarked: fused append + decode step")
    out, idx = sj.decode_step_append(k_new, v_new, pos, wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, k)
    torch.cuda.synchronize()
    # the appended token's rows are in place
    assert torch.equal(wl.K[:, :, n - 1].view(torch.int16), k_new[:, :, 0].view(torch.int16))
    fmt = "fp8" if fp8 else "bf16"
    say("full size as benchmarked: copying the inputs to the host")
    q, K, V, M = bits(wl.q), bits(wl.K), bits(wl.V), wl.M.cpu().numpy()
    P = Kp.cpu().numpy() if fp8 else bits(Kp)
    _check_all_units(f"full size {fmt}", out, idx, q, K, V, P, M, n, k, fmt=fmt)
