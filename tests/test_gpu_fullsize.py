"""Parity at the full 128K batch-16 size, in the launch configuration the benchmark
times (B=16, 8 KV heads, G=4, n=131072, r=32, k=4096). The oracle checks a seeded
sample of (sequence, KV head) units one by one; the rest are checked for the
properties every index list must have."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_BF16, bits, check_unit, kproj_torch, say

pytestmark = pytest.mark.gpu


def test_long_batched_full_size():
    say("full size: generating B=16 n=131072 on the GPU")
    wl = workloads.long_batched(device="cuda")
    Kp = kproj_torch(wl.K, wl.M)
    say("full size: decode step")
    out, idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, wl.k)
    torch.cuda.synchronize()
    ix = idx.cpu().numpy()
    n, k = wl.capacity, wl.k
    # every unit: k distinct ascending positions in [0, n)
    assert np.all(ix >= 0) and np.all(ix < n)
    assert np.all(np.diff(ix, axis=-1) > 0)
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(0)
    units = [(0, 0), (15, 7)] + [(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 6), rng.integers(0, 8, 6))]
    q = bits(wl.q)
    M = wl.M.cpu().numpy()
    scale = jssa.default_sm_scale(128)
    for b, h in units:
        say(f"full size: oracle on unit ({b},{h})")
        Kb = bits(wl.K[b, h])[None, None]
        Vb = bits(wl.V[b, h])[None, None]
        Pb = bits(Kp[b, h])[None, None]
        qb = q[b:b + 1, h * 4:(h + 1) * 4]
        check_unit(o[b, h * 4:(h + 1) * 4], ix[b, h], qb, Kb, Vb, Pb, M[h:h + 1], 0, 0, 4, n, k, scale,
                   OUT_TOL_BF16, tag="full size")


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
    ix = idx.cpu().numpy()
    assert np.all(ix >= 0) and np.all(ix < n) and np.all(np.diff(ix, axis=-1) > 0)
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    # the appended token's rows are in place
    assert torch.equal(wl.K[:, :, n - 1].view(torch.int16), k_new[:, :, 0].view(torch.int16))
    rng = np.random.default_rng(1)
    units = [(0, 0), (15, 7)] + [(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 4), rng.integers(0, 8, 4))]
    q = bits(wl.q)
    M = wl.M.cpu().numpy()
    scale = jssa.default_sm_scale(128)
    fmt = "fp8" if fp8 else "bf16"
    for b, h in units:
        say(f"full size as benchmarked: oracle on unit ({b},{h})")
        Kb = bits(wl.K[b, h])[None, None]
        Vb = bits(wl.V[b, h])[None, None]
        Pb = (Kp[b, h].cpu().numpy() if fp8 else bits(Kp[b, h]))[None, None]
        qb = q[b:b + 1, h * 4:(h + 1) * 4]
        check_unit(o[b, h * 4:(h + 1) * 4], ix[b, h], qb, Kb, Vb, Pb, M[h:h + 1], 0, 0, 4, n, k, scale,
                   OUT_TOL_BF16, tag=f"full size {fmt}", fmt=fmt)
