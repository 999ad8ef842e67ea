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
