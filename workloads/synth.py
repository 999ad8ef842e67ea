"""Seeded synthetic inputs for one sparse-decode step.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no projection, no scoring, no selection, no attention and
no calibration. Both sides of every parity check (the HIP path and the CPU
oracle) receive the tensors built here.

Shapes follow the GQA decode workloads of the JSSA article ("JSSA 完全拆解:
联合 query-key 子空间打分与 gather-free 内核"): 32 query heads over 8 KV heads,
head dim 128, scoring rank 32, budgets of a few thousand tokens and 128K
contexts (section "投影打分缓存与校准成本" and the experiment setup). The pages
measure on model activations and public suites; none of those are available,
so seeded Gaussian tensors with the structure below stand in for them.

Layouts (all row-major, contiguous):
    q      [B, H_q, d]        bf16, H_q = H_kv * G; query head h_q maps to KV head h_q // G
    K, V   [B, H_kv, cap, d]  bf16
    M      [H_kv, r, d]       fp32, orthonormal rows
    seq_len[B]                int32
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

ROPE_BASE = 500000.0


@dataclass
class Workload:
    name: str
    batch: int
    n_kv_heads: int
    group: int
    head_dim: int
    rank: int
    capacity: int
    k: int
    seq_len: torch.Tensor            # [B] int32 (on the workload's device)
    q: torch.Tensor                  # [B, H_q, d] bf16
    K: torch.Tensor                  # [B, H_kv, cap, d] bf16
    V: torch.Tensor                  # [B, H_kv, cap, d] bf16
    M: Optional[torch.Tensor]        # [H_kv, r, d] fp32 (None until calibrated)
    sm_scale: float = 0.0            # 0 selects 1/sqrt(d)
    calib_q: Optional[torch.Tensor] = None   # [N, G, d] fp32 calibration query heads
    calib_k: Optional[torch.Tensor] = None   # [N, d] fp32 calibration keys
    extra: dict = field(default_factory=dict)

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def random_orthonormal(n_kv_heads: int, rank: int, head_dim: int, seed: int) -> torch.Tensor:
    """One random orthonormal r x d basis per KV head: the transposed Q factor of
    QR(N(0,1)^{d x r}), computed in fp64 on the host and stored as fp32."""
    g = _gen(seed, "cpu")
    out = torch.empty(n_kv_heads, rank, head_dim, dtype=torch.float64)
    for h in range(n_kv_heads):
        a = torch.randn(head_dim, rank, generator=g, dtype=torch.float64)
        qf, _ = torch.linalg.qr(a)
        out[h] = qf.T
    return out.to(torch.float32)


def rope_tables(positions: torch.Tensor, head_dim: int, base: float = ROPE_BASE):
    """cos/sin tables [len(positions), d/2] for rotate-half RoPE, computed in fp64."""
    half = head_dim // 2
    inv_freq = base ** (-torch.arange(0, half, dtype=torch.float64, device=positions.device) * 2.0 / head_dim)
    ang = positions.to(torch.float64)[:, None] * inv_freq[None, :]
    return torch.cos(ang), torch.sin(ang)


def apply_rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotate-half RoPE on the last dim of x (fp32); cos/sin broadcast over leading dims."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c = cos.to(x.dtype)
    s = sin.to(x.dtype)
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def gaussian(batch, n_kv_heads, group, head_dim, rank, n, k, *, seed, device="cpu",
             capacity=None, seq_len=None, with_basis=True, name="gaussian") -> Workload:
    """Plain N(0,1) q, K, V (bf16) with a random orthonormal basis. Used for edge cases:
    ragged seq_len per sequence, capacity above n, odd n."""
    cap = int(capacity if capacity is not None else n)
    g = _gen(seed, device)
    hq = n_kv_heads * group
    q = torch.randn(batch, hq, head_dim, generator=g, device=device).to(torch.bfloat16)
    K = torch.randn(batch, n_kv_heads, cap, head_dim, generator=g, device=device).to(torch.bfloat16)
    V = torch.randn(batch, n_kv_heads, cap, head_dim, generator=g, device=device).to(torch.bfloat16)
    if seq_len is None:
        seq_len = [n] * batch
    sl = torch.tensor(seq_len, dtype=torch.int32, device=device)
    M = random_orthonormal(n_kv_heads, rank, head_dim, seed + 7919).to(device) if with_basis else None
    return Workload(name, batch, n_kv_heads, group, head_dim, rank, cap, k, sl, q, K, V, M)


def tiny_single_head(seed: int = 1, device="cpu", n_calib: int = 512) -> Workload:
    """Tiny single-head step: B=1, one KV head, G=4, d=128, n=4096, r=16, k=256.

    q, K, V ~ N(0,1); 4 seeded key channels scaled by 8; 32 seeded positions whose
    keys are replaced by ||k_j|| * (0.6*u + 0.8*w), u the unit mean query direction
    and w a random unit vector orthogonal to u (cosine 0.6 with the mean query before
    bf16 rounding). The basis M is left to the caller's calibration over the
    n_calib seeded (query heads, key) samples returned in calib_q / calib_k, which
    follow the same law (query heads N(0,1); keys with the same outlier channels).
    """
    B, H, G, d, n, r, k = 1, 1, 4, 128, 4096, 16, 256
    g = _gen(seed, "cpu")
    q = torch.randn(B, H * G, d, generator=g).to(torch.bfloat16)
    Kf = torch.randn(B, H, n, d, generator=g)
    V = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    outlier_ch = torch.randperm(d, generator=g)[:4]
    Kf[..., outlier_ch] *= 8.0
    planted = torch.randperm(n, generator=g)[:32].sort().values
    # Direction of the group's mean query; only used to place the planted keys.
    u = q[0].to(torch.float64).mean(dim=0)
    u = u / u.norm()
    for j in planted.tolist():
        w = torch.randn(d, generator=g, dtype=torch.float64)
        w = w - (w @ u) * u
        w = w / w.norm()
        norm = Kf[0, 0, j].to(torch.float64).norm()
        Kf[0, 0, j] = (norm * (0.6 * u + 0.8 * w)).to(torch.float32)
    K = Kf.to(torch.bfloat16)
    calib_q = torch.randn(n_calib, G, d, generator=g)
    calib_k = torch.randn(n_calib, d, generator=g)
    calib_k[:, outlier_ch] *= 8.0
    wl = Workload("tiny-single-head-n4096-r16-k256", B, H, G, d, r, n, k,
                  torch.tensor([n], dtype=torch.int32), q, K, V, None,
                  calib_q=calib_q, calib_k=calib_k,
                  extra={"planted": planted, "outlier_channels": outlier_ch})
    return wl.to(device) if device != "cpu" else wl


def rope_gqa(batch, n_kv_heads, group, n, rank, k, *, seed, device="cpu", heavy_frac=0.0,
             head_dim=128, capacity=None, name="rope-gqa", n_q_sets=1, quiet=None) -> Workload:
    """LLaMA-3.1-8B-shaped decode layer: K, V ~ N(0,1) bf16 with rotate-half RoPE
    (base 500000, no frequency scaling) applied to K at positions 0..n-1 and to q at
    position n-1; a random orthonormal basis per KV head. With heavy_frac > 0, a
    seeded round(heavy_frac*n) positions per (b, h) get their key scaled by 4 (norm x4,
    V unchanged). n_q_sets > 1 draws that many independent query sets, stacked as
    extra["q_sets"] [n_q_sets, B, H_q, d]; q is the first. quiet = (period, rows, scale)
    scales the keys at positions p with p % period < rows by `scale` (after RoPE and
    the heavy hitters; a power of two keeps the bf16 values exact).

    K and V are drawn one sequence at a time on `device`, so the fp32 staging stays
    at one sequence's size.
    """
    cap = int(capacity if capacity is not None else n)
    d = head_dim
    g = _gen(seed, device)
    hq = n_kv_heads * group
    pos = torch.arange(n, device=device)
    cos, sin = rope_tables(pos, d)
    qcos, qsin = rope_tables(torch.tensor([n - 1], device=device), d)
    q_sets = []
    for _ in range(n_q_sets):
        qs = torch.randn(batch, hq, d, generator=g, device=device)
        q_sets.append(apply_rope(qs, qcos, qsin).to(torch.bfloat16))
    K = torch.empty(batch, n_kv_heads, cap, d, dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    n_heavy = int(round(heavy_frac * n))
    heavy = []
    for b in range(batch):
        kb = torch.randn(n_kv_heads, n, d, generator=g, device=device)
        kb = apply_rope(kb, cos, sin)
        hb = []
        if n_heavy > 0:
            for h in range(n_kv_heads):
                sel = torch.randperm(n, generator=g, device=device)[:n_heavy]
                kb[h, sel] *= 4.0
                hb.append(sel)
        if quiet is not None:
            period, rows, scale = quiet
            kb[:, (pos % period) < rows] *= scale
        K[b, :, :n] = kb.to(torch.bfloat16)
        del kb
        V[b, :, :n] = torch.randn(n_kv_heads, n, d, generator=g, device=device).to(torch.bfloat16)
        if cap > n:
            K[b, :, n:] = 0
            V[b, :, n:] = 0
        heavy.append(hb)
    M = random_orthonormal(n_kv_heads, rank, d, seed + 7919).to(device)
    sl = torch.full((batch,), n, dtype=torch.int32, device=device)
    extra = {"heavy": heavy}
    if n_q_sets > 1:
        extra["q_sets"] = torch.stack(q_sets)
    return Workload(name, batch, n_kv_heads, group, d, rank, cap, k, sl, q_sets[0], K, V, M,
                    extra=extra)


def llama8b_layer(seed: int = 2, device="cpu") -> Workload:
    """B=1, 32/8 heads (G=4), d=128, n=32768, r=32, k=2048, RoPE keys."""
    return rope_gqa(1, 8, 4, 32768, 32, 2048, seed=seed, device=device,
                    name="llama8b-layer-b1-n32768-r32-k2048")


def long_batched(seed: int = 3, device="cpu", n_q_sets: int = 1, batch: int = 16,
                 n: int = 131072) -> Workload:
    """B=16, 32/8 heads, d=128, n=131072, r=32, k=4096, RoPE keys plus 1% heavy hitters."""
    return rope_gqa(batch, 8, 4, n, 32, 4096, seed=seed, device=device, heavy_frac=0.01,
                    name=f"long-batched-b{batch}-n{n}-r32-k4096", n_q_sets=n_q_sets)


def long_batched_blind_spot(seed: int = 13, device="cpu", batch: int = 16, n: int = 131072,
                            k: int = 4096) -> Workload:
    """long_batched with the keys at positions p % (n/1024) < 2 scaled by 1/16 (n a
    multiple of 1024): the rows an evenly spaced sampler of 1024 adjacent pairs reads
    are the quietest of the sequence, so such a sample places any score threshold far
    below the true k-th score. The top-k lies entirely where the sample does not look."""
    return rope_gqa(batch, 8, 4, n, 32, k, seed=seed, device=device, heavy_frac=0.01,
                    name=f"long-batched-blind-spot-b{batch}-n{n}-r32-k{k}", quiet=(n // 1024, 2, 1.0 / 16.0))


def gated(batch, n_kv_heads, group, n, unit_size, k_units, *, seed, device="cpu", capacity=None,
          seq_len=None, name="gated-units") -> Workload:
    """Gated-logit (SAS-style) decode layer: K, V and q as in rope_gqa, plus one gate
    score per context unit of unit_size tokens, u ~ N(0,1) fp32, stored as
    extra["gate_scores"] [B, H_kv, ceil(cap/unit_size)]. seq_len (a list) makes the
    batch ragged; rows past a sequence's length are zero."""
    wl = rope_gqa(batch, n_kv_heads, group, n, 16, k_units * unit_size, seed=seed, device=device,
                  capacity=capacity, name=name)
    g = _gen(seed + 104729, device)
    n_u = (wl.capacity + unit_size - 1) // unit_size
    wl.extra["gate_scores"] = torch.randn(batch, n_kv_heads, n_u, generator=g, device=device)
    wl.extra["unit_size"] = unit_size
    wl.extra["k_units"] = k_units
    wl.M = None
    if seq_len is not None:
        wl.seq_len = torch.tensor(seq_len, dtype=torch.int32, device=device)
        for b, nb in enumerate(seq_len):
            wl.K[b, :, max(nb, 0):] = 0
            wl.V[b, :, max(nb, 0):] = 0
    return wl


def gated_config(seed: int = 4, device="cpu") -> Workload:
    """B=1, 32/8 heads (G=4), d=128, n=32768 in 512 units of 64 tokens, budget 32 units."""
    return gated(1, 8, 4, 32768, 64, 32, seed=seed, device=device, name="gated-b1-n32768-u64-k32")


def blocks(batch, n_kv_heads, group, n, block_size, k_blocks, *, seed, device="cpu", capacity=None,
           seq_len=None, name="block-sparse") -> Workload:
    """Block-sparse decode layer: K, V and q as in rope_gqa (no scoring basis);
    extra["block_size"], extra["k_blocks"]. seq_len (a list) makes the batch ragged;
    rows past a sequence's length are zero."""
    wl = rope_gqa(batch, n_kv_heads, group, n, 16, k_blocks * block_size, seed=seed, device=device,
                  capacity=capacity, name=name)
    wl.M = None
    wl.extra["block_size"] = block_size
    wl.extra["k_blocks"] = k_blocks
    if seq_len is not None:
        wl.seq_len = torch.tensor(seq_len, dtype=torch.int32, device=device)
        for b, nb in enumerate(seq_len):
            wl.K[b, :, max(nb, 0):] = 0
            wl.V[b, :, max(nb, 0):] = 0
    return wl


def block_config(seed: int = 5, device="cpu") -> Workload:
    """B=4, 64/8 heads (G=8), d=128, n=65536 in 1024 blocks of 64, 16 blocks kept."""
    return blocks(4, 8, 8, 65536, 64, 16, seed=seed, device=device, name="blocks-b4-g8-n65536-bs64-k16")


def new_token(wl: Workload, seed: int, T: int = 1):
    """k_new, v_new [B, H_kv, T, d] bf16 for an append of T tokens."""
    dev = wl.q.device
    g = _gen(seed, dev)
    shape = (wl.batch, wl.n_kv_heads, T, wl.head_dim)
    k_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    return k_new, v_new


def _to(self: Workload, device) -> Workload:
    def mv(t):
        return t.to(device) if isinstance(t, torch.Tensor) else t
    extra = {k: mv(v) for k, v in self.extra.items()}
    return Workload(self.name, self.batch, self.n_kv_heads, self.group, self.head_dim, self.rank,
                    self.capacity, self.k, mv(self.seq_len), mv(self.q), mv(self.K), mv(self.V),
                    mv(self.M), self.sm_scale, mv(self.calib_q), mv(self.calib_k), extra)


Workload.to = _to

