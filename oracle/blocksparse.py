"""CPU oracle for the block-sparse decode step (NSA-style block selection with a
parameter-free block key, and an INT4 selector cache).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the benchmark's
cpu_baseline leg may import anything under oracle/. Nothing here is shared with
the HIP path.

Sources:
  * the NSA tutorial page, "稀疏注意力:每个 query 只挑一部分历史去读"
    (learn-llm.fim.ai): a block's summary key is visible only once the block is
    complete; the selection score of a block is softmax(q . summary_key /
    sqrt(head_size)) over the visible blocks, the query heads that share a K/V head
    add their scores and select together; the current block is always selected,
    and the paper's 16 selected blocks always include the first block and the two
    local blocks;
  * the SpotAttention abstract page ("SpotAttention: Plug-In Block-Sparse Routing
    for Pretrained Long-Context Transformers", paperdaily.cn): the selector's key
    cache can be held in INT4 at no accuracy cost.

What one decode step computes per sequence b and KV head h, blocks being
block_size consecutive positions (block j covers [j*bs, (j+1)*bs)):
  1. block keys kc_j for the complete blocks (j < floor(n/bs));
  2. per query head g: p_g = softmax_j(sm_scale * q_g . kc_j) over the complete
     blocks; the block score is s_j = sum_g p_g,j;
  3. the kept blocks: the forced ones (the first n_init blocks and the n_local
     blocks ending with the current block, which holds position n-1) plus the
     largest-score complete blocks until k_blocks are kept (ties: lower block);
     every block when there are at most k_blocks;
  4. exact softmax attention of every query head over the kept blocks' positions.

Readings taken where the pages are silent (each is also listed in the design notes):
  * the summary key: the pages learn a compression MLP (or a Linear with block
    position terms); with no trained weights here, the block key is the mean of
    the block's keys, computed exactly and rounded once to bf16;
  * the softmax runs over every complete block (forced ones included), without the
    learnable sink slot the tutorial adds to its compression branch;
  * the current block is forced (the tutorial gives it a score of 1e4); with
    n_local = 2 the two local blocks are the current block and the one before it;
  * the kept blocks' positions are listed ascending, padded with -1 to
    k_blocks * block_size entries; the attention is the selection branch alone
    (no compression or sliding-window branch, no branch gates);
  * INT4 selector cache: symmetric, one scale per group of 64 consecutive elements
    of a block key; scale = fp16(fp32(absmax) / 7) (fp32 division, then round to
    nearest even into binary16, saturating at 65504); code = clamp(rint(fp32(x /
    scale)), -7, 7) with an fp32 division, 0 when the scale is 0; the stored key
    value is code * scale. The quantized value is the bf16 block key.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32, fp16_to_f32, round_to_bf16, round_to_fp16

INT4_GROUP = 64
INT4_MAX = 7


def complete_blocks(n: int, block: int) -> int:
    return int(n) // block


def total_blocks(n: int, block: int) -> int:
    return (int(n) + block - 1) // block


def block_keys(K_bits: np.ndarray, n: int, block: int) -> np.ndarray:
    """Keys of the complete blocks: bf16 of the exact mean of each block's keys.
    K_bits [>= n, d] bf16 bits -> [floor(n/block), d] bf16 bits."""
    m = complete_blocks(n, block)
    if m == 0:
        return np.zeros((0, K_bits.shape[1]), dtype=np.uint16)
    k = bf16_to_f32(K_bits[:m * block]).astype(np.float64).reshape(m, block, -1)
    # the fp64 sum is exact while the block mixes magnitudes less than 2^44 apart
    return round_to_bf16(k.sum(axis=1) / block)


def int4_quantize(kc_bits: np.ndarray):
    """INT4 selector cache of bf16 block keys [m, d]: codes int8 [m, d] in -7..7 and
    fp16 scale bits [m, d/64] (see the module's reading)."""
    x = bf16_to_f32(kc_bits).astype(np.float32)
    m, d = x.shape
    g = x.reshape(m, d // INT4_GROUP, INT4_GROUP)
    absmax = np.abs(g).max(axis=2)
    s32 = (absmax / np.float32(INT4_MAX)).astype(np.float32)
    s16 = round_to_fp16(np.minimum(s32.astype(np.float64), 65504.0))
    scale = fp16_to_f32(s16)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / scale[:, :, None]).astype(np.float32)
    codes = np.where(scale[:, :, None] > 0, np.clip(np.rint(ratio), -INT4_MAX, INT4_MAX), 0.0)
    return codes.reshape(m, d).astype(np.int8), s16


def int4_dequantize(codes: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    m, d = codes.shape
    s = fp16_to_f32(scales_bits).astype(np.float32)
    v = codes.astype(np.float32).reshape(m, d // INT4_GROUP, INT4_GROUP) * s[:, :, None]
    return v.reshape(m, d)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement codes per byte: element 2i in the low nibble,
    element 2i+1 in the high nibble. [m, d] int8 -> [m, d/2] uint8."""
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def block_scores(q_heads_bits: np.ndarray, kc: np.ndarray, sm_scale: float) -> np.ndarray:
    """s_j = sum_g softmax_j(sm_scale * q_g . kc_j) over the given complete blocks
    (kc fp32 values [m, d]); fp64 throughout."""
    m = kc.shape[0]
    if m == 0:
        return np.zeros(0, dtype=np.float64)
    q = bf16_to_f32(q_heads_bits).astype(np.float64)
    z = (q @ kc.astype(np.float64).T) * float(np.float32(sm_scale))      # [G, m]
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def forced_blocks(n: int, block: int, n_init: int, n_local: int) -> np.ndarray:
    nb = total_blocks(n, block)
    if nb == 0:
        return np.zeros(0, dtype=np.int64)
    cur = nb - 1
    f = set(range(min(n_init, nb))) | set(range(max(cur - n_local + 1, 0), cur + 1))
    return np.array(sorted(f), dtype=np.int64)


def select_blocks(s: np.ndarray, n: int, block: int, k_blocks: int, n_init: int, n_local: int) -> np.ndarray:
    """Kept blocks, ascending: the forced ones, then complete blocks by descending
    score (ties: lower block) until k_blocks are kept; all blocks if there are at
    most k_blocks."""
    assert n_init + n_local <= k_blocks, "the forced blocks must fit the budget"
    nb = total_blocks(n, block)
    if nb <= k_blocks:
        return np.arange(nb, dtype=np.int64)
    forced = forced_blocks(n, block, n_init, n_local)
    room = max(k_blocks - forced.size, 0)
    m = complete_blocks(n, block)
    eligible = np.setdiff1d(np.arange(m), forced)
    order = eligible[np.argsort(-np.asarray(s, dtype=np.float64)[eligible], kind="stable")]
    return np.sort(np.concatenate([forced, order[:room]])).astype(np.int64)


def block_tokens(blocks: np.ndarray, n: int, block: int, k_blocks: int) -> np.ndarray:
    out = np.full(k_blocks * block, -1, dtype=np.int32)
    toks = [np.arange(j * block, min((j + 1) * block, n)) for j in blocks]
    if toks:
        t = np.concatenate(toks)
        out[:t.size] = t
    return out


def decode_unit(q_heads_bits, K_bits, V_bits, kc_values, n, block, k_blocks, n_init, n_local, sm_scale):
    """One (sequence, KV head). kc_values: fp32 values of the stored block keys
    [>= floor(n/block), d] (bf16 decoded, or INT4 dequantized). Returns (out fp64
    [G, d], idx int32 [k_blocks*block], kept blocks, block scores)."""
    from .jssa import attend
    m = complete_blocks(n, block)
    s = block_scores(q_heads_bits, kc_values[:m], sm_scale)
    blocks = select_blocks(s, n, block, k_blocks, n_init, n_local)
    idx = block_tokens(blocks, n, block, k_blocks)
    out = attend(q_heads_bits, K_bits[:n], V_bits[:n], idx, sm_scale)
    return out, idx, blocks, s
