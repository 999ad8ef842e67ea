"""GPU parity of the block-sparse path: block keys (bf16 and INT4) against the
oracle, incremental appends against a bulk build, and the decode step's kept
blocks and output against the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import blocksparse as bs
from oracle import jssa
from oracle.numerics import bf16_to_f32
from tests.gpu_helpers import OUT_TOL_BF16, OUT_TOL_F32, bits, say

pytestmark = pytest.mark.gpu


def _keys(wl, bsz, int4=False):
    Kc, Kq, Ks = sj.block_cache(wl.K, bsz, int4=int4)
    sj.block_keys(wl.K, wl.seq_len, bsz, Kc, Kq, Ks)
    torch.cuda.synchronize()
    return Kc, Kq, Ks


def _np_u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def test_block_keys_bf16_and_int4():
    say("block keys: bf16 mean keys and their INT4 form")
    wl = workloads.blocks(2, 2, 4, 5000, 64, 8, seed=80, device="cuda", seq_len=[5000, 1000], capacity=5000)
    Kc, Kq, Ks = _keys(wl, 64, int4=True)
    K = bits(wl.K)
    kc = bits(Kc)
    for b, n in ((0, 5000), (1, 1000)):
        m = n // 64
        for h in range(2):
            ref = bs.block_keys(K[b, h], n, 64)
            # the GPU sums in fp32, the oracle rounds the exact mean once: one bf16 ulp
            # plus the fp32 summation bound apart at most, identical almost always
            exact = float(np.mean(kc[b, h, :m] == ref))
            g = bf16_to_f32(kc[b, h, :m]).astype(np.float64)
            r = bf16_to_f32(ref).astype(np.float64)
            kf = np.abs(bf16_to_f32(K[b, h, :m * 64]).astype(np.float64)).reshape(m, 64, 128).sum(axis=1) / 64
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(g), np.abs(r)), 2.0 ** -126))) - 7)
            assert np.all(np.abs(g - r) <= ulp + kf * 64 * 2.0 ** -24), (b, h)
            assert exact >= 0.999, (b, h, exact)
            assert np.all(kc[b, h, m:] == 0)                    # incomplete and unused blocks untouched
            # INT4: the oracle's quantization of the GPU's own bf16 keys, bit for bit
            codes, scales = bs.int4_quantize(kc[b, h, :m])
            assert np.array_equal(Kq[b, h, :m].cpu().numpy(), bs.pack_int4(codes)), (b, h)
            assert np.array_equal(_np_u16(Ks[b, h, :m]), scales), (b, h)


def test_block_append_matches_bulk_build():
    say("block append: token by token and in chunks equals the bulk build")
    wl = workloads.blocks(2, 2, 4, 700, 32, 8, seed=81, device="cuda", capacity=704)
    Kc0, Kq0, Ks0 = _keys(wl, 32, int4=True)
    K = torch.zeros_like(wl.K)
    V = torch.zeros_like(wl.V)
    Kc, Kq, Ks = sj.block_cache(wl.K, 32, int4=True)
    t = 0
    for step in [1, 1, 30, 1, 64, 100, 3, 200, 300]:          # sums to 700
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        sj.block_append(wl.K[:, :, t:t + step].contiguous(), wl.V[:, :, t:t + step].contiguous(), pos, K, V, 32,
                        Kc, Kq, Ks)
        t += step
    torch.cuda.synchronize()
    assert torch.equal(K.view(torch.int16), wl.K.view(torch.int16))
    assert torch.equal(Kc.view(torch.int16), Kc0.view(torch.int16))
    assert torch.equal(Kq, Kq0) and torch.equal(Ks.view(torch.int16), Ks0.view(torch.int16))


def _check_step(wl, bsz, k_blocks, keys, n_init=1, n_local=2, out_f32=True, tag="", int4=False, exact_sets=False):
    Kc, Kq, Ks = keys
    if int4:
        out, idx = sj.block_decode_step(wl.q, wl.K, wl.V, wl.seq_len, bsz, k_blocks, None, Kq, Ks, n_init, n_local,
                                        out_f32=out_f32)
    else:
        out, idx = sj.block_decode_step(wl.q, wl.K, wl.V, wl.seq_len, bsz, k_blocks, Kc, None, None, n_init, n_local,
                                        out_f32=out_f32)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ix = idx.cpu().numpy()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    G = wl.group
    scale = jssa.default_sm_scale(128)
    tol = OUT_TOL_F32 if out_f32 else OUT_TOL_BF16
    for b in range(wl.batch):
        n = min(max(int(wl.seq_len[b]), 0), wl.capacity)
        for h in range(wl.n_kv_heads):
            m = n // bsz
            if int4:
                kcv = bs.int4_dequantize(bs.unpack_int4(Kq[b, h, :m].cpu().numpy()), _np_u16(Ks[b, h, :m]))
            else:
                kcv = bf16_to_f32(bits(Kc[b, h, :m]))
            qh = q[b, h * G:(h + 1) * G]
            ref_out, ref_idx, ref_blocks, s = bs.decode_unit(qh, K[b, h], V[b, h], kcv, n, bsz, k_blocks, n_init,
                                                             n_local, scale)
            gi = ix[b, h]
            # positions: whole kept blocks, ascending, -1 padded
            valid = gi[gi >= 0]
            assert np.all(np.diff(valid) > 0) and np.all(gi[valid.size:] == -1), (tag, b, h)
            got_blocks = np.unique(valid // bsz)
            assert np.array_equal(bs.block_tokens(got_blocks, n, bsz, k_blocks), gi), (tag, b, h)
            # kept blocks: identical, or differing only inside the score band at the boundary
            if not np.array_equal(got_blocks, ref_blocks):
                assert not exact_sets, (tag, b, h, got_blocks, ref_blocks)
                assert got_blocks.size == ref_blocks.size
                forced = bs.forced_blocks(n, bsz, n_init, n_local)
                assert np.all(np.isin(forced, got_blocks))
                chosen = np.setdiff1d(ref_blocks, forced)
                T = s[chosen].min()
                diff = np.setxor1d(got_blocks, ref_blocks)
                assert np.all(np.abs(s[diff] - T) <= 1e-3 * abs(T)), (tag, b, h, diff, s[diff], T)
            mine = jssa.attend(qh, K[b, h][:n], V[b, h][:n], gi, scale)
            err = np.max(np.abs(o[b, h * G:(h + 1) * G] - mine)) if n else np.max(np.abs(o[b, h * G:(h + 1) * G]))
            assert err <= tol, (tag, b, h, err)
            if np.array_equal(got_blocks, ref_blocks) and n:
                assert np.max(np.abs(o[b, h * G:(h + 1) * G] - ref_out)) <= tol
    return out, idx


def test_block_step_config_shape_bf16_and_int4():
    say("block step: B=4, 64/8 heads, n=65536, 1024 blocks of 64, 16 kept (bf16 and INT4 keys)")
    wl = workloads.block_config(device="cuda")
    keys = _keys(wl, 64, int4=True)
    _check_step(wl, 64, 16, keys, tag="bf16")
    _check_step(wl, 64, 16, keys, tag="int4", int4=True)
    _check_step(wl, 64, 16, keys, out_f32=False, tag="bf16 out")


@pytest.mark.parametrize("G,bsz,k_blocks", [(1, 64, 8), (2, 16, 20), (4, 32, 5), (8, 128, 3)])
def test_block_step_ragged(G, bsz, k_blocks):
    say(f"block step ragged G={G} bs={bsz} k={k_blocks}")
    seq = [3000, 1, 0, bsz * 9, bsz * 3 + 5, 2049]
    wl = workloads.blocks(6, 2, G, 3000, bsz, k_blocks, seed=82 + G, device="cuda", capacity=3003, seq_len=seq)
    keys = _keys(wl, bsz, int4=True)
    _check_step(wl, bsz, k_blocks, keys, tag=f"bf16 G{G} bs{bsz}")
    _check_step(wl, bsz, k_blocks, keys, tag=f"int4 G{G} bs{bsz}", int4=True)
    _check_step(wl, bsz, k_blocks, keys, n_init=0, n_local=0, tag="no forced")
    _check_step(wl, bsz, k_blocks, keys, n_init=k_blocks // 2, n_local=k_blocks - k_blocks // 2, tag="all forced")


def test_block_step_duplicated_keys_tie_to_lower_block():
    say("block step: duplicated block keys tie exactly")
    wl = workloads.blocks(1, 2, 4, 64 * 200, 64, 10, seed=86, device="cuda")
    Kc, _, _ = _keys(wl, 64)
    Kc[:, :, 100:200] = Kc[:, :, 0:100]                  # every block key appears twice
    _check_step(wl, 64, 10, (Kc, None, None), tag="dup", exact_sets=True)


def test_block_step_many_blocks_scores_from_global():
    # 10000 complete blocks per sequence: more scores than the selection stages in LDS
    say("block step: 10000 blocks of 4")
    wl = workloads.blocks(1, 1, 4, 40000, 4, 50, seed=87, device="cuda", seq_len=[39999], capacity=40000)
    keys = _keys(wl, 4, int4=True)
    _check_step(wl, 4, 50, keys, tag="many bf16")
    _check_step(wl, 4, 50, keys, tag="many int4", int4=True)


def test_block_step_largest_budget_and_clamped_lengths():
    # the largest block budget (4096 blocks of one position: every key its own block),
    # a capacity that is not a multiple of the block size, lengths above the capacity
    say("block step: 4096-block budget; capacity not a multiple of bs; seq_len above capacity")
    wl = workloads.blocks(2, 1, 4, 9000, 1, 4096, seed=88, device="cuda", capacity=9000)
    wl.seq_len = torch.tensor([20000, 7777], dtype=torch.int32, device="cuda")
    keys = _keys(wl, 1, int4=True)
    _check_step(wl, 1, 4096, keys, tag="budget 4096")
    wl2 = workloads.blocks(2, 2, 2, 1000, 48, 6, seed=89, device="cuda", capacity=1001, seq_len=[1001, 999])
    keys2 = _keys(wl2, 48, int4=True)
    _check_step(wl2, 48, 6, keys2, tag="bs 48 cap 1001")
    _check_step(wl2, 48, 6, keys2, tag="bs 48 cap 1001 int4", int4=True)


def test_block_toy_by_hand_on_gpu():
    from tests import golden_variants as gv
    from tests.util import from_bits
    say("block step: hand-worked toy (bf16 and INT4 keys)")
    g = gv.load("block_toy")
    q = from_bits(gv.padded_bits(g["q_heads"]))[None].cuda()
    K = from_bits(gv.padded_bits(g["K"]))[None, None].cuda()
    V = from_bits(gv.padded_bits(g["V"]))[None, None].cuda()
    sl = torch.tensor([g["n"]], dtype=torch.int32, device="cuda")
    bsz = g["block_size"]
    Kc, Kq, Ks = sj.block_cache(K, bsz, int4=True)
    sj.block_keys(K, sl, bsz, Kc, Kq, Ks)
    for keys in ((Kc, None, None), (None, Kq, Ks)):
        out, idx = sj.block_decode_step(q, K, V, sl, bsz, g["k_blocks"], *keys, g["n_init"], g["n_local"],
                                        sm_scale=1.0, out_f32=True)
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0, 0]) == g["idx"]
        o = out.cpu().numpy()[0]
        assert np.max(np.abs(o[:, :4] - gv.matrix(g["out"]))) < 1e-5
        assert np.all(o[:, 4:] == 0)
