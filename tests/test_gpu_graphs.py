"""Steps captured once as a HIP graph and replayed with new inputs copied into the
captured buffers: every replay must give exactly what the same call gives eagerly
with the same inputs. Covered: the gated-logit step, the block-sparse step (bf16 and
INT4 block keys) and the allocation-free decode step (whose scratch array the
replays share). Between replays the same step runs eagerly, with buffers of its
own, as the reference."""
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _capture(calls):
    """calls() once outside the capture (on a side stream, as warm-up), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    return graph


def _bitwise(a, b, what):
    x = a.view(torch.uint8) if a.dtype != torch.int32 else a
    y = b.view(torch.uint8) if b.dtype != torch.int32 else b
    assert torch.equal(x, y), f"{what} differs"


def _randn_like(t, g):
    return torch.randn(t.shape, generator=g, device="cuda").to(t.dtype)


def test_gated_step_graph_replays():
    say("graph: gated step, 3 replays")
    unit, k_units = 16, 20
    wl = workloads.gated(2, 2, 4, 3000, unit, k_units, seed=160, device="cuda", seq_len=[3000, 2049])
    q_in = wl.q.clone()
    gates_in = wl.extra["gate_scores"].clone()
    out = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")
    idx = torch.empty(2, 2, unit * k_units, dtype=torch.int32, device="cuda")
    ws = sj.gated_workspace(sj.gated_shape(wl.q, wl.K, True), unit, k_units)

    def calls():
        sj.gated_decode_step(q_in, wl.K, wl.V, gates_in, wl.seq_len, unit, k_units, lam=1.5, out=out, idx=idx,
                             workspace=ws, out_f32=True)

    graph = _capture(calls)
    g = torch.Generator(device="cuda")
    g.manual_seed(161)
    for rep in range(3):
        q, gates = _randn_like(q_in, g), _randn_like(gates_in, g)
        q_in.copy_(q)
        gates_in.copy_(gates)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_idx = sj.gated_decode_step(q, wl.K, wl.V, gates, wl.seq_len, unit, k_units, lam=1.5,
                                                out_f32=True)
        torch.cuda.synchronize()
        _bitwise(idx, ref_idx, f"gated replay {rep}: idx")
        _bitwise(out, ref_out, f"gated replay {rep}: out")


@pytest.mark.parametrize("int4", [False, True])
def test_block_step_graph_replays(int4):
    say(f"graph: block step (int4 keys: {int4}), 3 replays")
    bsz, k_blocks = 32, 6
    wl = workloads.blocks(3, 2, 8, 3000, bsz, k_blocks, seed=170, device="cuda", capacity=3003,
                          seq_len=[3000, 2049, bsz * 4 + 5])
    Kc, Kq, Ks = sj.block_cache(wl.K, bsz, int4=True)
    sj.block_keys(wl.K, wl.seq_len, bsz, Kc, Kq, Ks)
    keys = (None, Kq, Ks) if int4 else (Kc, None, None)
    q_in = wl.q.clone()
    out = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")
    idx = torch.empty(3, 2, bsz * k_blocks, dtype=torch.int32, device="cuda")
    ws = sj.block_workspace(sj.gated_shape(wl.q, wl.K, True), bsz, k_blocks)

    def calls():
        sj.block_decode_step(q_in, wl.K, wl.V, wl.seq_len, bsz, k_blocks, *keys, out=out, idx=idx, workspace=ws,
                             out_f32=True)

    graph = _capture(calls)
    g = torch.Generator(device="cuda")
    g.manual_seed(171)
    for rep in range(3):
        q = _randn_like(q_in, g)
        q_in.copy_(q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_idx = sj.block_decode_step(q, wl.K, wl.V, wl.seq_len, bsz, k_blocks, *keys, out_f32=True)
        torch.cuda.synchronize()
        _bitwise(idx, ref_idx, f"block replay {rep}: idx")
        _bitwise(out, ref_out, f"block replay {rep}: out")


def test_noalloc_step_graph_replays():
    # the allocation-free step is meant for code under graph capture: captured with its
    # new-token append, replayed with new queries and tokens, each replay against the
    # workspace step run eagerly on a copy of the caches
    say("graph: allocation-free decode step, 3 replays")
    B, Hkv, G, r, cap, k = 2, 2, 4, 32, 9216, 400
    seq = [9000, 7001]
    wl = workloads.gaussian(B, Hkv, G, 128, r, max(seq), k, seed=180, capacity=cap, device="cuda", seq_len=seq)
    Kp = torch.zeros(B, Hkv, cap, r, dtype=torch.bfloat16, device="cuda")
    sj.append_kv(wl.K, wl.V, wl.M, torch.zeros(B, dtype=torch.int32, device="cuda"), wl.K.clone(), wl.V.clone(), Kp)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    pos = seq_len - 1
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    q_in = wl.q.clone()
    kn_in, vn_in = workloads.new_token(wl, seed=181)
    out = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device="cuda")

    def calls():
        sj.decode_step_append_noalloc(kn_in, vn_in, pos, q_in, K, V, P, wl.M, seq_len, k, out, idx)

    graph = _capture(calls)
    g = torch.Generator(device="cuda")
    g.manual_seed(182)
    for rep in range(3):
        q, kn, vn = _randn_like(q_in, g), _randn_like(kn_in, g), _randn_like(vn_in, g)
        q_in.copy_(q)
        kn_in.copy_(kn)
        vn_in.copy_(vn)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        K2, V2, P2 = wl.K.clone(), wl.V.clone(), Kp.clone()
        ref_out, ref_idx = sj.decode_step_append(kn, vn, pos, q, K2, V2, P2, wl.M, seq_len, k)
        torch.cuda.synchronize()
        for name, a, b in (("K", K, K2), ("V", V, V2), ("Kproj", P, P2), ("idx", idx, ref_idx), ("out", out, ref_out)):
            _bitwise(a, b, f"noalloc replay {rep}: {name}")
