"""The fused prep + scan launch (sjsa_prep_scan, which the decode steps use) against
the separate prep and scan launches: identical index lists, outputs and caches over
ragged lengths, both cache formats, every rank, with and without the appended token;
the appended token's own key (taken from the prep's published row, not from memory);
repeated steps on one workspace; a captured graph replayed with new queries; and
the exact fallback when the scan workgroups stop waiting."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa
from tests.gpu_helpers import OUT_TOL_F32, bits, check_unit, say

pytestmark = pytest.mark.gpu


def _cache(wl, fp8):
    """Projected cache of every slot, written by the library's append."""
    Kp = torch.zeros(wl.batch, wl.n_kv_heads, wl.capacity, wl.rank, dtype=torch.uint8 if fp8 else torch.bfloat16,
                     device="cuda")
    pos0 = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    sj.append_kv(wl.K, wl.V, wl.M, pos0, wl.K.clone(), wl.V.clone(), Kp)
    return Kp


def _step(wl, Kp, q, seq_len, k, mode, new=None, ws=None, wait_us=0):
    """One step on copies of the caches through the stage calls: mode "separate" (prep
    or prep_append, then scan) or "fused" (prep_scan, its scan workgroups waiting at
    most wait_us for the prep; 0 = the default, negative = no wait); then select and
    attend. Returns the caches after the step, idx and the fp32 output."""
    fp8 = Kp.dtype == torch.uint8
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    shape = sj.make_shape(wl.batch, wl.n_kv_heads, wl.group, 128, wl.rank, wl.capacity, kproj_fp8=fp8,
                          fused_wait_us=wait_us)
    if ws is None:
        ws = sj.alloc_workspace(shape, k)
    if mode == "separate":
        if new is None:
            sj.prep(shape, q, wl.M, P, seq_len, k, ws)
        else:
            sj.prep_append(shape, new[0], new[1], new[2], q, K, V, wl.M, P, seq_len, k, ws)
        sj.scan(shape, P, seq_len, ws)
    else:
        if new is None:
            sj.prep_scan(shape, q, wl.M, P, seq_len, k, ws)
        else:
            sj.prep_scan(shape, q, wl.M, P, seq_len, k, ws, k_new=new[0], v_new=new[1], pos=new[2], K=K, V=V)
    idx = sj.select(shape, P, seq_len, k, ws)
    out = sj.attend(q, K, V, idx, seq_len, workspace=ws, out_f32=True, rank=wl.rank)
    torch.cuda.synchronize()
    return K, V, P, idx, out


def _same(a, b, tag):
    for name, x, y in zip(("K", "V", "Kproj", "idx", "out"), a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y), f"{tag}: {name} differs"


def _oracle(wl, res, q, seq, k, fp8, tag, units):
    K, V, P, idx, out = res
    Kb, Vb, qb = bits(K), bits(V), bits(q)
    Pb = P.cpu().numpy() if fp8 else bits(P)
    M = wl.M.cpu().numpy()
    o, ix = out.cpu().numpy(), idx.cpu().numpy()
    G = wl.group
    for b, h in units:
        check_unit(o[b, h * G:(h + 1) * G], ix[b, h], qb, Kb, Vb, Pb, M, b, h, G, seq[b], k,
                   jssa.default_sm_scale(128), OUT_TOL_F32, tag, fmt="fp8" if fp8 else "bf16")


@pytest.mark.parametrize("r,G,fp8,append", [(32, 4, False, True), (32, 4, True, True), (16, 1, False, False),
                                            (64, 8, False, True), (64, 2, True, False), (16, 2, True, True)])
def test_fused_matches_separate(r, G, fp8, append):
    seq = [9000, 4097, 1, 20000]
    k = 512
    tag = f"prep_scan r={r} G={G} fp8={fp8} append={append}"
    say(tag)
    wl = workloads.gaussian(4, 2, G, 128, r, max(seq), k, seed=60 + r + G, capacity=20480, device="cuda",
                            seq_len=seq)
    Kp = _cache(wl, fp8)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    new = None
    if append:
        k_new, v_new = workloads.new_token(wl, seed=61, T=1)
        new = (k_new, v_new, seq_len - 1)        # the new token is the last of each sequence
    ref = _step(wl, Kp, wl.q, seq_len, k, "separate", new)
    got = _step(wl, Kp, wl.q, seq_len, k, "fused", new)
    _same(ref, got, tag)
    # and the library's decode step (which makes the fused launch) gives the same
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    if append:
        out, idx = sj.decode_step_append(new[0], new[1], new[2], wl.q, K, V, P, wl.M, seq_len, k, out_f32=True)
    else:
        out, idx = sj.decode_step(wl.q, K, V, P, wl.M, seq_len, k, out_f32=True)
    torch.cuda.synchronize()
    _same(ref, (K, V, P, idx, out), tag + " decode step")
    _oracle(wl, got, wl.q, seq, k, fp8, tag, [(0, 0), (1, 1), (2, 0), (3, 1)])


@pytest.mark.parametrize("fp8,sign", [(False, 1.0), (False, -1.0), (True, 1.0)])
def test_appended_token_ranks_by_its_new_key(fp8, sign):
    # the new token's key is the (scaled) mean query of its group: it scores highest
    # (sign +1) or lowest (-1) in its unit, while the slot it overwrites held an
    # ordinary key; the fused scan must rank it by the new key
    tag = f"appended token key fp8={fp8} sign={sign}"
    say(tag)
    seq = [12000, 5000]
    k = 256
    wl = workloads.gaussian(2, 2, 4, 128, 32, max(seq), k, seed=70, capacity=12288, device="cuda", seq_len=seq)
    Kp = _cache(wl, fp8)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    qbar = wl.q.float().view(2, 2, 4, 128).mean(dim=2)                  # [B, H_kv, d]
    k_new = (sign * 3.0 * qbar / qbar.norm(dim=-1, keepdim=True) * 11.0).to(torch.bfloat16).unsqueeze(2).contiguous()
    _, v_new = workloads.new_token(wl, seed=71, T=1)
    new = (k_new, v_new, seq_len - 1)
    ref = _step(wl, Kp, wl.q, seq_len, k, "separate", new)
    got = _step(wl, Kp, wl.q, seq_len, k, "fused", new)
    _same(ref, got, tag)
    ix = got[3].cpu().numpy()
    for b in range(2):
        for h in range(2):
            assert ((seq[b] - 1) in ix[b, h]) == (sign > 0), f"{tag}: unit ({b},{h})"
    _oracle(wl, got, wl.q, seq, k, fp8, tag, [(0, 0), (0, 1), (1, 0), (1, 1)])


def test_repeated_steps_on_one_workspace():
    # four decode steps in a row on one workspace (new query and new token each time):
    # each equals the separate-launch step on a fresh workspace
    say("prep_scan: repeated steps on one workspace")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 8000, 300, seed=75, capacity=8192, device="cuda", seq_len=[8000, 6000])
    Kp = _cache(wl, False)
    shape = sj.make_shape(2, 2, 4, 128, 32, 8192)
    ws = sj.alloc_workspace(shape, 300)
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    seq = torch.tensor([8000, 6000], dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(76)
    for step in range(4):
        q = torch.randn(wl.q.shape, generator=g, device="cuda").to(torch.bfloat16)
        k_new = torch.randn(2, 2, 1, 128, generator=g, device="cuda").to(torch.bfloat16)
        v_new = torch.randn(2, 2, 1, 128, generator=g, device="cuda").to(torch.bfloat16)
        seq = seq + 1
        pos = seq - 1
        wl_now = workloads.Workload(wl.name, 2, 2, 4, 128, 32, 8192, 300, seq, q, K, V, wl.M)
        ref = _step(wl_now, P, q, seq, 300, "separate", (k_new, v_new, pos))
        out, idx = sj.decode_step_append(k_new, v_new, pos, q, K, V, P, wl.M, seq, 300, out_f32=True, workspace=ws)
        torch.cuda.synchronize()
        _same(ref, (K, V, P, idx, out), f"step {step}")


def test_graph_replay_with_new_queries():
    # the step captured once as a HIP graph and replayed with new queries copied into
    # its input: every replay equals an eager step (the hand-over tags must change
    # from replay to replay although the captured launch arguments do not)
    say("prep_scan: graph replays")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 9000, 400, seed=80, capacity=9216, device="cuda",
                            seq_len=[9000, 7000])
    Kp = _cache(wl, False)
    shape = sj.make_shape(2, 2, 4, 128, 32, 9216, out_f32=True)
    ws = sj.alloc_workspace(shape, 400)
    q_in = wl.q.clone()
    out = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")
    idx = torch.empty(2, 2, 400, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up outside the capture
        sj.decode_step(q_in, wl.K, wl.V, Kp, wl.M, wl.seq_len, 400, out=out, idx=idx, workspace=ws, out_f32=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sj.decode_step(q_in, wl.K, wl.V, Kp, wl.M, wl.seq_len, 400, out=out, idx=idx, workspace=ws, out_f32=True)
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda")
    g.manual_seed(81)
    for rep in range(4):
        q = torch.randn(wl.q.shape, generator=g, device="cuda").to(torch.bfloat16)
        q_in.copy_(q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_idx = sj.decode_step(q, wl.K, wl.V, Kp, wl.M, wl.seq_len, 400, out_f32=True)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {rep}: idx"
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"replay {rep}: out"


@pytest.mark.parametrize("fp8,wait_us", [(False, 0), (False, -1), (True, 0), (True, -1)])
def test_graph_replay_of_the_appending_stage_calls(fp8, wait_us):
    # the appending step's stage calls (append + prep + scan in one launch, select,
    # attend + merge) captured once and replayed with new queries and new tokens copied
    # into the captured inputs. Each replay gives the caches, index lists and outputs of
    # the same calls made eagerly on a copy of the caches. This holds on the candidate
    # path and with every unit on the exact path (wait_us < 0), whose arrival counts
    # each replay's prep clears again.
    tag = f"prep_scan: graph replays of the appending step (fp8 {fp8}, wait {wait_us})"
    say(tag)
    k = 400
    wl = workloads.gaussian(2, 2, 4, 128, 32, 9000, k, seed=87, capacity=9216, device="cuda",
                            seq_len=[9000, 7001])
    Kp = _cache(wl, fp8)
    seq_len = wl.seq_len
    pos = (seq_len - 1).to(torch.int32)
    shape = sj.make_shape(2, 2, 4, 128, 32, 9216, kproj_fp8=fp8, fused_wait_us=wait_us)
    ws = sj.alloc_workspace(shape, k)
    K, V, P = wl.K.clone(), wl.V.clone(), Kp.clone()
    q_in = wl.q.clone()
    kn_in, vn_in = workloads.new_token(wl, seed=88)
    idx = torch.empty(2, 2, k, dtype=torch.int32, device="cuda")
    out = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")

    def calls():
        sj.prep_scan(shape, q_in, wl.M, P, seq_len, k, ws, k_new=kn_in, v_new=vn_in, pos=pos, K=K, V=V)
        sj.select(shape, P, seq_len, k, ws, idx=idx)
        sj.attend(q_in, K, V, idx, seq_len, out=out, workspace=ws, out_f32=True, rank=32)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda")
    g.manual_seed(89)
    for rep in range(4):
        q = torch.randn(wl.q.shape, generator=g, device="cuda").to(torch.bfloat16)
        kn = torch.randn(kn_in.shape, generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn(vn_in.shape, generator=g, device="cuda").to(torch.bfloat16)
        q_in.copy_(q)
        kn_in.copy_(kn)
        vn_in.copy_(vn)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = _step(wl, Kp, q, seq_len, k, "fused", new=(kn, vn, pos), wait_us=wait_us)
        _same((K, V, P, idx, out), ref, f"{tag}, replay {rep}")


def test_zero_wait_limit_falls_back_exactly():
    # scan workgroups that do not wait (a negative limit in the shape) mark their tiles
    # unusable; the selection then recomputes those units exactly, so the results do
    # not change
    say("prep_scan: zero wait limit")
    wl = workloads.gaussian(4, 2, 4, 128, 32, 30000, 700, seed=85, capacity=30720, device="cuda",
                            seq_len=[30000, 17, 12345, 4096])
    Kp = _cache(wl, False)
    seq = [30000, 17, 12345, 4096]
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=86, T=1)
    new = (k_new, v_new, seq_len - 1)
    ref = _step(wl, Kp, wl.q, seq_len, 700, "separate", new)
    got = _step(wl, Kp, wl.q, seq_len, 700, "fused", new, wait_us=-1)
    _same(ref, got, "zero wait")
    _oracle(wl, got, wl.q, seq, 700, False, "zero wait", [(0, 0), (2, 1), (3, 0)])


@pytest.mark.parametrize("r,G,fp8", [(16, 1, False), (16, 2, True), (32, 4, True), (64, 8, False), (64, 4, True)])
def test_every_unit_exact_equals_candidate_path(r, G, fp8):
    # every rank and cache format of the exact path (scores recomputed by several
    # workgroups per unit, dense selection) against the candidate path: the same
    # index lists and outputs bit for bit, over ragged lengths and a budget past the
    # dense selection's lists (k > 8192) for one of them
    k = 9000 if r == 64 and not fp8 else 700
    seq = [30000, 17, 12345, 4096 + 3]
    tag = f"exact path r={r} G={G} fp8={fp8} k={k}"
    say(tag)
    wl = workloads.gaussian(4, 2, G, 128, r, 30000, k, seed=95 + r + G, capacity=30000, device="cuda", seq_len=seq)
    Kp = _cache(wl, fp8)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    ref = _step(wl, Kp, wl.q, seq_len, k, "fused")
    got = _step(wl, Kp, wl.q, seq_len, k, "fused", wait_us=-1)
    _same(ref, got, tag)
    _oracle(wl, got, wl.q, seq, k, fp8, tag, [(0, 1), (2, 0), (3, 1)])


@pytest.mark.parametrize("fp8", [False, True])
def test_exact_path_with_one_workgroup_per_unit(fp8):
    # 256 units fill the GPU with their selectors, so the selection launch has no
    # exact-path helpers and the exact path recomputes and selects each unit in one
    # workgroup: the same index lists and outputs as the candidate path, bit for bit,
    # over ragged lengths
    seq = [3000 - 37 * b for b in range(32)]
    k = 200
    tag = f"exact path, one workgroup per unit, fp8={fp8}"
    say(tag)
    wl = workloads.gaussian(32, 8, 4, 128, 32, 3000, k, seed=141 + fp8, capacity=3000, device="cuda", seq_len=seq)
    Kp = _cache(wl, fp8)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    ref = _step(wl, Kp, wl.q, seq_len, k, "fused")
    got = _step(wl, Kp, wl.q, seq_len, k, "fused", wait_us=-1)
    _same(ref, got, tag)
    _oracle(wl, got, wl.q, seq, k, fp8, tag, [(0, 0), (17, 5), (31, 7)])


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_edge_lengths(fp8):
    # capacity not a multiple of the 4096-row tile, an empty sequence, a sequence no
    # longer than the budget (every position taken), one exactly a tile long, one whose
    # appended slot lies past its length; fused step against the separate launches
    seq = [0, 300, 4096, 10001, 7000]
    pos = [5, 299, 4095, 10000, 9000]          # the last: a slot past the sequence's length
    k = 300
    tag = f"prep_scan edge lengths fp8={fp8}"
    say(tag)
    wl = workloads.gaussian(5, 2, 4, 128, 32, max(seq), k, seed=90, capacity=10001, device="cuda", seq_len=seq)
    Kp = _cache(wl, fp8)
    seq_len = torch.tensor(seq, dtype=torch.int32, device="cuda")
    k_new, v_new = workloads.new_token(wl, seed=91, T=1)
    new = (k_new, v_new, torch.tensor(pos, dtype=torch.int32, device="cuda"))
    ref = _step(wl, Kp, wl.q, seq_len, k, "separate", new)
    got = _step(wl, Kp, wl.q, seq_len, k, "fused", new)
    _same(ref, got, tag)
    ix = got[3].cpu().numpy()
    assert np.all(ix[0] == -1)                                   # empty sequence: nothing selected
    assert np.array_equal(ix[1, 0, :300], np.arange(300))        # n <= k: every position
    _oracle(wl, got, wl.q, seq, k, fp8, tag, [(1, 0), (2, 1), (3, 0), (4, 1)])
