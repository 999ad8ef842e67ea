"""GPU parity of the gated-logit (SAS) decode step against the oracle: the kept
units' positions exactly, the biased attention output within tolerance."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import jssa, sas
from tests.gpu_helpers import OUT_TOL_BF16, OUT_TOL_F32, bits, say

pytestmark = pytest.mark.gpu


def _check(wl, unit, k_units, lam, out_f32=True, tag="", gates=None):
    u = wl.extra["gate_scores"] if gates is None else gates
    out, idx = sj.gated_decode_step(wl.q, wl.K, wl.V, u, wl.seq_len, unit, k_units, lam=lam, out_f32=out_f32)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ix = idx.cpu().numpy()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    un = u.cpu().numpy()
    G = wl.group
    tol = OUT_TOL_F32 if out_f32 else OUT_TOL_BF16
    scale = jssa.default_sm_scale(128)
    for b in range(wl.batch):
        n = min(max(int(wl.seq_len[b]), 0), wl.capacity)
        for h in range(wl.n_kv_heads):
            ref_out, ref_idx, _ = sas.gated_decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], un[b, h], n,
                                                        unit, k_units, lam, scale)
            assert np.array_equal(ix[b, h], ref_idx), f"{tag} unit ({b},{h}): positions differ"
            err = np.max(np.abs(o[b, h * G:(h + 1) * G] - ref_out))
            assert err <= tol, f"{tag} unit ({b},{h}): max |out - oracle| = {err}"
    return out, idx


def test_gated_config_512_units_of_64():
    say("gated step: B=1, 32/8 heads, n=32768, 512 units of 64, budget 32")
    wl = workloads.gated_config(device="cuda")
    for lam, out_f32 in ((1.0, True), (1.0, False), (2.5, True)):
        _check(wl, 64, 32, lam, out_f32=out_f32, tag=f"config lam={lam}")


# (4, 1, 300) has 3003 units: more than the attention launch selects for itself, so the
# separate selection kernel runs; (4, 64, 64) keeps every one of its 47 units
@pytest.mark.parametrize("G,unit,k_units", [(1, 64, 8), (2, 16, 20), (4, 1, 300), (8, 64, 3), (4, 64, 64)])
def test_gated_ragged(G, unit, k_units):
    say(f"gated ragged G={G} unit={unit} k_units={k_units}")
    seq = [3000, 1, 0, 64 * 9, 2049]
    wl = workloads.gated(5, 2, G, 3000, unit, k_units, seed=60 + G + unit, device="cuda", capacity=3003,
                         seq_len=seq)
    _check(wl, unit, k_units, 1.0, tag=f"ragged G{G} u{unit} k{k_units}")


def test_gated_many_units_with_ties():
    # 1500 units per sequence; integer scores tie often, so the boundary key is shared
    say("gated 1500 units with ties")
    wl = workloads.gated(2, 2, 4, 6000, 4, 100, seed=70, device="cuda", seq_len=[6000, 5999])
    g = torch.randint(-3, 4, wl.extra["gate_scores"].shape, generator=torch.Generator().manual_seed(71))
    gates = g.float().cuda()
    _check(wl, 4, 100, 1.0, tag="radix ties", gates=gates)
    _check(wl, 4, 100, 1.0, tag="radix normal")


def test_gated_scores_read_from_global():
    # 10000 single-token units: more scores than the kernel stages in LDS
    say("gated 10000 units, scores read from global memory")
    wl = workloads.gated(1, 2, 4, 10000, 1, 500, seed=75, device="cuda", seq_len=[9999])
    _check(wl, 1, 500, 1.0, tag="unstaged")
    g = torch.randint(-2, 3, wl.extra["gate_scores"].shape, generator=torch.Generator().manual_seed(76))
    _check(wl, 1, 500, 1.0, tag="unstaged ties", gates=g.float().cuda())


def test_gated_ties_and_budget_one():
    say("gated ties; budget of one unit")
    wl = workloads.gated(2, 2, 4, 4000, 8, 40, seed=72, device="cuda", seq_len=[4000, 3333])
    g = torch.randint(-2, 3, wl.extra["gate_scores"].shape, generator=torch.Generator().manual_seed(73))
    _check(wl, 8, 40, 1.0, tag="ties", gates=g.float().cuda())
    _check(wl, 8, 1, 1.0, tag="current unit only")


def test_gated_lambda_zero_equals_plain_attention_bitwise():
    say("gated lambda=0 vs attend over the same positions")
    wl = workloads.gated(2, 2, 4, 5000, 64, 16, seed=74, device="cuda", seq_len=[5000, 4100])
    out, idx = sj.gated_decode_step(wl.q, wl.K, wl.V, wl.extra["gate_scores"], wl.seq_len, 64, 16, lam=0.0)
    ref = sj.attend(wl.q, wl.K, wl.V, idx, wl.seq_len, rank=32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_gated_is_deterministic():
    say("gated determinism")
    wl = workloads.gated_config(device="cuda")
    u = wl.extra["gate_scores"]
    a = sj.gated_decode_step(wl.q, wl.K, wl.V, u, wl.seq_len, 64, 32)
    b = sj.gated_decode_step(wl.q, wl.K, wl.V, u, wl.seq_len, 64, 32)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_gated_largest_unit_budget_and_clamped_lengths():
    # the largest unit budget the library takes (4096 units), single-token units, and
    # sequence lengths beyond the capacity (clamped to it)
    say("gated: 4096-unit budget; seq_len above capacity")
    wl = workloads.gated(2, 1, 4, 9000, 1, 4096, seed=77, device="cuda", capacity=9000)
    wl.seq_len = torch.tensor([12000, 5000], dtype=torch.int32, device="cuda")
    _check(wl, 1, 4096, 1.0, tag="budget 4096")
    wl2 = workloads.gated(1, 2, 2, 3000, 64, 4096, seed=78, device="cuda")     # every unit fits the budget
    _check(wl2, 64, 4096, 0.5, tag="all units kept")


def test_gated_toy_by_hand_on_gpu():
    from tests import golden_variants as gv
    from tests.util import from_bits
    say("gated: hand-worked toy")
    g = gv.load("gated_toy")
    q = from_bits(gv.padded_bits(g["q_heads"]))[None].cuda()
    K = from_bits(gv.padded_bits(g["K"]))[None, None].cuda()
    V = from_bits(gv.padded_bits(g["V"]))[None, None].cuda()
    u = torch.tensor([[[gv.value(x) for x in g["u"]]]], dtype=torch.float32, device="cuda")
    sl = torch.tensor([g["n"]], dtype=torch.int32, device="cuda")
    for c in g["cases"]:
        out, idx = sj.gated_decode_step(q, K, V, u, sl, g["unit_size"], g["k_units"], lam=c["lambda"], sm_scale=1.0,
                                        out_f32=True)
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0, 0]) == g["idx"]
        o = out.cpu().numpy()[0]
        assert np.max(np.abs(o[:, :4] - gv.matrix(c["out"]))) < 1e-5
        assert np.all(o[:, 4:] == 0)


@pytest.mark.parametrize("unit,k_units", [(64, 32), (1, 300)])
def test_gated_minus_inf_scores(unit, k_units):
    # scores of -inf (gate 0), among them the current unit's and the first units' (which
    # are a thread's first scores in the running softmax sum): the positions they hold get
    # zero weight, checked against the oracle; (1, 300) runs the separate selection kernel
    say(f"gated -inf scores unit={unit} k_units={k_units}")
    seq = [3000, 2049, 640]
    wl = workloads.gated(3, 2, 4, 3000, unit, k_units, seed=95, device="cuda", capacity=3003, seq_len=seq)
    gates = wl.extra["gate_scores"].clone()
    gates[:, :, :3] = -float("inf")
    gates[:, 0, 5::7] = -float("inf")
    for b, n in enumerate(seq):
        gates[b, 1, (n + unit - 1) // unit - 1] = -float("inf")      # the current unit of head 1
    for lam in (1.0, 0.0):
        out, _ = _check(wl, unit, k_units, lam, tag=f"-inf scores lam={lam}", gates=gates)
        assert torch.isfinite(out).all()
