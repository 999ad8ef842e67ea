"""End-to-end GPU parity of sjsa_decode_step (and the stage calls) against the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
import workloads
from oracle import calib, jssa
from oracle.numerics import bf16_to_f32
from tests import golden_toy
from tests.gpu_helpers import (OUT_TOL_BF16, OUT_TOL_F32, bits, check_unit, from_bits, kproj_oracle, say)

pytestmark = pytest.mark.gpu


def _run_and_check(wl, kproj_bits, k, out_f32=True, tag=""):
    Kp = from_bits(kproj_bits).cuda()
    out, idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, k, out_f32=out_f32)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ix = idx.cpu().numpy()
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.cpu().numpy()
    scale = jssa.default_sm_scale(128)
    G = wl.group
    tol = OUT_TOL_F32 if out_f32 else OUT_TOL_BF16
    msgs = []
    for b in range(wl.batch):
        n = min(max(int(wl.seq_len[b]), 0), wl.capacity)
        for h in range(wl.n_kv_heads):
            msgs.append(check_unit(o[b, h * G:(h + 1) * G], ix[b, h], q, K, V, kproj_bits, M, b, h, G, n, k,
                                   scale, tol, tag))
    return o, ix, msgs


def test_tiny_single_head_calibrated():
    say("step tiny single head, calibrated basis")
    wl = workloads.tiny_single_head()
    M = calib.calibrate(wl.calib_q.numpy(), wl.calib_k.numpy(), wl.rank).astype(np.float32)
    wl.M = torch.from_numpy(M)[None].contiguous()
    wl = wl.to("cuda")
    kp = kproj_oracle(bits(wl.K), M[None])
    for out_f32 in (True, False):
        _run_and_check(wl, kp, wl.k, out_f32=out_f32, tag="tiny")


def test_llama8b_layer():
    say("step llama8b-shaped layer n=32768 k=2048")
    wl = workloads.llama8b_layer(device="cuda")
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    _run_and_check(wl, kp, wl.k, out_f32=False, tag="llama8b")


@pytest.mark.parametrize("r,G", [(16, 1), (32, 2), (64, 4), (32, 8)])
def test_ragged_batches(r, G):
    say(f"step ragged r={r} G={G}")
    seq = [7000, 1, 0, 4099, 6999]
    wl = workloads.gaussian(5, 2, G, 128, r, 7000, 300, seed=r * 10 + G, device="cuda", seq_len=seq,
                            capacity=7003)
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    for k in (300, 1, 7000):
        _run_and_check(wl, kp, k, tag=f"ragged r{r} G{G} k{k}")


@pytest.mark.parametrize("r", [32, 64])
def test_sequence_past_one_gather_chunk(r):
    # 150,001 rows: more scan tiles per unit than the selection gathers in one round trip
    # (64 tiles of 2048 rows at r = 32, 128 of 1024 at r = 64), so its later chunks run;
    # the second sequence ends short of the capacity, inside the second chunk
    say(f"step: sequences past one selection gather chunk r={r}")
    seq = [150001, 140000]
    wl = workloads.gaussian(2, 1, 4, 128, r, 150001, 1024, seed=77 + r, device="cuda", seq_len=seq,
                            capacity=150001)
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    _run_and_check(wl, kp, 1024, tag=f"two gather chunks r{r}")


@pytest.mark.parametrize("r,k", [(32, 12000), (32, 20000), (16, 30000)])
def test_budgets_near_and_above_the_candidate_lists(r, k):
    # k = 12000: the candidates (about 1.7 k) exceed the 16384 the selection keeps, so
    # the exact path runs; k > 16384 always takes it. The attention splits the budget
    # over many chunks; the second sequence is shorter than k
    say(f"step large budget r={r} k={k}")
    seq = [60000, 25001]
    wl = workloads.gaussian(2, 2, 4, 128, r, 60000, k, seed=90 + r + k, device="cuda", seq_len=seq)
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    _run_and_check(wl, kp, k, tag=f"large budget r{r} k{k}")


def test_budget_at_least_context_is_dense():
    say("step k >= n")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 900, 1000, seed=21, device="cuda", seq_len=[900, 333])
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    o, ix, _ = _run_and_check(wl, kp, 1000, tag="dense")
    assert np.array_equal(ix[0, 0, :900], np.arange(900)) and np.all(ix[0, 0, 900:] == -1)
    assert np.array_equal(ix[1, 1, :333], np.arange(333)) and np.all(ix[1, 1, 333:] == -1)


@pytest.mark.parametrize("k", [4999, 4998])
def test_budget_just_below_the_context(k):
    # all but one or two positions selected: the candidate lists cannot hold them, so the
    # exact path selects; the second sequence is shorter than k (every position taken)
    say(f"step k = n - {5000 - k}")
    wl = workloads.gaussian(2, 2, 4, 128, 32, 5000, k, seed=31 + k, device="cuda", seq_len=[5000, 4000])
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    o, ix, _ = _run_and_check(wl, kp, k, tag=f"k = {k}")
    assert np.array_equal(ix[1, 0, :4000], np.arange(4000)) and np.all(ix[1, 0, 4000:] == -1)


def test_duplicated_kproj_rows_tie_to_lower_position():
    say("step exact ties from duplicated rows")
    wl = workloads.gaussian(1, 1, 4, 128, 32, 8192, 512, seed=22, device="cuda")
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    kp[0, 0, 4096:] = kp[0, 0, :4096]          # every projected row appears twice
    o, ix, msgs = _run_and_check(wl, kp, 512, tag="dup")
    # bit-equal scores on both sides: the sets must be identical (no band needed)
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    _, ref_idx, _ = jssa.decode_unit(q[0], K[0, 0], V[0, 0], kp[0, 0], wl.M.cpu().numpy()[0], 8192, 512,
                                     jssa.default_sm_scale(128))
    assert np.array_equal(ix[0, 0], ref_idx)


def test_zero_query_all_scores_tie():
    say("step zero query")
    wl = workloads.gaussian(1, 2, 4, 128, 16, 3000, 100, seed=23, device="cuda")
    wl.q.zero_()
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    o, ix, _ = _run_and_check(wl, kp, 100, tag="zero-q")
    assert np.array_equal(ix[0, 0], np.arange(100))       # all scores are +-0: lowest positions


def test_zero_query_sequence_in_a_batch_takes_the_first_positions():
    # a padded slot: sequence 1's query heads are zero, so every score of its units is
    # +-0 (one key), every row is a candidate and those units take the exact path,
    # whose crowded first-digit bin holds the whole row: the first k positions; the
    # other sequence is an ordinary one in the same launch
    say("step zero-query sequence in a batch")
    n, k = 40000, 1500
    wl = workloads.gaussian(2, 2, 4, 128, 32, n, k, seed=29, device="cuda")
    wl.q[1].zero_()
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    o, ix, _ = _run_and_check(wl, kp, k, tag="zero-query slot")
    for h in range(2):
        assert np.array_equal(ix[1, h], np.arange(k))


def test_nan_query_sequence_selects_its_first_positions():
    # one sequence's queries are NaN: every score is NaN (ranked last, all equal), so its
    # units select their first k positions through the exact path; the other sequence
    # in the launch is unaffected
    say("step NaN-query sequence")
    n, k = 20000, 700
    wl = workloads.gaussian(2, 2, 4, 128, 32, n, k, seed=33, device="cuda")
    wl.q[1] = float("nan")
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    Kp = from_bits(kp).cuda()
    out, idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, k, out_f32=True)
    torch.cuda.synchronize()
    ix, o = idx.cpu().numpy(), out.cpu().numpy()
    for h in range(2):
        assert np.array_equal(ix[1, h], np.arange(k))
    q, K, V, M = bits(wl.q), bits(wl.K), bits(wl.V), wl.M.cpu().numpy()
    for h in range(2):
        check_unit(o[0, 4 * h:4 * h + 4], ix[0, h], q, K, V, kp, M, 0, h, 4, n, k, jssa.default_sm_scale(128),
                   OUT_TOL_F32, "NaN-query batch")


def test_stage_calls_equal_fused_step_and_are_deterministic():
    say("stages vs fused step, determinism")
    wl = workloads.gaussian(3, 2, 4, 128, 32, 20000, 700, seed=24, device="cuda", seq_len=[20000, 15000, 9])
    Kp = from_bits(kproj_oracle(bits(wl.K), wl.M.cpu().numpy())).cuda()
    shape = sj.shape_of(wl.q, wl.K, wl.M)
    ws = sj.alloc_workspace(shape, 700)
    o1, i1 = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, 700, workspace=ws)
    o2, i2 = sj.decode_step(wl.q, wl.K, wl.V, Kp, wl.M, wl.seq_len, 700, workspace=ws)
    sc = sj.score(wl.q, Kp, wl.M, wl.seq_len, 700, ws, write_scores=True)
    i3 = sj.select(shape, Kp, wl.seq_len, 700, ws)
    o3 = sj.attend(wl.q, wl.K, wl.V, i3, wl.seq_len, workspace=ws, rank=32)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(i1, i3)
    # stored scores against the oracle's scores, within the fp32 error bound
    q = bits(wl.q)
    M = wl.M.cpu().numpy()
    kp = bits(Kp)
    s_gpu = sc.cpu().numpy()
    for b, n in ((0, 20000), (1, 15000), (2, 9)):
        for h in range(2):
            qbar = jssa.mean_query(q[b, 4 * h:4 * h + 4])
            qhat = jssa.project_query(qbar, M[h])
            s_ref = jssa.score_positions(qhat, kp[b, h, :n]).astype(np.float64)
            kf = np.abs(bf16_to_f32(kp[b, h, :n]).astype(np.float64))
            a = np.abs(M[h]).astype(np.float64) @ np.abs(qbar.astype(np.float64))
            bound = 1e-5 * (kf @ np.abs(qhat.astype(np.float64)) + kf @ a) + 1e-30
            assert np.all(np.abs(s_gpu[b, h, :n] - s_ref) <= bound)


def test_golden_toy_hand_worked_on_gpu():
    say("step golden toy")
    g = golden_toy.load()
    q, K, V, M = golden_toy.padded(g)
    kp = jssa.project_keys(K, M)
    qt = from_bits(q[None]).cuda()
    Kt = from_bits(K[None, None]).cuda()
    Vt = from_bits(V[None, None]).cuda()
    Kpt = from_bits(kp[None, None]).cuda()
    Mt = torch.from_numpy(M[None]).cuda()
    sl = torch.tensor([5], dtype=torch.int32, device="cuda")
    for c in g["cases"]:
        out, idx = sj.decode_step(qt, Kt, Vt, Kpt, Mt, sl, c["k"], sm_scale=g["sm_scale"], out_f32=True)
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0, 0]) == c["idx"]
        if c["out"] is not None:
            o = out.cpu().numpy()[0]
            assert np.max(np.abs(o[:, :4] - c["out"])) <= 1e-6
            assert np.all(o[:, 4:] == 0)


def _ties_check(wl, kp, k, tag):
    """Exact index-set equality (scores tie bit-for-bit on both sides) plus output parity."""
    o, ix, _ = _run_and_check(wl, kp, k, tag=tag)
    q, K, V = bits(wl.q), bits(wl.K), bits(wl.V)
    M = wl.M.cpu().numpy()
    for b in range(wl.batch):
        n = int(wl.seq_len[b])
        for h in range(wl.n_kv_heads):
            _, ref_idx, _ = jssa.decode_unit(q[b, 4 * h:4 * h + 4], K[b, h], V[b, h], kp[b, h], M[h], n, k,
                                             jssa.default_sm_scale(128))
            assert np.array_equal(ix[b, h], ref_idx), (tag, b, h)


def test_candidate_overflow_falls_back_exactly():
    # every projected row identical: all scores tie, every row reaches the threshold,
    # and 40000 candidates exceed what the selection keeps in LDS
    say("step candidate overflow -> exact fallback")
    wl = workloads.gaussian(1, 2, 4, 128, 16, 40000, 1500, seed=25, device="cuda")
    kp = kproj_oracle(bits(wl.K[:, :, :1].contiguous()), wl.M.cpu().numpy())
    kp = np.ascontiguousarray(np.repeat(kp, 40000, axis=2))
    _ties_check(wl, kp, 1500, "overflow")


def test_candidate_underflow_falls_back_exactly():
    # the prep stage samples 1024 pairs of adjacent rows (2*floor(i*n/2048) and the row
    # after it); the first row of every pair scores high, all others low: the sampled
    # threshold lands on the high score, and only 1024 rows (fewer than k) reach it
    say("step candidate underflow -> exact fallback")
    n, k = 40000, 2000
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, k, seed=26, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    low = jssa.project_keys(bits(wl.K[0, 0, :1].contiguous()), M[0])[0]
    high = (np.sign(qhat) * 4.0)
    from oracle.numerics import round_to_bf16
    high = round_to_bf16(high)
    kp = np.tile(low, (1, 1, n, 1)).astype(np.uint16)
    first_of_pair = 2 * ((np.arange(1024, dtype=np.int64) * n) // 2048)
    kp[0, 0, first_of_pair] = high
    _ties_check(wl, kp, k, "underflow")


def test_constant_unit_with_spread_high_rows_falls_back_exactly():
    # 1000 high rows spread over a unit whose other rows are all equal: every row is
    # a candidate, and in the exact path the crowded boundary bin holds one key value
    say("step constant unit with spread high rows -> exact fallback")
    n, k = 40000, 1500
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, k, seed=28, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    low = jssa.project_keys(bits(wl.K[0, 0, :1].contiguous()), M[0])[0]
    from oracle.numerics import round_to_bf16
    high = round_to_bf16(np.sign(qhat) * 4.0)
    kp = np.tile(low, (1, 1, n, 1)).astype(np.uint16)
    kp[0, 0, np.random.default_rng(28).choice(n, 1000, replace=False)] = high
    _ties_check(wl, kp, k, "constant unit, high rows")


def test_scan_stage_overflow_falls_back_exactly():
    # the first 4096 rows (one scan tile) all score high, the rest low: every wave of
    # that tile finds 1024 candidates, more than it can stage; the total (4096) would
    # fit the selection, so only the overflow flag keeps the result exact
    say("step scan stage overflow -> exact fallback")
    n, k = 40000, 1500
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, k, seed=27, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    low = jssa.project_keys(bits(wl.K[0, 0, :1].contiguous()), M[0])[0]
    from oracle.numerics import round_to_bf16
    high = round_to_bf16(np.sign(qhat) * 4.0)
    kp = np.tile(low, (1, 1, n, 1)).astype(np.uint16)
    kp[0, 0, :4096] = high
    _ties_check(wl, kp, k, "stage overflow")


@pytest.mark.parametrize("k", [100, 400])
def test_outliers_between_sampled_rows(k):
    # 300 rows score far above every other row and sit between the sampled pairs
    # (rows 2*floor(i*n/2048) and the one after), so the sampled threshold and key
    # range know nothing of them: their candidate keys saturate. With k = 100 the
    # boundary lies among the outliers, with k = 400 every outlier is taken whole.
    say(f"step unsampled outliers k={k}")
    n = 40000
    wl = workloads.gaussian(1, 2, 4, 128, 16, n, k, seed=28, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    kp = kproj_oracle(bits(wl.K), M)
    from oracle.numerics import round_to_bf16
    starts = 2 * ((np.arange(1024, dtype=np.int64) * n) // 2048)
    rows = (starts + 10)[::3][:300]
    assert not np.isin(rows, np.concatenate([starts, starts + 1])).any()
    rng = np.random.default_rng(29)
    for h in range(2):
        qhat = jssa.project_query(jssa.mean_query(q[0, 4 * h:4 * h + 4]), M[h]).astype(np.float64)
        mag = rng.uniform(64.0, 128.0, size=(300, 1))
        kp[0, h, rows] = round_to_bf16(np.sign(qhat)[None, :] * mag)
    o, ix, _ = _run_and_check(wl, kp, k, tag=f"outliers k{k}")
    for h in range(2):
        if k == 400:
            assert np.isin(rows, ix[0, h]).all()
        else:
            assert np.isin(ix[0, h], rows).all()


def test_many_equal_keys_at_the_boundary_with_shifted_keys():
    # projected rows c * sign(q_hat): the score grows with c. Most rows take c spread
    # over [0.1, 4] (a wide key range, so the candidates' relative keys are shifted),
    # 200 identical rows take c = 2 and the budget ends halfway through them: the
    # selection meets 200 entries on one relative key and ranks them by exact key,
    # then by position
    say("step many equal keys at the boundary")
    n = 20000
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, 64, seed=33, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    from oracle.numerics import round_to_bf16, bf16_to_f32 as b2f
    rng = np.random.default_rng(34)
    c = b2f(round_to_bf16(rng.uniform(0.1, 4.0, size=n))).astype(np.float64)
    cluster = np.sort(rng.choice(n, size=200, replace=False))
    c[cluster] = 2.0
    kp = round_to_bf16(np.sign(qhat)[None, :] * c[:, None])[None, None]
    k = int(np.sum(c > 2.0)) + 100
    _ties_check(wl, np.ascontiguousarray(kp), k, "equal keys at the boundary")


def test_saturated_boundary_ties_resolve_by_position():
    # 300 outliers between the sampled rows (their candidate keys saturate) in four groups
    # of identical rows: the budget of 100 takes the whole top group and part of the
    # next, so the selection meets 300 entries on the saturated relative key, ranks them
    # by exact key and breaks the ties by position, exactly as the oracle does
    say("step saturated boundary with ties")
    n, k = 40000, 100
    wl = workloads.gaussian(1, 1, 4, 128, 16, n, k, seed=36, device="cuda")
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    kp = kproj_oracle(bits(wl.K), M)
    from oracle.numerics import round_to_bf16
    starts = 2 * ((np.arange(1024, dtype=np.int64) * n) // 2048)
    rows = (starts + 7)[:300]
    assert not np.isin(rows, np.concatenate([starts, starts + 1])).any()
    qhat = jssa.project_query(jssa.mean_query(q[0, 0:4]), M[0]).astype(np.float64)
    mag = np.array([64.0, 80.0, 96.0, 112.0])[np.random.default_rng(37).integers(0, 4, size=300)]
    kp[0, 0, rows] = round_to_bf16(np.sign(qhat)[None, :] * mag[:, None])
    assert np.sum(mag == 112.0) < k < np.sum(mag >= 96.0)
    _ties_check(wl, kp, k, "saturated boundary ties")


def test_units_on_different_paths_in_one_launch():
    # one launch where unit (0,0) has every row identical (its 20001 candidates overflow
    # the lists), (1,0) has the first row of every sampled pair scoring high (1024
    # candidates, fewer than k) and (0,1), (1,1) are ordinary: the exact-path units are
    # recomputed by four workgroups each (over lengths that split unevenly), the others
    # select from their candidates
    say("step units on different paths")
    n, k = 20001, 1500
    seq = [20001, 18000]
    wl = workloads.gaussian(2, 2, 4, 128, 16, n, k, seed=38, device="cuda", capacity=20001, seq_len=seq)
    M = wl.M.cpu().numpy()
    q = bits(wl.q)
    kp = kproj_oracle(bits(wl.K), M)
    kp[0, 0, :] = kp[0, 0, :1]
    qhat = jssa.project_query(jssa.mean_query(q[1, 0:4]), M[0]).astype(np.float64)
    from oracle.numerics import round_to_bf16
    first_of_pair = 2 * ((np.arange(1024, dtype=np.int64) * 18000) // 2048)
    kp[1, 0, :] = kp[1, 0, :1]
    kp[1, 0, first_of_pair] = round_to_bf16(np.sign(qhat) * 4.0)
    _ties_check(wl, np.ascontiguousarray(kp), k, "mixed paths")


def test_blind_spot_input_takes_the_exact_path():
    # the sampled rows are the quietest of every sequence (keys x 1/16): the threshold
    # falls far below the k-th score, every unit's candidates exceed the lists and the
    # exact path selects; every unit against the oracle
    say("step sampler blind spot")
    wl = workloads.long_batched_blind_spot(batch=2, n=32768, k=2048, device="cuda")
    kp = kproj_oracle(bits(wl.K), wl.M.cpu().numpy())
    _run_and_check(wl, kp, 2048, out_f32=False, tag="blind spot")
