#!/usr/bin/env python3
"""Benchmark one sparse decode step of the 128K batched-decode workload on one MI355X.

A step is the whole hot path on one batch: append the current token (K, V and its
projected scoring row), scoring prep and the full-context score scan (one launch:
the prep workgroups hand q_hat and the threshold to the scan workgroups), per-KV-head
top-k, and gather-free attention with the split merge. Inputs are resident in HBM
before timing starts. Throughput comes from steps run back to back between one
pair of events; a second timed pass brackets every stage with HIP events on the
stream the kernels run on, which gives the prep + scan kernel's own duration.

Prints one JSON line. Default: --gpus 1 --steps 200 --warmup 20.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOAD = ("long-batched decode step: batch 16, 32 query / 8 KV heads (G=4), d=128, n=131072 cached tokens "
            "per sequence, scoring rank r=32, budget k=4096; bf16 K/V with RoPE (base 500000) and 1% heavy "
            "hitters (key x4), random orthonormal basis per KV head, 8 query sets cycled")
PMC_FILE = os.path.join(ROOT, "profiles", "prep_scan_kernel_long_batched_pmc.json")
SCAN_SOURCES = [os.path.join(ROOT, "token_level_sparse_kv_amd", "csrc", f)
                for f in ("score.hip", "sjsa_device.h", "key_proj.h")]


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of known size, for scaling rocprofv3 counters."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def traffic_from_profile(scan_bytes_per_launch):
    """HBM bytes per prep + scan launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    try:
        with open(PMC_FILE) as f:
            p = json.load(f)
    except (OSError, ValueError):
        return None
    try:
        if p.get("source_sha256") != source_hash(SCAN_SOURCES):
            return None
    except OSError:
        return None
    fetch = p["fetch_kib_per_launch"] * 1024.0 / p["copy_fetch_factor"]
    write = p["write_kib_per_launch"] * 1024.0 / p["copy_write_factor"]
    return fetch + write


def cpu_baseline(host, units, k, scale, gpu_out, gpu_idx):
    """The oracle, as it stands, on a sample of (sequence, KV head) units of the same
    step, with a thread pool over units. Also checks the GPU results of those units."""
    import numpy as np
    from oracle import jssa
    q, K, V, Kp, M, G = host["q"], host["K"], host["V"], host["Kp"], host["M"], host["G"]
    n = K.shape[1]                      # K is [units, n, d]
    workers = max(1, min(16, os.cpu_count() or 1))

    def run(i):
        b, h = units[i]
        return jssa.decode_unit(q[b, h * G:(h + 1) * G], K[i], V[i], Kp[i], M[h], n, k, scale)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(run, range(len(units))))
    dt = time.perf_counter() - t0
    ok = True
    worst = 0.0
    for i, (b, h) in enumerate(units):
        ref_out, ref_idx, s = res[i]
        g = gpu_idx[i]
        T = np.sort(s[ref_idx])[0]
        diff = np.setxor1d(g, ref_idx)
        ok &= bool(np.all(np.diff(g) > 0)) and bool(np.all(np.abs(s[diff] - T) <= 1e-3 * abs(T)))
        mine = jssa.attend(q[b, h * G:(h + 1) * G], K[i], V[i], g, scale)
        worst = max(worst, float(np.max(np.abs(gpu_out[i] - mine))))
    return dt, workers, ok, worst


def oracle_timing(jobs):
    """Wall time of the oracle jobs (callables) on a thread pool, and the thread count."""
    workers = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(lambda f: f(), jobs))
    return time.perf_counter() - t0, workers, res


def _bits(t):
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def fp8_variant(sj, wl, K, V, M, seq_len, q_sets, k_new, v_new, pos_new, steps, warmup, step_bytes, peak,
                cpu=False):
    """The same step over an FP8 E4M3 scoring cache (one byte per element), timed the
    same way. Reported beside the bf16 figure, which stays the headline."""
    import numpy as np
    import torch
    B, Hkv, G, d, r, n, k = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim, wl.rank, wl.capacity, wl.k
    dev = K.device
    K, V = K.clone(), V.clone()
    Kp8 = torch.empty(B, Hkv, n, r, dtype=torch.uint8, device=dev)
    T = 8192
    for t0 in range(0, n, T):
        pos = torch.full((B,), t0, dtype=torch.int32, device=dev)
        sj.append_kv(K[:, :, t0:t0 + T].contiguous(), V[:, :, t0:t0 + T].contiguous(), M, pos, K, V, Kp8)
    shape = sj.make_shape(B, Hkv, G, d, r, n, kproj_fp8=True)
    ws = sj.alloc_workspace(shape, k, dev)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hkv * G, d, dtype=torch.bfloat16, device=dev)

    def step(i):
        q = q_sets[i % q_sets.shape[0]]
        sj.prep_scan(shape, q, M, Kp8, seq_len, k, ws, k_new=k_new, v_new=v_new, pos=pos_new, K=K, V=V)
        sj.select(shape, Kp8, seq_len, k, ws, idx=idx)
        sj.attend(q, K, V, idx, seq_len, out=out, workspace=ws, rank=r)

    for i in range(warmup):
        step(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    tb = step_bytes(B, Hkv, G, d, r, n, k, kb=1)
    gbs = tb["total"] / (ms * 1e-3) / 1e9
    res = {"kproj_dtype": "fp8_e4m3", "value": round(1000.0 / ms, 2), "unit": "steps/s",
           "ms_per_step": round(ms, 5), "algorithmic_bytes_per_step": tb["total"], "hbm_gbs": round(gbs, 1),
           "hbm_frac_of_peak": round(gbs / peak, 4)}
    if cpu:
        from oracle import jssa
        units = [(b, h) for b in range(0, B, 4) for h in range(0, Hkv, 2)]       # 16 of 128
        q = _bits(q_sets[0])
        Mh = M.cpu().numpy()
        scale = jssa.default_sm_scale(d)
        jobs = []
        for b, h in units:
            Kb, Vb, Pb = _bits(K[b, h]), _bits(V[b, h]), Kp8[b, h].cpu().numpy()
            jobs.append(lambda b=b, h=h, Kb=Kb, Vb=Vb, Pb=Pb: jssa.decode_unit(
                q[b, h * G:(h + 1) * G], Kb, Vb, Pb, Mh[h], n, k, scale, "fp8"))
        dt, workers, _ = oracle_timing(jobs)
        scale_up = B * Hkv / len(units)
        res["cpu_baseline"] = {"value": round(1.0 / (dt * scale_up), 4), "unit": "steps/s", "cores": workers,
                               "kind": "oracle", "sample": f"{len(units)} of {B * Hkv} units of one step, wall "
                                                           f"time scaled by {scale_up:g}"}
    return res


GATED_WORKLOAD = ("gated-logit decode step: batch 1, 32 query / 8 KV heads (G=4), d=128, n=32768 in 512 units of "
                  "64 tokens, budget 32 units (current unit kept), lambda=1; gate scores ~ N(0,1); 4 input sets "
                  "rotated so the K/V rows are not cache resident")


def gated_variant(sj, workloads, steps, warmup, peak, cpu=False):
    """The gated-logit (unit-gated) step at its own workload, timed back to back over
    4 rotating input sets (together larger than the last-level cache)."""
    import torch
    sets = [workloads.gated_config(seed=4 + i, device="cuda") for i in range(4)]
    wl = sets[0]
    unit, k_units = wl.extra["unit_size"], wl.extra["k_units"]
    shape = sj.gated_shape(wl.q, wl.K)
    ws = sj.gated_workspace(shape, unit, k_units)
    out = torch.empty_like(wl.q)
    idx = torch.empty(wl.batch, wl.n_kv_heads, unit * k_units, dtype=torch.int32, device="cuda")

    def step(i):
        w = sets[i % len(sets)]
        sj.gated_decode_step(w.q, w.K, w.V, w.extra["gate_scores"], w.seq_len, unit, k_units, lam=1.0, out=out,
                             idx=idx, workspace=ws)

    for i in range(warmup):
        step(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    units = wl.batch * wl.n_kv_heads
    ktok = unit * k_units
    kv = units * ktok * wl.head_dim * 2 * 2
    nbytes = (kv + units * (wl.capacity // unit) * 4 + 2 * wl.q.numel() * 2 + units * ktok * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": GATED_WORKLOAD, "value": round(1000.0 / ms, 2), "unit": "steps/s",
           "us_per_step": round(ms * 1000.0, 2), "algorithmic_bytes_per_step": nbytes, "kv_row_bytes": kv,
           "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / peak, 4), "bound": "latency"}
    if cpu:
        from oracle import jssa, sas
        q = _bits(wl.q)
        u = wl.extra["gate_scores"].cpu().numpy()
        G = wl.group
        n = int(wl.seq_len[0])
        jobs = []
        for h in range(wl.n_kv_heads):
            Kb, Vb = _bits(wl.K[0, h]), _bits(wl.V[0, h])
            jobs.append(lambda h=h, Kb=Kb, Vb=Vb: sas.gated_decode_unit(
                q[0, h * G:(h + 1) * G], Kb, Vb, u[0, h], n, unit, k_units, 1.0, jssa.default_sm_scale(128)))
        dt, workers, _ = oracle_timing(jobs)
        res["cpu_baseline"] = {"value": round(1.0 / dt, 2), "unit": "steps/s", "cores": workers, "kind": "oracle",
                               "sample": "all 8 (sequence, KV head) units of one step"}
    return res


BLOCK_WORKLOAD = ("block-sparse decode step: batch 4, 64 query / 8 KV heads (G=8), d=128, n=65536 in 1024 blocks "
                  "of 64, 16 blocks kept (first block and the two local blocks forced); mean block keys; K/V with "
                  "RoPE; 4 input sets rotated so the K/V rows are not cache resident")


def block_variant(sj, workloads, steps, warmup, peak, int4, cpu=False):
    """The block-sparse step at its own workload (bf16 or INT4 block keys), timed back
    to back over 4 rotating input sets."""
    import torch
    sets = []
    for i in range(4):
        w = workloads.block_config(seed=5 + i, device="cuda")
        bsz = w.extra["block_size"]
        w.extra["keys"] = sj.block_cache(w.K, bsz, int4=int4, bf16=not int4)
        sj.block_keys(w.K, w.seq_len, bsz, *w.extra["keys"])
        sets.append(w)
    wl = sets[0]
    bsz, k_blocks = wl.extra["block_size"], wl.extra["k_blocks"]
    shape = sj.gated_shape(wl.q, wl.K)
    ws = sj.block_workspace(shape, bsz, k_blocks)
    out = torch.empty_like(wl.q)
    idx = torch.empty(wl.batch, wl.n_kv_heads, bsz * k_blocks, dtype=torch.int32, device="cuda")

    def step(i):
        w = sets[i % len(sets)]
        Kc, Kq, Ks = w.extra["keys"]
        sj.block_decode_step(w.q, w.K, w.V, w.seq_len, bsz, k_blocks, Kc, Kq, Ks, 1, 2, out=out, idx=idx,
                             workspace=ws)

    for i in range(warmup):
        step(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    units = wl.batch * wl.n_kv_heads
    nblk = wl.capacity // bsz
    key_bytes = units * nblk * (wl.head_dim // 2 + 2 * (wl.head_dim // 64) if int4 else wl.head_dim * 2)
    kv = units * k_blocks * bsz * wl.head_dim * 2 * 2
    nbytes = key_bytes + kv + 2 * wl.q.numel() * 2 + units * k_blocks * bsz * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": BLOCK_WORKLOAD, "block_keys": "int4" if int4 else "bf16", "value": round(1000.0 / ms, 2),
           "unit": "steps/s", "us_per_step": round(ms * 1000.0, 2), "algorithmic_bytes_per_step": nbytes,
           "block_key_bytes": key_bytes, "kv_row_bytes": kv, "hbm_gbs": round(gbs, 1),
           "hbm_frac_of_peak": round(gbs / peak, 4), "bound": "latency"}
    if cpu:
        from oracle import blocksparse, jssa
        from oracle.numerics import bf16_to_f32
        q = _bits(wl.q)
        G = wl.group
        n = int(wl.seq_len[0])
        m = n // bsz
        Kc, Kq, Ks = wl.extra["keys"]
        units = [(b, h) for b in range(wl.batch) for h in (0, 5)]                 # 8 of 32
        jobs = []
        for b, h in units:
            Kb, Vb = _bits(wl.K[b, h]), _bits(wl.V[b, h])
            if int4:
                kcv = blocksparse.int4_dequantize(blocksparse.unpack_int4(Kq[b, h, :m].cpu().numpy()),
                                                  _bits(Ks[b, h, :m]))
            else:
                kcv = bf16_to_f32(_bits(Kc[b, h, :m]))
            jobs.append(lambda b=b, h=h, Kb=Kb, Vb=Vb, kcv=kcv: blocksparse.decode_unit(
                q[b, h * G:(h + 1) * G], Kb, Vb, kcv, n, bsz, k_blocks, 1, 2, jssa.default_sm_scale(128)))
        dt, workers, _ = oracle_timing(jobs)
        units_total = wl.batch * wl.n_kv_heads
        scale_up = units_total / len(units)
        res["cpu_baseline"] = {"value": round(1.0 / (dt * scale_up), 3), "unit": "steps/s", "cores": workers,
                               "kind": "oracle", "sample": f"{len(units)} of {units_total} units of one step, "
                                                           f"wall time scaled by {scale_up:g}"}
    return res


CALIB_WORKLOAD = ("calibration accumulation: one 131072-token prefill, 32 query / 8 KV heads (G=4), d=128; "
                  "second-moment sums of the group-mean query and of the key per KV head")
# fp32 FMA peak for non-packed instructions: 256 CUs x 64 FMA lanes per clock x 2 flops x
# 2.4 GHz. The published 157.3 TFLOP/s counts packed FP32 (two FMAs per lane per
# instruction), which this build does not emit.
FP32_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
FP32_PACKED_PEAK_TFLOPS = 157.3


def calib_variant(sj, reps, warmup, cpu=False):
    """Second-moment accumulation over one prefill of 131072 tokens (the pages'
    calibration sequence length), timed over repeated calls."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    T, Hkv, G = 131072, 8, 4
    q = torch.randn(1, Hkv * G, T, 128, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, Hkv, T, 128, generator=g, device="cuda").to(torch.bfloat16)
    SQ = torch.zeros(Hkv, 128, 128, dtype=torch.float64, device="cuda")
    SK = torch.zeros_like(SQ)
    ws = sj.calib_workspace(q, k)
    for _ in range(warmup):
        sj.calib_accumulate(q, k, SQ, SK, workspace=ws)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        sj.calib_accumulate(q, k, SQ, SK, workspace=ws)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    flops = 2 * Hkv * T * 128 * 128 * 2            # both moment matrices, multiply + add per element
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": CALIB_WORKLOAD, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
           "ms_per_prefill": round(ms, 4), "bound": "alu", "achieved_tflops": round(tf, 2),
           "peak_tflops": round(FP32_PEAK_TFLOPS, 2), "frac": round(tf / FP32_PEAK_TFLOPS, 4),
           "packed_fp32_peak_tflops": FP32_PACKED_PEAK_TFLOPS,
           "input_bytes": q.numel() * 2 + k.numel() * 2}
    if cpu:
        from oracle import calib
        P = 4096                                    # positions per sampled KV head
        heads = [0, 3, 6, 7]
        jobs = []
        for h in heads:
            qh = _bits(q[0, h * G:(h + 1) * G, :P]).transpose(1, 0, 2).copy()      # [P, G, d]
            kh = _bits(k[0, h, :P])
            jobs.append(lambda qh=qh, kh=kh: calib.accumulate_moments(qh, kh))
        dt, workers, _ = oracle_timing(jobs)
        sampled = P * len(heads)
        res["cpu_baseline"] = {"value": round(sampled / Hkv / dt, 1), "unit": "tokens/s", "cores": workers,
                               "kind": "oracle", "sample": f"{P} positions of {len(heads)} of {Hkv} KV heads; "
                                                           f"tokens/s = positions per KV head / wall time"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-units", type=int, default=16, help="units sampled for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-fp8-variant", action="store_true", help="skip the FP8 scoring-cache measurement")
    ap.add_argument("--no-gated-variant", action="store_true", help="skip the gated-logit step measurement")
    ap.add_argument("--no-block-variant", action="store_true", help="skip the block-sparse step measurements")
    ap.add_argument("--no-calib-variant", action="store_true", help="skip the calibration accumulation measurement")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (this build measures the "
              f"single-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(1 << 30, 5)
        return

    import numpy as np
    import torch

    import token_level_sparse_kv_amd as sj
    import workloads
    from token_level_sparse_kv_amd.perfmodel import MI355X_HBM_PEAK_GBS, step_bytes

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.time()
    wl = workloads.long_batched(device=dev, n_q_sets=8)
    B, Hkv, G, d, r, n, k = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim, wl.rank, wl.capacity, wl.k
    q_sets = wl.extra["q_sets"]
    K, V, M, seq_len = wl.K, wl.V, wl.M, wl.seq_len
    # projected scoring cache, built by the library's append over every cached token
    Kp = torch.empty(B, Hkv, n, r, dtype=torch.bfloat16, device=dev)
    T = 8192
    for t0 in range(0, n, T):
        pos = torch.full((B,), t0, dtype=torch.int32, device=dev)
        sj.append_kv(K[:, :, t0:t0 + T].contiguous(), V[:, :, t0:t0 + T].contiguous(), M, pos, K, V, Kp)
    k_new, v_new = workloads.new_token(wl, seed=99)
    pos_new = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
    shape = sj.make_shape(B, Hkv, G, d, r, n)
    ws = sj.alloc_workspace(shape, k, dev)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hkv * G, d, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    def step(i, ev=None):
        # the stage calls of sjsa_decode_step_append: one launch appends the new token
        # (K, V and projected rows), preps and scans; then select, attend + merge
        q = q_sets[i % q_sets.shape[0]]
        if ev is not None:
            ev[0].record()
        sj.prep_scan(shape, q, M, Kp, seq_len, k, ws, k_new=k_new, v_new=v_new, pos=pos_new, K=K, V=V)
        if ev is not None:
            ev[1].record()
        sj.select(shape, Kp, seq_len, k, ws, idx=idx)
        if ev is not None:
            ev[2].record()
        sj.attend(q, K, V, idx, seq_len, out=out, workspace=ws, rank=r)
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # throughput: K whole steps back to back, bracketed by one pair of events (an event
    # between two kernels delays the second by several microseconds, so the steps
    # themselves carry none)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    # stage durations: the same K steps again with an event between consecutive
    # stages, all on the stream the kernels run on (torch's current stream); each
    # interval also holds the launch latency of its first kernel, so these figures
    # slightly overstate the kernels' own durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    names = ["append+prep+scan", "select", "attend"]
    stage_ms = {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, nm in enumerate(names)}

    tb = step_bytes(B, Hkv, G, d, r, n, k)
    gbs = tb["total"] / (ms_per_step * 1e-3) / 1e9
    # the prep + scan launch moves the projected cache, q, M and the appended rows
    scan_bytes = tb["scan_kproj"] + tb["q"] + tb["M"] + tb["append"]
    scan_gbs = scan_bytes / (stage_ms["append+prep+scan"] * 1e-3) / 1e9
    traffic = traffic_from_profile(scan_bytes)

    line = {
        "metric": "sparse decode steps/s + achieved HBM GB/s (% of peak) at 128K ctx",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": B, "n_q_heads": Hkv * G, "n_kv_heads": Hkv, "head_dim": d,
                   "context": n, "rank": r, "k": k, "kproj_dtype": "bf16"},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / MI355X_HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": tb["total"],
        "stage_us": {kk: round(v * 1000.0, 2) for kk, v in stage_ms.items()},
        "roofline": {"kernel": "prep + score scan (prep_scan_kernel<32,2,true>)", "bound": "hbm",
                     "achieved": round(scan_gbs, 1), "bytes_per_launch": scan_bytes,
                     "peak": MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / MI355X_HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "setup_s": round(t_setup, 2),
    }

    print(f"timed: {ms_per_step * 1000:.1f} us/step, stages (us) {line['stage_us']}", file=sys.stderr, flush=True)
    if not args.no_gated_variant:
        line["gated_variant"] = gated_variant(sj, workloads, args.steps, args.warmup, MI355X_HBM_PEAK_GBS,
                                              cpu=not args.no_cpu_baseline)
    if not args.no_block_variant:
        line["block_variant"] = block_variant(sj, workloads, args.steps, args.warmup, MI355X_HBM_PEAK_GBS, False,
                                              cpu=not args.no_cpu_baseline)
        line["block_int4_variant"] = block_variant(sj, workloads, args.steps, args.warmup, MI355X_HBM_PEAK_GBS,
                                                   True, cpu=not args.no_cpu_baseline)
    if not args.no_calib_variant:
        line["calib_variant"] = calib_variant(sj, max(2, args.steps // 20), 1, cpu=not args.no_cpu_baseline)
    if not args.no_fp8_variant:
        line["kproj_fp8_variant"] = fp8_variant(sj, wl, K, V, M, seq_len, q_sets, k_new, v_new, pos_new, args.steps,
                                                args.warmup, step_bytes, MI355X_HBM_PEAK_GBS,
                                                cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        rng = np.random.default_rng(3)
        all_units = [(b, h) for b in range(B) for h in range(Hkv)]
        pick = sorted(rng.choice(len(all_units), size=min(args.cpu_units, len(all_units)), replace=False))
        units = [all_units[i] for i in pick]
        step(0)
        torch.cuda.synchronize()
        q0 = q_sets[0]

        def bits(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        host = {"q": bits(q0), "M": M.cpu().numpy(), "G": G,
                "K": np.stack([bits(K[b, h]) for b, h in units]),
                "V": np.stack([bits(V[b, h]) for b, h in units]),
                "Kp": np.stack([bits(Kp[b, h]) for b, h in units])}
        go = out.float().cpu().numpy()
        gi = idx.cpu().numpy()
        gpu_out = np.stack([go[b, h * G:(h + 1) * G] for b, h in units])
        gpu_idx = np.stack([gi[b, h] for b, h in units])
        dt, workers, ok, worst = cpu_baseline(host, units, k, 1.0 / np.sqrt(d), gpu_out, gpu_idx)
        scale_up = len(all_units) / len(units)
        line["cpu_baseline"] = {"value": round(1.0 / (dt * scale_up), 4), "unit": "steps/s", "cores": workers,
                                "kind": "oracle",
                                "sample": f"{len(units)} of {len(all_units)} (sequence, KV head) units of one "
                                          f"step (scoring, top-k, exact attention), wall time scaled by "
                                          f"{scale_up:g}; NumPy, thread pool over units"}
        line["parity_sample"] = {"units": len(units), "idx_band_ok": bool(ok), "max_abs_out_err": worst}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
