#!/usr/bin/env python3
"""Benchmark one sparse decode step of the 128K batched-decode workload on one MI355X.

A step is the whole hot path on one batch: append the current token (K, V and its
projected scoring row), scoring prep and the full-context score scan (one launch:
the prep workgroups hand q_hat and the threshold to the scan workgroups), per-KV-head
top-k, and gather-free attention with the split merge. Inputs are resident in HBM
before timing starts.

Timings of the headline step (all on the stream the kernels run on):
  * throughput: K steps back to back between one pair of events (`value`,
    `ms_per_step`);
  * per-step percentiles: the K steps again with an event between consecutive steps;
  * stages: an event between consecutive stages (the prep + scan kernel's own time);
  * flushed: a 1 GiB write between steps, outside each step's events;
  * rotated: two full input sets (about 19 GB) alternated back to back;
  * graph: 8 steps captured as one HIP graph and replayed;
  * the read ceiling of the same GPU: a plain streaming-read kernel.
Variants (their own workloads and entry points) follow: the exact fallback (scan
workgroups that never wait), an input that blinds the threshold sampler, the FP8
scoring cache, the gated-logit and block-sparse steps (eager and graph-replayed),
and the calibration accumulation. The oracle is timed on the whole step (all 128
units, median of 3) on the host's cores, and every unit's GPU result is checked
against it.

Prints one JSON line. Default: --gpus 1 --steps 200 --warmup 20.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import os
import platform
import statistics
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
                for f in ("score.hip", "sjsa_device.h", "key_proj.h", "sjsa_internal.h")]
MEMBW_LIB = os.path.join(ROOT, "token_level_sparse_kv_amd", "lib", "libsjsa_membw.so")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


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


def traffic_from_profile():
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


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # the oracle's thread pool: at most 16 threads, whatever the OS reports as available
    pool = max(1, min(16, avail))
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": avail, "pool_threads": pool}


# ------------------------------------------------------------------ GPU timing helpers
def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def back_to_back_us(fn, steps, warmup):
    """Mean microseconds per call of fn(i) over `steps` calls between one pair of events."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = _ev(), _ev()
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1000.0


def percentiles_us(fn, steps, between=None):
    """p10 / p50 / p90 of per-call times, an event pair around every call; `between`
    runs before each call, outside its events."""
    import numpy as np
    import torch
    torch.cuda.synchronize()
    pairs = []
    for i in range(steps):
        if between is not None:
            between()
        a, b = _ev(), _ev()
        a.record()
        fn(i)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    x = np.array([a.elapsed_time(b) * 1000.0 for a, b in pairs])
    return {"p10": round(float(np.percentile(x, 10)), 2), "p50": round(float(np.median(x)), 2),
            "p90": round(float(np.percentile(x, 90)), 2)}


def graph_us(fn, n_per_graph, steps):
    """Microseconds per call of fn(i) when n_per_graph calls (i = 0 ..) are captured as
    one HIP graph and the graph is replayed back to back."""
    import torch
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):                 # warm-up on the capture stream
        for i in range(n_per_graph):
            fn(i)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_per_graph):
            fn(i)
    torch.cuda.synchronize()
    reps = max(2, steps // n_per_graph)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    a, b = _ev(), _ev()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / (reps * n_per_graph) * 1000.0
    del g
    return us


def read_ceiling_gbs(buf):
    """Best streaming-read rate over a few launch shapes (libsjsa_membw), GB/s."""
    import torch
    lib = ctypes.CDLL(MEMBW_LIB)
    lib.sjsa_membw_read.restype = ctypes.c_int
    lib.sjsa_membw_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    sink = torch.zeros(32768, dtype=torch.int32, device=buf.device)
    best = 0.0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for wgs in (2048, 4096, 8192, 16384, 32768):
        def run(_i, wgs=wgs):
            if lib.sjsa_membw_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, ctypes.c_void_p(sink.data_ptr()),
                                   stream) != 0:
                raise RuntimeError("read probe launch failed")
        us = back_to_back_us(run, 10, 3)
        best = max(best, nbytes / (us * 1e-6) / 1e9)
    return best


def _bits(t):
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ oracle on the host
def oracle_step(host, units, k, scale, pool, reps=1, fmt="bf16"):
    """The oracle (as it stands) on `units` (a list of (b, h)), a thread pool over units.
    Returns (median wall seconds over reps, per-unit results)."""
    from oracle import jssa
    q, K, V, Kp, M, G, n = host["q"], host["K"], host["V"], host["Kp"], host["M"], host["G"], host["n"]

    def run(u):
        b, h = u
        return jssa.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], Kp[b, h], M[h], n, k, scale, fmt)

    times, res = [], None
    with cf.ThreadPoolExecutor(max_workers=pool) as ex:
        for _ in range(reps):
            t0 = time.perf_counter()
            res = list(ex.map(run, units))
            times.append(time.perf_counter() - t0)
    return statistics.median(times), res


def parity_summary(host, units, results, gpu_out, gpu_idx, scale):
    """Band rule on idx and max |out - oracle attention over the GPU's idx| per unit."""
    import numpy as np
    from oracle import jssa
    q, K, V, G, n = host["q"], host["K"], host["V"], host["G"], host["n"]
    ok, worst, diff_units = True, 0.0, 0
    for (b, h), (ref_out, ref_idx, s) in zip(units, results):
        g = gpu_idx[b, h]
        T = np.sort(s[ref_idx[ref_idx >= 0]])[0]
        diff = np.setxor1d(g[g >= 0], ref_idx[ref_idx >= 0])
        diff_units += int(diff.size > 0)
        ok &= bool(np.all(np.diff(g[g >= 0]) > 0)) and bool(np.all(np.abs(s[diff] - T) <= 1e-3 * abs(T)))
        mine = jssa.attend(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], g, scale)
        worst = max(worst, float(np.max(np.abs(gpu_out[b, h * G:(h + 1) * G] - mine))))
    return {"units": len(units), "idx_band_ok": bool(ok), "units_with_band_differences": diff_units,
            "max_abs_out_err": worst, "out_tol": 2e-2}


# ------------------------------------------------------------------ variants
def fp8_variant(sj, wl, K, V, M, seq_len, q_sets, k_new, v_new, pos_new, steps, warmup, step_bytes, peak,
                cpu=None):
    """The same step over an FP8 E4M3 scoring cache (one byte per element), timed the
    same way. Reported beside the bf16 figure, which stays the headline."""
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

    def step(i, ev=None):
        q = q_sets[i % q_sets.shape[0]]
        if ev is not None:
            ev[0].record()
        sj.prep_scan(shape, q, M, Kp8, seq_len, k, ws, k_new=k_new, v_new=v_new, pos=pos_new, K=K, V=V)
        if ev is not None:
            ev[1].record()
        sj.select(shape, Kp8, seq_len, k, ws, idx=idx)
        if ev is not None:
            ev[2].record()
        sj.attend(q, K, V, idx, seq_len, out=out, workspace=ws, rank=r)
        if ev is not None:
            ev[3].record()

    us = back_to_back_us(step, steps, warmup)
    evs = [[_ev() for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stages = {nm: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps * 1000.0, 2)
              for j, nm in enumerate(["append+prep+scan", "select", "attend"])}
    tb = step_bytes(B, Hkv, G, d, r, n, k, kb=1)
    gbs = tb["total"] / (us * 1e-6) / 1e9
    scan_bytes = tb["scan_kproj"] + tb["q"] + tb["M"] + tb["append"]
    res = {"kproj_dtype": "fp8_e4m3", "value": round(1e6 / us, 2), "unit": "steps/s",
           "ms_per_step": round(us / 1000.0, 5), "algorithmic_bytes_per_step": tb["total"], "hbm_gbs": round(gbs, 1),
           "hbm_frac_of_peak": round(gbs / peak, 4), "stage_us": stages,
           "scan_hbm_frac_of_peak": round(scan_bytes / (stages["append+prep+scan"] * 1e-6) / 1e9 / peak, 4),
           "graph_us_per_step": round(graph_us(step, 8, steps), 2)}
    say(f"fp8: {us:.1f} us/step, stages {stages}")
    if cpu is not None:
        from oracle import jssa
        units = [(b, h) for b in range(B) for h in range(Hkv)]
        step(0)
        torch.cuda.synchronize()
        host = {"q": _bits(q_sets[0]), "K": _bits(K), "V": _bits(V), "Kp": Kp8.cpu().numpy(), "M": M.cpu().numpy(),
                "G": G, "n": n}
        dt, results = oracle_step(host, units, k, jssa.default_sm_scale(d), cpu["pool_threads"], fmt="fp8")
        res["cpu_baseline"] = {"value": round(1.0 / dt, 4), "unit": "steps/s", "cores": cpu["pool_threads"],
                               "kind": "oracle", "sample": f"all {len(units)} units of one step (one run)",
                               **{kk: cpu[kk] for kk in ("cpu_model", "os_cpu_count")}}
        res["parity_all_units"] = parity_summary(host, units, results, out.float().cpu().numpy(), idx.cpu().numpy(),
                                                 jssa.default_sm_scale(d))
        del host
    return res


GATED_WORKLOAD = ("gated-logit decode step: batch 1, 32 query / 8 KV heads (G=4), d=128, n=32768 in 512 units of "
                  "64 tokens, budget 32 units (current unit kept), lambda=1; gate scores ~ N(0,1); 4 input sets "
                  "rotated so the K/V rows are not cache resident")


def gated_variant(sj, workloads, steps, warmup, peak, cpu=None):
    """The gated-logit (unit-gated) step at its own workload, timed back to back over
    4 rotating input sets (together larger than the last-level cache), eagerly and as
    a replayed graph of 4 steps."""
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

    us = back_to_back_us(step, steps, warmup)
    gus = graph_us(step, len(sets), steps)
    units = wl.batch * wl.n_kv_heads
    ktok = unit * k_units
    kv = units * ktok * wl.head_dim * 2 * 2
    nbytes = (kv + units * (wl.capacity // unit) * 4 + 2 * wl.q.numel() * 2 + units * ktok * 4)
    best = min(us, gus)
    gbs = nbytes / (best * 1e-6) / 1e9
    res = {"workload": GATED_WORKLOAD, "value": round(1e6 / best, 2), "unit": "steps/s",
           "us_per_step": round(best, 2), "eager_us_per_step": round(us, 2), "graph_us_per_step": round(gus, 2),
           "algorithmic_bytes_per_step": nbytes, "kv_row_bytes": kv,
           "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / peak, 4), "bound": "latency"}
    if cpu is not None:
        from oracle import jssa, sas
        q = _bits(wl.q)
        u = wl.extra["gate_scores"].cpu().numpy()
        G = wl.group
        n = int(wl.seq_len[0])
        Kb, Vb = _bits(wl.K), _bits(wl.V)
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=cpu["pool_threads"]) as ex:
            list(ex.map(lambda h: sas.gated_decode_unit(q[0, h * G:(h + 1) * G], Kb[0, h], Vb[0, h], u[0, h], n,
                                                        unit, k_units, 1.0, jssa.default_sm_scale(128)),
                        range(wl.n_kv_heads)))
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(1.0 / dt, 2), "unit": "steps/s", "cores": cpu["pool_threads"],
                               "kind": "oracle", "sample": "all 8 (sequence, KV head) units of one step"}
    return res


BLOCK_WORKLOAD = ("block-sparse decode step: batch 4, 64 query / 8 KV heads (G=8), d=128, n=65536 in 1024 blocks "
                  "of 64, 16 blocks kept (first block and the two local blocks forced); mean block keys; K/V with "
                  "RoPE; 4 input sets rotated so the K/V rows are not cache resident")


def block_variant(sj, workloads, steps, warmup, peak, int4, cpu=None):
    """The block-sparse step at its own workload (bf16 or INT4 block keys), timed back
    to back over 4 rotating input sets, eagerly and as a replayed graph of 4 steps."""
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

    us = back_to_back_us(step, steps, warmup)
    gus = graph_us(step, len(sets), steps)
    units = wl.batch * wl.n_kv_heads
    nblk = wl.capacity // bsz
    key_bytes = units * nblk * (wl.head_dim // 2 + 2 * (wl.head_dim // 64) if int4 else wl.head_dim * 2)
    kv = units * k_blocks * bsz * wl.head_dim * 2 * 2
    nbytes = key_bytes + kv + 2 * wl.q.numel() * 2 + units * k_blocks * bsz * 4
    best = min(us, gus)
    gbs = nbytes / (best * 1e-6) / 1e9
    res = {"workload": BLOCK_WORKLOAD, "block_keys": "int4" if int4 else "bf16", "value": round(1e6 / best, 2),
           "unit": "steps/s", "us_per_step": round(best, 2), "eager_us_per_step": round(us, 2),
           "graph_us_per_step": round(gus, 2), "algorithmic_bytes_per_step": nbytes,
           "block_key_bytes": key_bytes, "kv_row_bytes": kv, "hbm_gbs": round(gbs, 1),
           "hbm_frac_of_peak": round(gbs / peak, 4), "bound": "latency"}
    if cpu is not None:
        from oracle import blocksparse, jssa
        from oracle.numerics import bf16_to_f32
        q = _bits(wl.q)
        G = wl.group
        n = int(wl.seq_len[0])
        m = n // bsz
        Kc, Kq, Ks = wl.extra["keys"]
        Kb, Vb = _bits(wl.K), _bits(wl.V)
        units_l = [(b, h) for b in range(wl.batch) for h in range(wl.n_kv_heads)]
        if int4:
            kq, ks = Kq[:, :, :m].cpu().numpy(), _bits(Ks[:, :, :m])
            kcv = {u: blocksparse.int4_dequantize(blocksparse.unpack_int4(kq[u]), ks[u]) for u in units_l}
        else:
            kcf = bf16_to_f32(_bits(Kc[:, :, :m]))
            kcv = {u: kcf[u] for u in units_l}
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=cpu["pool_threads"]) as ex:
            list(ex.map(lambda u: blocksparse.decode_unit(q[u[0], u[1] * G:(u[1] + 1) * G], Kb[u[0], u[1]],
                                                          Vb[u[0], u[1]], kcv[u], n, bsz, k_blocks, 1, 2,
                                                          jssa.default_sm_scale(128)), units_l))
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(1.0 / dt, 3), "unit": "steps/s", "cores": cpu["pool_threads"],
                               "kind": "oracle", "sample": f"all {len(units_l)} units of one step"}
    return res


CALIB_WORKLOAD = ("calibration accumulation: one 131072-token prefill, 32 query / 8 KV heads (G=4), d=128; "
                  "second-moment sums of the group-mean query and of the key per KV head")
# Published dense matrix-core peaks: fp32 (the mean-query moment's products) and bf16
# (the key moment's products, exact in fp32).
MFMA_FP32_PEAK_TFLOPS = 157.3
MFMA_BF16_PEAK_TFLOPS = 2500.0


def calib_variant(sj, reps, warmup, cpu=None):
    """Second-moment accumulation over one prefill of 131072 tokens (the pages'
    calibration sequence length), timed over repeated calls."""
    import torch
    from token_level_sparse_kv_amd.perfmodel import MI355X_HBM_PEAK_GBS
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    T, Hkv, G = 131072, 8, 4
    q = torch.randn(1, Hkv * G, T, 128, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, Hkv, T, 128, generator=g, device="cuda").to(torch.bfloat16)
    SQ = torch.zeros(Hkv, 128, 128, dtype=torch.float64, device="cuda")
    SK = torch.zeros_like(SQ)
    ws = sj.calib_workspace(q, k)
    us = back_to_back_us(lambda i: sj.calib_accumulate(q, k, SQ, SK, workspace=ws), reps, warmup)
    ms = us / 1000.0
    in_bytes = q.numel() * 2 + k.numel() * 2
    gbs = in_bytes / (ms * 1e-3) / 1e9
    # products formed on the matrix cores: the 36 upper-triangle 16 x 16 tiles of each
    # 128 x 128 moment, one multiply-add per element per position
    tri_flops = Hkv * T * 36 * 256 * 2
    floor_us = (tri_flops / (MFMA_FP32_PEAK_TFLOPS * 1e12) + tri_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
    res = {"workload": CALIB_WORKLOAD, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
           "ms_per_prefill": round(ms, 4), "bound": "hbm", "achieved_gbps": round(gbs, 1),
           "peak_gbps": MI355X_HBM_PEAK_GBS, "frac": round(gbs / MI355X_HBM_PEAK_GBS, 4), "input_bytes": in_bytes,
           "mfma": {"query_fp32_gflop": round(tri_flops / 1e9, 2), "key_bf16_gflop": round(tri_flops / 1e9, 2),
                    "peak_fp32_tflops": MFMA_FP32_PEAK_TFLOPS, "peak_bf16_tflops": MFMA_BF16_PEAK_TFLOPS,
                    "floor_us": round(floor_us, 1), "frac_of_floor": round(floor_us / us, 4)}}
    if cpu is not None:
        from oracle import calib
        P = 4096                                    # positions per sampled KV head
        heads = [0, 3, 6, 7]
        jobs = []
        for h in heads:
            qh = _bits(q[0, h * G:(h + 1) * G, :P]).transpose(1, 0, 2).copy()      # [P, G, d]
            kh = _bits(k[0, h, :P])
            jobs.append(lambda qh=qh, kh=kh: calib.accumulate_moments(qh, kh))
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=cpu["pool_threads"]) as ex:
            list(ex.map(lambda f: f(), jobs))
        dt = time.perf_counter() - t0
        sampled = P * len(heads)
        res["cpu_baseline"] = {"value": round(sampled / Hkv / dt, 1), "unit": "tokens/s", "cores": cpu["pool_threads"],
                               "kind": "oracle", "sample": f"{P} positions of {len(heads)} of {Hkv} KV heads; "
                                                           f"tokens/s = positions per KV head / wall time"}
    return res


def recall_diagnostic(sj, workloads):
    """The tiny single-head workload (32 planted keys at cosine 0.6 with the mean query,
    4 outlier key channels), its basis calibrated by the library from the workload's
    512 samples: how much of the full-dimension top-k (the exact mean-query ranking)
    the rank-16 selection recovers, and how many planted keys each set holds. A
    diagnostic of the method on this input, not a parity check."""
    import numpy as np
    import torch
    from oracle import jssa
    from oracle.numerics import bf16_to_f32
    wl = workloads.tiny_single_head(device="cuda")
    G, d, r, n, k = wl.group, wl.head_dim, wl.rank, wl.capacity, wl.k
    cq = wl.calib_q.permute(1, 0, 2).unsqueeze(0).contiguous().to(torch.bfloat16)       # [1, G, N, d]
    ck = wl.calib_k.unsqueeze(0).unsqueeze(0).contiguous().to(torch.bfloat16)          # [1, 1, N, d]
    SQ = torch.zeros(1, d, d, dtype=torch.float64, device="cuda")
    SK = torch.zeros_like(SQ)
    sj.calib_accumulate(cq, ck, SQ, SK)
    torch.cuda.synchronize()
    M, _ = sj.calib_basis(SQ, SK, r)
    M = torch.from_numpy(M).cuda()
    Kp = torch.empty(1, 1, n, r, dtype=torch.bfloat16, device="cuda")
    sj.append_kv(wl.K, wl.V, M, torch.zeros(1, dtype=torch.int32, device="cuda"), wl.K.clone(), wl.V.clone(), Kp)
    _, idx = sj.decode_step(wl.q, wl.K, wl.V, Kp, M, wl.seq_len, k)
    torch.cuda.synchronize()
    sel = set(idx.cpu().numpy()[0, 0].tolist())
    qbar = jssa.mean_query(_bits(wl.q)[0]).astype(np.float64)
    full = bf16_to_f32(_bits(wl.K)[0, 0]).astype(np.float64) @ qbar
    top_full = set(jssa.select_topk(full.astype(np.float32), k).tolist())
    planted = set(wl.extra["planted"].tolist())
    return {"workload": "tiny single-head step: B=1, one KV head, G=4, d=128, n=4096, r=16, k=256; 32 planted "
                        "keys (cosine 0.6 with the mean query), 4 outlier key channels; basis calibrated by the "
                        "library (sjsa_calib_accumulate + sjsa_calib_basis) from 512 seeded samples",
            "recall_of_full_dim_topk": round(len(sel & top_full) / k, 4),
            "planted_in_selection": len(sel & planted), "planted_in_full_dim_topk": len(top_full & planted),
            "planted": len(planted), "kind": "diagnostic, not parity"}


def batch_sweep(sj, workloads, batches, steps, warmup, peak_gbs):
    """The 128K decode step (the headline's heads, rank and budget) at other batch sizes,
    bf16 and FP8 scoring caches: steps back to back, and the mean time of each stage with
    an event between stages. Shows how the stages' shares move with the batch."""
    import numpy as np
    import torch
    from token_level_sparse_kv_amd.perfmodel import step_bytes
    dev = torch.device("cuda:0")
    rows = []
    for B in batches:
        for fp8 in (False, True):
            say(f"sweep: batch {B}, {'FP8' if fp8 else 'bf16'} scoring cache")
            wl = workloads.long_batched(device=dev, n_q_sets=8, batch=B)
            Hkv, G, d, r, n, k = wl.n_kv_heads, wl.group, wl.head_dim, wl.rank, wl.capacity, wl.k
            K, V, M, seq_len, q_sets = wl.K, wl.V, wl.M, wl.seq_len, wl.extra["q_sets"]
            Kp = torch.empty(B, Hkv, n, r, dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
            for t0 in range(0, n, 8192):
                pos = torch.full((B,), t0, dtype=torch.int32, device=dev)
                sj.append_kv(K[:, :, t0:t0 + 8192].contiguous(), V[:, :, t0:t0 + 8192].contiguous(), M, pos, K, V,
                             Kp)
            k_new, v_new = workloads.new_token(wl, seed=99)
            pos_new = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
            shape = sj.make_shape(B, Hkv, G, d, r, n, kproj_fp8=fp8)
            ws = sj.alloc_workspace(shape, k, dev)
            idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
            out = torch.empty(B, Hkv * G, d, dtype=torch.bfloat16, device=dev)

            def step(i, ev=None):
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

            us = back_to_back_us(step, steps, warmup)
            evs = [[_ev() for _ in range(4)] for _ in range(steps)]
            torch.cuda.synchronize()
            for i in range(steps):
                step(i, evs[i])
            torch.cuda.synchronize()
            stages = {nm: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1000.0, 2)
                      for j, nm in enumerate(["append+prep+scan", "select", "attend+merge"])}
            tb = step_bytes(B, Hkv, G, d, r, n, k, kb=1 if fp8 else 2)
            rows.append({"batch": B, "kproj_dtype": "fp8_e4m3" if fp8 else "bf16", "us_per_step": round(us, 2),
                         "algorithmic_bytes_per_step": tb["total"],
                         "hbm_frac_of_peak": round(tb["total"] / (us * 1e-6) / 1e9 / peak_gbs, 4),
                         "stage_us": stages})
            say(json.dumps(rows[-1]))
            del wl, K, V, M, Kp, ws, q_sets, idx, out
            torch.cuda.empty_cache()
    return rows


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["headline", "fp8", "exact", "gated", "block", "calib", "sweep"],
                    help="run one measurement only, for profiling: the headline step's passes (one JSON line, no "
                         "variants), or one variant (its JSON object alone); sweep: the step at batch 1 to 64 "
                         "(not part of the default run)")
    ap.add_argument("--no-fp8-variant", action="store_true", help="skip the FP8 scoring-cache measurement")
    ap.add_argument("--no-gated-variant", action="store_true", help="skip the gated-logit step measurement")
    ap.add_argument("--no-block-variant", action="store_true", help="skip the block-sparse step measurements")
    ap.add_argument("--no-calib-variant", action="store_true", help="skip the calibration accumulation measurement")
    ap.add_argument("--no-fallback-variants", action="store_true",
                    help="skip the exact-fallback and sampler blind-spot measurements")
    args = ap.parse_args()

    only = args.only
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the step is measured on "
              f"one GPU's share of the batch)", file=sys.stderr)
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
    cpu = None if args.no_cpu_baseline or only else host_info()
    steps, warmup = args.steps, args.warmup
    if only == "gated":
        print(json.dumps({"gated_variant": gated_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS)}))
        return
    if only == "block":
        print(json.dumps({"block_variant": block_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS, False),
                          "block_int4_variant": block_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS,
                                                              True)}))
        return
    if only == "sweep":
        print(json.dumps({"batch_sweep": batch_sweep(sj, workloads, [1, 2, 4, 8, 16, 32, 64], min(steps, 100),
                                                     warmup, MI355X_HBM_PEAK_GBS)}))
        return
    if only == "calib":
        print(json.dumps({"calib_variant": calib_variant(sj, max(5, steps // 20), 2)}))
        return
    t_setup = time.time()
    wl = workloads.long_batched(device=dev, n_q_sets=8)
    B, Hkv, G, d, r, n, k = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim, wl.rank, wl.capacity, wl.k

    def kproj_cache(K, V, M):
        # projected scoring cache, built by the library's append over every cached token
        Kp = torch.empty(B, Hkv, n, r, dtype=torch.bfloat16, device=dev)
        for t0 in range(0, n, 8192):
            pos = torch.full((B,), t0, dtype=torch.int32, device=dev)
            sj.append_kv(K[:, :, t0:t0 + 8192].contiguous(), V[:, :, t0:t0 + 8192].contiguous(), M, pos, K, V, Kp)
        return Kp

    q_sets = wl.extra["q_sets"]
    K, V, M, seq_len = wl.K, wl.V, wl.M, wl.seq_len
    if only == "fp8":
        k_new, v_new = workloads.new_token(wl, seed=99)
        pos_new = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
        print(json.dumps({"kproj_fp8_variant": fp8_variant(sj, wl, K, V, M, seq_len, q_sets, k_new, v_new, pos_new,
                                                           steps, warmup, step_bytes, MI355X_HBM_PEAK_GBS)}))
        return
    Kp = kproj_cache(K, V, M)
    k_new, v_new = workloads.new_token(wl, seed=99)
    pos_new = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
    shape = sj.make_shape(B, Hkv, G, d, r, n)
    ws = sj.alloc_workspace(shape, k, dev)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hkv * G, d, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    def make_step(shape, ws, K, V, Kp, q_sets):
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
        return step

    def stage_us(step):
        evs = [[_ev() for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        names = ["append+prep+scan", "select", "attend"]
        return {nm: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1000.0, 2)
                for j, nm in enumerate(names)}

    def padded_slot(steps_, warmup_):
        # sequence 0's query heads all zero (a padded batch slot): every score of its
        # units is 0, every row a candidate, and those units take the exact path
        qz = q_sets.clone()
        qz[:, 0].zero_()
        wsz = sj.alloc_workspace(shape, k, dev)
        step_z = make_step(shape, wsz, K, V, Kp, qz)
        us = back_to_back_us(step_z, steps_, warmup_)
        res = {"us_per_step": round(us, 2), "stage_us": stage_us(step_z)}
        step_z(0)
        torch.cuda.synchronize()
        res["first_positions"] = bool(torch.equal(idx[0].cpu(), torch.arange(k, dtype=torch.int32).expand(Hkv, k)))
        del wsz, qz
        return res

    step = make_step(shape, ws, K, V, Kp, q_sets)
    if only == "exact":
        # every unit on the exact path (no scan workgroup takes what its prep publishes)
        shape_fb = sj.make_shape(B, Hkv, G, d, r, n, fused_wait_us=-1)
        step_fb = make_step(shape_fb, sj.alloc_workspace(shape_fb, k, dev), K, V, Kp, q_sets)
        fb = back_to_back_us(step_fb, steps, warmup)
        print(json.dumps({"fallback_variant": {"us_per_step": round(fb, 2), "stage_us": stage_us(step_fb)}}))
        print(json.dumps({"padded_slot_variant": padded_slot(steps, warmup)}))
        return
    # throughput: K whole steps back to back, bracketed by one pair of events (an event
    # between two kernels delays the second by several microseconds, so the steps
    # themselves carry none)
    us_step = back_to_back_us(step, steps, warmup)
    ms_per_step = us_step / 1000.0
    say(f"headline: {us_step:.1f} us/step")
    stages = stage_us(step)
    pct = percentiles_us(step, steps)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    pct_flushed = percentiles_us(step, steps, between=lambda: flush.fill_(7))
    del flush
    g_us = graph_us(step, 8, steps)
    ceiling = read_ceiling_gbs(K)
    step(0)
    torch.cuda.synchronize()
    ref_idx, ref_out = idx.clone(), out.clone()
    say(f"stages {stages}, per-step {pct}, flushed {pct_flushed}, graph {g_us:.1f} us, read ceiling {ceiling:.0f} GB/s")

    tb = step_bytes(B, Hkv, G, d, r, n, k)
    gbs = tb["total"] / (ms_per_step * 1e-3) / 1e9
    # the prep + scan launch moves the projected cache, q, M and the appended rows
    scan_bytes = tb["scan_kproj"] + tb["q"] + tb["M"] + tb["append"]
    scan_gbs = scan_bytes / (stages["append+prep+scan"] * 1e-6) / 1e9
    traffic = traffic_from_profile()

    line = {
        "metric": "sparse decode steps/s + achieved HBM GB/s (% of peak) at 128K ctx",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
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
        "hbm_frac_of_read_ceiling": round(gbs / ceiling, 4),
        "read_ceiling_gbs": round(ceiling, 1),
        "algorithmic_bytes_per_step": tb["total"],
        "step_us": pct,
        "step_us_flushed": {**pct_flushed, "flush": "1 GiB device write between steps, outside the events"},
        "graph_us_per_step": round(g_us, 2),
        "stage_us": stages,
        "roofline": {"kernel": "prep + score scan (prep_scan_kernel<32,2,true>)", "bound": "hbm",
                     "achieved": round(scan_gbs, 1), "bytes_per_launch": scan_bytes,
                     "peak": MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / MI355X_HBM_PEAK_GBS, 4),
                     "read_ceiling": round(ceiling, 1), "frac_of_read_ceiling": round(scan_gbs / ceiling, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "setup_s": round(t_setup, 2),
    }

    if not only:
        # two full input sets alternated, so no step finds the previous one's rows cached
        wl2 = workloads.long_batched(seed=13, device=dev, n_q_sets=8)
        K2, V2 = wl2.K, wl2.V
        Kp2 = kproj_cache(K2, V2, M)
        ws2 = sj.alloc_workspace(shape, k, dev)
        step2 = make_step(shape, ws2, K2, V2, Kp2, wl2.extra["q_sets"])
        rot = back_to_back_us(lambda i: (step if i % 2 == 0 else step2)(i), steps, warmup)
        line["rotated_us_per_step"] = round(rot, 2)
        line["rotated_sets"] = "two full input sets (K, V, Kproj: 2 x 9.66 GB) alternated back to back"
        del wl2, K2, V2, Kp2, ws2, step2
        torch.cuda.empty_cache()
        say(f"rotated: {rot:.1f} us/step")

    if not only and not args.no_fallback_variants:
        # every scan workgroup gives up at once (no wait), so every unit is recomputed
        # and selected exactly by the selection kernel
        shape_fb = sj.make_shape(B, Hkv, G, d, r, n, fused_wait_us=-1)
        ws_fb = sj.alloc_workspace(shape_fb, k, dev)
        step_fb = make_step(shape_fb, ws_fb, K, V, Kp, q_sets)
        fb = back_to_back_us(step_fb, steps, warmup)
        fb_st = {kk: v for kk, v in stage_us(step_fb).items()}
        step_fb(0)
        torch.cuda.synchronize()
        same = bool(torch.equal(idx, ref_idx) and torch.equal(out.view(torch.int16), ref_out.view(torch.int16)))
        line["fallback_variant"] = {
            "what": "the headline step with sjsa_shape.fused_wait_us < 0: no scan workgroup takes what its prep "
                    "publishes, so every unit takes the exact path (scores recomputed by four workgroups per unit, "
                    "dense radix selection)",
            "us_per_step": round(fb, 2), "ratio_to_headline": round(fb / us_step, 3), "stage_us": fb_st,
            "results_equal_headline": same}
        del ws_fb
        say(f"fallback: {fb:.1f} us/step ({fb / us_step:.2f}x), stages {fb_st}, same results {same}")
        pz = padded_slot(steps, warmup)
        line["padded_slot_variant"] = {
            "what": "the headline step with every query head of sequence 0 zero (a padded batch slot): its 8 units "
                    "score every row 0, so every row is a candidate and they take the exact path; the result is "
                    "their first k positions",
            **pz, "ratio_to_headline": round(pz["us_per_step"] / us_step, 3)}
        say(f"padded slot: {pz['us_per_step']:.1f} us/step ({pz['us_per_step'] / us_step:.2f}x)")
        # an input whose top-k the threshold sampler cannot see
        wb = workloads.long_batched_blind_spot(device=dev)
        Kb_, Vb_ = wb.K, wb.V
        Kpb = kproj_cache(Kb_, Vb_, M)
        wsb = sj.alloc_workspace(shape, k, dev)
        step_b = make_step(shape, wsb, Kb_, Vb_, Kpb, q_sets)
        bl = back_to_back_us(step_b, steps, warmup)
        bl_st = stage_us(step_b)
        line["blind_spot_variant"] = {
            "workload": "the headline workload with the keys at positions p % 128 < 2 scaled by 1/16: the rows an "
                        "evenly spaced sampler of 1024 pairs would read are the quietest, so a threshold placed from "
                        "them would lie far below the k-th score; the prep draws each pair's offset in its stratum "
                        "anew for every unit and step, so its threshold sees through the arrangement",
            "us_per_step": round(bl, 2), "ratio_to_headline": round(bl / us_step, 3), "stage_us": bl_st}
        say(f"blind spot: {bl:.1f} us/step, stages {bl_st}")
        if cpu is not None:
            from oracle import jssa
            step_b(0)
            torch.cuda.synchronize()
            units = [(b, h) for b in range(0, B, 4) for h in range(0, Hkv, 2)]      # 16 of 128
            hostb = {"q": _bits(q_sets[0]), "K": _bits(Kb_), "V": _bits(Vb_), "Kp": _bits(Kpb), "M": M.cpu().numpy(),
                     "G": G, "n": n}
            _, resb = oracle_step(hostb, units, k, jssa.default_sm_scale(d), cpu["pool_threads"])
            line["blind_spot_variant"]["parity_sample"] = parity_summary(
                hostb, units, resb, out.float().cpu().numpy(), idx.cpu().numpy(), jssa.default_sm_scale(d))
            del hostb
        del wb, Kb_, Vb_, Kpb, wsb, step_b
        torch.cuda.empty_cache()

    if not only and not args.no_gated_variant:
        line["gated_variant"] = gated_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS, cpu=cpu)
    if not only and not args.no_block_variant:
        line["block_variant"] = block_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS, False, cpu=cpu)
        line["block_int4_variant"] = block_variant(sj, workloads, steps, warmup, MI355X_HBM_PEAK_GBS, True, cpu=cpu)
    if not only and not args.no_calib_variant:
        line["calib_variant"] = calib_variant(sj, max(5, steps // 20), 2, cpu=cpu)
    if not only and not args.no_fp8_variant:
        line["kproj_fp8_variant"] = fp8_variant(sj, wl, K, V, M, seq_len, q_sets, k_new, v_new, pos_new, steps,
                                                warmup, step_bytes, MI355X_HBM_PEAK_GBS, cpu=cpu)
        torch.cuda.empty_cache()
    if cpu is not None:
        from oracle import jssa
        # the oracle on the whole step: every (sequence, KV head) unit, median of 3 runs
        step(0)
        torch.cuda.synchronize()
        units = [(b, h) for b in range(B) for h in range(Hkv)]
        host = {"q": _bits(q_sets[0]), "K": _bits(K), "V": _bits(V), "Kp": _bits(Kp), "M": M.cpu().numpy(), "G": G,
                "n": n}
        scale = jssa.default_sm_scale(d)
        dt, results = oracle_step(host, units, k, scale, cpu["pool_threads"], reps=3)
        line["cpu_baseline"] = {"value": round(1.0 / dt, 4), "unit": "steps/s", "cores": cpu["pool_threads"],
                                "kind": "oracle",
                                "sample": f"the whole step: all {len(units)} (sequence, KV head) units (scoring, "
                                          f"top-k, exact attention), median of 3 runs; NumPy, thread pool over units",
                                "cpu_model": cpu["cpu_model"], "os_cpu_count": cpu["os_cpu_count"],
                                "affinity_cpus": cpu["affinity_cpus"]}
        line["parity_all_units"] = parity_summary(host, units, results, out.float().cpu().numpy(), idx.cpu().numpy(),
                                                  scale)
        del host, results
        line["recall_diagnostic"] = recall_diagnostic(sj, workloads)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
