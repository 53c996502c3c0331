#!/usr/bin/env python3
"""Benchmark of one paged MLA decode step on one MI355X.

A step is the whole hot path over one batch: split-KV schedule, decode
(mla_decode_paged) and combine (mla_combine).  The schedule is a launch of
its own (mla_get_metadata), except for workgroups of at most 16 query rows
and at most 1024 sequences, where the decode computes the same partition
itself at the start of the launch (tile_metadata NULL); --schedule separate
forces the separate launch.
Inputs are seeded synthetic workloads (workloads.CONFIGS), resident in HBM
before timing starts; R replicas of the cache / queries / tables rotate so
that consecutive steps never hit the 256 MB Infinity Cache with the same KV.
Steps are replayed through a captured HIP graph (no memset nodes), so host
launch overhead does not enter the GPU time.

Prints ONE JSON line (rank 0, N = 1).  `value` is the whole-step throughput
in algorithmic HBM bytes per second; the roofline object is for the decode
kernel, timed with HIP events on the stream it runs on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
METRIC = "paged MLA decode achieved HBM GB/s and bf16 TFLOPS (fraction of roofline)"
WORKLOAD_NAMES = {
    1: "tiny_decode",
    2: "memory_bound_decode",
    3: "compute_bound_decode",
    4: "multi_token_causal_decode",
    5: "skewed_long_context_decode",
}


def algorithmic_work(case):
    """Bytes the method must move and flops it must do (each visible KV token
    read once: one latent serves every head)."""
    L = case.cache_seqlens.astype(np.int64)
    b, s_q, h_q = case.batch, case.s_q, case.h_q
    R = s_q * h_q
    pages = (L + 63) // 64
    nbytes = (1152 * L.sum() + 1152 * b * R + 1024 * b * R + 4 * b * R + 4 * pages.sum() + 4 * b)
    vis = 0
    for i in range(s_q):
        n = (L - s_q + 1 + i) if case.causal else L
        vis += np.clip(n, 0, L).sum()
    flops = 2 * (576 + 512) * h_q * vis
    return int(nbytes), int(flops)


def _host_info():
    """CPU model and the BLAS library numpy calls (name, version, threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {}
    try:
        from threadpoolctl import threadpool_info

        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"name": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "arch": i.get("architecture")}
                break
    except Exception:  # pragma: no cover
        pass
    return model, blas


def _time_oracle(case, chosen, min_s):
    """Seconds per pass of the oracle over the chosen sequences (repeated
    until about min_s of work has been timed)."""
    import oracle

    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_ref(case, batches=chosen)
        reps += 1
        if time.perf_counter() - t0 >= min_s:
            break
    return (time.perf_counter() - t0) / reps, reps


def _subcase(case, chosen):
    return type(case)(q=case.q[chosen], kv=case.kv, block_table=case.block_table[chosen],
                      cache_seqlens=case.cache_seqlens[chosen], softmax_scale=case.softmax_scale,
                      causal=case.causal)


def cpu_baseline(case, budget_s=20.0, min_s=10.0):
    """Time the oracle (as it stands) on a bounded sample of the workload,
    with every BLAS thread the host gives this process; then one thread on
    the two smallest workloads (tiny, memory-bound) in full."""
    import oracle
    from workloads import make_config_case

    model, blas = _host_info()
    threads = int(blas.get("threads") or len(os.sched_getaffinity(0)))
    L = case.cache_seqlens.astype(np.int64)
    order = list(range(case.batch))
    # estimate per-sequence cost by its tokens and take sequences until the budget
    t0 = time.perf_counter()
    oracle.decode_ref(case, batches=[order[0]])
    per_tok = (time.perf_counter() - t0) / max(1, int(L[order[0]]))
    chosen, est = [], 0.0
    for b in order:
        c = per_tok * max(1, int(L[b]))
        if chosen and est + c > budget_s:
            break
        chosen.append(b)
        est += c
    dt, reps = _time_oracle(case, chosen, min_s)
    nbytes, flops = algorithmic_work(_subcase(case, chosen))
    single = {}
    try:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1, user_api="blas"):
            for k in (1, 2):
                c = make_config_case(k)
                t1, r1 = _time_oracle(c, list(range(c.batch)), 3.0)
                nb, fl = algorithmic_work(c)
                single[WORKLOAD_NAMES[k]] = {"s_per_step": round(t1, 4),
                                             "GB_per_s": round(nb / t1 / 1e9, 4),
                                             "GFLOP_per_s": round(fl / t1 / 1e9, 3)}
    except Exception as e:  # pragma: no cover
        single = {"skipped": str(e)}
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle over {len(chosen)} of {case.batch} sequences "
                  f"({int(L[chosen].sum())} cached tokens), {reps} timed pass(es) of "
                  f"{dt:.3f} s each; {flops / dt / 1e9:.2f} GFLOP/s",
        "GFLOP_per_s": round(flops / dt / 1e9, 3),
        "cpu_model": model,
        "blas": blas,
        "single_thread": single,
    }


# what the decode kernels are built from (the HBM counters belong to them)
KERNEL_SOURCES = (
    "mla_paged_kv_06_amd/csrc/mla_decode_t16.hip",
    "mla_paged_kv_06_amd/csrc/mla_decode.hip",
    "mla_paged_kv_06_amd/csrc/mla_decode_sv64.hip",
    "mla_paged_kv_06_amd/csrc/mla_decode_common.h",
    "mla_paged_kv_06_amd/csrc/mla_sched_inlaunch.h",
    "mla_paged_kv_06_amd/csrc/mla_device.h",
    "mla_paged_kv_06_amd/csrc/mla_api.hip",
    "include",
    "mla_paged_kv_06_amd/build.py",
)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """sha256 over the sources, headers and build flags of the decode kernels."""
    import hashlib

    h = hashlib.sha256()
    files = []
    for entry in KERNEL_SOURCES:
        path = os.path.join(ROOT, entry)
        if os.path.isdir(path):
            files += [os.path.join(path, f) for f in sorted(os.listdir(path))
                      if f.endswith((".hip", ".h"))]
        else:
            files.append(path)
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter record, if it was
    taken on the current kernel sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w:
        return None
    return int(w["fetch_bytes"] + w["write_bytes"])


def absorption_rates(mla, b, s_q, h_q, seed, dev, launches_per_rep=None):
    """Time the query and output absorption products (the row next to the
    decode) on this workload's token and head counts, synthetic weights; each
    launch reads a different replica (more than 1 GiB in all) so that no
    weight is served from the 256 MB last-level cache.  Returns per product:
    average launch time (HIP events around a graph of back-to-back launches
    on the launch stream), algorithmic bytes and flops per launch, and the
    fraction of the HBM peak (both products are weight/activation streams at
    2 flops per weight byte per token)."""
    import torch
    from workloads import make_absorb_case

    case = make_absorb_case(b, s_q, h_q, seed)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    M = b * s_q
    qb = h_q * 512 * 128 * 2 + M * h_q * (128 + 64 + 576) * 2
    ob = h_q * 128 * 512 * 2 + M * h_q * (512 + 128) * 2
    fl = 2 * M * h_q * 128 * 512
    R = max(2, math.ceil((1 << 30) / (qb + ob)))
    base = [up(case.q_nope), up(case.q_rope), up(case.w_uk_t), up(case.lat_out), up(case.w_uv)]
    reps = [base] + [[t.clone() for t in base] for _ in range(R - 1)]
    q_out = [torch.empty((b, s_q, h_q, 576), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    o = [torch.empty((b, s_q, h_q, 128), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    out = {}
    for name, fn, nb in (
            ("query", lambda r: mla.absorb_query(reps[r][0], reps[r][1], reps[r][2], q_out[r]), qb),
            ("output", lambda r: mla.absorb_output(reps[r][3], reps[r][4], o[r]), ob)):
        for r in range(R):
            fn(r)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for r in range(R):
                fn(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / R)
        ms = float(np.mean(times))
        gbs = nb / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 3), "bytes": nb, "flops": fl,
                     "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "TFLOP_per_s": round(fl / (ms * 1e-3) / 1e12, 2)}
    out["replicas"] = R
    return out


def query_token_rates(mla, seqlens, s_q, h_q, seed, dev):
    """Time whole decode steps (schedule + decode + combine, the schedule
    inside the decode where it can go) with s_q query tokens per sequence,
    causal: several speculative tokens, or a chunk of new tokens at every
    head.  The same kernels as the workloads above, more rows per sequence.
    Replicas of cache, queries and tables (over 1 GiB in all) rotate in a
    graph of back-to-back steps; HIP events around replays on the launch
    stream."""
    import ctypes

    import torch
    from workloads import make_case

    case = make_case(seqlens, s_q, h_q, True, seed=seed, pool_factor=1.0)
    nbytes, flops = algorithmic_work(case)
    b = case.batch
    lib = mla.load_library()
    footprint = case.kv.nbytes + 2 * case.q.nbytes
    R = max(2, math.ceil((1 << 30) / footprint))
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    base = (up(case.q), up(case.kv), torch.from_numpy(case.block_table).to(dev),
            torch.from_numpy(case.cache_seqlens).to(dev))
    reps = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    parts = mla.num_partitions(s_q, h_q)
    ws_bytes = mla.workspace_bytes(b, s_q, h_q)
    in_decode = mla.prefers_in_decode(b, s_q, h_q, case.max_pages)
    bufs = [dict(meta=torch.empty((parts, mla.META_INTS), dtype=torch.int32, device=dev),
                 splits=torch.empty((b + 1,), dtype=torch.int32, device=dev),
                 ws=torch.empty((ws_bytes,), dtype=torch.uint8, device=dev),
                 out=torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev),
                 lse=torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev))
            for _ in range(R)]
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def step(r):
        q, kv, bt, sl = reps[r]
        o = bufs[r]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        s1 = 0 if in_decode else lib.mla_get_metadata(vp(sl), b, s_q, h_q, 0, vp(o["meta"]),
                                                      vp(o["splits"]), st)
        s2 = lib.mla_decode_paged(vp(q), vp(kv), vp(bt), vp(sl), b, s_q, h_q, case.num_pages,
                                  case.max_pages, case.softmax_scale, 1,
                                  None if in_decode else vp(o["meta"]), vp(o["splits"]), 0,
                                  vp(o["ws"]), ws_bytes, vp(o["out"]), vp(o["lse"]), st)
        s3 = lib.mla_combine(vp(o["ws"]), ws_bytes, vp(o["splits"]), b, s_q, h_q, 0,
                             vp(o["out"]), vp(o["lse"]), st)
        if s1 or s2 or s3:
            raise RuntimeError(f"library status {s1} {s2} {s3}")

    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for r in range(R):
            step(r)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(5):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / R)
    ms = float(np.mean(times))
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return {"batch": b, "s_q": s_q, "h_q": h_q, "rows_per_sequence": s_q * h_q, "causal": True,
            "sum_seqlen": int(case.cache_seqlens.sum()), "partitions": parts,
            "us_per_step": round(ms * 1e3, 2), "bytes": nbytes, "flops": flops,
            "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP_per_s": round(tf, 2), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "replicas": R}


def fp8_cache_rates(mla, case, dev):
    """Time the decode step over the FP8 latent cache (schedule + FP8 decode
    + combine) on this workload's sequences and queries, the cache quantized
    on the GPU beforehand; replicas of cache, queries and tables (over 1 GiB)
    rotate in a graph of back-to-back steps, HIP events on the launch stream.
    Algorithmic bytes count 656 per cached token instead of 1152."""
    import ctypes

    import torch

    b, s_q, h_q = case.batch, case.s_q, case.h_q
    if s_q * h_q > 16:
        return {"skipped": "the FP8-cache decode takes at most 16 query rows per sequence"}
    lib = mla.load_library()
    L = case.cache_seqlens.astype(np.int64)
    R_ = s_q * h_q
    nbytes = int(656 * L.sum() + 1152 * b * R_ + 1024 * b * R_ + 4 * b * R_ +
                 4 * ((L + 63) // 64).sum() + 4 * b)
    q0 = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv0 = mla.kv_quantize_fp8(torch.from_numpy(case.kv.view(np.int16)).to(dev).view(torch.bfloat16))
    bt0 = torch.from_numpy(case.block_table).to(dev)
    sl0 = torch.from_numpy(case.cache_seqlens).to(dev)
    R = max(2, math.ceil((1 << 30) / (kv0.numel() + 2 * q0.numel())))
    reps = [(q0, kv0, bt0, sl0)] + [(q0.clone(), kv0.clone(), bt0.clone(), sl0.clone())
                                   for _ in range(R - 1)]
    parts = mla.num_partitions(s_q, h_q)
    ws_bytes = mla.workspace_bytes(b, s_q, h_q)
    bufs = [dict(meta=torch.empty((parts, mla.META_INTS), dtype=torch.int32, device=dev),
                 splits=torch.empty((b + 1,), dtype=torch.int32, device=dev),
                 ws=torch.empty((ws_bytes,), dtype=torch.uint8, device=dev),
                 out=torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev),
                 lse=torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev))
            for _ in range(R)]
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def step(r, full=True):
        q, kv, bt, sl = reps[r]
        o = bufs[r]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        s1 = lib.mla_get_metadata(vp(sl), b, s_q, h_q, 0, vp(o["meta"]), vp(o["splits"]), st) \
            if full else 0
        s2 = lib.mla_decode_paged_fp8(vp(q), vp(kv), vp(bt), vp(sl), b, s_q, h_q,
                                      kv.shape[0], case.max_pages, case.softmax_scale,
                                      int(case.causal), vp(o["meta"]), vp(o["splits"]), 0,
                                      vp(o["ws"]), ws_bytes, vp(o["out"]), vp(o["lse"]), st)
        s3 = lib.mla_combine(vp(o["ws"]), ws_bytes, vp(o["splits"]), b, s_q, h_q, 0,
                             vp(o["out"]), vp(o["lse"]), st) if full else 0
        if s1 or s2 or s3:
            raise RuntimeError(f"library status {s1} {s2} {s3}")

    res = {}
    for name, full in (("step", True), ("decode", False)):
        for r in range(R):
            step(r, True)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for r in range(R):
                step(r, full)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / R)
        res[name] = float(np.mean(times))
    gbs = nbytes / (res["step"] * 1e-3) / 1e9
    dgbs = nbytes / (res["decode"] * 1e-3) / 1e9
    return {"us_per_step": round(res["step"] * 1e3, 2), "decode_us": round(res["decode"] * 1e3, 2),
            "bytes": nbytes, "GB_per_s": round(gbs, 1), "decode_GB_per_s": round(dgbs, 1),
            "decode_hbm_frac": round(dgbs / HBM_PEAK_GBS, 4), "token_bytes": 656,
            "replicas": R}


def kv_append_rates(mla, seqlens, n_new, seed, dev, R=32):
    """Time mla_kv_append appending n_new tokens to every sequence of this
    workload (its lengths; a pool of exactly the held pages plus the free
    ones).  Each of R launches in a graph works on its own copy of the
    lengths and of the free count, reset before every replay outside the
    timed region, so every launch does the same allocation and copies.  A
    latency-bound step: a few hundred KB per launch."""
    import torch

    rng = np.random.Generator(np.random.PCG64(seed))
    batch = len(seqlens)
    held = [(int(L) + 63) // 64 for L in seqlens]
    need = [(int(L) + n_new + 63) // 64 - h for L, h in zip(seqlens, held)]
    max_pages = max(h + k for h, k in zip(held, need))
    free = sum(need) + 8
    num_pages = sum(held) + free
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((batch, max_pages), -1, dtype=np.int32)
    k = 0
    for b, h in enumerate(held):
        bt[b, :h] = perm[k:k + h]
        k += h
    kv = torch.empty((num_pages, 64, 576), dtype=torch.bfloat16, device=dev)
    bt_d = torch.from_numpy(bt).to(dev)
    fp = torch.from_numpy(perm[k:].copy()).to(dev)
    new_kv = torch.randn((batch, n_new, 576), dtype=torch.float32, device=dev).to(torch.bfloat16)
    sl0 = torch.tensor(np.asarray(seqlens, dtype=np.int32), device=dev)
    sls = [sl0.clone() for _ in range(R)]
    fcs = [torch.full((1,), free, dtype=torch.int32, device=dev) for _ in range(R)]
    sts = [torch.empty((1,), dtype=torch.int32, device=dev) for _ in range(R)]

    def reset():
        for r in range(R):
            sls[r].copy_(sl0)
            fcs[r].fill_(free)
        torch.cuda.synchronize()

    def launches():
        for r in range(R):
            mla.kv_append(kv, bt_d, sls[r], new_kv, fp, fcs[r], sts[r])

    reset()
    launches()
    torch.cuda.synchronize()
    if any(int(st.cpu()[0]) != 0 for st in sts):
        raise RuntimeError("kv_append reported a shortage in the timing setup")
    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launches()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(5):
        reset()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / R)
    ms = float(np.mean(times))
    nb = 2 * batch * n_new * 576 * 2 + 8 * batch + 4 * sum(need) * 2
    gbs = nb / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 3), "bytes": int(nb), "tokens": batch * n_new,
            "new_pages": int(sum(need)), "GB_per_s": round(gbs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 5), "launches_per_call": 2}


def prefill_rates(mla, seqlens, h_q, seed, dev, reps=5):
    """Time MLA prefill in per-head form on packed prompts: the expansion of
    the latents into per-head keys and values (two launches) and the causal
    attention, each alone, HIP events on the launch stream around a graph of
    back-to-back launches.  Attention flops: 2 * (192 + 128) per (query,
    visible key) pair and head; expansion: 2 * 512 * 128 * 2 per token and
    head."""
    import torch
    from workloads import make_prefill_case

    case = make_prefill_case(seqlens, h_q, seed)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(  # noqa
        torch.bfloat16)
    lat, q, wk, wv = up(case.latent), up(case.q), up(case.w_uk), up(case.w_uv)
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    T = case.tokens
    k_nope = torch.empty((T, h_q, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k_nope)
    o = torch.empty_like(k_nope)
    lse = torch.empty((T, h_q), dtype=torch.float32, device=dev)
    ms = int(max(seqlens))
    L = np.asarray(seqlens, dtype=np.int64)
    pairs = int((L * (L + 1) // 2).sum())
    att_flops = 2 * (192 + 128) * h_q * pairs
    exp_flops = 2 * 2 * 512 * 128 * h_q * T

    def expand():
        mla.prefill_expand_kv(lat, wk, wv, k_nope, v)

    def attend():
        mla.prefill_attention(q, k_nope, lat[:, 512:], v, cu, ms, case.softmax_scale, True, o, lse)

    out = {"prompts": [int(x) for x in seqlens], "heads": h_q, "tokens": T}
    for name, fn, fl in (("expand_kv", expand, exp_flops), ("attention", attend, att_flops)):
        fn()
        torch.cuda.synchronize()
        g = _capture(lambda: [fn() for _ in range(reps)])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(3):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        t = float(np.median(ts))
        tf = fl / (t * 1e-3) / 1e12
        out[name] = {"us": round(t * 1e3, 2), "flops": int(fl), "TFLOP_per_s": round(tf, 1),
                     "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    return out


def copy_calibration(mib, launches=5):
    """Plain device-to-device copies of a known size, for scaling the HBM byte
    counters (run under rocprofv3 --pmc)."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": launches}), flush=True)


def _capture(fn):
    """A HIP graph of fn()'s launches on a side stream, replayed once."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return g


def _pct(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(xs.mean()), 3), "p10": round(float(np.percentile(xs, 10)), 3),
            "p50": round(float(np.percentile(xs, 50)), 3),
            "p90": round(float(np.percentile(xs, 90)), 3), "n": int(xs.size)}


def measure_workload(mla, k, steps, warmup, dev, replicas=0, schedule="auto", use_graph=True,
                     per_launch=20):
    """Time whole steps (schedule + decode + combine) and the decode kernel
    alone on workload k.  Returns the measurement dict and the case."""
    import ctypes

    import torch
    from workloads import CONFIGS, make_config_case

    spec = CONFIGS[k]
    case = make_config_case(k)
    nbytes, flops = algorithmic_work(case)
    print(f"# workload {k} ({spec.name}): batch {case.batch} s_q {case.s_q} h_q {case.h_q} "
          f"sum L {int(case.cache_seqlens.sum())} pool {case.num_pages} pages; "
          f"{nbytes / 1e6:.2f} MB, {flops / 1e9:.2f} GFLOP per step", file=sys.stderr, flush=True)
    footprint = case.kv.nbytes + case.q.nbytes + case.block_table.nbytes
    R = replicas or max(2, math.ceil((1 << 30) / footprint))
    q0 = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv0 = torch.from_numpy(case.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    bt0 = torch.from_numpy(case.block_table).to(dev)
    sl0 = torch.from_numpy(case.cache_seqlens).to(dev)
    reps = [(q0, kv0, bt0, sl0)] + [(q0.clone(), kv0.clone(), bt0.clone(), sl0.clone())
                                   for _ in range(R - 1)]
    b, s_q, h_q = case.batch, case.s_q, case.h_q
    parts = mla.num_partitions(s_q, h_q)
    ws_bytes = mla.workspace_bytes(b, s_q, h_q)
    bufs = [dict(meta=torch.empty((parts, mla.META_INTS), dtype=torch.int32, device=dev),
                 splits=torch.empty((b + 1,), dtype=torch.int32, device=dev),
                 ws=torch.empty((ws_bytes,), dtype=torch.uint8, device=dev),
                 out=torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev),
                 lse=torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev))
            for _ in range(R)]
    lib = mla.load_library()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    in_decode = schedule == "in_decode" or (
        schedule == "auto" and mla.prefers_in_decode(b, s_q, h_q, case.max_pages))

    def decode(r):
        q, kv, bt, sl = reps[r]
        o = bufs[r]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        s2 = lib.mla_decode_paged(vp(q), vp(kv), vp(bt), vp(sl), b, s_q, h_q, case.num_pages,
                                  case.max_pages, case.softmax_scale, int(case.causal),
                                  None if in_decode else vp(o["meta"]), vp(o["splits"]), 0,
                                  vp(o["ws"]), ws_bytes, vp(o["out"]), vp(o["lse"]), st)
        if s2:
            raise RuntimeError(f"decode status {s2}")

    def step(r):
        sl = reps[r][3]
        o = bufs[r]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if not in_decode:
            s1 = lib.mla_get_metadata(vp(sl), b, s_q, h_q, 0, vp(o["meta"]), vp(o["splits"]), st)
            if s1:
                raise RuntimeError(f"metadata status {s1}")
        decode(r)
        s3 = lib.mla_combine(vp(o["ws"]), ws_bytes, vp(o["splits"]), b, s_q, h_q, 0,
                             vp(o["out"]), vp(o["lse"]), st)
        if s3:
            raise RuntimeError(f"combine status {s3}")

    # eager warmup (also sanity: every replica once)
    for i in range(max(warmup, R)):
        step(i % R)
    torch.cuda.synchronize()

    # graphs of G = min(K, R) steps (each on its own replica) and of the
    # remainder, so that the timed region is K steps replayed from graphs
    K = steps
    G = min(K, R)
    full, rem = divmod(K, G)
    timing = "hip-graph"
    graph = rgraph = None
    if use_graph:
        try:
            graph = _capture(lambda: [step(r) for r in range(G)])
            if rem:
                rgraph = _capture(lambda: [step(r) for r in range(rem)])
        except Exception as e:  # capture not available: eager launches
            print(f"# graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph = rgraph = None
    if graph is None:
        timing = "eager"

    # ---- timed region: exactly K whole steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(full):
            graph.replay()
        if rgraph is not None:
            rgraph.replay()
    else:
        for i in range(K):
            step(i % R)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K

    # ---- decode kernel: HIP events on the launch stream around a graph of
    # back-to-back decode launches (one per replica, schedules built above)
    dgraph = None
    if graph is not None:
        try:
            dgraph = _capture(lambda: [decode(r) for r in range(R)])
        except Exception as e:
            print(f"# decode graph capture failed ({e})", file=sys.stderr)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_rep = max(5, K // R)
    dec_ms = []
    for _ in range(n_rep):
        e0.record()
        if dgraph is not None:
            dgraph.replay()
        else:
            for r in range(R):
                decode(r)
        e1.record()
        torch.cuda.synchronize()
        dec_ms.append(e0.elapsed_time(e1) / R)
    dec_avg_ms = float(np.mean(dec_ms))
    # ---- spread: each launch alone between two events (eager; the markers
    # add about a microsecond, which matters only for the smallest workloads)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(per_launch)]
    for i, (a, z) in enumerate(evs):
        a.record()
        decode(i % R)
        z.record()
    torch.cuda.synchronize()
    each_us = [a.elapsed_time(z) * 1e3 for a, z in evs]

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (dec_avg_ms * 1e-3) / 1e9
    dec_tflops = flops / (dec_avg_ms * 1e-3) / 1e12
    # the bound of the decode kernel: its arithmetic intensity against the
    # ridge of the two peaks
    mfma_bound = flops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(dec_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roofline["traffic"] = measured_traffic(WORKLOAD_NAMES[k])
    m = {
        "workload": WORKLOAD_NAMES[k], "config_index": k,
        "batch": b, "s_q": s_q, "h_q": h_q, "causal": bool(case.causal),
        "cache_seqlens": list(spec.lengths), "sum_seqlen": int(case.cache_seqlens.sum()),
        "seed": 1000 + k, "replicas": R, "timing": timing,
        "graph_steps": G if graph is not None else 0,
        "graph_replays": (full + (1 if rgraph is not None else 0)) if graph is not None else 0,
        "schedule": "in-decode" if in_decode else "separate-launch",
        "value_GB_per_s": round(value, 2), "ms_per_step": round(ms_per_step, 5),
        "step_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "algorithmic": {"bytes_per_step": int(nbytes), "flops_per_step": int(flops)},
        "decode_kernel_ms": round(dec_avg_ms, 5),
        "decode_us_graph": _pct([x * 1e3 for x in dec_ms]),
        "decode_us_per_launch": _pct(each_us),
        "decode_launches_timed": n_rep * R,
        "decode_GB_per_s": round(achieved, 1), "decode_tflops": round(dec_tflops, 3),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "mfma_frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4),
        "roofline": roofline,
    }
    del reps, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return m, case


def machine_limits(mla, dev):
    """What this GPU reaches on plain work: a streaming read of 2 GiB (HBM)
    and a loop of bf16 16x16x32 matrix instructions (matrix cores), with the
    shader clock sampled under matrix load."""
    import ctypes

    import torch

    lib = mla.load_library()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    blocks = 2048
    sink = torch.empty(max(blocks, 256 * 4), dtype=torch.int32, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for it in range(6):
        e0.record()
        rc = lib.mla_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                       ctypes.c_void_p(sink.data_ptr()), blocks, st())
        e1.record()
        torch.cuda.synchronize()
        if rc:
            raise RuntimeError(f"probe status {rc}")
        if it:
            ts.append(e0.elapsed_time(e1))
    read_gbs = nbytes / (float(np.median(ts)) * 1e-3) / 1e9
    # the 64-row decode's page copies alone (LDS-DMA, four-slot ring, two
    # slots ahead, 256 workgroups): cycles per 36 KiB slot and the time from
    # the end of a slot's issue to the end of the wait for it
    ring = {}
    rblocks, rsteps = 256, 2000
    rsink = torch.empty(rblocks * 512, dtype=torch.int32, device=dev)
    rclk = torch.zeros(2 * rblocks, dtype=torch.int64, device=dev)
    for name, kind, slots in (("l2_resident_alone", 0, 2), ("l2_resident_beside_key_reads", 1, 2),
                              ("l2_resident_beside_68_mfma_per_simd", 2, 2),
                              ("hbm_stream_alone", 0, 200)):
        assert rblocks * slots * 36864 <= nbytes
        cyc, lat = [], []
        for it in range(3):
            rc = lib.mla_probe_copy_ring(kind, ctypes.c_void_p(buf.data_ptr()), slots, rsteps, rblocks,
                                         ctypes.c_void_p(rsink.data_ptr()),
                                         ctypes.c_void_p(rclk.data_ptr()), st())
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"probe status {rc}")
            if it:
                c = rclk.cpu().numpy().reshape(rblocks, 2).astype(np.float64)
                cyc.append(float(c[:, 0].mean()) / rsteps)
                lat.append(float(c[:, 1].mean()))
        per_slot = float(np.median(cyc))
        ring[name] = {"cycles_per_slot": round(per_slot, 1),
                      "bytes_per_clock_per_cu": round(36864 / per_slot, 1),
                      "issue_to_landed_cycles": round(float(np.median(lat)), 1)}
    ring["work"] = ("256 workgroups x 8 waves; waves 4-7 copy 36 KiB slots (nine 1 KiB LDS-DMA "
                    "copies each) two slots ahead into a 4-slot ring, one barrier per slot; "
                    "waves 0-3 idle, read 576 B of key fragments per lane, or run 68 bf16 "
                    "16x16x32 MFMA per slot; 2 slots per workgroup stay in L2, 200 stream from HBM")
    del buf
    # matrix loop: 256 workgroups of 8 waves, 4 chains each
    mblocks, iters = 256, 20000
    msink = torch.empty(mblocks * 512, dtype=torch.float32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    ts, ghz = [], []
    for it in range(4):
        e0.record()
        rc = lib.mla_probe_mfma(iters, mblocks, ctypes.c_void_p(msink.data_ptr()),
                                ctypes.c_void_p(clk.data_ptr()), st())
        e1.record()
        torch.cuda.synchronize()
        if rc:
            raise RuntimeError(f"probe status {rc}")
        if it:
            ts.append(e0.elapsed_time(e1))
            c = clk.cpu().numpy()
            ghz.append(float(c[0]) / (float(c[1]) / 100e6) / 1e9)
    mflops = mblocks * 8 * iters * 4 * 16384
    mfma_tf = mflops / (float(np.median(ts)) * 1e-3) / 1e12
    # LDS reads per compute unit: bytes per shader clock of workgroup 0
    lds = {}
    lsink = torch.empty(256 * 512, dtype=torch.int32, device=dev)
    for kind, name, nbytes_lane in ((0, "ds_read_b128_key_fragments", 16),
                                    (1, "ds_read_b64_tr_b16_value_fragments", 8)):
        per_clk = []
        for it in range(3):
            rc = lib.mla_probe_lds(kind, 4000, 256, ctypes.c_void_p(lsink.data_ptr()),
                                   ctypes.c_void_p(clk.data_ptr()), st())
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"probe status {rc}")
            if it:
                per_clk.append(4000 * 16 * 512 * nbytes_lane / float(clk.cpu().numpy()[0]))
        lds[name] = round(float(np.median(per_clk)), 1)
    # matrix work in one wave of each SIMD beside vector work in the other:
    # launch time together against each alone (1.0 of the sum: no overlap)
    isink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    iclk = torch.zeros(2, dtype=torch.int64, device=dev)
    t_kind = {}
    for kind in range(5):
        ts = []
        for it in range(3):
            e0.record()
            rc = lib.mla_probe_issue(kind, 20000, 256, ctypes.c_void_p(isink.data_ptr()),
                                     ctypes.c_void_p(iclk.data_ptr()), st())
            e1.record()
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"probe status {rc}")
            if it:
                ts.append(e0.elapsed_time(e1) * 1e3)
        t_kind[kind] = float(np.median(ts))
    issue = {"us_mfma_alone": round(t_kind[0], 1), "us_fma_alone": round(t_kind[1], 1),
             "us_exp_alone": round(t_kind[2], 1), "us_mfma_with_fma": round(t_kind[3], 1),
             "us_mfma_with_exp": round(t_kind[4], 1),
             "fma_together_over_sum": round(t_kind[3] / (t_kind[0] + t_kind[1]), 3),
             "exp_together_over_sum": round(t_kind[4] / (t_kind[0] + t_kind[2]), 3),
             "work": "256 workgroups x 8 waves, 20000 trips: waves 0-3 4 bf16 16x16x32 MFMA a "
                     "trip, waves 4-7 16 fp32 FMA or 4 v_exp_f32 a trip"}
    torch.cuda.empty_cache()
    return {"stream_read_GB_per_s": round(read_gbs, 1),
            "stream_read_frac_of_spec": round(read_gbs / HBM_PEAK_GBS, 4),
            "stream_read_bytes": nbytes,
            "mfma_loop_TFLOP_per_s": round(mfma_tf, 1),
            "mfma_loop_frac_of_spec": round(mfma_tf / BF16_PEAK_TFLOPS, 4),
            "shader_clock_GHz_under_mfma": round(float(np.median(ghz)), 3),
            "spec_clock_GHz": 2.4,
            "lds_read_bytes_per_clock_per_cu": lds,
            "matrix_beside_vector_work": issue,
            "page_copy_ring": ring}


def trace_stats(path):
    """Per-kernel dispatch durations (count, mean, p10, p50, p90 in us) from a
    rocprofv3 kernel-trace CSV."""
    import csv

    dur = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            name = row.get("Kernel_Name") or row.get("KernelName") or "?"
            t = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            dur.setdefault(name, []).append(t / 1e3)
    out = {}
    for name, xs in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        out[name] = _pct(xs)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="headline workload (default 4, the largest)")
    ap.add_argument("--others", default="2,3,5",
                    help="workloads measured beside the headline ('' for none)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1 GiB")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the streaming-read and matrix-loop machine limits")
    ap.add_argument("--schedule", choices=["auto", "separate", "in_decode"], default="auto",
                    help="auto: the decode schedules itself where that is faster")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the rows next to the decode")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--probes-only", action="store_true",
                    help="only run the machine-limit probes and print them")
    ap.add_argument("--trace-stats", default="", metavar="CSV",
                    help="only summarise a rocprofv3 kernel-trace CSV (no GPU)")
    args = ap.parse_args()

    if args.trace_stats:
        trace_stats(args.trace_stats)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X; "
              "a multi-GPU run is not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import mla_paged_kv_06_amd as mla
    from workloads import make_config_case

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mla.load_library()
    dev = torch.device("cuda:0")
    if args.probes_only:
        print(json.dumps(machine_limits(mla, dev)), flush=True)
        return

    k = args.config
    head, case = measure_workload(mla, k, args.steps, args.warmup, dev, args.replicas,
                                  args.schedule, not args.no_graph)
    limits = None if args.no_probes else machine_limits(mla, dev)
    roofline = dict(head["roofline"])
    if limits:
        if roofline["bound"] == "mfma":
            roofline["frac_of_measured_peak"] = round(
                roofline["achieved"] / limits["mfma_loop_TFLOP_per_s"], 4)
        else:
            roofline["frac_of_measured_peak"] = round(
                roofline["achieved"] / limits["stream_read_GB_per_s"], 4)
    res = {
        "metric": METRIC,
        "value": head["value_GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "batch": head["batch"], "s_q": head["s_q"], "h_q": head["h_q"], "head_dim": 576,
            "v_dim": 512, "page": 64, "cache_seqlens": head["cache_seqlens"],
            "sum_seqlen": head["sum_seqlen"], "causal": head["causal"], "seed": head["seed"],
            "replicas": head["replicas"], "timing": head["timing"],
            "graph_steps": head["graph_steps"], "graph_replays": head["graph_replays"],
            "decode_launches_timed": head["decode_launches_timed"],
            "schedule": head["schedule"],
        },
        "algorithmic": head["algorithmic"],
        "tflops": head["step_tflops"],
        "decode_kernel_ms": head["decode_kernel_ms"],
        "decode_us_graph": head["decode_us_graph"],
        "decode_us_per_launch": head["decode_us_per_launch"],
        "decode_tflops": head["decode_tflops"],
        "roofline": roofline,
        "hbm_frac": head["hbm_frac"],
        "mfma_frac": head["mfma_frac"],
    }
    if limits:
        res["machine_limits"] = limits
    others = [int(x) for x in args.others.split(",") if x.strip()] if args.others else []
    res["workloads"] = {}
    for k2 in others:
        if k2 == k:
            continue
        m2, _ = measure_workload(mla, k2, args.steps, args.warmup, dev, 0, args.schedule,
                                 not args.no_graph)
        if limits:
            r2 = m2["roofline"]
            ref = limits["mfma_loop_TFLOP_per_s"] if r2["bound"] == "mfma" else \
                limits["stream_read_GB_per_s"]
            r2["frac_of_measured_peak"] = round(r2["achieved"] / ref, 4)
        res["workloads"][m2["workload"]] = m2
    if not args.no_next_rows:
        b, s_q, h_q = case.batch, case.s_q, case.h_q
        c2 = make_config_case(2)
        res["next_rows"] = {
            "absorption": absorption_rates(mla, b, s_q, h_q, 2000 + k, dev),
            "kv_append": kv_append_rates(mla, [int(x) for x in case.cache_seqlens], s_q,
                                         3000 + k, dev),
            # the FP8 cache decode takes at most 16 rows: the memory-bound workload
            "fp8_cache": fp8_cache_rates(mla, c2, dev),
            # more query tokens per sequence: 2, 4 and 8 speculative tokens
            # on the memory-bound workload's sequences (32, 64 and 128 rows),
            # and a 512-token chunk at 128 heads over a 4096-token cache
            "query_tokens": {
                "speculative_s_q2": query_token_rates(
                    mla, [int(x) for x in c2.cache_seqlens], 2, 16, 4001, dev),
                "speculative_s_q4": query_token_rates(
                    mla, [int(x) for x in c2.cache_seqlens], 4, 16, 4002, dev),
                "speculative_s_q8": query_token_rates(
                    mla, [int(x) for x in c2.cache_seqlens], 8, 16, 4004, dev),
                "chunk_512x128": query_token_rates(mla, [4096], 512, 128, 4003, dev),
            },
            # MLA prefill in per-head form: one 4096-token prompt at 128 heads
            "prefill": prefill_rates(mla, [4096], 128, 5001, dev),
        }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
