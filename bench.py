#!/usr/bin/env python3
"""Benchmark of the fused lightning-indexer top-k (lid_topk) on one MI355X.

One step = one lid_topk call over one batch of the workload (all of it:
scoring, mask, streaming top-k and, for split plans, the merge).  The timed
steps are replayed from HIP graphs (a short decode call is otherwise bound by
the host's launch rate), each replay between two HIP events, which gives the
mean, median and minimum time per step; the eager per-call time and the
scoring kernel's own duration (HIP events around it, eager) are reported
beside it.  Inputs are seeded synthetic tensors already resident in device
memory; at least 1 GiB of device copies is rotated, in an order that never
comes back to a copy before all the others were read, so no step re-reads
bytes out of the 256 MB last-level cache.  Prints one JSON line on stdout
(progress goes to stderr).

    python bench.py [--workload c2|c3|c4|c5|dec1m] [--steps K] [--warmup W]

Without --workload the line is the multi-sequence workload c5 (4 sequences x
512 queries over 4 key blocks of 262144, the largest configuration, K timed
steps) with the CPU oracle timed beside it, and the other graded workloads
(single-token decode over 32768 and 1048576 keys, the 512 x 16384 and
2048 x 131072 prefills) are timed in the same run with their own step counts
and reported under "workloads".
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer scored (query,key) pairs/sec + top-k tokens/sec; % MFMA / % HBM peak"
PEAK_HBM_BPS = 8.0e12        # MI355X HBM3E, published
PEAK_MFMA_F16 = 2.5e15       # MI355X dense f16/bf16 MFMA, published
PEAK_MFMA_FP8 = 5.0e15       # MI355X dense FP8 MFMA, published
PEAK_F32_VALU = 157.3e12     # MI355X fp32 vector, published (256 CUs x 2.4 GHz x 256 flops per CU-clock)
DEFAULT_STEPS = {"c2": 2000, "dec1m": 300, "c3": 400, "c4": 40, "c5": 20}
# the other graded workloads, timed in the default run beside the headline
SECONDARY = {"c2": 400, "dec1m": 200, "c3": 200, "c4": 20}
HEADLINE = "c5"
DEFAULT_FORM = {"c2": "none", "dec1m": "none", "c3": "mask", "c4": "mask", "c5": "ranges"}
DESCRIPTION = {
    "c2": "single-token decode, n_tok 1 x n_kv 32768",
    "dec1m": "single-token decode, n_tok 1 x n_kv 1048576",
    "c3": "prefill ubatch, n_tok 512 x n_kv 16384, causal f16 mask",
    "c4": "long-context prefill, n_tok 2048 x n_kv 131072, causal f16 mask",
    "c5": "multi-sequence ubatch, 4 seqs x 512 queries, 4 key blocks x 262144, per-query ranges",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# the sources each plan's scoring kernel is compiled from
PLAN_SOURCES = {
    "decode": ["k_decode.hip", "lid_device.h", "lid_budget.h", "lid_kernels.h", "lid_merge.h", "lid_select.h"],
    "prefill": ["k_prefill.hip", "lid_device.h", "lid_budget.h", "lid_kernels.h"],
    "generic": ["k_generic.hip", "lid_device.h", "lid_budget.h", "lid_kernels.h"],
    "shared": ["k_shared.hip", "lid_device.h", "lid_budget.h", "lid_kernels.h", "lid_merge.h", "lid_select.h"],
    "attn": ["k_attn.hip", "lid_device.h", "lid_budget.h", "lid_kernels.h"],
}


def kernel_source_hash(plan: str = None) -> str:
    """sha256 over the HIP sources of a plan's scoring kernel (all sources
    when plan is None); a stored traffic figure is only reported while the
    kernel it was measured on is unchanged."""
    import hashlib
    csrc = os.path.join(ROOT, "sparse_attention_token_lid_amd", "csrc")
    names = PLAN_SOURCES.get(plan) or [n for n in os.listdir(csrc) if n.endswith((".hip", ".h"))]
    h = hashlib.sha256()
    for name in sorted(names):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, plan: str, splits: int):
    """HBM bytes per scoring-kernel launch measured with rocprofv3 counters
    (profiles/traffic.json), or None if absent or measured on other kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    # a workload's record under another entry point's kernel is keyed "<workload>:<plan>"
    rec = data.get(f"{workload}:{plan}") or data.get(workload)
    if not rec or rec.get("kernel_hash") != kernel_source_hash(plan):
        return None
    if rec.get("plan") != plan or rec.get("splits") != splits:
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy(nbytes: int, reps: int = 5):
    """A plain device-to-device copy of a known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}), flush=True)


def visible_pairs(wl, ranges):
    if ranges is None:
        return wl.n_tok * wl.n_kv
    return int((ranges[:, 1].astype("int64") - ranges[:, 0]).clip(min=0).sum())


def cpu_baseline(d, form, seconds, gpu_idx=None):
    """Time the CPU oracle on a bounded sample of the same workload.  With
    the GPU's output rows (gpu_idx, host array), also report how many of the
    sampled rows have exactly the oracle's index set ("exact_match")."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    wl = d["wl"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    ranges = d["ranges"]
    mask = d["mask"] if form == "mask" else None
    rng_arg = ranges if form == "ranges" else None

    last = {}

    def run(rows):
        t0 = time.perf_counter()
        o_idx = oracle.topk(d["q"], d["k"], d["w"], mask=mask, kv_range=rng_arg, k_top=wl.k_top, rows=rows,
                            threads=threads)[0]
        last["rows"], last["idx"] = list(rows), o_idx
        return time.perf_counter() - t0

    def exact_match():
        if gpu_idx is None:
            return None
        pairs = dict(zip(last["rows"], last["idx"]))   # distinct rows (the decode copies are one row)
        same = sum(set(gpu_idx[r][gpu_idx[r] >= 0].tolist()) == set(o[o >= 0].tolist()) for r, o in pairs.items())
        return {"rows": len(pairs), "identical_index_sets": int(same)}

    def pairs_of(rows):
        if ranges is None:
            return len(rows) * wl.n_kv
        r = ranges[rows]
        return int((r[:, 1].astype(np.int64) - r[:, 0]).sum())

    if wl.n_tok == 1:
        # one query: the oracle parallelises over queries, so the whole
        # workload runs as one copy per host thread (independent decode
        # requests of this shape), repeated until the time budget is used
        copies = [0] * threads
        reps, spent = 0, 0.0
        while spent < seconds and (reps == 0 or spent / reps * (reps + 1) <= 3 * seconds):
            spent += run(copies)
            reps += 1
        return {"value": pairs_of(copies) * reps / spent, "unit": "pairs/s", "cores": threads, "kind": "oracle",
                "sample": f"the full workload (1 query x {wl.n_kv} keys) as {threads} concurrent copies, "
                          f"run {reps} times, {spent:.1f} s",
                "exact_match": exact_match()}
    # many queries: spread a row sample over the host's cores, sized to the budget
    m = min(wl.n_tok, threads)
    rows = list(range(0, wl.n_tok, max(1, wl.n_tok // m)))[:m]
    t = run(rows)
    if t < seconds / 3:
        m2 = min(wl.n_tok, int(len(rows) * seconds / max(t, 1e-3)))
        rows = list(range(0, wl.n_tok, max(1, wl.n_tok // max(m2, 1))))[:max(m2, 1)]
        t = run(rows)
    return {"value": pairs_of(rows) / t, "unit": "pairs/s", "cores": min(threads, len(rows)), "kind": "oracle",
            "sample": f"{len(rows)} of {wl.n_tok} queries (evenly spaced) with all their visible keys, {t:.1f} s",
            "exact_match": exact_match()}


# sparse-attention consumer: the prefill ubatch's shape (512 queries over
# 16384 keys, 512 selected per query) with a synthetic attention shape (64
# heads, latent rows of 512, bf16): the pages fix only the latent width
ATTN_SHAPE = {"n_tok": 512, "n_kv": 16384, "n_head": 64, "latent_dim": 512, "k_sel": 512, "dtype": "bf16"}


def bench_attn(args):
    """Time lid_sparse_attn (one kernel per call) on ATTN_SHAPE."""
    import numpy as np
    import torch

    import lid_inputs as li
    import sparse_attention_token_lid_amd as L

    c = ATTN_SHAPE
    n_tok, n_kv, H, Ld, k_sel = c["n_tok"], c["n_kv"], c["n_head"], c["latent_dim"], c["k_sel"]
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else max(3, steps // 10)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = L.load()
    log("[bench] generating the sparse-attention inputs")
    qa_h, kv_h = li.draw_attn(n_tok, n_kv, H, Ld, c["dtype"], seed=21)
    idx_h = li.draw_selection(n_tok, n_kv, k_sel, seed=22)
    scale = 1.0 / math.sqrt(Ld)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    qa0, kv0, idx0 = bf(qa_h), bf(kv_h), torch.from_numpy(idx_h).to(dev)
    per_copy = sum(t.numel() * t.element_size() for t in (qa0, kv0, idx0))
    copies = max(2, min(64, math.ceil((1 << 30) / per_copy)))
    sets = [(qa0, kv0, idx0)] + [tuple(t.clone() for t in (qa0, kv0, idx0)) for _ in range(copies - 1)]
    out = torch.empty((n_tok, H, Ld), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    calls = [(n_tok, n_kv, H, Ld, k_sel, L.LID_BF16, a.data_ptr(), b.data_ptr(), i.data_ptr(), scale,
              out.data_ptr()) for (a, b, i) in sets]
    log(f"[bench] mode=attn copies={copies} ({per_copy / 2**20:.1f} MiB each) steps={steps} warmup={warmup}")

    def step(i, st=stream):
        rc = lib.lid_sparse_attn(*calls[i % copies], st)
        if rc != 0:
            raise L.LidError(rc, "lid_sparse_attn")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    hip = L.hip_runtime()
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2 * steps):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e)
    torch.cuda.synchronize()
    for i in range(steps):
        L.set_profile_events(evs[2 * i], evs[2 * i + 1])
        step(warmup + i)
    torch.cuda.synchronize()
    L.set_profile_events(None, None)
    kern = []
    for i in range(steps):
        f = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(f), evs[2 * i], evs[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        kern.append(f.value)
    for e in evs:
        hip.hipEventDestroy(e)
    event_ms = sum(kern) / len(kern)
    # timed steps: replayed from HIP graphs, continuing the copy rotation
    total_ms, per_step, G = graph_timing(lambda i, st: step(i, st), steps, copies, (warmup + steps) % copies,
                                         event_ms)
    ms_per_step = total_ms / steps
    log(f"[bench] attn graph: {steps} steps: {total_ms:.3f} ms, {ms_per_step * 1e3:.2f} us/step "
        f"(median {_median(per_step) * 1e3:.2f}, min {min(per_step) * 1e3:.2f}; event pairs {event_ms * 1e3:.2f} us)")
    assert bool(torch.isfinite(out).all()), "non-finite attention output"
    kern_ms = min(event_ms, ms_per_step)   # one kernel per call: the replay is back-to-back launches
    # per (query, head, selected key): 2 L flops for the score, 2 L for the
    # weighted sum (the plain definition; the kernel's split of the weights
    # into two 16-bit parts makes its MFMA work 1.5 times this).  Latent width
    # 512 runs on MFMA (bf16 dense peak); other widths on the fp32 vector ALU.
    flops = 4.0 * n_tok * H * k_sel * Ld
    achieved = flops / (kern_ms * 1e-3)
    mfma = Ld == 512
    pairs = n_tok * k_sel
    res = {
        "metric": "sparse attention (query, selected key) pairs/sec; % MFMA peak",
        "value": pairs * steps / (total_ms * 1e-3), "unit": "pairs/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"sparse attention: n_tok {n_tok} x {k_sel} selected of n_kv {n_kv}, "
                               f"{H} heads, latent {Ld}",
                   **c, "parallelism": "single GPU", "mode": "attn"},
        "timing": f"HIP-graph replays of {G} steps each, every replay between two HIP events",
        "ms_per_step_median": _median(per_step), "ms_per_step_min": min(per_step),
        "kernel_us": kern_ms * 1e3, "kernel_event_us": event_ms * 1e3,
        "kernel_hash": kernel_source_hash("attn"),
        "roofline": {"bound": "mfma" if mfma else "alu", "achieved": achieved / 1e12,
                     "peak": (PEAK_MFMA_F16 if mfma else PEAK_F32_VALU) / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / (PEAK_MFMA_F16 if mfma else PEAK_F32_VALU),
                     "traffic": stored_traffic("attn", "attn", 1) if mfma else None,
                     "traffic_unit": "HBM bytes per launch", "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
        # the first m queries (all of them when they fit the time budget), run
        # repeatedly until about cpu_seconds have been spent
        m = max(1, min(n_tok, threads))
        t0 = time.perf_counter()
        oracle.sparse_attn(qa_h[:m], kv_h, idx_h[:m], scale, qk_dtype="bf16", threads=threads)
        t = time.perf_counter() - t0
        if t < args.cpu_seconds / 3:
            m = max(1, min(n_tok, int(m * args.cpu_seconds / max(t, 1e-3))))
        reps, t = 0, 0.0
        while t < args.cpu_seconds and (reps == 0 or t / reps * (reps + 1) <= 3 * args.cpu_seconds):
            t0 = time.perf_counter()
            oracle.sparse_attn(qa_h[:m], kv_h, idx_h[:m], scale, qk_dtype="bf16", threads=threads)
            t += time.perf_counter() - t0
            reps += 1
        res["cpu_baseline"] = {"value": m * k_sel * reps / t, "unit": "pairs/s", "cores": min(threads, m * H),
                               "kind": "oracle",
                               "sample": f"the first {m} of {n_tok} queries, run {reps} times, {t:.1f} s"}
    print(json.dumps(res), flush=True)


def graph_timing(make_call, steps, copies, base, step_est_ms):
    """Time `steps` calls replayed from HIP graphs.

    make_call(i, stream) issues the call on input copy i.  G calls go in one
    graph (G divides steps; G x the estimated step time >= about 0.3 ms, so a
    replay outlasts its host-side launch), and step j of the timed region uses
    copy (base + j) % copies: the graphs are captured per starting copy, so
    the rotation never comes back to a copy before every other was read.
    Every replay sits between two HIP events.  Returns (total_ms, per-step
    samples in ms (one per replay), G)."""
    import torch
    dev = torch.cuda.current_device()
    want = max(1, math.ceil(0.3 / max(step_est_ms, 1e-4)))
    G = next((g for g in range(1, min(steps, 64) + 1) if steps % g == 0 and g >= want),
             max(g for g in range(1, min(steps, 64) + 1) if steps % g == 0))
    replays = steps // G
    n_graphs = min(replays, copies // math.gcd(G, copies))
    cap = torch.cuda.Stream(dev)
    graphs = []
    torch.cuda.synchronize()
    for r in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            s_cap = torch.cuda.current_stream(dev).cuda_stream
            for i in range(G):
                make_call((base + r * G + i) % copies, s_cap)
        graphs.append(g)
    # one untimed replay of each graph (the first replay of a graph uploads it)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    evs[0].record()
    for j in range(replays):
        graphs[j % n_graphs].replay()
        evs[j + 1].record()
    torch.cuda.synchronize()
    per = [evs[j].elapsed_time(evs[j + 1]) / G for j in range(replays)]
    total = evs[0].elapsed_time(evs[-1])
    del graphs
    return total, per, G


def _median(x):
    y = sorted(x)
    n = len(y)
    return 0.5 * (y[(n - 1) // 2] + y[n // 2])


def run_topk(args, name, steps, warmup, cpu_seconds):
    """Bench one workload of the fused top-k (or the score-only / shared
    modes); returns the result dict of the JSON line."""
    import numpy as np
    import torch

    import lid_inputs as li
    import sparse_attention_token_lid_amd as L

    form = args.form or DEFAULT_FORM[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L.load()

    log(f"[bench] generating {name} ({form})")
    d = li.make(name, with_mask=(form == "mask"))
    wl = d["wl"]
    if form == "mask" and d["mask"] is None:
        raise SystemExit("dense mask form is not generated on the host for this workload; use --form ranges")
    pairs = visible_pairs(wl, d["ranges"] if form != "none" else None)

    def dev_tensor(a, kind):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if kind in ("f16bits",) else a)
        t = t.to(dev)
        return t.view(torch.float16) if kind == "f16bits" else t

    q0 = torch.from_numpy(d["q"]).to(dev)
    k0 = torch.from_numpy(d["k"]).to(dev)
    w0 = torch.from_numpy(d["w"]).to(dev)
    m0 = dev_tensor(d["mask"], "f16bits") if form == "mask" else None
    r0 = torch.from_numpy(d["ranges"]).to(dev) if form == "ranges" else None
    fp8 = args.qk == "fp8"
    qs0 = ks0 = None
    if fp8:
        if args.mode != "topk":
            raise SystemExit("--qk fp8 goes with --mode topk")
        # per-row max scaling to E4M3 (synthetic inputs: the pages give no indexer scale convention)
        qs0 = q0.float().abs().amax(dim=2).clamp(min=1e-20) / 448.0
        ks0 = k0.float().abs().amax(dim=1).clamp(min=1e-20) / 448.0
        q0 = (q0.float() / qs0[:, :, None]).to(torch.float8_e4m3fn)
        k0 = (k0.float() / ks0[:, None]).to(torch.float8_e4m3fn)
    per_copy = sum(t.numel() * t.element_size() for t in (q0, k0, w0, m0, r0, qs0, ks0) if t is not None)
    # at least 1 GiB of copies (4x the last-level cache), and at least 2
    copies = max(2, min(64, math.ceil((1 << 30) / per_copy)))
    sets = [(q0, k0, w0, m0, r0, qs0, ks0)]
    for _ in range(copies - 1):
        sets.append(tuple(None if t is None else t.clone() for t in (q0, k0, w0, m0, r0, qs0, ks0)))
    shape = L.shape_for(q0, k0, wl.k_top, m0, splits=args.splits)
    plan, splits = L.plan_of(shape)
    ws_bytes = L.workspace_size(shape)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # the counter region starts at zero
    idx = torch.empty((wl.n_tok, wl.k_top), dtype=torch.int32, device=dev)
    sc = torch.empty((wl.n_tok, wl.k_top), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    lib = L.load()
    scores_mode = args.mode == "scores"
    shared_mode = args.mode == "shared"
    if shared_mode:
        # one ubatch-wide selection: every (query, key) pair is scored
        lib.lid_topk_shared_workspace_size.restype = ctypes.c_size_t
        ws_bytes = int(lib.lid_topk_shared_workspace_size(ctypes.byref(shape)))
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        idx = torch.empty((wl.k_top,), dtype=torch.int32, device=dev)
        sc = torch.empty((wl.k_top,), dtype=torch.float32, device=dev)
        plan, splits = "shared", 1
        pairs = wl.n_tok * wl.n_kv
    if scores_mode:
        sout = torch.empty((wl.n_tok, wl.n_kv), dtype=torch.float32, device=dev)
        pshape = L.shape_for(q0, k0, wl.k_top, m0, plan=L.PLAN_PREFILL)
        plan, splits = "prefill (score-only)", L.plan_of(pshape)[1]
        ws_bytes = 0
    calls = []
    for (q, k, w, m, r, qs, ks) in sets:
        ptrs = [t.data_ptr() if t is not None else None for t in (q, k, w, m, r)]
        if scores_mode:
            calls.append((ctypes.byref(shape), *ptrs, sout.data_ptr(), wl.n_kv))
        elif fp8:
            calls.append((ctypes.byref(shape), ptrs[0], qs.data_ptr(), ptrs[1], ks.data_ptr(), *ptrs[2:],
                          idx.data_ptr(), sc.data_ptr(), ws.data_ptr(), ws_bytes))
        else:
            calls.append((ctypes.byref(shape), *ptrs, idx.data_ptr(), sc.data_ptr(), ws.data_ptr(), ws_bytes))
    log(f"[bench] {name}: mode={args.mode} plan={plan} splits={splits} workspace={ws_bytes} B copies={copies} "
        f"({per_copy / 2**20:.1f} MiB each) steps={steps} warmup={warmup}")
    entry = lib.lid_scores if scores_mode else (lib.lid_topk_shared if shared_mode else
                                                (lib.lid_topk_fp8 if fp8 else lib.lid_topk))

    def call(i, st):
        rc = entry(*calls[i % copies], st)
        if rc != 0:
            raise L.LidError(rc)

    for i in range(warmup):
        call(i, stream)
    torch.cuda.synchronize()

    hip = L.hip_runtime()
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2 * steps):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        L.set_profile_events(evs[2 * i], evs[2 * i + 1])
        call(warmup + i, stream)
    t1.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    L.set_profile_events(None, None)
    total_ms = t0.elapsed_time(t1)
    kern = []
    for i in range(steps):
        f = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(f), evs[2 * i], evs[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        kern.append(f.value)
    for e in evs:
        hip.hipEventDestroy(e)
    kern_ms = sum(kern) / len(kern)
    eager_ms_per_step = total_ms / steps
    log(f"[bench] {name} eager: {steps} steps: {total_ms:.3f} ms GPU ({(wall1 - wall0) * 1e3:.1f} ms wall), "
        f"{eager_ms_per_step * 1e3:.2f} us/step, scoring kernel {kern_ms * 1e3:.2f} us")

    # The timed steps proper, replayed from HIP graphs (see graph_timing),
    # continuing the copy rotation where the eager steps left it.
    total_ms, per_step, G = graph_timing(call, steps, copies, (warmup + steps) % copies, kern_ms)
    ms_per_step = total_ms / steps
    log(f"[bench] {name} graph: {steps} steps ({steps // G} replays of {G}): {total_ms:.3f} ms GPU, "
        f"{ms_per_step * 1e3:.2f} us/step (median {_median(per_step) * 1e3:.2f}, min {min(per_step) * 1e3:.2f})")
    # the graph's last replay left a real result in idx / sc: spot-check it is a valid row
    if scores_mode:
        assert bool(torch.isfinite(sout[-1]).any()), "no visible score in the last row"
    else:
        got = (idx if shared_mode else idx[0]).cpu().numpy()
        assert got.max() < wl.n_kv and (got[got >= 0].size == np.unique(got[got >= 0]).size), "invalid top-k row"

    H, D, K = wl.n_head, wl.head_dim, wl.k_top
    value = pairs * steps / (total_ms * 1e-3)
    # The roofline's kernel duration.  A HIP event pair around one eager launch
    # also counts the dispatch in front of the kernel (a few us, which the
    # rocprofv3 trace does not); when a call is this one kernel alone (decode;
    # prefill with one split or up to 16 splits finished in the kernel), the
    # graph replay's mean time per step is back-to-back launches of it and
    # agrees with the trace, so that is used; other calls keep the event pairs.
    n2 = 1 << max(0, (K - 1).bit_length())
    one_kernel = not scores_mode and not shared_mode and (
        plan == "decode" or (plan == "prefill" and (splits == 1 or (splits <= 16 and 256 <= n2 <= 1024 and K % 2 == 0))))
    event_kern_ms = kern_ms
    if one_kernel:
        kern_ms = min(kern_ms, ms_per_step)
    if scores_mode:
        flops = 2.0 * H * D * pairs
        out_bytes = wl.n_tok * wl.n_kv * 4
        in_bytes = wl.n_kv * D * 2 + wl.n_tok * (H * D * 2 + H * 4) + (pairs * 2 if form == "mask" else 0)
        f_mfma = flops / (kern_ms * 1e-3) / PEAK_MFMA_F16
        f_hbm = (in_bytes + out_bytes) / (kern_ms * 1e-3) / PEAK_HBM_BPS
        if f_mfma >= f_hbm:
            roof = {"bound": "mfma", "achieved": flops / (kern_ms * 1e-3) / 1e12, "peak": PEAK_MFMA_F16 / 1e12,
                    "unit": "TFLOP/s", "frac": f_mfma, "traffic": None, "traffic_unit": "HBM bytes per launch",
                    "algorithmic_flops": flops, "output_bytes": out_bytes}
        else:
            roof = {"bound": "hbm", "achieved": (in_bytes + out_bytes) / (kern_ms * 1e-3) / 1e9,
                    "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s", "frac": f_hbm, "traffic": None,
                    "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": in_bytes + out_bytes}
    elif plan == "decode":
        eb = 1 if fp8 else 2   # bytes per q / k element
        key_bytes = pairs * (D * eb + (4 if fp8 else 0))
        alg_bytes = key_bytes + wl.n_tok * (H * D * eb + H * (8 if fp8 else 4)) + (pairs * 2 if form == "mask" else 0) \
            + wl.n_tok * K * 8
        achieved = alg_bytes / (kern_ms * 1e-3)
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_BPS, "traffic": None if fp8 else stored_traffic(name, plan, splits),
                "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": alg_bytes}
    else:
        flops = 2.0 * H * D * pairs
        achieved = flops / (kern_ms * 1e-3)
        peak = PEAK_MFMA_FP8 if fp8 else PEAK_MFMA_F16   # a contraction takes the peak of its own dtype
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None if fp8 else stored_traffic(name, plan, splits),
                "traffic_unit": "HBM bytes per launch", "algorithmic_flops": flops}
    out = {
        "metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f8e4m3" if fp8 else wl.dtype, "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTION[name]}", "n_tok": wl.n_tok, "n_kv": wl.n_kv, "n_head": H,
                   "head_dim": D, "k_top": K, "visible_pairs": pairs, "visibility": form, "plan": plan,
                   "splits": splits, "workspace_bytes": ws_bytes, "parallelism": "single GPU", "mode": args.mode},
        "topk_tokens_per_s": wl.n_tok * steps / (total_ms * 1e-3),
        "timing": f"HIP-graph replays of {G} steps each, every replay between two HIP events",
        "ms_per_step_median": _median(per_step), "ms_per_step_min": min(per_step),
        "input_copies": copies, "input_copy_bytes": per_copy,
        "eager_ms_per_step": eager_ms_per_step,
        "scoring_kernel_us": kern_ms * 1e3,
        "scoring_kernel_timing": "graph replay mean, one kernel per call" if one_kernel
        else "HIP events around each eager launch",
        "scoring_kernel_event_us": event_kern_ms * 1e3,
        "scoring_kernel_event_us_median": _median(kern) * 1e3,
        "kernel_hash": kernel_source_hash(plan),
        "roofline": roof,
    }
    if cpu_seconds and not scores_mode and not fp8 and not shared_mode:
        log(f"[bench] timing the CPU oracle (~{cpu_seconds:.0f} s)")
        # the last replay left the workload's result in idx: the oracle's
        # sampled rows are compared with it
        out["cpu_baseline"] = cpu_baseline(d, form, cpu_seconds, gpu_idx=idx.cpu().numpy())
    del sets, calls
    torch.cuda.empty_cache()
    return out


def summary_of(r):
    """The per-workload fields of a secondary workload's result."""
    roof = r["roofline"]
    return {"workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"], "steps": r["steps"],
            "ms_per_step": r["ms_per_step"], "ms_per_step_median": r["ms_per_step_median"],
            "ms_per_step_min": r["ms_per_step_min"], "plan": r["config"]["plan"], "splits": r["config"]["splits"],
            "visibility": r["config"]["visibility"], "kernel_hash": r["kernel_hash"],
            "scoring_kernel_us": r["scoring_kernel_us"],
            "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None, choices=sorted(DEFAULT_STEPS),
                    help="bench this workload alone (default: the headline c5 plus the other graded workloads)")
    ap.add_argument("--form", default=None, choices=["none", "mask", "ranges"])
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--qk", default="f16", choices=["f16", "fp8"],
                    help="f16: the workload's f16 q and k (the default); fp8: the same values quantised to "
                         "OCP E4M3 with per-row scales (max |row| / 448), run through lid_topk_fp8")
    ap.add_argument("--mode", default="topk", choices=["topk", "scores", "shared", "attn"],
                    help="topk: the fused top-k (the default); scores: the score-only mode (lid_scores), "
                         "which writes the n_tok x n_kv f32 scores; shared: the per-ubatch top-k "
                         "(lid_topk_shared); attn: the sparse attention over a selection (lid_sparse_attn)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="without --workload: time the headline workload only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the indexer path here is a single-GPU build "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.mode == "attn":
        bench_attn(args)
        return

    name = args.workload or HEADLINE
    steps = args.steps if args.steps is not None else DEFAULT_STEPS[name]
    warmup = args.warmup if args.warmup is not None else max(3, steps // 10)
    cpu = None if args.no_cpu_baseline else args.cpu_seconds
    secondary = args.workload is None and not args.no_secondary and args.mode == "topk" and args.qk == "f16" \
        and args.form is None and args.splits == 0
    others = {}
    if secondary:
        # the other graded workloads first (their inputs are freed before the
        # headline's), each with its own step count
        for w2, k2 in SECONDARY.items():
            others[w2] = summary_of(run_topk(args, w2, k2, max(3, k2 // 10), None))
    out = run_topk(args, name, steps, warmup, cpu)
    if secondary:
        out["workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
