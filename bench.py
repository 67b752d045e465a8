#!/usr/bin/env python3
"""Throughput of the CSA / HCA hot path on one MI355X.

Default workload: CSA decode at 64K context -- 32 sequences x 16,384
compressed entries, bf16, 64 query heads x 512, indexer 64 x 128, top-k 1024,
window 128.  A step is one pass of the path for the whole batch:
indexer_score -> topk_select -> sparse_mqa_attend (query RMSNorm + RoPE fused
into the attention prologue, inverse RoPE into its epilogue).

Inputs are resident in HBM before the timed region.  Every decode read set is
below the 256 MiB Infinity Cache, so the timed steps rotate through several
copies of the caches at distinct addresses (cold-cache protocol).

Prints ONE JSON line.  ``value`` = query tokens/s (decode) or TFLOP/s
(prefill).  ``roofline`` rates the longest single kernel of the step against
its bound (per-call time from HIP events around back-to-back launches on the
launch stream); ``roofline_step`` rates the whole step (median of per-step
event times) against the same peak and a measured device-copy rate, with each
call's own fraction; ``cpu_baseline`` times the fp64 oracle on a bounded
sample of the same workload on this host (with the host's CPU count and
model), and the MXFP4 workload adds the top-k recall against the fp64
oracle.  ``tiny_csa`` / ``tiny_hca`` report time only.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

METRIC = "CSA decode query-tokens/s @64K–1M ctx, % HBM roofline; prefill TFLOP/s"

# HBM traffic of the roofline kernel, per launch: rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), each scaled by bytes / counter of a plain copy
# of known size (--copy-probe).  An entry holds for the kernel source it was
# taken on (sha256 of the .hip file); after any change it reports null.
TRAFFIC = {
    'decode_64k': {"kernel": "indexer_mfma_kernel", "src": "indexer.hip", "sha256": "11edc41b8d401743b8505978f26a4f4bd07674f12674e731507cd4bd8cfe797c", "fetch_kib": 67723.0, "write_kib": 2048.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'decode_1m_fp4': {"kernel": "indexer_mfma_kernel", "src": "indexer.hip", "sha256": "11edc41b8d401743b8505978f26a4f4bd07674f12674e731507cd4bd8cfe797c", "fetch_kib": 69941.3, "write_kib": 4096.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'prefill_32k': {"kernel": "attend_pf_kernel", "src": "attend.hip", "sha256": "7ecf3628d32825a140dc0e8963b807f6116a1d2a6f0b1f10e08a7e180c5977b0", "fetch_kib": 3585243.6, "write_kib": 2097152.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'prefill_32k_mxfp4': {"kernel": "attend_pf_kernel", "src": "attend.hip", "sha256": "7ecf3628d32825a140dc0e8963b807f6116a1d2a6f0b1f10e08a7e180c5977b0", "fetch_kib": 3528917.9, "write_kib": 2097152.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'oproj_decode': {"kernel": "grouped_out_proj", "src": "oproj.hip", "sha256": "fdf6181d79947eb13a3532a65336dabd0336924f79cbadcfe230d06ce9d3d945", "fetch_kib": 80943.6, "write_kib": 8968.2, "fetch_scale": 1.9998, "write_scale": 1.0},
    'oproj_prefill': {"kernel": "grouped_out_proj", "src": "oproj.hip", "sha256": "fdf6181d79947eb13a3532a65336dabd0336924f79cbadcfe230d06ce9d3d945", "fetch_kib": 4495578.3, "write_kib": 842334.2, "fetch_scale": 1.9998, "write_scale": 1.0},
    'hca_decode_1m': {"kernel": "attend_mfma_kernel + attend_combine_kernel", "src": "attend.hip", "sha256": "7ecf3628d32825a140dc0e8963b807f6116a1d2a6f0b1f10e08a7e180c5977b0", "fetch_kib": 75833.2, "write_kib": 17536.0, "fetch_scale": 1.9998, "write_scale": 1.0},
}


# ------------------------------------------------------------------ algorithmic bytes
def decode_bytes(sp, N):
    """Algorithmic bytes per query token (one sequence).  `total` is what the
    method must move: index keys, the indexer query and weights, the selected
    KV rows and the window, the query and the output.  The per-stage figures
    add each kernel's own output and the intermediates it reads (scores,
    indices), which a fused path would not move."""
    c, d_r = sp.c, sp.d_r
    row = {"bf16": 2 * c, "fp8mix": (c - d_r) + 2 * d_r, "f32": 4 * c}[sp.kv_format]
    q = sp.nh * c * 2
    out = sp.nh * c * 2
    win = sp.n_win * row
    if sp.kind == "hca_decode":
        attend = N * row + win + q + out
        return dict(attend=attend, total=attend)
    if sp.index_format == "mxfp4":
        kI = N * (sp.cI // 2 + sp.cI // 32)
        qI = sp.nI * (sp.cI // 2 + sp.cI // 32)
        score = 2
    else:
        kI = N * sp.cI * 2
        qI = sp.nI * sp.cI * 2
        score = 4
    method_indexer = kI + qI + sp.nI * 4
    attend = min(sp.k, N) * row + win + q + out
    return dict(indexer=method_indexer + N * score, topk=N * score + sp.k * 4, attend=attend,
                total=method_indexer + attend)


# the kernels behind each call of the decode step
DECODE_KERNELS = {"indexer": "indexer_mfma_kernel",
                  "topk": "topk_fine_hist_kernel + topk_fine_emit_kernel (2^14 < N); topk_kernel",
                  "attend": "attend_mfma_kernel + attend_combine_kernel"}


def prefill_flops(sp, T):
    """Algorithmic flops of indexer + attention over a causal prefill."""
    fi = fa = 0
    for q in range(T):
        nv = (q + 1) // sp.m
        fi += nv * sp.nI * sp.cI * 2
        fa += (min(sp.k, nv) + min(q + 1, sp.n_win)) * sp.nh * sp.c * 4
    return fi, fa


# ------------------------------------------------------------------ timing helpers
def timed_steps(torch, stream, run_step, steps):
    """K steps back to back on `stream`, bracketed by a synchronize on both
    sides and nothing between the steps: wall seconds (the value).  Then K
    more with a HIP event at each step boundary: per-step GPU microseconds
    (the distribution; each event adds its own dispatch gap, a few us).
    Also the host seconds spent launching the K steps of the first pass."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps):
            run_step(i)
    host = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for i in range(steps):
            run_step(i)
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return wall, np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]), host


def stage_times(torch, stream, stages, reps):
    """Each call of the path launched `reps` times back to back (over the
    rotated inputs) between two HIP events on its launch stream: microseconds
    per call, the period a call takes in a full queue.  Events between the
    calls of a step would add their own dispatch gaps (4-7 us per call here);
    this period matches the kernel trace's durations."""
    out = {}
    for name, fn in stages:
        with torch.cuda.stream(stream):
            fn(0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                fn(i)
            e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / reps
    return out


def distribution(us):
    return dict(median=float(np.median(us)), p10=float(np.percentile(us, 10)),
                p90=float(np.percentile(us, 90)), mean=float(np.mean(us)))


def copy_bandwidth(torch, stream, nbytes=1 << 30, reps=10):
    """Read + write GB/s of a plain device copy (the streaming rate a kernel can
    reach), measured here."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    with torch.cuda.stream(stream):
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            b.copy_(a)
        e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


# ------------------------------------------------------------------ CPU baseline
def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return dict(host_cpus=os.cpu_count(), cpus_available=affinity, cpu_model=model,
                blas_threads=blas_threads())


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline_decode(inp, budget_s=12.0):
    from oracle import pipeline as OP
    sp = inp["spec"]
    t0 = time.perf_counter()
    n = 0
    while True:
        OP.decode_reference(inp, n % sp.B)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="query-tokens/s", cores=blas_threads(), kind="oracle",
                sample=f"{n} query tokens (sequences cycled) of the same workload, fp64 numpy, "
                       f"{dt:.1f} s", **host_info())


def fp4_recall(inp, gpu_idx, seqs=(0, -1)):
    """Top-k recall of the timed selection (MXFP4 index keys and queries,
    bf16 scores) against the fp64 oracle's top-k over the unquantised keys and
    queries, for a sample of sequences."""
    from oracle import csa as O
    sp = inp["spec"]
    rec = []
    t0 = time.perf_counter()
    for b in sorted({s % sp.B for s in seqs}):
        N, p = int(inp["n_entries"][b]), int(inp["q_pos"][b, 0])
        nv = int(O.n_visible(p, sp.m, N))
        ref = set(O.topk(O.index_scores(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv),
                         nv, sp.k).tolist())
        got = {int(x) for x in gpu_idx[b, 0] if x >= 0}
        rec.append(len(ref & got) / min(sp.k, nv))
    return dict(value=float(np.mean(rec)), per_sequence=rec,
                against="fp64 oracle top-k over the unquantised index keys and queries",
                seconds=round(time.perf_counter() - t0, 1),
                context="the pages quote 99.7% for a trained model; these keys are N(0,1)")


def cpu_baseline_prefill(inp, rows, budget_s=12.0):
    from oracle import pipeline as OP
    sp = inp["spec"]
    t0 = time.perf_counter()
    caches = OP.prefill_caches(inp)       # compression is not part of the timed path
    t1 = time.perf_counter()
    done, flops = 0, 0.0
    for r in rows:
        OP.prefill_reference(inp, caches, [r])
        p = int(inp["q_pos"][r])
        nv = (p + 1) // sp.m
        flops += nv * sp.nI * sp.cI * 2 + (min(sp.k, nv) + min(p + 1, sp.n_win)) * sp.nh * sp.c * 4
        done += 1
        if time.perf_counter() - t1 > budget_s:
            break
    dt = time.perf_counter() - t1
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=blas_threads(), kind="oracle",
                sample=f"{done} query rows spread over the sequence (indexer+top-k+attention, "
                       f"fp64 numpy, {dt:.1f} s; compression done beforehand in {t1 - t0:.1f} s)",
                **host_info())


# ------------------------------------------------------------------ decode bench
def run_decode(args, torch, I, G):
    sp = I.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    inp = I.decode_inputs(sp)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        base = G.upload_decode(inp, dev, stream)
        if args.paged:                           # caches moved into a hybrid page pool
            G.page_decode(base, seed=1, drop_dense=True)
        copies = [base]
        for _ in range(args.copies - 1):
            c = G.Decode(**{k: getattr(base, k) for k in base.__dataclass_fields__})
            for name in ("kv", "win", "kI", "kI_scale", "qI", "qI_scale", "w", "q", "scores",
                         "idx", "out"):
                v = getattr(base, name)
                if v is not None:
                    setattr(c, name, v.clone())
            if base.pool is not None:
                c.pool = base.pool.clone()
            c.ws = None
            c.ws_topk = None
            copies.append(c)
        for c in copies:                         # workspace sizing outside the timed region
            G.decode_step(c, stream)
    torch.cuda.synchronize()
    print(f"[bench] {args.copies} cache copies resident", file=sys.stderr, flush=True)
    kinds = ["indexer", "topk", "attend"] if sp.kind == "decode" else ["attend"]
    call = {"indexer": G.decode_indexer, "topk": G.decode_topk,
            "attend": lambda c, s: G.decode_attend(c, stream=s)}
    # the step: eager launches (measured faster here than HIP graph replay of
    # the same calls), or one HIP graph per cache copy with --graph
    side = torch.cuda.Stream()

    def step_fn(c):
        if args.chunks > 1:
            G.decode_step_overlapped(c, [stream, side], args.chunks)
        else:
            G.decode_step(c, stream)
    with torch.cuda.stream(stream):
        for c in copies:                         # sizes the chunk workspaces
            step_fn(c)
    torch.cuda.synchronize()
    if args.graph:
        graphs = []
        for c in copies:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                step_fn(c)
            graphs.append(gr)
        torch.cuda.synchronize()
        run_step = lambda i: graphs[i % len(graphs)].replay()
    else:
        run_step = lambda i: step_fn(copies[i % len(copies)])
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            run_step(i)
    torch.cuda.synchronize()
    # the timed steps (value, and the distribution of the step)
    elapsed, step_us, host_s = timed_steps(torch, stream, run_step, args.steps)
    # per-call times: each call back to back over the rotated copies
    stages = [(kind, (lambda i, k=kind: call[k](copies[i % len(copies)], stream)))
              for kind in kinds]
    avg = stage_times(torch, stream, stages, max(args.steps, 12))
    copy_gbs = copy_bandwidth(torch, stream)
    ms_step = elapsed / args.steps * 1e3
    N = inp["Nmax"]
    by = decode_bytes(sp, N)
    value = sp.B * args.steps / elapsed
    dist = distribution(step_us)
    step_bytes = by["total"] * sp.B
    step_gbs = step_bytes / (dist["median"] * 1e-6) / 1e9
    per = {}
    for k in kinds:
        gbs = by[k] * sp.B / (avg[k] * 1e-6) / 1e9
        per[k] = dict(kernels=DECODE_KERNELS[k], us=round(avg[k], 2), bytes=by[k] * sp.B,
                      achieved_gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    # the dominant kernel: the longest single kernel of the step, the indexer
    # in CSA decode (the attention call is two kernels, each shorter; every
    # call's own fraction is under roofline_step.kernels); HCA decode has only
    # the attention call
    dom = "indexer" if "indexer" in kinds else "attend"
    dom_bytes = by[dom] * sp.B
    achieved = dom_bytes / (avg[dom] * 1e-6) / 1e9
    res = dict(
        metric=METRIC, value=value, unit="query-tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype=("bf16" if sp.index_format == "bf16" else "mxfp4+fp8/bf16"),
        data="synthetic",
        config=dict(workload=sp.name, batch=sp.B, context=sp.L, compressed_entries=N, m=sp.m,
                    heads=sp.nh, head_dim=sp.c, rope_dims=sp.d_r, top_k=sp.k or None,
                    indexer=(f"{sp.nI}x{sp.cI} {sp.index_format}" if sp.nI else None),
                    kv_format=sp.kv_format, window=sp.n_win, cache_copies=args.copies,
                    cache=(f"paged: {base.pool.page_bytes}-byte pages of 32 CSA rows + 32 index "
                           "keys + 1 HCA row, random page order" if base.pool is not None
                           else "dense")),
        roofline=dict(bound="hbm", kernel=DECODE_KERNELS[dom], achieved=achieved,
                      peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS, traffic=None,
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=avg[dom],
                      timing="HIP events around back-to-back launches of the call over the "
                             "rotated copies, on its launch stream, after the timed steps"),
        roofline_step=dict(bound="hbm", achieved=step_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                           frac=step_gbs / HBM_PEAK_GBS, algorithmic_bytes=step_bytes,
                           step_us=dist, host_launch_us=round(host_s / args.steps * 1e6, 2),
                           copy_gbs=round(copy_gbs, 1),
                           frac_of_copy=step_gbs / copy_gbs, kernels=per,
                           launch=("HIP graph per cache copy" if args.graph else "eager launches")
                           + (f"; batch in {args.chunks} groups on 2 streams"
                              if args.chunks > 1 else "")),
    )
    return res, (inp, copies[0])


# ------------------------------------------------------------------ output projection
# the Flash shape of the configuration table: 64 heads x 512, 8 groups of rank
# 1024, hidden 4096; decode = one step's 32 query rows, prefill = 32K rows
OPROJ = dict(oproj_decode=32, oproj_prefill=32768)


def run_oproj(args, torch):
    import long_context_sparse_10_amd as L
    R, nh, c, g, d_g, d = OPROJ[args.config], 64, 512, 8, 1024, 4096
    K1, Ku = nh // g * c, g * d_g
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(1007)
    bf = torch.bfloat16
    o = torch.randn(R, nh, c, generator=gen, device=dev).to(bf)
    # weight copies rotated so the 128 MiB of weights do not stay in the
    # 256 MiB Infinity Cache between calls (decode)
    ncopy = 3 if R <= 64 else 1
    Ws = [((torch.randn(g, d_g, K1, generator=gen, device=dev) / math.sqrt(K1)).to(bf),
           (torch.randn(d, Ku, generator=gen, device=dev) / math.sqrt(Ku)).to(bf))
          for _ in range(ncopy)]
    y = torch.empty(R, d, dtype=bf, device=dev)
    stream = torch.cuda.Stream()
    ws = None
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, ncopy)):
            Wa, Wb = Ws[i % ncopy]
            ws = L.grouped_out_proj(o, L.BF16, R, nh, c, g, d_g, Wa, Wb, d, y, L.BF16, ws, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            Wa, Wb = Ws[i % ncopy]
            L.grouped_out_proj(o, L.BF16, R, nh, c, g, d_g, Wa, Wb, d, y, L.BF16, ws, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    call_us = e0.elapsed_time(e1) * 1e3 / args.steps
    ms = elapsed / args.steps * 1e3
    flops = 2.0 * R * (nh * c * d_g + Ku * d)
    # algorithmic bytes: both weight matrices, o, y, and u written and read once
    nbytes = 2 * (g * d_g * K1 + d * Ku + R * nh * c + R * d + 2 * R * Ku)
    cfg = dict(workload=args.config, rows=R, heads=nh, head_dim=c, groups=g, rank_per_group=d_g,
               hidden=d, weight_copies=ncopy)
    res = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=ms,
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
               data="synthetic", config=cfg,
               step=dict(call_us=call_us, kernels="u = per-group o.W_a^T, then y = u.W_b^T"))
    if R <= 64:
        gbs = nbytes / (call_us * 1e-6) / 1e9
        res.update(value=R / (ms * 1e-3), unit="query-tokens/s",
                   roofline=dict(bound="hbm", kernel="grouped_out_proj", achieved=gbs,
                                 peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                                 traffic=None, algorithmic_bytes_per_launch=nbytes,
                                 avg_launch_us=call_us))
    else:
        tf = flops / (call_us * 1e-6) / 1e12
        res.update(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s",
                   roofline=dict(bound="mfma", kernel="grouped_out_proj", achieved=tf,
                                 peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=tf / BF16_PEAK_TFLOPS,
                                 traffic=None, algorithmic_flops_per_launch=flops,
                                 avg_launch_us=call_us))
    return res, (o, Ws[0], R, nh, c, g, d_g, d)


def cpu_baseline_oproj(case, budget_s=10.0):
    """The oracle's grouped projection on a bounded sample of rows."""
    from oracle import csa as O
    o, (Wa, Wb), R, nh, c, g, d_g, d = case
    rows = min(R, 32)
    oo = o[:rows].float().cpu().numpy()
    Wa_, Wb_ = Wa.float().cpu().numpy(), Wb.float().cpu().numpy()
    t0 = time.perf_counter()
    n = 0
    while True:
        O.grouped_out_proj(oo, Wa_, Wb_)
        n += rows
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="query-tokens/s", cores=blas_threads(), kind="oracle",
                sample=f"{n} rows ({rows} per call) of the same shape, fp64 numpy, {dt:.1f} s",
                **host_info())


# ------------------------------------------------------------------ prefill bench
def run_prefill(args, torch, I, G):
    sp = I.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    inp = I.prefill_inputs(sp)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        p = G.upload_prefill(inp, dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        G.prefill_compress(p, stream)
        e1.record(stream)
        G.prefill_attention_path(p, stream)
    torch.cuda.synchronize()
    t_comp = e0.elapsed_time(e1)
    n = sp.T // sp.m
    for _ in range(args.warmup):
        with torch.cuda.stream(stream):
            G.prefill_attention_path(p, stream)
    torch.cuda.synchronize()
    import long_context_sparse_10_amd as L
    sfmt = L.BF16 if sp.index_format == "mxfp4" else L.F32
    scale = 1.0 / math.sqrt(sp.c)
    elapsed, step_us, host_s = timed_steps(torch, stream, lambda i: G.prefill_attention_path(p, stream),
                                   args.steps)
    stages = [
        ("indexer", lambda i: G.prefill_indexer(p, stream)),
        ("topk", lambda i: L.topk_select(p.scores, sfmt, p.q_pos, p.n_entries, 1, sp.T, n, sp.m,
                                         sp.k, p.idx, None, stream)),
        ("attend", lambda i: L.sparse_mqa_attend(p.q, L.BF16, p.gamma, 1e-6, sp.d_r, 1e4, p.q_pos,
                                                 p.kv, L.BF16, n, p.idx, sp.k, p.win, sp.T,
                                                 sp.n_win, p.sink, scale, 1, sp.T, sp.nh, sp.c,
                                                 p.out, L.BF16, p.ws_attend, stream)),
    ]
    avg = stage_times(torch, stream, stages, args.steps)
    fi, fa = prefill_flops(sp, sp.T)
    ms = elapsed / args.steps * 1e3
    tflops = (fi + fa) / (ms * 1e-3) / 1e12
    dist = distribution(step_us)
    step_tf = (fi + fa) / (dist["median"] * 1e-6) / 1e12
    att = fa / (avg["attend"] * 1e-6) / 1e12
    idx_tf = fi / (avg["indexer"] * 1e-6) / 1e12
    per = dict(indexer=dict(kernels="indexer_rows_kernel", us=round(avg["indexer"], 1),
                            flops=fi, tflops=round(idx_tf, 1),
                            frac=round(idx_tf / BF16_PEAK_TFLOPS, 4)),
               topk=dict(kernels="topk_kernel", us=round(avg["topk"], 1)),
               attend=dict(kernels="attend_pf_kernel", us=round(avg["attend"], 1), flops=fa,
                           tflops=round(att, 1), frac=round(att / BF16_PEAK_TFLOPS, 4)))
    res = dict(
        metric=METRIC, value=tflops, unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16" if sp.index_format == "bf16" else "bf16+mxfp4 indexer",
        data="synthetic",
        config=dict(workload=sp.name, seq_len=sp.T, hidden=sp.d, heads=sp.nh, head_dim=sp.c,
                    top_k=sp.k, indexer=f"{sp.nI}x{sp.cI} {sp.index_format}", window=sp.n_win),
        roofline=dict(bound="mfma", kernel="attend_pf_kernel", achieved=att,
                      peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=att / BF16_PEAK_TFLOPS,
                      traffic=None, algorithmic_flops_per_launch=fa, avg_launch_us=avg["attend"],
                      timing="HIP events around back-to-back launches of the call, on its "
                             "launch stream, after the timed steps"),
        roofline_step=dict(bound="mfma", achieved=step_tf, peak=BF16_PEAK_TFLOPS,
                           unit="TFLOP/s", frac=step_tf / BF16_PEAK_TFLOPS,
                           algorithmic_flops=fi + fa, step_us=dist, kernels=per,
                           compress_ms_untimed=t_comp),
    )
    return res, inp


# ------------------------------------------------------------------ compression
def compress_flops(sp, T):
    """Algorithmic flops of the prefill compressor: the projections (main KV
    2 or 4, index keys 4, window rows 1) of every token, 2 flops per MAC."""
    nkv = 4 if sp.m == 4 else 2
    f = nkv * T * sp.c * sp.d * 2 + T * sp.c * sp.d * 2
    if sp.nI:
        f += 4 * T * sp.cI * sp.d * 2
    return f


def run_compress(args, torch, I, G):
    """The prefill workload's compression alone (csa_compress for the main KV
    entries, the index keys and the per-token window rows): not part of the
    prefill metric, measured as its own row."""
    sp = I.CONFIGS["prefill_32k"]
    dev = torch.device("cuda", 0)
    inp = I.prefill_inputs(sp)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        p = G.upload_prefill(inp, dev)
        for _ in range(max(args.warmup, 1)):
            G.prefill_compress(p, stream)
    torch.cuda.synchronize()
    elapsed, step_us, host_s = timed_steps(torch, stream, lambda i: G.prefill_compress(p, stream), args.steps)
    fl = compress_flops(sp, sp.T)
    dist = distribution(step_us)
    tf = fl / (dist["median"] * 1e-6) / 1e12
    ms = elapsed / args.steps * 1e3
    return dict(
        metric=METRIC, value=fl / (ms * 1e-3) / 1e12, unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload="compress_32k", seq_len=sp.T, hidden=sp.d, m=sp.m, head_dim=sp.c,
                    indexer_dim=sp.cI, calls="main KV (4 projections), index keys (4), window (1)"),
        roofline=dict(bound="mfma", kernel="csa_compress (3 calls: weight transposes, "
                      "oproj_big_kernel, pool_kernel)", achieved=tf, peak=BF16_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=tf / BF16_PEAK_TFLOPS, traffic=None,
                      algorithmic_flops_per_launch=fl, avg_launch_us=dist["median"],
                      timing="HIP events at the step boundaries (median step)"),
        step=dict(step_us=dist),
        cpu_baseline=None,
    )


# ------------------------------------------------------------------ tiny configurations
def run_tiny(args, torch, I, G):
    """Tiny CSA / HCA: one sequence of 1024 tokens, hidden 256, fp32.  A step is
    the whole path: compression (main KV, index keys, window rows), then
    indexer, top-k and sparse attention (CSA) or dense attention (HCA).  Time
    only: every kernel runs a few microseconds, launch latency decides."""
    sp = I.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    inp = I.prefill_inputs(sp)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        p = G.upload_prefill(inp, dev)

    def step(i):
        G.prefill_compress(p, stream)
        G.prefill_attention_path(p, stream)
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, 1)):
            step(i)
    torch.cuda.synchronize()
    elapsed, step_us, host_s = timed_steps(torch, stream, step, args.steps)
    stages = [("compress", lambda i: G.prefill_compress(p, stream)),
              ("attention_path", lambda i: G.prefill_attention_path(p, stream))]
    avg = stage_times(torch, stream, stages, args.steps)
    ms = elapsed / args.steps * 1e3
    res = dict(
        metric=METRIC, value=sp.T / (ms * 1e-3), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload=sp.name, seq_len=sp.T, hidden=sp.d, heads=sp.nh, head_dim=sp.c,
                    rope_dims=sp.d_r, m=sp.m, top_k=sp.k or None,
                    indexer=(f"{sp.nI}x{sp.cI} f32" if sp.nI else None), window=sp.n_win),
        roofline=None,
        step=dict(step_us=distribution(step_us), kernel_us={k: round(v, 1) for k, v in avg.items()},
                  note="time only: launch-latency bound at this size"),
        cpu_baseline=None,
    )
    return res


def kernel_traffic(config, kernel):
    """Measured HBM bytes per launch of the roofline kernel, or None (no
    counters for this kernel, or its source changed since they were taken)."""
    t = TRAFFIC.get(config)
    if t is None or t.get("kernel") != kernel:
        return None
    import hashlib
    src = os.path.join(ROOT, "long_context_sparse_10_amd", "csrc", t["src"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["sha256"]:
            return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def copy_probe(torch):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "dispatches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_64k",
                    choices=["decode_64k", "hca_decode_1m", "decode_1m_fp4", "prefill_32k",
                             "prefill_32k_mxfp4", "oproj_decode", "oproj_prefill", "tiny_csa",
                             "tiny_hca", "compress_32k"])
    ap.add_argument("--copies", type=int, default=6, help="cache copies rotated (cold cache)")
    ap.add_argument("--graph", action="store_true", help="decode: replay each step as a HIP graph")
    ap.add_argument("--chunks", type=int, default=1,
                    help="decode: batch groups whose chains run on two streams (1 = one chain)")
    ap.add_argument("--paged", action="store_true",
                    help="decode: caches in a hybrid page pool (block-table indirection)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the decode batch shards by sequence; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(torch)
        return
    import csa_inputs as I
    from long_context_sparse_10_amd import pipeline as G
    if args.config.startswith("tiny"):
        print(json.dumps(run_tiny(args, torch, I, G)), flush=True)
        return
    if args.config == "compress_32k":
        print(json.dumps(run_compress(args, torch, I, G)), flush=True)
        return
    if args.config in OPROJ:
        res, case = run_oproj(args, torch)
        res["roofline"]["traffic"] = kernel_traffic(args.config, res["roofline"]["kernel"])
        res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_oproj(case)
        print(json.dumps(res), flush=True)
        return
    if args.config.startswith("prefill"):
        args.copies = 1
        res, inp = run_prefill(args, torch, I, G)
    else:
        res, (inp, first) = run_decode(args, torch, I, G)
    res["roofline"]["traffic"] = kernel_traffic(args.config, res["roofline"]["kernel"])
    if not args.no_cpu_baseline:
        if args.config.startswith("prefill"):
            rows = np.linspace(0, inp["T"] - 1, 64).astype(int)
            res["cpu_baseline"] = cpu_baseline_prefill(inp, rows)
        else:
            res["cpu_baseline"] = cpu_baseline_decode(inp)
            if inp["spec"].index_format == "mxfp4":
                res["recall"] = fp4_recall(inp, first.idx.cpu().numpy())
    else:
        res["cpu_baseline"] = None
        if not args.config.startswith("prefill") and inp["spec"].index_format == "mxfp4":
            res["recall"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
