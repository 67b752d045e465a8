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
(prefill).  ``roofline`` rates the dominant kernel against its bound, from HIP
events on the launch stream; ``cpu_baseline`` times the fp64 oracle on a
bounded sample of the same workload on this host.
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
    'decode_64k': {"src": "indexer.hip", "sha256": "11edc41b8d401743b8505978f26a4f4bd07674f12674e731507cd4bd8cfe797c", "fetch_kib": 67722.4, "write_kib": 2048.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'hca_decode_1m': {"src": "attend.hip", "sha256": "ae43da131e40bab8930d9ee5ceba58df2972325b9233c721d116c4efef778fcf", "fetch_kib": 75822.0, "write_kib": 17536.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'decode_1m_fp4': {"src": "indexer.hip", "sha256": "11edc41b8d401743b8505978f26a4f4bd07674f12674e731507cd4bd8cfe797c", "fetch_kib": 69941.2, "write_kib": 4096.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    'prefill_32k': {"src": "attend.hip", "sha256": "ae43da131e40bab8930d9ee5ceba58df2972325b9233c721d116c4efef778fcf", "fetch_kib": 3574817.2, "write_kib": 2097152.9, "fetch_scale": 1.9998, "write_scale": 1.0},
    'prefill_32k_mxfp4': {"src": "attend.hip", "sha256": "ae43da131e40bab8930d9ee5ceba58df2972325b9233c721d116c4efef778fcf", "fetch_kib": 3405804.8, "write_kib": 2097155.9, "fetch_scale": 1.9998, "write_scale": 1.0},
    'oproj_decode': {"src": "oproj.hip", "sha256": "99d8386e33f20e6b4550c52e1cad5985505842be7148f54ce0c4b5e890c9f760", "fetch_kib": 80948.4, "write_kib": 8967.4, "fetch_scale": 1.9998, "write_scale": 1.0},
    'oproj_prefill': {"src": "oproj.hip", "sha256": "99d8386e33f20e6b4550c52e1cad5985505842be7148f54ce0c4b5e890c9f760", "fetch_kib": 4553178.6, "write_kib": 842469.5, "fetch_scale": 1.9998, "write_scale": 1.0},
}


# ------------------------------------------------------------------ algorithmic bytes
def decode_bytes(sp, N):
    """Bytes the method must move per query token (one sequence)."""
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
    else:
        kI = N * sp.cI * 2
        qI = sp.nI * sp.cI * 2
    indexer = kI + qI + sp.nI * 4
    attend = min(sp.k, N) * row + win + q + out
    return dict(indexer=indexer, attend=attend, total=indexer + attend)


def prefill_flops(sp, T):
    """Algorithmic flops of indexer + attention over a causal prefill."""
    fi = fa = 0
    for q in range(T):
        nv = (q + 1) // sp.m
        fi += nv * sp.nI * sp.cI * 2
        fa += (min(sp.k, nv) + min(q + 1, sp.n_win)) * sp.nh * sp.c * 4
    return fi, fa


# ------------------------------------------------------------------ CPU baseline
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
                       f"{dt:.1f} s")


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
                       f"fp64 numpy, {dt:.1f} s; compression done beforehand in {t1 - t0:.1f} s)")


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
    # per-kernel launch time: each call back to back over the rotated copies
    # (the queue stays full, so an event pair brackets kernel time only)
    avg = {}
    for kind in kinds:
        reps = max(args.steps, 12)
        with torch.cuda.stream(stream):
            for i in range(len(copies)):
                call[kind](copies[i], stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                call[kind](copies[i % len(copies)], stream)
            e1.record(stream)
        torch.cuda.synchronize()
        avg[kind] = e0.elapsed_time(e1) * 1e3 / reps
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            run_step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    gpu_ms = e0.elapsed_time(e1)
    ms_step = elapsed / args.steps * 1e3
    N = inp["Nmax"]
    by = decode_bytes(sp, N)
    dom = "indexer" if sp.kind == "decode" else "attend"
    dom_bytes = by[dom] * sp.B
    achieved = dom_bytes / (avg[dom] * 1e-6) / 1e9
    value = sp.B * args.steps / elapsed
    step_gbs = by["total"] * sp.B / (ms_step * 1e-3) / 1e9
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
        roofline=dict(bound="hbm", kernel=dom, achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=None,
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=avg[dom]),
        step=dict(algorithmic_bytes=by["total"] * sp.B, achieved_gbs=step_gbs,
                  frac_of_hbm_peak=step_gbs / HBM_PEAK_GBS, gpu_ms_per_step=gpu_ms / args.steps,
                  launch=("HIP graph per cache copy" if args.graph else "eager launches")
                  + (f"; batch in {args.chunks} groups on 2 streams" if args.chunks > 1 else ""),
                  kernel_us={k: round(v, 2) for k, v in avg.items()}),
    )
    return res, inp


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
                sample=f"{n} rows ({rows} per call) of the same shape, fp64 numpy, {dt:.1f} s")


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
    kinds = ["indexer", "topk", "attend"]
    n = sp.T // sp.m
    for _ in range(args.warmup):
        with torch.cuda.stream(stream):
            G.prefill_attention_path(p, stream)
    torch.cuda.synchronize()
    import long_context_sparse_10_amd as L
    sfmt = L.BF16 if sp.index_format == "mxfp4" else L.F32
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    scale = 1.0 / math.sqrt(sp.c)
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            e = ev[i]
            e[0].record(stream)
            G.prefill_indexer(p, stream)
            e[1].record(stream)
            L.topk_select(p.scores, sfmt, p.q_pos, p.n_entries, 1, sp.T, n, sp.m, sp.k, p.idx,
                          None, stream)
            e[2].record(stream)
            L.sparse_mqa_attend(p.q, L.BF16, p.gamma, 1e-6, sp.d_r, 1e4, p.q_pos, p.kv, L.BF16, n,
                                p.idx, sp.k, p.win, sp.T, sp.n_win, p.sink, scale, 1, sp.T, sp.nh,
                                sp.c, p.out, L.BF16, p.ws_attend, stream)
            e[3].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    avg = {k: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) * 1e3
           for j, k in enumerate(kinds)}
    fi, fa = prefill_flops(sp, sp.T)
    ms = elapsed / args.steps * 1e3
    tflops = (fi + fa) / (ms * 1e-3) / 1e12
    att = fa / (avg["attend"] * 1e-6) / 1e12
    res = dict(
        metric=METRIC, value=tflops, unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16" if sp.index_format == "bf16" else "bf16+mxfp4 indexer",
        data="synthetic",
        config=dict(workload=sp.name, seq_len=sp.T, hidden=sp.d, heads=sp.nh, head_dim=sp.c,
                    top_k=sp.k, indexer=f"{sp.nI}x{sp.cI} {sp.index_format}", window=sp.n_win),
        roofline=dict(bound="mfma", kernel="attend", achieved=att, peak=BF16_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=att / BF16_PEAK_TFLOPS, traffic=None,
                      algorithmic_flops_per_launch=fa, avg_launch_us=avg["attend"]),
        step=dict(indexer_tflops=fi / (avg["indexer"] * 1e-6) / 1e12,
                  attend_tflops=att, kernel_us={k: round(v, 1) for k, v in avg.items()},
                  compress_ms_untimed=t_comp),
    )
    return res, inp


def kernel_traffic(config):
    """Measured HBM bytes per launch of the roofline kernel, or None."""
    t = TRAFFIC.get(config)
    if t is None:
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
                             "prefill_32k_mxfp4", "oproj_decode", "oproj_prefill"])
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
    if args.config in OPROJ:
        res, case = run_oproj(args, torch)
        res["roofline"]["traffic"] = kernel_traffic(args.config)
        res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_oproj(case)
        print(json.dumps(res), flush=True)
        return
    if args.config.startswith("prefill"):
        args.copies = 1
        res, inp = run_prefill(args, torch, I, G)
    else:
        res, inp = run_decode(args, torch, I, G)
    res["roofline"]["traffic"] = kernel_traffic(args.config)
    if not args.no_cpu_baseline:
        if args.config.startswith("prefill"):
            rows = np.linspace(0, inp["T"] - 1, 64).astype(int)
            res["cpu_baseline"] = cpu_baseline_prefill(inp, rows)
        else:
            res["cpu_baseline"] = cpu_baseline_decode(inp)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
