"""Device-side composition of the CSA calls for whole workloads.

Uploads the seeded synthetic inputs, builds the caches with the library's own
kernels (``csa_prep_rows`` / ``csa_compress``) and runs one step of the hot
path: ``indexer_score`` -> ``topk_select`` -> ``sparse_mqa_attend`` for CSA,
``hca_attend`` for HCA.  Every arithmetic step runs in libcsa; torch provides
device memory and streams only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import _lib as C

ROPE_THETA = 10000.0
EPS = 1e-6
FMT = {"f32": C.F32, "bf16": C.BF16, "fp8mix": C.FP8MIX, "mxfp4": C.MXFP4}


def _row_bytes(fmt, c, d_r):
    return {C.F32: 4 * c, C.BF16: 2 * c, C.FP8MIX: (c - d_r) + 2 * d_r, C.MXFP4: c // 2}[fmt]


def to_dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload an fp32 array holding values of ``dtype`` ("f32" / "bf16")."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def encode_rows(x: torch.Tensor, fmt: int, rows: int, c: int, *, norm_w=None, d_r=0,
                pos=None, rows_per_seq=1, pos_stride=1, pos_offset=0, stream=None):
    """Run ``csa_prep_rows`` on ``rows`` rows of ``x`` into a new buffer of
    format ``fmt``; returns (rows tensor, scales or None)."""
    out = torch.empty(rows * _row_bytes(fmt, c, d_r), dtype=torch.uint8, device=x.device)
    sc = torch.empty(rows * (c // 32), dtype=torch.uint8, device=x.device) if fmt == C.MXFP4 else None
    xt = C.BF16 if x.dtype == torch.bfloat16 else C.F32
    C.csa_prep_rows(x, xt, rows, c, norm_w, EPS, d_r, ROPE_THETA, pos, rows_per_seq, pos_stride,
                    pos_offset, out, sc, fmt, stream)
    return out, sc


# ============================================================ paged caches
@dataclass
class PagePool:
    """A hybrid page pool (Evidence Ledger Section 3.5.1; "G2C Brief -- DeepSeek
    V4", "Hybrid attention creates a hybrid cache"):
    one page per 128-token block of a sequence, each series of entries in its
    own section of the page.  ``sections[name] = (byte offset, entries_log2,
    row bytes)``; ``table[b, j]`` is the page of block j of sequence b."""
    pool: torch.Tensor
    table: torch.Tensor
    page_bytes: int
    sections: dict

    def base(self, name) -> int:
        """Device address of slot 0 of page 0 of a series."""
        return self.pool.data_ptr() + self.sections[name][0]

    def pages(self, name) -> "C.Pages":
        return C.Pages(self.table, self.sections[name][1], self.page_bytes)

    def _section(self, name):
        off, lg, rb = self.sections[name]
        return self.pool[:, off:off + (rb << lg)], 1 << lg, rb

    def scatter(self, name, rows):
        """Store dense rows (a [B, N, ...] tensor of N rows per sequence, any
        dtype, read as bytes) as entries 0..N-1 of each sequence's pages."""
        sec, E, rb = self._section(name)
        B, nb = self.table.shape
        r = rows.contiguous().view(torch.uint8).reshape(B, -1, rb)
        if r.shape[1] < nb * E:
            pad = torch.full((B, nb * E - r.shape[1], rb), 0xFF, dtype=torch.uint8,
                             device=r.device)
            r = torch.cat([r, pad], 1)
        sec[self.table.reshape(-1).long()] = r.reshape(B * nb, E * rb)

    def gather(self, name, N):
        """Entries 0..N-1 of every sequence as dense rows [B, N, row bytes]."""
        sec, E, rb = self._section(name)
        B, nb = self.table.shape
        return sec[self.table.reshape(-1).long()].reshape(B, nb * E, rb)[:, :N]

    def clone(self) -> "PagePool":
        return PagePool(self.pool.clone(), self.table, self.page_bytes, dict(self.sections))


def hybrid_pool(B, max_blocks, series, device, seed=0, spare=2) -> PagePool:
    """A pool of B * max_blocks pages (+ ``spare``), assigned to the blocks in a
    seeded random order.  ``series``: (name, entries_log2, row bytes) per
    section, each section 256-byte aligned.  Every byte starts as 0xFF, which
    no stored row holds (NaN in fp32 / bf16 / e4m3 and e8m0)."""
    off, sections = 0, {}
    for name, lg, rb in series:
        sections[name] = (off, lg, rb)
        off += ((rb << lg) + 255) // 256 * 256
    n_pages = B * max_blocks + spare
    pool = torch.full((n_pages, off), 0xFF, dtype=torch.uint8, device=device)
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * max_blocks]
    table = torch.from_numpy(perm.astype(np.int32).reshape(B, max_blocks)).to(device)
    return PagePool(pool, table, off, sections)


def _row_bytes_of(fmt, c, d_r):
    return {C.F32: 4 * c, C.BF16: 2 * c, C.FP8MIX: (c - d_r) + 2 * d_r, C.MXFP4: c // 2}[fmt]


# ============================================================ decode
@dataclass
class Decode:
    spec: object
    B: int
    Nmax: int
    q: torch.Tensor
    q_pos: torch.Tensor
    n_entries: torch.Tensor
    sink: torch.Tensor
    gamma: torch.Tensor
    kv: torch.Tensor
    win: torch.Tensor
    kv_fmt: int
    qI: Optional[torch.Tensor] = None
    qI_scale: Optional[torch.Tensor] = None
    kI: Optional[torch.Tensor] = None
    kI_scale: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None
    index_fmt: int = C.BF16
    score_fmt: int = C.F32
    scores: Optional[torch.Tensor] = None
    idx: Optional[torch.Tensor] = None
    out: Optional[torch.Tensor] = None
    ws: Optional[torch.Tensor] = None
    ws_topk: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)
    pool: Optional[PagePool] = None    # set: the caches live in pages (kv / kI / kI_scale unused)
    win_len: int = 0                   # slots of the window ring (n_win or more)


def upload_decode(inp: dict, device="cuda", stream=None) -> Decode:
    """Device buffers for one decode step: the compressed caches (RMSNorm +
    RoPE at position m*i, stored in the config's KV format), the window ring
    (RoPE at each slot's own position), index keys and the query side."""
    sp = inp["spec"]
    B, Nmax, c, d_r = sp.B, inp["Nmax"], sp.c, sp.d_r
    kv_fmt = FMT[sp.kv_format]
    gamma = torch.ones(c, dtype=torch.float32, device=device)
    raw = torch.from_numpy(inp["kv_raw"]).to(device)
    kv, _ = encode_rows(raw, kv_fmt, B * Nmax, c, norm_w=gamma, d_r=d_r, rows_per_seq=Nmax,
                        pos_stride=sp.m, stream=stream)
    del raw
    wraw = torch.from_numpy(inp["win_raw"]).to(device)
    wpos = torch.from_numpy(inp["win_pos"].reshape(-1)).to(device)
    win_len = int(inp["win_raw"].shape[1])
    win, _ = encode_rows(wraw, kv_fmt, B * win_len, c, norm_w=gamma, d_r=d_r, pos=wpos,
                         stream=stream)
    d = Decode(spec=sp, B=B, Nmax=Nmax, q=to_dev(inp["q"], sp.dtype, device),
               q_pos=torch.from_numpy(inp["q_pos"]).to(device),
               n_entries=torch.from_numpy(inp["n_entries"]).to(device),
               sink=torch.from_numpy(inp["sink"]).to(device), gamma=gamma, kv=kv, win=win,
               kv_fmt=kv_fmt, win_len=win_len)
    d.out = torch.empty(B, 1, sp.nh, c, dtype=torch.bfloat16, device=device)
    if sp.kind == "decode":
        d.index_fmt = FMT[sp.index_format]
        if d.index_fmt == C.MXFP4:
            kraw = torch.from_numpy(inp["kI"]).to(device)
            d.kI, d.kI_scale = encode_rows(kraw, C.MXFP4, B * Nmax, sp.cI, stream=stream)
            del kraw
            qraw = torch.from_numpy(inp["qI"]).to(device)
            d.qI, d.qI_scale = encode_rows(qraw, C.MXFP4, B * sp.nI, sp.cI, stream=stream)
            d.score_fmt = C.BF16
        else:
            d.kI = to_dev(inp["kI"], sp.index_format, device)
            d.qI = to_dev(inp["qI"], sp.index_format, device)
            d.score_fmt = C.F32
        d.w = torch.from_numpy(inp["w"]).to(device)
        sdt = torch.bfloat16 if d.score_fmt == C.BF16 else torch.float32
        d.scores = torch.empty(B, 1, Nmax, dtype=sdt, device=device)
        d.idx = torch.empty(B, 1, sp.k, dtype=torch.int32, device=device)
    return d


def page_decode(d: Decode, seed=0, drop_dense=False) -> PagePool:
    """Move a decode batch's caches into a hybrid pool: one page per 128-token
    block holding 32 CSA main rows, 32 index keys (+ their MXFP4 scales) and 1
    HCA row.  A CSA workload fills the CSA sections, an HCA workload the HCA
    section; the other sections belong to the other layer type and stay unused
    here."""
    sp = d.spec
    rb = _row_bytes_of(d.kv_fmt, sp.c, sp.d_r)
    rbi = _row_bytes_of(d.index_fmt, sp.cI or 128, 0)
    csa = sp.kind == "decode"
    series = [("csa_kv", 5, rb), ("kI", 5, rbi)]
    if csa and d.index_fmt == C.MXFP4:
        series.append(("kI_scale", 5, (sp.cI or 128) // 32))
    series.append(("hca_kv", 0, rb))
    per_block = 32 if csa else 1
    nb = (d.Nmax + per_block - 1) // per_block
    pool = hybrid_pool(d.B, nb, series, d.kv.device, seed)
    if csa:
        pool.scatter("csa_kv", d.kv)
        pool.scatter("kI", d.kI)
        if d.kI_scale is not None:
            pool.scatter("kI_scale", d.kI_scale)
    else:
        pool.scatter("hca_kv", d.kv)
    d.pool = pool
    if drop_dense:
        d.kv = d.kI = d.kI_scale = None
    return pool


def _kv_series(d: Decode):
    return "csa_kv" if d.spec.kind == "decode" else "hca_kv"


def decode_indexer(d: Decode, stream=None):
    sp = d.spec
    if d.pool is not None:
        kI, ks = d.pool.base("kI"), (d.pool.base("kI_scale") if d.index_fmt == C.MXFP4 else None)
        C.indexer_score(d.qI, d.qI_scale, d.index_fmt, d.w, kI, ks, d.index_fmt, d.q_pos,
                        d.n_entries, d.B, 1, sp.nI, sp.cI, d.Nmax, sp.m, d.scores, d.score_fmt,
                        stream, pages=d.pool.pages("kI"))
        return
    C.indexer_score(d.qI, d.qI_scale, d.index_fmt, d.w, d.kI, d.kI_scale, d.index_fmt, d.q_pos,
                    d.n_entries, d.B, 1, sp.nI, sp.cI, d.Nmax, sp.m, d.scores, d.score_fmt, stream)


def decode_topk(d: Decode, stream=None):
    sp = d.spec
    d.ws_topk = C.topk_select(d.scores, d.score_fmt, d.q_pos, d.n_entries, d.B, 1, d.Nmax, sp.m,
                              sp.k, d.idx, d.ws_topk, stream)


def decode_attend(d: Decode, idx=None, stream=None):
    sp = d.spec
    qt = C.BF16 if d.q.dtype == torch.bfloat16 else C.F32
    scale = 1.0 / math.sqrt(sp.c)
    kv, pages = d.kv, None
    if d.pool is not None:
        kv, pages = d.pool.base(_kv_series(d)), d.pool.pages(_kv_series(d))
    if sp.kind == "hca_decode":
        d.ws = C.hca_attend(d.q, qt, d.gamma, EPS, sp.d_r, ROPE_THETA, d.q_pos, kv, d.kv_fmt,
                            d.Nmax, d.n_entries, sp.m, d.win, d.win_len, sp.n_win, d.sink, scale,
                            d.B, 1, sp.nh, sp.c, d.out, C.BF16, d.ws, stream, pages=pages)
    else:
        d.ws = C.sparse_mqa_attend(d.q, qt, d.gamma, EPS, sp.d_r, ROPE_THETA, d.q_pos, kv,
                                   d.kv_fmt, d.Nmax, d.idx if idx is None else idx, sp.k, d.win,
                                   d.win_len, sp.n_win, d.sink, scale, d.B, 1, sp.nh, sp.c, d.out,
                                   C.BF16, d.ws, stream, pages=pages)


def decode_step(d: Decode, stream=None):
    """One decode step of the hot path for every sequence of the batch."""
    if d.spec.kind == "decode":
        decode_indexer(d, stream)
        decode_topk(d, stream)
    decode_attend(d, stream=stream)


def _batch_slice(t, b0, b1, B):
    """Sequences b0..b1-1 of a batch-major tensor (or of a flat per-sequence
    byte buffer) as a view."""
    if t is None:
        return None
    if t.shape[0] == B:
        return t[b0:b1]
    per = t.shape[0] // B
    return t[b0 * per:b1 * per]


def decode_chunks(d: Decode, chunks: int):
    """The batch cut into ``chunks`` contiguous groups of sequences, each a
    Decode of views with its own workspaces (made once, kept on ``d``)."""
    key = ("chunks", chunks)
    if key not in d.extra:
        bounds = np.linspace(0, d.B, min(chunks, d.B) + 1).astype(int)
        subs = []
        for b0, b1 in zip(bounds[:-1], bounds[1:]):
            kw = {k: getattr(d, k) for k in d.__dataclass_fields__}
            for name in ("q", "q_pos", "n_entries", "kv", "win", "qI", "qI_scale", "kI",
                         "kI_scale", "w", "scores", "idx", "out"):
                kw[name] = _batch_slice(kw[name], b0, b1, d.B)
            kw.update(B=int(b1 - b0), ws=None, ws_topk=None, extra={})
            if d.pool is not None:   # the group's rows of the block table
                kw["pool"] = PagePool(d.pool.pool, d.pool.table[b0:b1], d.pool.page_bytes,
                                      d.pool.sections)
            subs.append(Decode(**kw))
        d.extra[key] = subs
    return d.extra[key]


def decode_step_overlapped(d: Decode, streams, chunks: int = 2):
    """The decode step with the batch in ``chunks`` groups whose chains
    (indexer -> top-k -> attention) run on ``streams`` in rotation, so one
    group's latency-bound top-k overlaps another group's streaming kernels.
    ``streams[0]`` is the caller's stream: the others fork from it and join
    back into it.  Every call is per sequence (the attention split plan never
    depends on the batch), so the result equals ``decode_step`` bit for bit."""
    main = streams[0]
    subs = decode_chunks(d, chunks)
    fork = torch.cuda.Event()
    fork.record(main)
    for s in streams[1:]:
        s.wait_event(fork)
    for i, sub in enumerate(subs):
        decode_step(sub, streams[i % len(streams)])
    for s in streams[1:]:
        join = torch.cuda.Event()
        join.record(s)
        main.wait_event(join)


# ============================================================ prefill
@dataclass
class Prefill:
    spec: object
    T: int
    dt: int
    H: torch.Tensor
    W: dict
    q: torch.Tensor
    qI: Optional[torch.Tensor]
    w: Optional[torch.Tensor]
    q_pos: torch.Tensor
    n_entries: torch.Tensor
    sink: torch.Tensor
    gamma: torch.Tensor
    kv: Optional[torch.Tensor] = None
    kI: Optional[torch.Tensor] = None
    kI_scale: Optional[torch.Tensor] = None
    qI_scale: Optional[torch.Tensor] = None
    win: Optional[torch.Tensor] = None
    scores: Optional[torch.Tensor] = None
    idx: Optional[torch.Tensor] = None
    out: Optional[torch.Tensor] = None
    ws: Optional[torch.Tensor] = None
    ws_attend: Optional[torch.Tensor] = None


def upload_prefill(inp: dict, device="cuda") -> Prefill:
    sp = inp["spec"]
    T, dt = inp["T"], sp.dtype
    names = [k for k in inp if k.startswith("W") or k.startswith("bias")]
    W = {}
    for k in names:
        W[k] = to_dev(inp[k], dt, device) if k.startswith("W") else torch.from_numpy(inp[k]).to(device)
    p = Prefill(spec=sp, T=T, dt=FMT[dt], H=to_dev(inp["H"], dt, device), W=W,
                q=to_dev(inp["q"], dt, device),
                qI=to_dev(inp["qI"], dt, device) if sp.nI else None,
                w=torch.from_numpy(inp["w"]).to(device) if sp.nI else None,
                q_pos=torch.from_numpy(inp["q_pos"]).to(device),
                n_entries=torch.tensor([T // sp.m], dtype=torch.int32, device=device),
                sink=torch.from_numpy(inp["sink"]).to(device),
                gamma=torch.ones(sp.c, dtype=torch.float32, device=device))
    if sp.nI and sp.index_format == "mxfp4":
        # MXFP4 index queries, encoded by the library from the bf16 values
        p.qI, p.qI_scale = encode_rows(p.qI.float(), C.MXFP4, T * sp.nI, sp.cI)
    return p


def prefill_compress(p: Prefill, stream=None):
    """Compress the sequence: main KV entries (RMSNorm + RoPE at m*i), index keys
    (second compressor, no norm / RoPE) and per-token window rows (m = 1)."""
    sp, T = p.spec, p.T
    n = T // sp.m
    kv_fmt = FMT[sp.kv_format]
    dev = p.H.device
    p.kv = torch.empty(max(n, 1) * _row_bytes(kv_fmt, sp.c, sp.d_r), dtype=torch.uint8, device=dev)
    overlap = sp.m == 4
    W = p.W
    p.ws = C.csa_compress(p.H, p.dt, 1, T, sp.d, W["W_kv_a"], W["W_z_a"],
                          W.get("W_kv_b"), W.get("W_z_b"), W["bias_a"], W.get("bias_b"), sp.m,
                          int(overlap), sp.c, p.gamma, EPS, sp.d_r, ROPE_THETA, sp.m, 0, p.kv, None,
                          kv_fmt, p.ws, stream)
    if sp.nI:
        ifmt = FMT[sp.index_format]
        p.kI = torch.empty(max(n, 1) * _row_bytes(ifmt, sp.cI, 0), dtype=torch.uint8, device=dev)
        if ifmt == C.MXFP4:
            p.kI_scale = torch.empty(max(n, 1) * (sp.cI // 32), dtype=torch.uint8, device=dev)
        p.ws = C.csa_compress(p.H, p.dt, 1, T, sp.d, W["WI_kv_a"], W["WI_z_a"], W["WI_kv_b"],
                              W["WI_z_b"], W["biasI_a"], W["biasI_b"], sp.m, 1, sp.cI, None, EPS, 0,
                              ROPE_THETA, sp.m, 0, p.kI, p.kI_scale, ifmt, p.ws, stream)
    p.win = torch.empty(T * _row_bytes(kv_fmt, sp.c, sp.d_r), dtype=torch.uint8, device=dev)
    p.ws = C.csa_compress(p.H, p.dt, 1, T, sp.d, W["W_win"], None, None, None, None, None, 1, 0,
                          sp.c, p.gamma, EPS, sp.d_r, ROPE_THETA, 1, 0, p.win, None, kv_fmt, p.ws,
                          stream)


def prefill_indexer(p: Prefill, stream=None):
    """Causal indexer scores of every query row of the prefill."""
    sp = p.spec
    ifmt = FMT[sp.index_format]
    sfmt = C.BF16 if ifmt == C.MXFP4 else C.F32
    C.indexer_score(p.qI, p.qI_scale, ifmt, p.w, p.kI, p.kI_scale, ifmt, p.q_pos, p.n_entries, 1,
                    p.q_pos.numel(), sp.nI, sp.cI, max(p.T // sp.m, 1), sp.m, p.scores, sfmt,
                    stream)


def prefill_attention_path(p: Prefill, stream=None):
    """Indexer -> top-k -> sparse attention (CSA), or dense HCA attention."""
    sp, T = p.spec, p.T
    Tq = p.q_pos.numel()
    n = max(T // sp.m, 1)
    dev = p.H.device
    scale = 1.0 / math.sqrt(sp.c)
    if p.out is None:
        p.out = torch.empty(1, Tq, sp.nh, sp.c, dtype=p.q.dtype, device=dev)
    ot = C.BF16 if p.q.dtype == torch.bfloat16 else C.F32
    kv_fmt = FMT[sp.kv_format]
    if sp.nI:
        ifmt = FMT[sp.index_format]
        sfmt = C.BF16 if ifmt == C.MXFP4 else C.F32   # MXFP4 indexer: bf16 scores
        if p.scores is None:
            sdt = torch.bfloat16 if sfmt == C.BF16 else torch.float32
            p.scores = torch.empty(1, Tq, n, dtype=sdt, device=dev)
            p.idx = torch.empty(1, Tq, sp.k, dtype=torch.int32, device=dev)
        prefill_indexer(p, stream)
        C.topk_select(p.scores, sfmt, p.q_pos, p.n_entries, 1, Tq, n, sp.m, sp.k, p.idx, None,
                      stream)
        p.ws_attend = C.sparse_mqa_attend(p.q, ot, p.gamma, EPS, sp.d_r, ROPE_THETA, p.q_pos, p.kv,
                                          kv_fmt, n, p.idx, sp.k, p.win, T, sp.n_win, p.sink, scale,
                                          1, Tq, sp.nh, sp.c, p.out, ot, p.ws_attend, stream)
    else:
        p.ws_attend = C.hca_attend(p.q, ot, p.gamma, EPS, sp.d_r, ROPE_THETA, p.q_pos, p.kv, kv_fmt,
                                   n, p.n_entries, sp.m, p.win, T, sp.n_win, p.sink, scale, 1, Tq,
                                   sp.nh, sp.c, p.out, ot, p.ws_attend, stream)
