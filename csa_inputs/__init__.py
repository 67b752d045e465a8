"""Seeded synthetic inputs for the CSA / HCA path.

This module holds random draws, dtype casts and array layout only -- none of the
method's arithmetic.  Both the HIP path (through the tests and ``bench.py``) and
the fp64 oracle consume exactly the arrays it returns, so the two sides share
inputs and nothing else.

Distributions follow the five workloads (the pages measure on no dataset; these
synthetic inputs stand in):

* tiny_csa / tiny_hca -- one sequence of 1024 tokens, hidden 256 ~ N(0, 1),
  weights ~ N(0, 1/fan_in), positional biases ~ N(0, 0.1), sinks ~ N(0, 1), all
  fp32 (N(mean, variance) throughout).  8 heads of dim 64 (RoPE on the last 16),
  indexer 4 x 32, top-k 32, window 128.
* decode_64k -- 32 sequences x 65,536 tokens (16,384 entries), bf16 KV of 512
  (RoPE 64), 64 query heads, indexer 64 x 128 bf16, top-k 1024.
* prefill_32k -- one sequence of 32,768 tokens, hidden 4096 bf16, compressor
  weights ~ N(0, 1/4096), 64 heads x 512, indexer 64 x 128, top-k 1024.
  prefill_32k_mxfp4 is the same prefill with MXFP4 index keys and queries.
* hca_decode_1m -- 16 sequences x 1,048,576 tokens, m' = 128 (8,192 entries),
  bf16 KV, 64 heads.
* decode_1m_fp4 -- 8 sequences x 1,048,576 tokens (262,144 entries), 128
  heads, MXFP4 index keys and queries, FP8/BF16 KV, top-k 1024.

Query-side inputs of the large workloads (q, q^I, w) are drawn directly from
N(0, 1): their projections sit upstream of the path.  The tiny workloads derive
them from the hidden states instead, through a rank-64 query latent
c^Q = h W^DQ (Evidence Ledger Section 2.3.1: the indexer queries come from the
same compressed query latent as the attention queries): q = c^Q W^UQ,
q^I = c^Q W^IUQ and w = h W^w, with weights ~ N(0, 1/fan_in), products in fp64
rounded once to fp32.  Raw KV / window / index-key values are
drawn N(0, 1) in fp32; normalisation, RoPE and format encoding are done by
each side itself.  Arrays tagged bf16 are fp32 arrays holding bf16 values
(rounded with torch's RNE cast).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEEDS = {"tiny_csa": 1001, "tiny_hca": 1001, "decode_64k": 1002, "prefill_32k": 1003,
         "hca_decode_1m": 1004, "decode_1m_fp4": 1005}


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    kind: str                 # "prefill", "decode", "hca_decode"
    m: int
    c: int
    d_r: int
    nh: int
    n_win: int = 128
    # prefill
    T: int = 0
    d: int = 0
    # decode
    B: int = 1
    L: int = 0
    # indexer / top-k
    nI: int = 0
    cI: int = 0
    k: int = 0
    dtype: str = "bf16"       # activations / weights / q
    latent_rank: int = 0      # > 0: q, q^I, w derived from h through a query latent of this rank
    kv_format: str = "bf16"   # "f32", "bf16", "fp8mix"
    index_format: str = "bf16"  # "f32", "bf16", "mxfp4"
    seed: int = 0

    @property
    def N(self):
        return self.L // self.m if self.kind != "prefill" else self.T // self.m

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny_csa": Spec("tiny_csa", "prefill", m=4, c=64, d_r=16, nh=8, T=1024, d=256, nI=4, cI=32,
                     k=32, dtype="f32", kv_format="f32", index_format="f32", seed=1001,
                     latent_rank=64),
    "tiny_hca": Spec("tiny_hca", "prefill", m=128, c=64, d_r=16, nh=8, T=1024, d=256,
                     dtype="f32", kv_format="f32", seed=1001, latent_rank=64),
    "decode_64k": Spec("decode_64k", "decode", m=4, c=512, d_r=64, nh=64, B=32, L=65536, nI=64,
                       cI=128, k=1024, seed=1002),
    "prefill_32k": Spec("prefill_32k", "prefill", m=4, c=512, d_r=64, nh=64, T=32768, d=4096,
                        nI=64, cI=128, k=1024, seed=1003),
    # the prefill with MXFP4 index keys and queries (bf16 scores): the same
    # seeded inputs, only the indexer's storage format differs
    "prefill_32k_mxfp4": Spec("prefill_32k_mxfp4", "prefill", m=4, c=512, d_r=64, nh=64, T=32768,
                              d=4096, nI=64, cI=128, k=1024, index_format="mxfp4", seed=1003),
    "hca_decode_1m": Spec("hca_decode_1m", "hca_decode", m=128, c=512, d_r=64, nh=64, B=16,
                          L=1 << 20, seed=1004),
    "decode_1m_fp4": Spec("decode_1m_fp4", "decode", m=4, c=512, d_r=64, nh=128, B=8,
                          L=1 << 20, nI=64, cI=128, k=1024, kv_format="fp8mix",
                          index_format="mxfp4", seed=1005),
}


# ---------------------------------------------------------------- draws
def _normal(rng, shape, var=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array holding values of ``dtype`` ("f32" or "bf16"; RNE via torch)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def decode_inputs(spec: Spec, seed: Optional[int] = None, lengths=None, win_len=None):
    """One decode step for ``spec.B`` sequences.

    ``lengths`` (per-sequence context lengths) defaults to ``spec.L`` for all.
    Returns a dict of numpy arrays; the query of sequence b sits at position
    lengths[b] - 1 and the cache holds n_entries[b] = lengths[b] // m entries.
    The window ring has ``win_len`` slots (default n_win): slot s holds the
    newest position p <= L-1 with p % win_len == s (-1 while empty).
    """
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    B, c, m = spec.B, spec.c, spec.m
    lengths = np.full(B, spec.L, dtype=np.int64) if lengths is None else np.asarray(lengths, np.int64)
    n_entries = (lengths // m).astype(np.int32)
    Nmax = int(max(1, n_entries.max()))
    out = dict(spec=spec, lengths=lengths, n_entries=n_entries, Nmax=Nmax,
               q_pos=(lengths - 1).astype(np.int32).reshape(B, 1))
    out["kv_raw"] = _normal(rng, (B, Nmax, c))
    # window ring: slot s holds the newest position p <= L-1 with p % win_len == s
    nw = spec.n_win if win_len is None else int(win_len)
    win_raw = _normal(rng, (B, nw, c))
    win_pos = np.full((B, nw), -1, dtype=np.int32)
    for b in range(B):
        for p in range(max(0, int(lengths[b]) - nw), int(lengths[b])):
            win_pos[b, p % nw] = p
    out["win_raw"], out["win_pos"] = win_raw, win_pos
    out["q"] = cast(_normal(rng, (B, 1, spec.nh, c)), spec.dtype)
    out["sink"] = _normal(rng, (spec.nh,))
    if spec.kind == "decode":
        if spec.index_format == "mxfp4":
            out["kI"] = _normal(rng, (B, Nmax, spec.cI))
            out["qI"] = _normal(rng, (B, 1, spec.nI, spec.cI))
        else:
            out["kI"] = cast(_normal(rng, (B, Nmax, spec.cI)), spec.index_format)
            out["qI"] = cast(_normal(rng, (B, 1, spec.nI, spec.cI)), spec.index_format)
        out["w"] = _normal(rng, (B, 1, spec.nI))
    return out


def prefill_inputs(spec: Spec, seed: Optional[int] = None, T: Optional[int] = None,
                   queries: Optional[np.ndarray] = None):
    """One prefill of a single sequence: hidden states, compressor weights and
    query-side inputs.  ``T`` overrides the length.  ``queries`` (sorted
    positions) restricts the query-side arrays to those rows; the weights and
    hidden states are the same draws whatever ``queries`` is."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    T = spec.T if T is None else T
    d, c, m, dt = spec.d, spec.c, spec.m, spec.dtype
    out = dict(spec=spec, T=T)
    out["H"] = cast(_normal(rng, (T, d)), dt)
    overlap = spec.kind == "prefill" and m == 4
    names = ["W_kv_a", "W_z_a"] + (["W_kv_b", "W_z_b"] if overlap else [])
    for nm in names:
        out[nm] = cast(_normal(rng, (d, c), 1.0 / d), dt)
    out["bias_a"] = _normal(rng, (m, c), 0.1)
    if overlap:
        out["bias_b"] = _normal(rng, (m, c), 0.1)
    out["W_win"] = cast(_normal(rng, (d, c), 1.0 / d), dt)
    if spec.nI:
        for nm in ("WI_kv_a", "WI_z_a", "WI_kv_b", "WI_z_b"):
            out[nm] = cast(_normal(rng, (d, spec.cI), 1.0 / d), dt)
        out["biasI_a"] = _normal(rng, (m, spec.cI), 0.1)
        out["biasI_b"] = _normal(rng, (m, spec.cI), 0.1)
    out["sink"] = _normal(rng, (spec.nh,))
    rows = np.arange(T) if queries is None else np.asarray(queries)
    out["q_pos"] = rows.astype(np.int32)
    if spec.latent_rank:
        out["q"], out["qI"], out["w"] = _latent_query_rows(rng, out, spec, rows)
        return out
    # query side, drawn row by row in blocks so a subset is cheap and identical
    out["q"], out["qI"], out["w"] = _query_rows(spec.seed if seed is None else seed, spec, T, rows)
    return out


def _latent_query_rows(rng, out, spec: Spec, rows: np.ndarray):
    """Query-side inputs from the hidden states through a rank-r query latent
    (the weights are drawn after every other array, which they leave unchanged):
    c^Q = h W^DQ, q = c^Q W^UQ, q^I = c^Q W^IUQ, w = h W^w; fp64, then fp32."""
    d, r = spec.d, spec.latent_rank
    out["W_DQ"] = _normal(rng, (d, r), 1.0 / d)
    out["W_UQ"] = _normal(rng, (r, spec.nh * spec.c), 1.0 / r)
    if spec.nI:
        out["W_IUQ"] = _normal(rng, (r, spec.nI * spec.cI), 1.0 / r)
        out["W_w"] = _normal(rng, (d, spec.nI), 1.0 / d)
    h = np.asarray(out["H"], np.float64)[rows]
    cq = h @ np.asarray(out["W_DQ"], np.float64)
    q = (cq @ np.asarray(out["W_UQ"], np.float64)).reshape(len(rows), spec.nh, spec.c)
    qI = w = None
    if spec.nI:
        qI = (cq @ np.asarray(out["W_IUQ"], np.float64)).reshape(len(rows), spec.nI, spec.cI)
        w = h @ np.asarray(out["W_w"], np.float64)
        qI, w = cast(qI, spec.dtype), cast(w, "f32")
    return cast(q, spec.dtype), qI, w


_QBLOCK = 256


def _query_rows(seed: int, spec: Spec, T: int, rows: np.ndarray):
    """Query-side draws in blocks of 256 positions, each block from its own
    seeded stream, so any subset of rows reproduces the full draw."""
    q = np.empty((len(rows), spec.nh, spec.c), np.float32)
    qI = np.empty((len(rows), spec.nI, spec.cI), np.float32) if spec.nI else None
    w = np.empty((len(rows), spec.nI), np.float32) if spec.nI else None
    blocks = sorted(set(int(r) // _QBLOCK for r in rows))
    for blk in blocks:
        brng = np.random.default_rng([seed, 7, blk])
        n = min(_QBLOCK, T - blk * _QBLOCK)
        bq = cast(_normal(brng, (n, spec.nh, spec.c)), spec.dtype)
        if spec.nI:
            bqi = cast(_normal(brng, (n, spec.nI, spec.cI)), spec.dtype)
            bw = _normal(brng, (n, spec.nI))
        sel = np.nonzero((rows // _QBLOCK) == blk)[0]
        loc = rows[sel] - blk * _QBLOCK
        q[sel] = bq[loc]
        if spec.nI:
            qI[sel] = bqi[loc]
            w[sel] = bw[loc]
    return q, qI, w


def random_index_sets(rng, n_vis: np.ndarray, k: int, holes: float = 0.0):
    """Random valid top-k outputs for attention-stage tests: for each row a
    sorted set of min(k, n_vis) distinct entries below n_vis, padded with -1;
    ``holes`` drops that fraction of the chosen entries (left as -1 slots)."""
    n_vis = np.asarray(n_vis).reshape(-1)
    out = np.full((n_vis.size, k), -1, dtype=np.int32)
    for r, n in enumerate(n_vis):
        n = int(n)
        pick = np.sort(rng.choice(n, size=min(k, n), replace=False)) if n else np.zeros(0, int)
        if holes and pick.size:
            pick = pick[rng.random(pick.size) >= holes]
        out[r, : pick.size] = pick
    return out
