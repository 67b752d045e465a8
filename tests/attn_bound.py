"""Per-element error bound of the matrix-core attention kernels (test helper).

The kernels compute one query row of shared-KV attention (Evidence Ledger Eqs
18-19, 27) as follows:
  * the prepared query (RMSNorm, RoPE at q) is scaled by tau * log2(e) in fp32
    and rounded to bf16: the matrix-core operand;
  * logits (log2 units) are fp32 sums of K = c exact bf16 products;
  * weights p' = 2^(logit - m) are fp32; their bf16 roundings feed the P.V
    product, the fp32 denominator sums the unrounded weights and the sink;
  * split slot lists store each split's O / l in bf16 and merge in fp32;
  * the output is rotated back by -q on its RoPE channels and stored in bf16.

``attend_ref_bound`` returns the fp64 reference built on the kernel's own bf16
query operand (the oracle's prepared query, scaled and rounded) and a bound on
|kernel - reference| per (head, channel), from first-order error propagation:

  Delta_y   = logit error of row y (nats): a one-ulp bf16 query flip on every
              element whose rounding the fp32 preparation could change, plus
              the fp32 accumulation c 2^-24 sum_j |q_j x_yj|;
  e_o       = sum_y p_y |x_y| Delta_y + |o| sum_y p_y Delta_y       (softmax)
            + (2^-8 + n 2^-24) sum_y p_y |x_y|                     (bf16 P, fp32 sums)
            + 2^-8 sum_s w_s |O_s / l_s|                           (bf16 split partials)
  bound     = 1.1 e_o, pairs of RoPE channels mixed as the rotation mixes them,
            + 2^-8 |out| (bf16 store) + 1e-6.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import csa as O
from oracle import formats as F

LOG2E = 1.0 / math.log(2.0)
U_BF16 = 2.0 ** -8            # unit roundoff of bf16 (8 significant bits)
U_F32 = 2.0 ** -24
RHO_QPREP = 2.0 ** -16        # relative error of the fp32 query preparation (c = 512 sum of squares)


def bf16_spacing(x):
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def attend_ref_bound(q_raw, X, sink, tau, d_r, pos, split_id=None, eps=1e-6, theta=1e4,
                     out_bf16=True):
    """Reference output [nh, c] of one query row over rows X [n, c] (in the
    kernel's slot order) and the per-element bound.  ``split_id`` [n] gives the
    slot split of each row (None: the list is not split)."""
    X = np.asarray(X, np.float64)
    sink = np.asarray(sink, np.float64)
    n, c = X.shape
    qp = O.prepare_query(q_raw, None, eps, d_r, theta, pos)
    s = tau * LOG2E
    qs = qp * s
    qb = F.bf16_round(qs)
    ulp = bf16_spacing(qs)
    ambiguous = np.abs(np.abs(qs - qb) - 0.5 * ulp) <= RHO_QPREP * np.abs(qs)
    dq = np.where(ambiguous, ulp, 0.0)
    if n == 0:
        out = np.zeros_like(qp)
        return out, np.full_like(out, 1e-6)
    aX = np.abs(X)
    lg = (qb @ X.T) / LOG2E                                # natural-unit logits [nh, n]
    M = np.maximum(sink, lg.max(axis=1))
    e = np.exp(lg - M[:, None])
    D = np.exp(sink - M) + e.sum(axis=1)
    p = e / D[:, None]
    o = p @ X
    delta = ((dq @ aX.T) + c * U_F32 * (np.abs(qb) @ aX.T)) / LOG2E + 1e-6
    pd = p * delta
    A = p @ aX
    gam = n * U_F32
    e_o = pd @ aX + np.abs(o) * pd.sum(axis=1, keepdims=True) + (U_BF16 + gam) * A + gam * np.abs(o)
    if split_id is not None:
        split_id = np.asarray(split_id)
        part = np.zeros_like(o)
        for sid in np.unique(split_id):
            rows = split_id == sid
            w = p[:, rows].sum(axis=1)
            Os = (p[:, rows] @ X[rows]) / np.maximum(w, 1e-300)[:, None]
            part += w[:, None] * np.abs(Os)
        e_o = e_o + U_BF16 * part
    e_o = 1.1 * e_o
    if d_r:
        # the rotation by -q mixes channel pairs (c-d_r+2u, c-d_r+2u+1): each
        # rotated channel's error is |cos| e_a + |sin| e_b at the pair's angle
        ang = -pos * O.rope_frequencies(d_r, theta)
        cs, sn = np.abs(np.cos(ang)), np.abs(np.sin(ang))
        a, b = e_o[:, c - d_r::2].copy(), e_o[:, c - d_r + 1::2].copy()
        e_o[:, c - d_r::2] = cs * a + sn * b
        e_o[:, c - d_r + 1::2] = sn * a + cs * b
    out = O.rope(o, -pos, d_r, theta)
    bound = e_o + (U_BF16 * np.abs(out) if out_bf16 else 0.0) + 1e-6
    return out, bound


# ---------------------------------------------------------------- the kernels' split plan
def split_plan(kslots, n_win, Tq=1, tile=32, table=2048):
    """(chunk, nsplit) of the matrix-core attention kernels for a slot list of
    kslots compressed slots plus n_win window slots: a function of the per-row
    slot count only."""
    total = kslots + n_win
    if (Tq > 1 or total <= 256) and total <= table:
        return -(-total // tile) * tile, 1
    want = 8 if total <= 4096 else 16
    ch = -(-(-(-total // want)) // tile) * tile
    ch = max(4 * tile, min(ch, table))
    return ch, -(-total // ch)


def slot_splits(sel_slots, kslots, n_win, pos, Tq=1):
    """Split id of every row the kernel reads, in slot order: the compressed
    rows at slots ``sel_slots`` (CSA: the v with idx[v] >= 0, kslots = k; HCA:
    0..N(q)-1, kslots = Nmax), then the window positions max(0, pos-n_win+1)..pos
    at slots kslots + j.  None when the list is not split."""
    ch, ns = split_plan(kslots, n_win, Tq)
    if ns == 1:
        return None
    ids = [v // ch for v in sel_slots]
    for j in range(n_win):
        if pos - n_win + 1 + j >= 0:
            ids.append((kslots + j) // ch)
    return np.asarray(ids)
