"""Plain fp64 CPU oracle of the Compressed Sparse Attention (CSA) hot path.

TEST INFRASTRUCTURE ONLY. This is the slow, obviously-correct reference the HIP
kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; the product path never does,
and it shares no code with the HIP library.

Every function follows a passage of the pages (cited by page title and section /
equation):

* "Evidence Ledger" (mailtotanvir, mastering-deepseek-v4-architecture) -- the
  CSA bullets (Section 2.3.1, Eqs 9-19), HCA (Section 2.3.2, Eqs 20-26), the
  shared attention details (Section 2.3.3, Eq 27) and mixed storage (2.3.4).
* "DeepSeek V4 study" (shuhuayu, studies/deepseek-v4) -- section 03 "Two
  resolutions of history": the score formula, the HCA pooling formula, the
  per-channel softmax over eight candidates, the configuration table.
* "DeepSeek-V4: What Remains After Compressing History?" (tianyi-zhang-02) --
  section 2 (the attention ledger) and section 3 (causal block boundaries).

Readings taken where the pages are silent (each is a parameter where cheap):

* N(q), the compressed entries visible to zero-based position q, is
  (q + 1) // m: entry i is complete once its last token m*i + m - 1 <= q.
* Entry 0 has no preceding block: its b-series candidates are absent.
* Positional biases are per (in-block position, channel): B_a, B_b in R^{m x c}.
* RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma, eps = 1e-6.
* RoPE rotates interleaved adjacent pairs (c - d_r + 2u, c - d_r + 2u + 1) of
  the last d_r channels by angle pos * theta^(-2u / d_r), theta = 10000.
  A compressed entry i sits at position pos_stride * i + pos_offset
  (default m * i, the first token of its block).
* Index keys come from a second compressor of the same form (output c_I) with
  no RMSNorm or RoPE; the indexer has no scale factor.
* Window rows are per-token projections with the same RMSNorm and RoPE at the
  token's own position; the window of query q is positions
  max(0, q - n_win + 1) .. q (the current token included).
* Top-k keeps the min(k, N(q)) largest scores, ties to the lower entry index,
  returned in ascending entry order and padded with -1.
* The attention logit is tau * (q . x) with tau = 1/sqrt(c); the sink enters
  the denominator as exp(z'_h) with no scaling; x serves as both K and V,
  including its RoPE channels, and the output is rotated back by -q.
* Grouped output projection: group j takes the consecutive heads
  j*nh/g .. (j+1)*nh/g - 1, their rotated-back outputs concatenated head by
  head; each group is projected to d_g by its own matrix and the g results,
  concatenated in group order, are projected to d.  No nonlinearity sits
  between the two products.  Weights follow the linear-layer convention
  [out, in].  The activation u between them may be rounded (bf16 in the
  kernels), passed in as ``round_u``.
"""
from __future__ import annotations

import numpy as np

ROPE_THETA = 10000.0
RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# visibility (strict block causality)
# --------------------------------------------------------------------------


def n_visible(q_pos, m: int, n_entries: int | None = None):
    """Compressed entries available to zero-based query position ``q_pos``.

    Evidence Ledger, CSA: a query attends only to blocks s < floor(t/m) with t
    the 1-based count of processed tokens; the tianyi-zhang-02 page (section 3)
    counts completed entries from the zero-based position plus one, divided by
    the block width.  Both give (q + 1) // m.
    ``n_entries`` caps it by what the cache holds.
    """
    n = (np.asarray(q_pos, dtype=np.int64) + 1) // m
    if n_entries is not None:
        n = np.minimum(n, n_entries)
    return n


# --------------------------------------------------------------------------
# RMSNorm and partial RoPE (Evidence Ledger, Section 2.3.3)
# --------------------------------------------------------------------------


def rms_norm(x, gamma=None, eps: float = RMS_EPS):
    """Per-row RMSNorm over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope_frequencies(d_r: int, theta: float = ROPE_THETA):
    u = np.arange(d_r // 2, dtype=np.float64)
    return theta ** (-2.0 * u / d_r)


def rope(x, pos, d_r: int, theta: float = ROPE_THETA):
    """Rotate the last ``d_r`` channels of ``x`` (adjacent pairs) by ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``; a negative position gives the
    inverse rotation used on the attention output.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    if d_r == 0:
        return y
    c = y.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_frequencies(d_r, theta)
    cs, sn = np.cos(ang), np.sin(ang)
    a = y[..., c - d_r::2].copy()
    b = y[..., c - d_r + 1::2].copy()
    y[..., c - d_r::2] = a * cs - b * sn
    y[..., c - d_r + 1::2] = a * sn + b * cs
    return y


# --------------------------------------------------------------------------
# compression (Evidence Ledger Eqs 9-12 and 20-26; shuhuayu section 03)
# --------------------------------------------------------------------------


def project(H, W):
    """Eqs 9-10: one projection series, H [T, d] @ W [d, c] in fp64."""
    return np.asarray(H, dtype=np.float64) @ np.asarray(W, dtype=np.float64)


def pool(C_a, Z_a, B_a, m: int, C_b=None, Z_b=None, B_b=None):
    """Per-channel softmax pooling of candidates into compressed entries.

    Entry i gathers its own block (positions m*i .. m*i+m-1) through the a-series
    and, when the b-series is given (CSA overlap), the preceding block
    (m*(i-1) .. m*i-1) through the b-series.  Each candidate r has logit
    Z[pos_r, j] + B[u_r, j] for in-block offset u_r; the weights are a softmax
    over the candidates, separately for each channel j, and the entry is the
    weighted sum of the candidates' C values (Eqs 11-12; HCA: c = sum_t
    softmax_t(z_t + b_t) * v_t over one block of m' tokens, no overlap).
    Entry 0 has no preceding block, so it pools its own m candidates only.
    """
    C_a = np.asarray(C_a, dtype=np.float64)
    Z_a = np.asarray(Z_a, dtype=np.float64)
    B_a = np.asarray(B_a, dtype=np.float64)
    T, c = C_a.shape
    n = T // m
    overlap = C_b is not None
    if overlap:
        C_b = np.asarray(C_b, dtype=np.float64)
        Z_b = np.asarray(Z_b, dtype=np.float64)
        B_b = np.asarray(B_b, dtype=np.float64)
    out = np.empty((n, c))
    for i in range(n):
        own = slice(m * i, m * i + m)
        logits = [Z_a[own] + B_a]                      # [m, c]
        values = [C_a[own]]
        if overlap and i > 0:
            prev = slice(m * (i - 1), m * i)
            logits.append(Z_b[prev] + B_b)
            values.append(C_b[prev])
        L = np.concatenate(logits, axis=0)             # [candidates, c]
        V = np.concatenate(values, axis=0)
        L = L - L.max(axis=0, keepdims=True)
        w = np.exp(L)
        w = w / w.sum(axis=0, keepdims=True)
        out[i] = (w * V).sum(axis=0)
    return out


def finish_entries(E, gamma, eps, d_r, theta, pos_stride, pos_offset, normalize=True):
    """Section 2.3.3: RMSNorm each compressed entry, then partial RoPE at the
    entry's position pos_stride * i + pos_offset."""
    E = np.asarray(E, dtype=np.float64)
    if normalize:
        E = rms_norm(E, gamma, eps)
    if d_r:
        pos = pos_stride * np.arange(E.shape[0]) + pos_offset
        E = rope(E, pos, d_r, theta)
    return E


def compress(H, W_kv_a, W_z_a, B_a, m, W_kv_b=None, W_z_b=None, B_b=None,
             gamma=None, eps=RMS_EPS, d_r=0, theta=ROPE_THETA,
             pos_stride=None, pos_offset=0, normalize=True):
    """Full compressor for one sequence: projections, pooling, norm, RoPE.

    ``W_z_a`` may be None only for m == 1 without overlap (the per-token window
    projection R_p = h_p W^KV, where pooling one candidate is the identity).
    """
    if pos_stride is None:
        pos_stride = m
    C_a = project(H, W_kv_a)
    if W_z_a is None:
        assert m == 1 and W_kv_b is None
        E = C_a
    else:
        Z_a = project(H, W_z_a)
        if W_kv_b is not None:
            E = pool(C_a, Z_a, B_a, m, project(H, W_kv_b), project(H, W_z_b), B_b)
        else:
            E = pool(C_a, Z_a, B_a, m)
    return finish_entries(E, gamma, eps, d_r, theta, pos_stride, pos_offset, normalize)


# --------------------------------------------------------------------------
# lightning indexer (Evidence Ledger Eqs 13-17; shuhuayu section 03)
# --------------------------------------------------------------------------


def index_scores(qI, w, kI, n_vis: int):
    """score(t, s) = sum_h w[t,h] * ReLU(qI[t,h] . kI[s]) for s < n_vis.

    qI [nI, cI], w [nI], kI [N, cI]; one key per entry shared by all indexer heads.
    """
    kI = np.asarray(kI, dtype=np.float64)[:n_vis]
    dots = kI @ np.asarray(qI, dtype=np.float64).T          # [n_vis, nI]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def index_scores_batch(qI, w, kI, q_pos, m, n_entries=None):
    """Scores for a block of queries of one sequence: qI [Tq, nI, cI], w [Tq, nI],
    kI [N, cI], q_pos [Tq].  Returns (scores [Tq, N] with -inf where invisible,
    n_vis [Tq])."""
    Tq = len(q_pos)
    N = kI.shape[0]
    nv = n_visible(q_pos, m, N if n_entries is None else n_entries)
    S = np.full((Tq, N), -np.inf)
    for t in range(Tq):
        S[t, : nv[t]] = index_scores(qI[t], w[t], kI, int(nv[t]))
    return S, nv


# --------------------------------------------------------------------------
# top-k selection (Evidence Ledger Eqs 13-17: top-k selects compressed blocks)
# --------------------------------------------------------------------------


def topk(scores, n_vis: int, k: int):
    """Indices of the min(k, n_vis) highest scores among entries 0..n_vis-1,
    ties to the lower index, ascending, padded with -1 to length k."""
    s = np.asarray(scores, dtype=np.float64)[:n_vis]
    order = np.lexsort((np.arange(n_vis), -s))     # primary key -score, then index
    chosen = np.sort(order[: min(k, n_vis)])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


# --------------------------------------------------------------------------
# core attention (Evidence Ledger Eqs 18-19, 27 and Section 2.3.3)
# --------------------------------------------------------------------------


def prepare_query(q_raw, gamma_q, eps, d_r, theta, pos):
    """RMSNorm on each query head, then partial RoPE at the query position."""
    return rope(rms_norm(q_raw, gamma_q, eps), pos, d_r, theta)


def attend_rows(q, X, sink, tau):
    """Shared-KV MQA of prepared heads q [nh, c] over rows X [n, c] in ONE softmax
    whose denominator also holds exp(z'_h):

        M   = max(z'_h, max_x tau q_h.x)
        D   = exp(z'_h - M) + sum_x exp(tau q_h.x - M)
        o_h = sum_x exp(tau q_h.x - M) / D * x
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    if X.shape[0] == 0:
        return np.zeros_like(q)
    logits = tau * (q @ X.T)                                  # [nh, n]
    M = np.maximum(sink, logits.max(axis=1))
    e = np.exp(logits - M[:, None])
    D = np.exp(sink - M) + e.sum(axis=1)
    return (e @ X) / D[:, None]


def window_positions(p: int, n_win: int):
    return np.arange(max(0, p - n_win + 1), p + 1)


def attend_query(q_raw, gamma_q, eps, d_r, theta, p, X, sink, tau):
    """One query: prepare q, attend over X, rotate the output back by -p."""
    q = prepare_query(q_raw, gamma_q, eps, d_r, theta, p)
    o = attend_rows(q, X, sink, tau)
    return rope(o, -p, d_r, theta)


def gather_rows(kv, idx, win, p, n_win, win_len):
    """Rows a query reads: the selected compressed entries (idx >= 0) followed by
    the window rows of positions max(0, p-n_win+1)..p, kept in ring slot
    pos % win_len.  Duplicated text in both parts is not deduplicated."""
    sel = [int(s) for s in idx if s >= 0]
    parts = []
    if sel:
        parts.append(np.asarray(kv, dtype=np.float64)[sel])
    wp = window_positions(p, n_win)
    if win is not None and wp.size:
        parts.append(np.asarray(win, dtype=np.float64)[wp % win_len])
    if not parts:
        return np.zeros((0, np.asarray(kv).shape[-1]))
    return np.concatenate(parts, axis=0)


def sparse_attend(q_raw, gamma_q, eps, d_r, theta, q_pos, kv, idx, win, n_win, win_len,
                  sink, tau):
    """CSA core attention for the queries of one sequence.
    q_raw [Tq, nh, c]; kv [N, c] prepared entries; idx [Tq, k]; win [win_len, c]."""
    out = np.empty(np.shape(q_raw), dtype=np.float64)
    for t, p in enumerate(np.asarray(q_pos)):
        X = gather_rows(kv, idx[t], win, int(p), n_win, win_len)
        out[t] = attend_query(q_raw[t], gamma_q, eps, d_r, theta, int(p), X, sink, tau)
    return out


def dense_attend(q_raw, gamma_q, eps, d_r, theta, q_pos, kv, m_prime, win, n_win, win_len,
                 sink, tau, n_entries=None):
    """HCA core attention: every visible compressed entry (s < (q+1)//m') plus
    the window and the sink in one softmax (Evidence Ledger, Section 2.3.2)."""
    N = np.shape(kv)[0] if n_entries is None else n_entries
    out = np.empty(np.shape(q_raw), dtype=np.float64)
    for t, p in enumerate(np.asarray(q_pos)):
        nv = int(n_visible(int(p), m_prime, N))
        X = gather_rows(kv, np.arange(nv), win, int(p), n_win, win_len)
        out[t] = attend_query(q_raw[t], gamma_q, eps, d_r, theta, int(p), X, sink, tau)
    return out


# --------------------------------------------------------------------------
# grouped output projection (Evidence Ledger, Section 2.3.1: n_h heads -> g
# groups -> d_g intermediates -> d; shuhuayu page section 03: outputs are
# rotated back before the grouped projection, configuration table: output
# groups / rank per group)
# --------------------------------------------------------------------------


def grouped_out_proj(o, W_a, W_b, round_u=None):
    """Grouped output projection of attention outputs.

    o    [R, nh, c]  per query row, the heads' outputs (already rotated by -q)
    W_a  [g, d_g, nh/g * c]  group j's projection (linear convention [out, in])
    W_b  [d, g * d_g]        the output projection

    u_j = concat(o[h] for h in group j) . W_a[j]^T   (R x d_g)
    y   = [u_0 | u_1 | ... | u_{g-1}] . W_b^T         (R x d)
    Returns (y, u) in fp64; ``round_u`` (if given) is applied to u before the
    second product."""
    o = np.asarray(o, dtype=np.float64)
    W_a = np.asarray(W_a, dtype=np.float64)
    W_b = np.asarray(W_b, dtype=np.float64)
    R, nh, c = o.shape
    g, d_g, K1 = W_a.shape
    if nh % g or K1 != nh // g * c or W_b.shape[1] != g * d_g:
        raise ValueError("inconsistent grouped projection shapes")
    hpg = nh // g
    u = np.empty((R, g, d_g))
    for j in range(g):
        oj = o[:, j * hpg:(j + 1) * hpg, :].reshape(R, K1)   # heads of group j, head-major
        u[:, j, :] = oj @ W_a[j].T
    u = u.reshape(R, g * d_g)
    if round_u is not None:
        u = np.asarray(round_u(u), dtype=np.float64)
    return u @ W_b.T, u


# --------------------------------------------------------------------------
# accounting (tianyi-zhang-02 page section 2; shuhuayu page sections 03, 06)
# --------------------------------------------------------------------------


def attention_ledger(history, light_ratio, heavy_ratio, selected, window):
    """Per-layer entry counts after ``history`` processed positions (the current
    query counted): completed compressed entries, the entries a query's core
    attention reads (selected CSA entries or all HCA entries, plus the local
    window, no deduplication, sink not counted) and the unfinished tail of the
    current block."""
    args = (history, light_ratio, heavy_ratio, selected, window)
    if not all(isinstance(v, int) and not isinstance(v, bool) and v > 0 for v in args):
        raise ValueError("counts must be positive integers")
    if not heavy_ratio > light_ratio:
        raise ValueError("the heavy ratio must exceed the light ratio")
    local = min(history, window)
    out = {}
    for name, ratio, cap in (("light", light_ratio, selected), ("heavy", heavy_ratio, None)):
        done, tail = divmod(history, ratio)
        out[name + "_stored"] = done
        out[name + "_main_reads"] = (done if cap is None else min(cap, done)) + local
        out[name + "_tail"] = tail
    return out


def kv_cache_bytes(context, n_csa, n_hca, n_swa, m=4, m_prime=128, n_win=128,
                   main_bytes=576, index_bytes=64):
    """Decoder KV payload at ``context`` tokens: CSA layers hold context//m main
    entries and as many index keys, HCA layers context//m' main entries, and
    every layer a saturated window of n_win uncompressed entries (shuhuayu
    section 06; 448 FP8 + 64 BF16 dims = 576 B, 128 FP4 dims = 64 B)."""
    csa = (context // m) * (main_bytes + index_bytes) + n_win * main_bytes
    hca = (context // m_prime) * main_bytes + n_win * main_bytes
    swa = n_win * main_bytes
    return n_csa * csa + n_hca * hca + n_swa * swa


def gqa8_cache_bytes(context, layers, kv_heads=8, head_dim=128, elem_bytes=2):
    """BF16 GQA-8 baseline: separate K and V, 8 KV heads of dim 128, every layer."""
    return layers * context * 2 * kv_heads * head_dim * elem_bytes
