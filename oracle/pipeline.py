"""The oracle's end-to-end runs on the seeded workloads (fp64, CPU).

TEST INFRASTRUCTURE ONLY (tests, smoke check and the CPU baseline of the
benchmark).  Takes the raw arrays of ``csa_inputs`` and applies the oracle's
own stage functions, including its own RMSNorm / RoPE of the caches and its own
format rounding (bf16, e4m3 + bf16, MXFP4) -- nothing comes from the HIP path.
"""
from __future__ import annotations

import math

import numpy as np

from . import csa as O
from . import formats as F

THETA = O.ROPE_THETA
EPS = O.RMS_EPS


def store(x, fmt, d_r):
    """Values a cache row holds after being stored in ``fmt``."""
    if fmt == "f32":
        return np.asarray(x, np.float64)
    if fmt == "bf16":
        return F.bf16_round(x)
    if fmt == "fp8mix":
        return F.fp8mix_round(x, d_r)
    raise ValueError(fmt)


def mxfp4_values(x):
    packed, scales = F.mxfp4_quantize(x)
    return F.mxfp4_dequantize(packed, scales), packed, scales


def decode_cache(inp, b, rows=None):
    """Prepared compressed entries of sequence b (all rows, or just ``rows``):
    RMSNorm, RoPE at position m*i, stored in the KV format."""
    sp = inp["spec"]
    raw = inp["kv_raw"][b] if rows is None else inp["kv_raw"][b][rows]
    idx = np.arange(raw.shape[0]) if rows is None else np.asarray(rows)
    E = O.rope(O.rms_norm(raw, None, EPS), sp.m * idx, sp.d_r, THETA)
    return store(E, sp.kv_format, sp.d_r)


def decode_window(inp, b):
    """The window ring of sequence b as stored: slot s holds the row of the
    newest position p with p % win_len == s (RMSNorm, RoPE at p), win_len being
    the ring's length (at least n_win)."""
    sp = inp["spec"]
    pos = inp["win_pos"][b]
    E = O.rope(O.rms_norm(inp["win_raw"][b], None, EPS), np.maximum(pos, 0), sp.d_r, THETA)
    return store(E, sp.kv_format, sp.d_r)


def decode_scores(inp, b):
    """Indexer scores of sequence b's query (and the visible count)."""
    sp = inp["spec"]
    N = int(inp["n_entries"][b])
    p = int(inp["q_pos"][b, 0])
    nv = int(O.n_visible(p, sp.m, N))
    if sp.index_format == "mxfp4":
        kI, _, _ = mxfp4_values(inp["kI"][b][:nv])
        qI, _, _ = mxfp4_values(inp["qI"][b, 0])
        s = O.index_scores(qI, inp["w"][b, 0], kI, nv)
        return F.bf16_round(s), nv
    return O.index_scores(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv), nv


def decode_attend(inp, b, idx):
    """Sparse (CSA) or dense (HCA) attention output of sequence b's query, with
    the caches prepared by the oracle itself; ``idx`` is the selected set."""
    sp = inp["spec"]
    p = int(inp["q_pos"][b, 0])
    tau = 1.0 / math.sqrt(sp.c)
    win = decode_window(inp, b)
    if sp.kind == "hca_decode":
        nv = int(O.n_visible(p, sp.m, int(inp["n_entries"][b])))
        sel = np.arange(nv)
    else:
        sel = np.asarray([s for s in idx if s >= 0], dtype=np.int64)
    kv_rows = decode_cache(inp, b, sel) if sel.size else np.zeros((0, sp.c))
    win_len = win.shape[0]                  # the ring's own length, n_win or more
    X = np.concatenate([kv_rows, win[O.window_positions(p, sp.n_win) % win_len]], axis=0)
    return O.attend_query(inp["q"][b, 0], None, EPS, sp.d_r, THETA, p, X, inp["sink"], tau)


def decode_reference(inp, b):
    """Whole decode step for sequence b: scores, top-k, attention output."""
    sp = inp["spec"]
    if sp.kind == "hca_decode":
        return dict(out=decode_attend(inp, b, None))
    s, nv = decode_scores(inp, b)
    idx = O.topk(s, nv, sp.k)
    return dict(scores=s, n_vis=nv, idx=idx, out=decode_attend(inp, b, idx))


# ----------------------------------------------------------------- prefill
def prefill_caches(inp):
    """Main entries, index keys and per-token window rows of a prefill."""
    sp = inp["spec"]
    H = inp["H"]
    overlap = sp.m == 4
    kv = O.compress(H, inp["W_kv_a"], inp["W_z_a"], inp["bias_a"], sp.m,
                    inp.get("W_kv_b") if overlap else None, inp.get("W_z_b") if overlap else None,
                    inp.get("bias_b") if overlap else None, None, EPS, sp.d_r, THETA, sp.m, 0)
    out = dict(kv=store(kv, sp.kv_format, sp.d_r))
    if sp.nI:
        kI = O.compress(H, inp["WI_kv_a"], inp["WI_z_a"], inp["biasI_a"], sp.m, inp["WI_kv_b"],
                        inp["WI_z_b"], inp["biasI_b"], normalize=False)
        out["kI_exact"] = kI
        out["kI"] = mxfp4_values(kI)[0] if sp.index_format == "mxfp4" else store(kI, sp.index_format, 0)
    win = O.compress(H, inp["W_win"], None, None, 1, d_r=sp.d_r, pos_stride=1, pos_offset=0)
    out["win"] = store(win, sp.kv_format, sp.d_r)
    return out


def prefill_reference(inp, caches, rows):
    """Scores / top-k / output for the query rows ``rows`` (indices into the
    query arrays of ``inp``)."""
    sp = inp["spec"]
    T = inp["T"]
    tau = 1.0 / math.sqrt(sp.c)
    res = []
    for r in rows:
        p = int(inp["q_pos"][r])
        d = dict(pos=p)
        if sp.nI:
            nv = int(O.n_visible(p, sp.m, T // sp.m))
            if sp.index_format == "mxfp4":
                # quantised-oracle mode: the same E2M1 values and scales, fp64, bf16 scores
                qq = mxfp4_values(inp["qI"][r])[0]
                s = F.bf16_round(O.index_scores(qq, inp["w"][r], caches["kI"], nv))
            else:
                s = O.index_scores(inp["qI"][r], inp["w"][r], caches["kI"], nv)
            idx = O.topk(s, nv, sp.k)
            X = O.gather_rows(caches["kv"], idx, caches["win"], p, sp.n_win, T)
            d.update(scores=s, n_vis=nv, idx=idx)
        else:
            nv = int(O.n_visible(p, sp.m, T // sp.m))
            X = O.gather_rows(caches["kv"], np.arange(nv), caches["win"], p, sp.n_win, T)
        d["out"] = O.attend_query(inp["q"][r], None, EPS, sp.d_r, THETA, p, X, inp["sink"], tau)
        res.append(d)
    return res


def tie_free(scores, nv, k, bound):
    """True when the k-th and (k+1)-th largest visible scores differ by more
    than ``bound`` (so any implementation within that error selects the same
    set)."""
    if nv <= k:
        return True
    s = np.sort(np.asarray(scores[:nv], dtype=np.float64))[::-1]
    return (s[k - 1] - s[k]) > bound
