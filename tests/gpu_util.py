"""Helpers shared by the GPU parity tests: device handle, decoding of the
library's stored rows with torch's own dtype views (independent of the oracle),
and the tolerance rules."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_10_amd as L


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def decode_rows(buf: torch.Tensor, fmt: int, rows: int, c: int, d_r: int) -> np.ndarray:
    """fp64 values of ``rows`` stored rows (torch dtype views do the decoding)."""
    b = buf.reshape(rows, -1)
    if fmt == L.F32:
        return b.view(torch.float32).double().cpu().numpy()
    if fmt == L.BF16:
        return b.view(torch.bfloat16).double().cpu().numpy()
    if fmt == L.FP8MIX:
        body = b[:, : c - d_r].contiguous().view(torch.float8_e4m3fn).double()
        rope = b[:, c - d_r:].contiguous().view(torch.bfloat16).double()
        return torch.cat([body, rope], 1).cpu().numpy()
    raise ValueError(fmt)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (for tolerances)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def e4m3_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -6)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 3)


def score_error_bound(qI, w, kI, nv, rel=1e-5):
    """A posteriori bound on |fp32 score - exact score| per entry:
    rel * sum_h |w_h| sum_j |qI_hj kI_sj|."""
    if nv == 0:
        return np.zeros(0)
    return rel * (np.abs(kI[:nv]) @ np.abs(qI).T) @ np.abs(w)


def mx_score_bound(inp, b, ref, nv):
    """Bound on |GPU bf16 score - quantised-oracle bf16 score| for MXFP4 keys:
    the fp32 accumulation error of the exact E2M1 products plus one bf16 step
    (the two sides may round to neighbouring bf16 values)."""
    from oracle import pipeline as OP
    kI, _, _ = OP.mxfp4_values(inp["kI"][b][:nv])
    qI, _, _ = OP.mxfp4_values(inp["qI"][b, 0])
    e = score_error_bound(qI, inp["w"][b, 0], kI, nv)
    return bf16_ulp(np.abs(ref) + e) + e


def report(name, **kv):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)


# ---------------------------------------------------------------- attention checks
def _row_bytes(fmt, c, d_r):
    return {L.F32: 4 * c, L.BF16: 2 * c, L.FP8MIX: (c - d_r) + 2 * d_r}[fmt]


def kernel_rows(kv, win, fmt, c, d_r, rows_per_seq, win_len, b, sel, pos, n_win):
    """The rows one query reads, decoded from the GPU's own stored bytes (so a
    check against them isolates the attention arithmetic): compressed entries
    ``sel`` of sequence b of a [B, rows_per_seq] cache, then the window ring's
    positions max(0, pos-n_win+1)..pos at slots p % win_len."""
    rb = _row_bytes(fmt, c, d_r)
    kvb = kv.reshape(-1).view(torch.uint8).reshape(-1, rows_per_seq, rb)
    winb = win.reshape(-1).view(torch.uint8).reshape(-1, win_len, rb)
    sel = np.asarray(sel, np.int64)
    parts = []
    if sel.size:
        g = kvb[b, torch.from_numpy(sel).to(kvb.device)].contiguous()
        parts.append(decode_rows(g, fmt, sel.size, c, d_r))
    wp = np.arange(max(0, pos - n_win + 1), pos + 1)
    if wp.size:
        g = winb[b, torch.from_numpy(wp % win_len).to(winb.device)].contiguous()
        parts.append(decode_rows(g, fmt, wp.size, c, d_r))
    return np.concatenate(parts, 0) if parts else np.zeros((0, c))


def check_attention(tag, got, q_raw, X, sink, tau, d_r, pos, sel_slots, kslots, n_win,
                    oracle_out, Tq=1, bar=2e-2, **kv):
    """Two checks of one query row's output [nh, c]: the acceptance bar against
    the oracle (its own caches and query), and the per-element bound of the
    kernels' arithmetic against the reference built on the same stored rows X
    (kernel slot order) and the kernel's bf16 query operand."""
    from tests.attn_bound import attend_ref_bound, slot_splits
    got = np.asarray(got, np.float64)
    sid = slot_splits(sel_slots, kslots, n_win, pos, Tq)
    ref, bound = attend_ref_bound(q_raw, X, sink, tau, d_r, pos, sid)
    over = np.abs(got - ref) - bound
    err = float(np.abs(got - oracle_out).max())
    ratio = float((np.abs(got - ref) / bound).max())
    report(tag, max_abs=err, bound_ratio=round(ratio, 3), **kv)
    assert err <= bar, (tag, err)
    assert np.all(over <= 0), (tag, float(over.max()), np.unravel_index(int(np.argmax(over)), over.shape))
    return err


def check_decode_attention(tag, g, inp, seq, idx_row, out_row, **kv):
    """check_attention for sequence b of an uploaded decode batch ``g``
    (pipeline.Decode with dense caches): CSA over ``idx_row``, or HCA over
    every visible entry when the workload is HCA."""
    import math
    from oracle import csa as O
    from oracle import pipeline as OP
    sp = inp["spec"]
    b = seq
    p = int(inp["q_pos"][b, 0])
    if sp.kind == "hca_decode":
        nv = int(O.n_visible(p, sp.m, int(inp["n_entries"][b])))
        sel_slots, sel, kslots = list(range(nv)), np.arange(nv), g.Nmax
        want = OP.decode_attend(inp, b, None)
    else:
        idx_row = np.asarray(idx_row)
        sel_slots = [v for v, s in enumerate(idx_row) if s >= 0]
        sel, kslots = idx_row[sel_slots], len(idx_row)
        want = OP.decode_attend(inp, b, idx_row)
    X = kernel_rows(g.kv, g.win, g.kv_fmt, sp.c, sp.d_r, g.Nmax, g.win_len, b, sel, p, sp.n_win)
    return check_attention(tag, out_row, inp["q"][b, 0], X, inp["sink"], 1 / math.sqrt(sp.c),
                           sp.d_r, p, sel_slots, kslots, sp.n_win, want, **kv)
