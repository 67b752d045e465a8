"""The attention error bound (tests/attn_bound.py) on the CPU, at the shape of
the 64K decode workload (one sequence: 16,384 entries, k = 1024, 128-slot
window, 64 heads x 512, bf16 rows; Evidence Ledger Eqs 18-19, 27):

  * an emulation of the kernels' rounding (bf16 query operand, fp32 logits,
    lazy running maximum per 32-slot tile, bf16 P, bf16 split partials merged
    in split order, bf16 output) stays inside it;
  * plausible mistakes fall outside it: one mis-gathered row, tau off by 2%,
    and -- with sinks strong enough to carry weight -- a dropped sink.
"""
import math

import numpy as np
import pytest

import csa_inputs as I
from oracle import csa as O
from oracle import formats as F
from oracle import pipeline as OP
from tests.attn_bound import LOG2E, attend_ref_bound, slot_splits, split_plan


def rows_in_slot_order(inp, b, idx):
    """Rows the kernel reads for sequence b, in slot order, and the slots of
    the compressed ones: selected entries (idx >= 0), then the window."""
    sp = inp["spec"]
    p = int(inp["q_pos"][b, 0])
    sel_slots = [v for v, s in enumerate(idx) if s >= 0]
    sel = np.asarray([idx[v] for v in sel_slots], np.int64)
    win = OP.decode_window(inp, b)
    wp = O.window_positions(p, sp.n_win)
    X = np.concatenate([OP.decode_cache(inp, b, sel), win[wp % win.shape[0]]], 0)
    return X, sel_slots


@pytest.fixture(scope="module")
def case():
    sp = I.CONFIGS["decode_64k"].replace(B=1)
    inp = I.decode_inputs(sp, seed=77)
    rng = np.random.default_rng(78)
    nv = int(O.n_visible(int(inp["q_pos"][0, 0]), sp.m, int(inp["n_entries"][0])))
    idx = I.random_index_sets(rng, np.array([nv]), sp.k)[0]
    X, sel_slots = rows_in_slot_order(inp, 0, idx)
    return sp, inp, idx, X, sel_slots


def emulate_kernel(q_raw, X, sink, tau, d_r, pos, chunk_rows):
    """The kernels' arithmetic in numpy: fp32 logits of the bf16 query operand,
    per 32-row tile a running maximum that moves only when a logit exceeds it
    by 8 nats, bf16 P in the numerator and fp32 sums in the denominator, bf16
    O / l per split (``chunk_rows``: row ranges of the splits, None = one),
    merge in split order with the sink, inverse RoPE, bf16 output."""
    qp = O.prepare_query(q_raw, None, 1e-6, d_r, 1e4, pos).astype(np.float32)
    qb = F.bf16_round((qp * np.float32(tau * LOG2E)).astype(np.float64)).astype(np.float32)
    Xf = X.astype(np.float32)
    nh = qb.shape[0]
    parts = []
    for r0, r1 in (chunk_rows or [(0, X.shape[0])]):
        m = np.full(nh, -3e38, np.float32)
        l = np.zeros(nh, np.float32)
        acc = np.zeros((nh, X.shape[1]), np.float32)
        for t0 in range(r0, r1, 32):
            t1 = min(t0 + 32, r1)
            lg = qb @ Xf[t0:t1].T                        # log2 units
            mx = lg.max(axis=1)
            grow = mx > m + np.float32(8 * LOG2E)
            m_new = np.where(grow, mx, m)
            alpha = np.exp2(m - m_new).astype(np.float32)
            l, acc, m = l * alpha, acc * alpha[:, None], m_new
            pw = np.exp2(lg - m[:, None]).astype(np.float32)
            l = l + pw.sum(axis=1, dtype=np.float32)
            acc = acc + F.bf16_round(pw.astype(np.float64)).astype(np.float32) @ Xf[t0:t1]
        parts.append((m * np.float32(1 / LOG2E), l, acc))
    z = np.asarray(sink, np.float64)
    if len(parts) == 1:
        m, l, acc = parts[0]
        M = np.maximum(m, z)
        o = acc * np.exp(m - M)[:, None] / (l * np.exp(m - M) + np.exp(z - M))[:, None]
    else:
        M = np.maximum(z, np.max([pm for pm, _, _ in parts], axis=0))
        den = np.exp(z - M)
        o = 0.0
        for pm, pl, pacc in parts:
            ob = F.bf16_round((pacc / np.maximum(pl, 1e-30)[:, None]).astype(np.float64))
            wgt = pl * np.exp(pm - M)
            den = den + wgt
            o = o + ob * wgt[:, None]
        o = o / den[:, None]
    return F.bf16_round(O.rope(o, -pos, d_r, 1e4))


def _chunk_rows(split_id):
    if split_id is None:
        return None
    edges = np.flatnonzero(np.diff(split_id)) + 1
    b = [0, *edges.tolist(), len(split_id)]
    return list(zip(b[:-1], b[1:]))


def test_plan_of_the_64k_decode_shape():
    assert split_plan(1024, 128) == (160, 8)       # 1152 slots: 8 splits of 5 tiles
    assert split_plan(64, 128) == (192, 1)         # short lists stay whole
    assert split_plan(1024, 128, Tq=4) == (1152, 1)


def test_kernel_emulation_inside_the_bound(case):
    sp, inp, idx, X, sel_slots = case
    p = int(inp["q_pos"][0, 0])
    tau = 1 / math.sqrt(sp.c)
    sid = slot_splits(sel_slots, sp.k, sp.n_win, p)
    ref, bound = attend_ref_bound(inp["q"][0, 0], X, inp["sink"], tau, sp.d_r, p, sid)
    emu = emulate_kernel(inp["q"][0, 0], X, inp["sink"], tau, sp.d_r, p, _chunk_rows(sid))
    err = np.abs(emu - ref)
    assert np.all(err <= bound), float((err - bound).max())
    # the bound is far inside the 2e-2 acceptance bar, and not vacuous
    assert np.median(bound) < 6e-3 and bound.max() < 2e-2 and err.max() > 1e-4
    # and the oracle itself (unrounded query) is within the acceptance bar
    assert np.abs(OP.decode_attend(inp, 0, idx) - emu).max() < 2e-2


def test_bound_rejects_a_mis_gathered_row(case):
    sp, inp, idx, X, sel_slots = case
    p = int(inp["q_pos"][0, 0])
    tau = 1 / math.sqrt(sp.c)
    sid = slot_splits(sel_slots, sp.k, sp.n_win, p)
    ref, bound = attend_ref_bound(inp["q"][0, 0], X, inp["sink"], tau, sp.d_r, p, sid)
    rng = np.random.default_rng(5)
    chosen = set(int(s) for s in idx if s >= 0)
    nv = int(inp["n_entries"][0])
    for _ in range(12):
        v = int(rng.integers(0, len(sel_slots)))
        other = int(rng.integers(0, nv))
        while other in chosen:
            other = int(rng.integers(0, nv))
        Xs = X.copy()
        Xs[v] = OP.decode_cache(inp, 0, [other])[0]        # row v read from the wrong entry
        wrong, _ = attend_ref_bound(inp["q"][0, 0], Xs, inp["sink"], tau, sp.d_r, p, sid)
        assert np.any(np.abs(wrong - ref) > bound), v


def test_bound_rejects_a_wrong_scale(case):
    sp, inp, idx, X, sel_slots = case
    p = int(inp["q_pos"][0, 0])
    tau = 1 / math.sqrt(sp.c)
    sid = slot_splits(sel_slots, sp.k, sp.n_win, p)
    ref, bound = attend_ref_bound(inp["q"][0, 0], X, inp["sink"], tau, sp.d_r, p, sid)
    for f in (1.02, 0.98):
        wrong, _ = attend_ref_bound(inp["q"][0, 0], X, inp["sink"], tau * f, sp.d_r, p, sid)
        assert np.any(np.abs(wrong - ref) > bound), f


def test_bound_rejects_a_dropped_sink_when_sinks_carry_weight(case):
    """With N(0,1) sinks the sink holds ~0.1% of the mass, below any rounding
    bound; shifted up by 6 it holds a large share, and dropping it is caught."""
    sp, inp, idx, X, sel_slots = case
    p = int(inp["q_pos"][0, 0])
    tau = 1 / math.sqrt(sp.c)
    sid = slot_splits(sel_slots, sp.k, sp.n_win, p)
    strong = inp["sink"] + 6.0
    ref, bound = attend_ref_bound(inp["q"][0, 0], X, strong, tau, sp.d_r, p, sid)
    emu = emulate_kernel(inp["q"][0, 0], X, strong, tau, sp.d_r, p, _chunk_rows(sid))
    assert np.all(np.abs(emu - ref) <= bound)
    no_sink, _ = attend_ref_bound(inp["q"][0, 0], X, np.full_like(strong, -1e4), tau, sp.d_r, p, sid)
    assert np.any(np.abs(no_sink - ref) > bound)
