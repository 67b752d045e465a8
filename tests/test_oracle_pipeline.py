"""Pins of the oracle's per-workload layer (``oracle/pipeline.py``), CPU only.

The decode references (caches prepared from raw entries, the window ring, the
quantised-oracle scores, top-k and attention) are checked against the prefill
references on the tiny workload: a decode step at position q of a sequence is
the prefill's query row q (tianyi-zhang-02 page, section 3: entries become
visible at q + 1 = m, 2m, ...; Evidence Ledger Eqs 18-19 and 27 for the
attention).  The prefill references are checked against the batch functions of
``oracle/csa.py`` (pinned on their own) and, for one query, against scalar
loops written from the equations.  ``tie_free`` is checked against its set
definition by brute force.
"""
import math

import numpy as np
import pytest

import csa_inputs as I
from oracle import csa as O
from oracle import formats as F
from oracle import pipeline as OP

QUERIES = [3, 4, 7, 8, 500, 1023]


@pytest.fixture(scope="module")
def tiny():
    sp = I.CONFIGS["tiny_csa"]
    inp = I.prefill_inputs(sp)
    return sp, inp, OP.prefill_caches(inp)


@pytest.fixture(scope="module")
def tiny_hca():
    sp = I.CONFIGS["tiny_hca"]
    inp = I.prefill_inputs(sp)
    return sp, inp, OP.prefill_caches(inp)


def decode_from_prefill(sp, inp, queries, win_len):
    """Decode-step inputs of the sequences that end at each query position of
    the tiny prefill: pooled (not yet normalised) entries, raw index keys,
    per-token window rows in a ring of ``win_len`` slots, the prefill's query
    row.  Built from projections and pooling only (no norm / RoPE / top-k)."""
    H = inp["H"]
    overlap = sp.m == 4
    E = O.compress(H, inp["W_kv_a"], inp["W_z_a"], inp["bias_a"], sp.m,
                   inp.get("W_kv_b") if overlap else None, inp.get("W_z_b") if overlap else None,
                   inp.get("bias_b") if overlap else None, normalize=False)
    R = O.project(H, inp["W_win"])
    B = len(queries)
    lengths = np.asarray(queries, np.int64) + 1
    n_entries = (lengths // sp.m).astype(np.int32)
    Nmax = int(max(1, n_entries.max()))
    kind = "decode" if sp.nI else "hca_decode"
    dsp = I.Spec("tiny_decode", kind, m=sp.m, c=sp.c, d_r=sp.d_r, nh=sp.nh, n_win=sp.n_win, B=B,
                 L=int(lengths.max()), nI=sp.nI, cI=sp.cI, k=sp.k, dtype="f32", kv_format="f32",
                 index_format="f32")
    win_raw = np.zeros((B, win_len, sp.c))
    win_pos = np.full((B, win_len), -1, np.int32)
    for b, L in enumerate(lengths):
        for p in range(max(0, int(L) - win_len), int(L)):
            win_raw[b, p % win_len] = R[p]
            win_pos[b, p % win_len] = p
    d = dict(spec=dsp, lengths=lengths, n_entries=n_entries, Nmax=Nmax,
             q_pos=(lengths - 1).astype(np.int32).reshape(B, 1),
             kv_raw=np.stack([E[:Nmax]] * B), win_raw=win_raw, win_pos=win_pos,
             q=inp["q"][queries][:, None], sink=inp["sink"])
    if sp.nI:
        kI = O.compress(H, inp["WI_kv_a"], inp["WI_z_a"], inp["biasI_a"], sp.m, inp["WI_kv_b"],
                        inp["WI_z_b"], inp["biasI_b"], normalize=False)
        d.update(kI=np.stack([kI[:Nmax]] * B), qI=inp["qI"][queries][:, None],
                 w=inp["w"][queries][:, None])
    return d


def test_decode_cache_and_window_equal_prefill_rows(tiny):
    """Entry i is stored at RoPE position m*i and window row p at p, ring slot
    p % win_len: the decode caches equal the prefill compressor's rows."""
    sp, inp, caches = tiny
    for win_len in (128, 160):
        d = decode_from_prefill(sp, inp, QUERIES, win_len)
        for b, q in enumerate(QUERIES):
            n = int(d["n_entries"][b])
            assert np.array_equal(OP.decode_cache(d, b)[:n], caches["kv"][:n])
            sel = np.arange(0, n, 3)
            assert np.array_equal(OP.decode_cache(d, b, sel), caches["kv"][sel])
            win = OP.decode_window(d, b)
            for p in range(max(0, q - win_len + 1), q + 1):
                assert np.array_equal(win[p % win_len], caches["win"][p]), (q, p)


@pytest.mark.parametrize("win_len", [128, 160])
def test_decode_reference_equals_prefill_row(tiny, win_len):
    """A decode step at position q (ring of 128 or 160 slots) reproduces the
    prefill's row q: visible count, scores, top-k set and output."""
    sp, inp, caches = tiny
    d = decode_from_prefill(sp, inp, QUERIES, win_len)
    refs = OP.prefill_reference(inp, caches, QUERIES)
    for b, (q, ref) in enumerate(zip(QUERIES, refs)):
        got = OP.decode_reference(d, b)
        assert got["n_vis"] == ref["n_vis"] == (q + 1) // sp.m
        assert np.allclose(got["scores"], ref["scores"], rtol=1e-12, atol=1e-12)
        assert np.array_equal(got["idx"], ref["idx"])
        assert np.allclose(got["out"], ref["out"], rtol=1e-10, atol=1e-12), q


def test_hca_decode_equals_prefill_row(tiny_hca):
    sp, inp, caches = tiny_hca
    qs = [3, 127, 128, 500, 1023]
    d = decode_from_prefill(sp, inp, qs, 128)
    refs = OP.prefill_reference(inp, caches, qs)
    for b, (q, ref) in enumerate(zip(qs, refs)):
        got = OP.decode_reference(d, b)["out"]
        assert np.allclose(got, ref["out"], rtol=1e-10, atol=1e-12), q


def test_prefill_reference_equals_batch_functions(tiny, tiny_hca):
    """prefill_reference row by row equals the csa.py batch calls over the
    whole sequence (scores with -inf beyond N(q), top-k, sparse / dense attend)."""
    sp, inp, caches = tiny
    T = inp["T"]
    rows = list(range(0, T, 37)) + [T - 1]
    S, nv = O.index_scores_batch(inp["qI"], inp["w"], caches["kI"], inp["q_pos"], sp.m)
    idx = np.stack([O.topk(S[t], int(nv[t]), sp.k) for t in range(T)])
    out = O.sparse_attend(inp["q"], None, OP.EPS, sp.d_r, OP.THETA, inp["q_pos"], caches["kv"],
                          idx, caches["win"], sp.n_win, T, inp["sink"], 1 / math.sqrt(sp.c))
    for r, ref in zip(rows, OP.prefill_reference(inp, caches, rows)):
        assert ref["n_vis"] == nv[r]
        assert np.allclose(ref["scores"], S[r, :nv[r]], rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(S[r, nv[r]:]))
        assert np.array_equal(ref["idx"], idx[r])
        assert np.allclose(ref["out"], out[r], rtol=1e-12, atol=1e-14)
    sp, inp, caches = tiny_hca
    out = O.dense_attend(inp["q"], None, OP.EPS, sp.d_r, OP.THETA, inp["q_pos"], caches["kv"],
                         sp.m, caches["win"], sp.n_win, T, inp["sink"], 1 / math.sqrt(sp.c))
    for r, ref in zip(rows, OP.prefill_reference(inp, caches, rows)):
        assert np.allclose(ref["out"], out[r], rtol=1e-12, atol=1e-14)


def _rot(x, pos, d_r, theta=10000.0):
    """Scalar RoPE: pair (c-d_r+2u, c-d_r+2u+1) turned by pos * theta^(-2u/d_r)."""
    y = list(x)
    c = len(x)
    for u in range(d_r // 2):
        a = pos * theta ** (-2.0 * u / d_r)
        i = c - d_r + 2 * u
        y[i] = x[i] * math.cos(a) - x[i + 1] * math.sin(a)
        y[i + 1] = x[i] * math.sin(a) + x[i + 1] * math.cos(a)
    return y


def test_one_query_against_scalar_loops(tiny):
    """Query 500 of the tiny prefill from scalar loops over the equations:
    indexer score, top-k by sorting, RMSNorm + RoPE of query and rows, one
    softmax over selected and window rows with exp(z'_h) in the denominator,
    output rotated back by -q."""
    sp, inp, caches = tiny
    q = 500
    c, d_r, m, eps = sp.c, sp.d_r, sp.m, 1e-6
    nv = (q + 1) // m
    kI = caches["kI"]
    score = []
    for s in range(nv):
        acc = 0.0
        for h in range(sp.nI):
            dot = sum(float(inp["qI"][q, h, j]) * float(kI[s, j]) for j in range(sp.cI))
            acc += float(inp["w"][q, h]) * max(dot, 0.0)
        score.append(acc)
    order = sorted(range(nv), key=lambda s: (-score[s], s))[:sp.k]
    sel = sorted(order)
    ref = OP.prefill_reference(inp, caches, [q])[0]
    assert list(ref["idx"][:len(sel)]) == sel
    # rows: entries from the raw pooled values, window rows from the raw projections
    E = O.compress(inp["H"], inp["W_kv_a"], inp["W_z_a"], inp["bias_a"], m, inp["W_kv_b"],
                   inp["W_z_b"], inp["bias_b"], normalize=False)
    R = O.project(inp["H"], inp["W_win"])

    def prep(x, pos):
        x = [float(v) for v in x]            # Python floats: fp64 throughout
        r = math.sqrt(sum(v * v for v in x) / len(x) + eps)
        return _rot([v / r for v in x], pos, d_r)
    rows = [prep(E[s], m * s) for s in sel] + [prep(R[p], p) for p in range(q - 127, q + 1)]
    tau = 1 / math.sqrt(c)
    out = []
    for h in range(sp.nh):
        qh = prep(inp["q"][q, h], q)
        logits = [tau * sum(a * b for a, b in zip(qh, x)) for x in rows]
        z = float(inp["sink"][h])
        M = max([z] + logits)
        den = math.exp(z - M) + sum(math.exp(v - M) for v in logits)
        o = [sum(math.exp(v - M) / den * x[j] for v, x in zip(logits, rows)) for j in range(c)]
        out.append(_rot(o, -q, d_r))
    assert np.allclose(ref["out"], np.array(out), rtol=1e-9, atol=1e-12)


# ----------------------------------------------------------------- tie_free
def _tie_free_by_sets(scores, nv, k, bound):
    """Definition: with more than k visible entries, every selected score
    exceeds every unselected one by more than ``bound``."""
    if nv <= k:
        return True
    sel = set(O.topk(scores, nv, k).tolist())
    lo = min(scores[s] for s in sel)
    hi = max(scores[s] for s in range(nv) if s not in sel)
    return lo - hi > bound


def test_tie_free_against_set_definition():
    rng = np.random.default_rng(11)
    cases = 0
    for _ in range(300):
        nv = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        s = np.round(rng.normal(size=nv + 5), int(rng.integers(0, 3)))  # rounding makes ties
        bound = float(rng.choice([0.0, 1e-3, 0.05, 0.5]))
        assert OP.tie_free(s, nv, k, bound) == _tie_free_by_sets(s, nv, k, bound)
        cases += 1
    assert cases == 300


def test_tie_free_edges():
    s = np.array([5.0, 3.0, 3.0, 1.0, 9.0])  # entry 4 is past nv for nv = 4
    assert OP.tie_free(s, 4, 4, 1.0)          # nv <= k: every entry is taken
    assert OP.tie_free(s, 3, 5, 0.0)
    assert not OP.tie_free(s, 4, 2, 0.0)       # the k-th and (k+1)-th tie exactly
    assert OP.tie_free(s, 4, 1, 1.9)           # gap 2 against a bound below it
    assert not OP.tie_free(s, 4, 1, 2.0)       # gap equal to the bound: not free
    assert OP.tie_free(s, 4, 3, 1.5) and not OP.tie_free(s, 4, 3, 2.5)
    # entries beyond nv never count, however large
    assert OP.tie_free(s, 4, 1, 1.0) and OP.tie_free(s, 5, 1, 3.9) and not OP.tie_free(s, 5, 1, 4.0)


# ----------------------------------------------------------------- quantised-oracle mode
def _mx_exact_rows(rng, n, c):
    """Rows whose MXFP4 encoding is exact: per 32-block, E2M1 grid values times
    2^s with one element of magnitude 6 * 2^s (so the block scale rule picks 2^s)."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(grid, size=(n, c)) * rng.choice([-1, 1], size=(n, c))
    x = x.reshape(n, c // 32, 32)
    x[:, :, 0] = 6.0 * rng.choice([-1, 1], size=(n, c // 32))
    s = rng.integers(-6, 3, size=(n, c // 32, 1)).astype(float)
    return (x * 2.0 ** s).reshape(n, c)


def test_mxfp4_decode_scores_quantise_both_sides_and_round_to_bf16():
    """The quantised-oracle mode (MXFP4 keys and queries, bf16 scores): inputs
    that MXFP4 holds exactly give bf16(exact score); scalar loops for the score."""
    rng = np.random.default_rng(12)
    sp = I.Spec("mx", "decode", m=4, c=64, d_r=16, nh=2, B=1, L=4 * 40, nI=4, cI=64, k=8,
                index_format="mxfp4")
    kI = _mx_exact_rows(rng, 40, 64)
    qI = _mx_exact_rows(rng, 4, 64)
    w = rng.normal(size=4)
    d = dict(spec=sp, n_entries=np.array([40]), q_pos=np.array([[4 * 40 - 1]]), kI=kI[None],
             qI=qI[None, None], w=w[None, None])
    s, nv = OP.decode_scores(d, 0)
    assert nv == 40
    for e in range(nv):
        acc = 0.0
        for h in range(4):
            acc += w[h] * max(0.0, sum(qI[h, j] * kI[e, j] for j in range(64)))
        assert s[e] == F.bf16_round(np.array([acc]))[0]
    # values MXFP4 cannot hold are quantised first: the scores move
    d["kI"] = (kI * 1.07)[None]
    s2, _ = OP.decode_scores(d, 0)
    assert not np.allclose(s2, F.bf16_round(s * 1.07))
