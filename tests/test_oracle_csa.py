"""Pins of the fp64 CSA oracle (CPU only): figures the pages print, closed forms,
invariants, brute force on tiny inputs and independent library routines."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ledger.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ============================================================ ledger / counts
def test_attention_ledger_page_asserts():
    for item in golden()["attention_ledger"]:
        assert O.attention_ledger(*item["args"])[item["key"]] == item["value"], item["cite"]


def test_attention_ledger_rejects_bad_counts():
    with pytest.raises(ValueError):
        O.attention_ledger(1024, 4, 4, 32, 128)
    with pytest.raises(ValueError):
        O.attention_ledger(0, 4, 128, 32, 128)


def test_stored_entries_at_1M_and_visibility():
    g = golden()
    for item in g["stored_entries_1M"]:
        # the last position of a 1M context is q = context - 1
        assert O.n_visible(item["context"] - 1, item["ratio"]) == item["value"], item["cite"]
        assert O.attention_ledger(item["context"], 4, 128, 1024, 128)[
            "light_stored" if item["ratio"] == 4 else "heavy_stored"] == item["value"]
    for item in g["visible_entries"]:
        assert O.n_visible(item["q"], item["m"]) == item["value"], item["cite"]


def test_kv_cache_ratio_about_two_percent():
    for item in golden()["kv_ratio_1M"]:
        L = 1 << 20
        v4 = O.kv_cache_bytes(L, item["n_csa"], item["n_hca"], item["n_swa"])
        base = O.gqa8_cache_bytes(L, item["layers"])
        assert abs(v4 / base - item["approx"]) < item["tol"], item["cite"]
    # derived figures (Pro): 5.18 GB against 262.0 GB
    v4 = O.kv_cache_bytes(1 << 20, 30, 31, 0)
    assert round(v4 / 1e9, 2) == 5.18
    assert round(O.gqa8_cache_bytes(1 << 20, 61) / 1e9, 1) == 262.0


def test_entry_bytes():
    from oracle import formats as F
    for item in golden()["entry_bytes"]:
        if "rope_dims" in item:
            row = F.fp8mix_encode(np.zeros((1, item["c"])), item["rope_dims"])
            assert row.shape[-1] == item["value"], item["cite"]
        else:
            packed, _ = F.mxfp4_quantize(np.zeros((1, item["c"])))
            assert packed.shape[-1] == item["value"], item["cite"]


# ============================================================ pooling (Eqs 11-12)
def brute_pool(C_a, Z_a, B_a, m, C_b=None, Z_b=None, B_b=None):
    """Scalar loops: for every entry and channel list the candidates, take a
    plain softmax of their logits and the weighted sum."""
    T, c = len(C_a), len(C_a[0])
    out = []
    for i in range(T // m):
        row = []
        for j in range(c):
            cands = [(Z_a[m * i + u][j] + B_a[u][j], C_a[m * i + u][j]) for u in range(m)]
            if C_b is not None and i > 0:
                cands += [(Z_b[m * (i - 1) + u][j] + B_b[u][j], C_b[m * (i - 1) + u][j])
                          for u in range(m)]
            top = max(l for l, _ in cands)
            ws = [math.exp(l - top) for l, _ in cands]
            row.append(sum(w * v for w, (_, v) in zip(ws, cands)) / sum(ws))
        out.append(row)
    return np.array(out)


def test_pool_matches_brute_force_overlap_and_hca():
    rng = np.random.default_rng(10)
    T, c, m = 24, 5, 4
    A = [rng.standard_normal((T, c)) for _ in range(4)]
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    np.testing.assert_allclose(O.pool(A[0], A[1], Ba, m, A[2], A[3], Bb),
                               brute_pool(A[0], A[1], Ba, m, A[2], A[3], Bb), rtol=1e-12, atol=1e-12)
    B8 = rng.standard_normal((8, c))
    np.testing.assert_allclose(O.pool(A[0], A[1], B8, 8), brute_pool(A[0], A[1], B8, 8),
                               rtol=1e-12, atol=1e-12)


def test_pool_uniform_logits_is_mean():
    """Uniform logits: entry i > 0 is the mean of its 2m candidates, entry 0 of m."""
    rng = np.random.default_rng(11)
    T, c, m = 16, 3, 4
    Ca, Cb = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    Z = np.full((T, c), 0.7)
    E = O.pool(Ca, Z, np.zeros((m, c)), m, Cb, Z, np.zeros((m, c)))
    np.testing.assert_allclose(E[0], Ca[0:4].mean(0), rtol=1e-13)
    for i in range(1, T // m):
        want = (Ca[4 * i:4 * i + 4].sum(0) + Cb[4 * i - 4:4 * i].sum(0)) / 8
        np.testing.assert_allclose(E[i], want, rtol=1e-13)


def test_pool_page_mean_example():
    """The page's lossy mean example: [1, 9] and [5, 5] both pool to 5."""
    g = golden()["mean_pool_example"]
    for blk in g["blocks"]:
        C = np.array(blk, dtype=float)[:, None]
        E = O.pool(C, np.zeros_like(C), np.zeros((2, 1)), 2)
        assert E[0, 0] == g["value"], g["cite"]


def test_pool_b_series_reads_preceding_block():
    """C_a = 0 and C_b[t] = t with uniform logits: entry i > 0 is the mean of the
    four zeros and of the preceding block's positions 4i-4..4i-1, i.e. (16i-10)/8."""
    T, m = 20, 4
    t = np.arange(T, dtype=float)[:, None]
    E = O.pool(np.zeros((T, 1)), np.zeros((T, 1)), np.zeros((m, 1)), m,
               t, np.zeros((T, 1)), np.zeros((m, 1)))
    assert E[0, 0] == 0.0
    for i in range(1, T // m):
        assert abs(E[i, 0] - (16 * i - 10) / 8) < 1e-13


def test_pool_bias_picks_in_block_offset_and_channel():
    """A dominant bias at in-block offset u (per channel) copies that candidate:
    channel 0 favours offset 2 of the own block, channel 1 offset 1 of the
    preceding block."""
    T, m = 16, 4
    t = np.arange(T, dtype=float)
    Ca = np.stack([t, t], 1)
    Cb = np.stack([-t, -t], 1)
    Ba = np.zeros((m, 2)); Bb = np.zeros((m, 2))
    Ba[2, 0] = 800.0
    Bb[1, 1] = 800.0
    E = O.pool(Ca, np.zeros((T, 2)), Ba, m, Cb, np.zeros((T, 2)), Bb)
    for i in range(T // m):
        assert E[i, 0] == 4 * i + 2
        if i > 0:
            assert E[i, 1] == -(4 * (i - 1) + 1)


def test_pool_identity_for_m1():
    rng = np.random.default_rng(12)
    C = rng.standard_normal((7, 4))
    np.testing.assert_array_equal(O.pool(C, rng.standard_normal((7, 4)), np.zeros((1, 4)), 1), C)


def test_pool_is_per_channel_softmax():
    """With channel-dependent logits the weights differ per channel: the result
    differs from pooling with the channel-0 weights applied to all channels."""
    rng = np.random.default_rng(13)
    Ca, Za = rng.standard_normal((8, 2)), rng.standard_normal((8, 2)) * 3
    E = O.pool(Ca, Za, np.zeros((4, 2)), 4)
    w0 = np.exp(Za[:4, 0] - Za[:4, 0].max()); w0 /= w0.sum()
    assert abs(E[0, 1] - (w0 * Ca[:4, 1]).sum()) > 1e-3


# ============================================================ RMSNorm / RoPE
def test_rms_norm_closed_forms():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((10, 64)) * 5
    y = O.rms_norm(x, None, 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-13)
    a = 0.01
    y = O.rms_norm(np.full((1, 8), a), np.full(8, 2.0), 1e-6)
    np.testing.assert_allclose(y, 2 * a / math.sqrt(a * a + 1e-6), rtol=1e-13)


def test_rope_is_textbook_rotation():
    """d_r = 4 on a 6-dim vector: dims 0-1 untouched; pair (2,3) rotated by
    p*theta^0, pair (4,5) by p*theta^(-1/2) (= p/100 for theta = 1e4)."""
    x = np.array([[1.0, 2.0, 3.0, 4.0, 5.0, 6.0]])
    p = 7
    y = O.rope(x, np.array([p]), 4)
    R = lambda a: np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
    np.testing.assert_array_equal(y[0, :2], x[0, :2])
    np.testing.assert_allclose(y[0, 2:4], R(p * 1.0) @ x[0, 2:4], rtol=1e-13)
    np.testing.assert_allclose(y[0, 4:6], R(p / 100.0) @ x[0, 4:6], rtol=1e-13)


def test_rope_norm_inverse_and_composition():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 64))
    p = rng.integers(0, 1 << 20, 5)
    y = O.rope(x, p, 16)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_allclose(O.rope(y, -p, 16), x, atol=1e-9)
    np.testing.assert_allclose(O.rope(O.rope(x, p, 16), 3 * p, 16), O.rope(x, 4 * p, 16), atol=1e-8)


# ============================================================ indexer / top-k
def test_index_scores_brute_force():
    rng = np.random.default_rng(30)
    nI, cI, N = 3, 5, 9
    q, w, k = rng.standard_normal((nI, cI)), rng.standard_normal(nI), rng.standard_normal((N, cI))
    want = []
    for s in range(7):
        tot = 0.0
        for h in range(nI):
            d = sum(q[h, j] * k[s, j] for j in range(cI))
            tot += w[h] * (d if d > 0 else 0.0)
        want.append(tot)
    np.testing.assert_allclose(O.index_scores(q, w, k, 7), want, rtol=1e-12, atol=1e-14)


def test_index_scores_special_cases_and_causality():
    rng = np.random.default_rng(31)
    q, k = rng.standard_normal((1, 6)), rng.standard_normal((10, 6))
    np.testing.assert_allclose(O.index_scores(q, np.ones(1), k, 10),
                               np.maximum(k @ q[0], 0), rtol=1e-13)
    # every dot product negative -> every score is 0 (a full tie)
    kneg = -np.abs(rng.standard_normal((10, 6)))
    assert np.all(O.index_scores(np.abs(q), np.ones(1), kneg, 10) == 0)
    S, nv = O.index_scores_batch(rng.standard_normal((4, 2, 6)), rng.standard_normal((4, 2)),
                                 k, np.array([2, 3, 7, 8]), 4)
    assert nv.tolist() == [0, 1, 2, 2]
    assert np.all(np.isinf(S[0])) and np.isfinite(S[1, 0]) and np.all(np.isinf(S[1, 1:]))


def brute_topk(scores, n, k):
    order = sorted(range(n), key=lambda s: (-scores[s], s))[:k]
    return sorted(order) + [-1] * (k - min(k, n))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(32)
    for trial in range(200):
        n = int(rng.integers(0, 40))
        k = int(rng.integers(1, 20))
        s = rng.integers(-3, 4, size=max(n, 1)).astype(float)   # many ties
        assert O.topk(s, n, k).tolist() == brute_topk(list(s), n, k)


def test_topk_tie_goes_to_lower_index():
    assert O.topk(np.zeros(10), 10, 3).tolist() == [0, 1, 2]
    assert O.topk(np.array([1.0, 5, 5, 5, 0]), 5, 2).tolist() == [1, 2]
    assert O.topk(np.array([1.0, 2.0]), 2, 4).tolist() == [0, 1, -1, -1]


# ============================================================ attention (Eqs 18-19, 27)
def test_single_row_with_sink_closed_form():
    """One row x, logit l = tau q.x: o = x e^l / (e^l + e^z'); the sink is not
    scaled by tau."""
    rng = np.random.default_rng(40)
    q, x = rng.standard_normal((2, 8)), rng.standard_normal((1, 8))
    z = np.array([0.3, -1.2])
    tau = 0.37
    o = O.attend_rows(q, x, z, tau)
    l = tau * (q @ x[0])
    np.testing.assert_allclose(o, (np.exp(l) / (np.exp(l) + np.exp(z)))[:, None] * x[0], rtol=1e-13)


def test_huge_sink_drives_output_to_zero():
    rng = np.random.default_rng(41)
    q, X = rng.standard_normal((3, 16)), rng.standard_normal((20, 16))
    o = O.attend_rows(q, X, np.full(3, 200.0), 0.25)
    assert np.abs(o).max() < 1e-60


def test_window_only_matches_torch_sdpa():
    """sink -> -inf, no compressed entries, no RoPE: textbook causal MQA over a
    sliding window with K = V, checked against torch's SDPA in fp64."""
    rng = np.random.default_rng(42)
    T, nh, c, n_win = 40, 3, 8, 6
    R = rng.standard_normal((T, c))
    qr = rng.standard_normal((T, nh, c))
    tau = 1 / math.sqrt(c)
    got = O.sparse_attend(qr, None, 1e-6, 0, 1e4, np.arange(T), np.zeros((1, c)),
                          np.full((T, 1), -1), R, n_win, T, np.full(nh, -1e300), tau)
    qn = O.rms_norm(qr)
    mask = np.zeros((T, T), dtype=bool)
    for p in range(T):
        mask[p, max(0, p - n_win + 1):p + 1] = True
    Q = torch.from_numpy(qn.transpose(1, 0, 2))                     # [nh, T, c]
    K = torch.from_numpy(R)[None].expand(nh, T, c)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, K, attn_mask=torch.from_numpy(mask), scale=tau).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def _tiny_stream(rng, T=64, d=12, c=8, cI=4, d_r=4):
    return dict(
        H=rng.standard_normal((T, d)),
        W=[rng.standard_normal((d, c)) / math.sqrt(d) for _ in range(5)],
        WI=[rng.standard_normal((d, cI)) / math.sqrt(d) for _ in range(4)],
        Ba=rng.standard_normal((4, c)) * 0.3, Bb=rng.standard_normal((4, c)) * 0.3,
        BIa=rng.standard_normal((4, cI)) * 0.3, BIb=rng.standard_normal((4, cI)) * 0.3,
        q=rng.standard_normal((T, 3, c)), qI=rng.standard_normal((T, 2, cI)),
        w=rng.standard_normal((T, 2)), sink=rng.standard_normal(3), c=c, d_r=d_r)


def _pipeline(s, k, n_win=8, pos_shift=0):
    """Whole CSA layer on one sequence with the oracle's stage functions."""
    T = s["H"].shape[0]
    c, d_r = s["c"], s["d_r"]
    W = s["W"]
    kv = O.compress(s["H"], W[0], W[1], s["Ba"], 4, W[2], W[3], s["Bb"], None, 1e-6, d_r,
                    1e4, 4, pos_shift)
    kI = O.compress(s["H"], *s["WI"][:2], s["BIa"], 4, *s["WI"][2:], s["BIb"], normalize=False)
    win = O.compress(s["H"], W[4], None, None, 1, d_r=d_r, pos_stride=1, pos_offset=pos_shift)
    qpos = np.arange(T)
    S, nv = O.index_scores_batch(s["qI"], s["w"], kI, qpos, 4)
    idx = np.stack([O.topk(S[t], int(nv[t]), k) for t in range(T)])
    out = O.sparse_attend(s["q"], None, 1e-6, d_r, 1e4, qpos + pos_shift, kv, idx, win,
                          n_win, T, s["sink"], 1 / math.sqrt(c))
    return out, idx, kv, win


def test_causality_future_tokens_do_not_leak():
    """Changing tokens after q must leave o(q) unchanged for the boundary
    positions 3, 4, 7, 8; changing a token at or before q must change it."""
    rng = np.random.default_rng(50)
    s = _tiny_stream(rng)
    base, _, _, _ = _pipeline(s, k=2)
    for q in (3, 4, 7, 8):
        s2 = {**s, "H": s["H"].copy()}
        s2["H"][q + 1:] += rng.standard_normal(s2["H"][q + 1:].shape)
        out2, _, _, _ = _pipeline(s2, k=2)
        np.testing.assert_array_equal(out2[:q + 1], base[:q + 1])
        s3 = {**s, "H": s["H"].copy()}
        s3["H"][q] += 1.0
        out3, _, _, _ = _pipeline(s3, k=2)
        assert np.abs(out3[q] - base[q]).max() > 1e-6


def test_shift_invariance_of_positions():
    """Shifting every position (query and rows) by the same amount leaves the
    output unchanged: RoPE makes the logits depend on differences only and the
    output is rotated back by -q."""
    rng = np.random.default_rng(51)
    c, d_r = 16, 8
    Xn = O.rms_norm(rng.standard_normal((30, c)))
    pos = rng.integers(0, 500, 30)
    qr = rng.standard_normal((4, c))
    z = rng.standard_normal(4)
    for delta in (1, 777, 123457):
        a = O.attend_query(qr, None, 1e-6, d_r, 1e4, 500, O.rope(Xn, pos, d_r), z, 0.25)
        b = O.attend_query(qr, None, 1e-6, d_r, 1e4, 500 + delta, O.rope(Xn, pos + delta, d_r),
                           z, 0.25)
        np.testing.assert_allclose(a, b, atol=1e-9)
    # whole layer: every position shifted by a multiple of the window array
    # length keeps the ring slots; queries past the first window are unaffected
    s = _tiny_stream(rng)
    T = s["H"].shape[0]
    a, _, _, _ = _pipeline(s, k=3)
    b, _, _, _ = _pipeline(s, k=3, pos_shift=193 * T)
    np.testing.assert_allclose(a[7:], b[7:], atol=1e-9)


def test_topk_at_least_visible_equals_dense():
    """k >= N(q): CSA reads every visible entry, the same as dense (HCA-style)
    attention over the same entries."""
    rng = np.random.default_rng(52)
    s = _tiny_stream(rng)
    T = s["H"].shape[0]
    out, idx, kv, win = _pipeline(s, k=T // 4)
    dense = O.dense_attend(s["q"], None, 1e-6, s["d_r"], 1e4, np.arange(T), kv, 4, win, 8, T,
                           s["sink"], 1 / math.sqrt(s["c"]))
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-13)


def test_shared_softmax_differs_from_per_branch_sum():
    """Normalising the compressed and the window branch separately and adding
    is not the shared softmax."""
    rng = np.random.default_rng(53)
    q = rng.standard_normal((2, 8))
    Xc, Xw = rng.standard_normal((5, 8)), rng.standard_normal((4, 8))
    z = np.array([0.1, 0.2])
    shared = O.attend_rows(q, np.concatenate([Xc, Xw]), z, 0.5)
    split = O.attend_rows(q, Xc, z, 0.5) + O.attend_rows(q, Xw, z, 0.5)
    assert np.abs(shared - split).max() > 1e-2


def test_window_includes_current_token_only_at_q0():
    rng = np.random.default_rng(54)
    R = rng.standard_normal((3, 4))
    assert O.gather_rows(np.zeros((1, 4)), [-1], R, 0, 128, 3).shape[0] == 1
    np.testing.assert_array_equal(O.gather_rows(np.zeros((1, 4)), [-1], R, 0, 128, 3)[0], R[0])
    # ring buffer: position 130 in a ring of 128 lives at slot 2
    ring = rng.standard_normal((128, 4))
    rows = O.gather_rows(np.zeros((1, 4)), [-1], ring, 130, 128, 128)
    assert rows.shape[0] == 128 and np.array_equal(rows[-1], ring[2])


# =================================================================== grouped output projection
def _oproj_case(rng, R=3, nh=8, c=6, g=4, d_g=5, d=7):
    o = rng.standard_normal((R, nh, c))
    W_a = rng.standard_normal((g, d_g, nh // g * c))
    W_b = rng.standard_normal((d, g * d_g))
    return o, W_a, W_b


def test_grouped_out_proj_is_a_block_diagonal_map():
    """The grouped projection is the block-diagonal matrix of the group
    projections (scipy's block_diag) applied to the flattened heads, then W_b:
    a transposed operand, a wrong flattening or a wrong group order fails."""
    from scipy.linalg import block_diag
    rng = np.random.default_rng(71)
    for shape in [dict(), dict(nh=6, g=3, c=4, d_g=2, d=5), dict(nh=4, g=1, c=3, d_g=6, d=2),
                  dict(nh=4, g=4, c=2, d_g=3, d=3)]:
        o, W_a, W_b = _oproj_case(rng, **shape)
        y, u = O.grouped_out_proj(o, W_a, W_b)
        R = o.shape[0]
        BD = block_diag(*W_a)                       # [g*d_g, nh*c]
        np.testing.assert_allclose(u, o.reshape(R, -1) @ BD.T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y, (o.reshape(R, -1) @ BD.T) @ W_b.T, rtol=1e-12, atol=1e-12)


def test_grouped_out_proj_groups_are_consecutive_heads():
    """Perturbing head h changes only u's block h // (nh/g)."""
    rng = np.random.default_rng(72)
    o, W_a, W_b = _oproj_case(rng)
    nh, g, d_g = o.shape[1], W_a.shape[0], W_a.shape[1]
    _, u0 = O.grouped_out_proj(o, W_a, W_b)
    for h in range(nh):
        o2 = o.copy()
        o2[:, h, :] += 1.0
        _, u2 = O.grouped_out_proj(o2, W_a, W_b)
        changed = [bool(np.any(u2[:, j * d_g:(j + 1) * d_g] != u0[:, j * d_g:(j + 1) * d_g]))
                   for j in range(g)]
        assert changed == [j == h // (nh // g) for j in range(g)], h


def test_grouped_out_proj_rounding_hook_and_shapes():
    """round_u acts on u only (bf16 keeps 8 significant bits, so rounding moves
    each u by at most 2^-8 |u| and y by at most 2^-8 |u| . |W_b|);
    inconsistent shapes are rejected."""
    import torch
    rng = np.random.default_rng(73)
    o, W_a, W_b = _oproj_case(rng, R=4, nh=8, c=16, g=2, d_g=32, d=9)
    y, u = O.grouped_out_proj(o, W_a, W_b)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    yb, ub = O.grouped_out_proj(o, W_a, W_b, round_u=bf)
    assert np.all(np.abs(ub - u) <= 2.0 ** -8 * np.abs(u))
    assert np.all(np.abs(yb - y) <= 2.0 ** -8 * (np.abs(u) @ np.abs(W_b).T) + 1e-12)
    with pytest.raises(ValueError):
        O.grouped_out_proj(o, W_a[:, :, :-1], W_b)
    with pytest.raises(ValueError):
        O.grouped_out_proj(o[:, :7], W_a, W_b)
