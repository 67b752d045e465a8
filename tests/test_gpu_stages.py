"""Stage-by-stage parity of the HIP path against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.
Every call goes through the C ABI (ctypes binding); both sides consume the same
seeded raw inputs and each side does its own normalisation, RoPE and encoding."""
import math

import numpy as np
import pytest
import torch

import csa_inputs as I
import long_context_sparse_10_amd as L
from long_context_sparse_10_amd import pipeline as G
from oracle import csa as O
from oracle import formats as F
from oracle import pipeline as OP
from tests.gpu_util import (bf16_ulp, check_decode_attention, decode_rows, dev, e4m3_ulp,
                            mx_score_bound, np64, report, score_error_bound)

pytestmark = pytest.mark.gpu


# =================================================================== row encoder
@pytest.mark.parametrize("c,d_r", [(512, 64), (64, 16)])
def test_prep_rows_norm_rope_formats(c, d_r):
    d = dev()
    rng = np.random.default_rng(100)
    rows = 777
    raw = rng.standard_normal((rows, c), dtype=np.float32) * 3
    pos = rng.integers(0, 1 << 20, rows).astype(np.int32)
    ref = O.rope(O.rms_norm(raw, None, 1e-6), pos, d_r)
    x = torch.from_numpy(raw).to(d)
    p = torch.from_numpy(pos).to(d)
    g = torch.ones(c, device=d)
    fmts = [L.F32, L.BF16] + ([L.FP8MIX] if c == 512 else [])
    for fmt in fmts:
        out, _ = G.encode_rows(x, fmt, rows, c, norm_w=g, d_r=d_r, pos=p)
        torch.cuda.synchronize()
        got = decode_rows(out, fmt, rows, c, d_r)
        if fmt == L.F32:
            err = np.abs(got - ref).max()
            report("prep f32", c=c, max_abs=err)
            assert err < 2e-5
            continue
        want = OP.store(ref, "bf16" if fmt == L.BF16 else "fp8mix", d_r)
        ulp = bf16_ulp(ref) if fmt == L.BF16 else np.concatenate(
            [e4m3_ulp(ref[:, : c - d_r]), bf16_ulp(ref[:, c - d_r:])], 1)
        mism = got != want
        report("prep", fmt=fmt, c=c, mismatches=int(mism.sum()), of=got.size)
        # a stored value may differ from the oracle's only by one step, and only
        # where the exact value sits within fp32 error of a rounding midpoint
        assert np.all(np.abs(got - ref) <= ulp * 0.5 + 1e-5 * np.abs(ref) + 1e-12)
        assert mism.mean() < 1e-3


def test_prep_rows_mxfp4_bit_exact():
    """Pure MXFP4 encoding of fp32 values is byte work: codes and scales must be
    bit-identical to the oracle's quantiser."""
    d = dev()
    rng = np.random.default_rng(101)
    rows, c = 1000, 128
    raw = rng.standard_normal((rows, c), dtype=np.float32)
    raw[3] = 0.0                                     # all-zero blocks
    raw[4, :32] = np.float32(6.0)                   # exact grid values
    raw[5, :32] = rng.standard_normal(32).astype(np.float32) * 1e-30
    out, sc = G.encode_rows(torch.from_numpy(raw).to(d), L.MXFP4, rows, c)
    packed, scales = F.mxfp4_quantize(raw.astype(np.float64))
    np.testing.assert_array_equal(out.cpu().numpy().reshape(rows, c // 2), packed)
    np.testing.assert_array_equal(sc.cpu().numpy().reshape(rows, c // 32), scales)


# =================================================================== compressor
@pytest.mark.parametrize("name", ["tiny_csa", "tiny_hca"])
def test_compress_tiny_f32(name):
    d = dev()
    sp = I.CONFIGS[name]
    inp = I.prefill_inputs(sp)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    torch.cuda.synchronize()
    ref = OP.prefill_caches(inp)
    n = sp.T // sp.m
    kv = decode_rows(p.kv, L.F32, n, sp.c, sp.d_r)
    win = decode_rows(p.win, L.F32, sp.T, sp.c, sp.d_r)
    e1, e2 = np.abs(kv - ref["kv"]).max(), np.abs(win - ref["win"]).max()
    report("compress", cfg=name, kv=e1, win=e2)
    assert e1 <= 1e-5 and e2 <= 1e-5
    if sp.nI:
        kI = decode_rows(p.kI, L.F32, n, sp.cI, 0)
        e3 = np.abs(kI - ref["kI"]).max()
        report("compress", cfg=name, index_keys=e3)
        assert e3 <= 1e-5


def test_compress_bf16_mfma_gemm():
    """bf16 hidden / weights (the prefill workload's dims, shorter sequence):
    the MFMA projection + pooling + norm + RoPE.  Stored bf16 the entries must
    sit within the bf16 bar (max-abs 2e-2) of the exact fp64 values; stored fp32
    the same kernels must agree to fp32-accumulation accuracy."""
    d = dev()
    sp = I.CONFIGS["prefill_32k"]
    T = 520                                            # 130 entries, ragged vs 128-row tiles
    inp = I.prefill_inputs(sp, T=T, queries=np.arange(4))
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    torch.cuda.synchronize()
    ref = OP.prefill_caches(inp)
    n = T // 4
    kv = decode_rows(p.kv, L.BF16, n, sp.c, sp.d_r)
    exact = O.compress(inp["H"], inp["W_kv_a"], inp["W_z_a"], inp["bias_a"], 4, inp["W_kv_b"],
                       inp["W_z_b"], inp["bias_b"], None, 1e-6, sp.d_r, 1e4, 4, 0)
    err = np.abs(kv - exact)
    mism = float((kv != ref["kv"]).mean())
    report("compress bf16", max_abs=err.max(), mism=mism)
    assert err.max() <= 2e-2 and mism < 1e-2
    kI = decode_rows(p.kI, L.BF16, n, sp.cI, 0)
    assert np.abs(kI - ref["kI_exact"]).max() <= 2e-2
    win = decode_rows(p.win, L.BF16, T, sp.c, sp.d_r)
    assert np.abs(win - ref["win"]).max() <= 2e-2
    # fp32 output of the same bf16 inputs isolates the kernels' own arithmetic
    out32 = torch.empty(n * sp.c * 4, dtype=torch.uint8, device=d)
    W = p.W
    L.csa_compress(p.H, L.BF16, 1, T, sp.d, W["W_kv_a"], W["W_z_a"], W["W_kv_b"], W["W_z_b"],
                   W["bias_a"], W["bias_b"], 4, 1, sp.c, p.gamma, 1e-6, sp.d_r, 1e4, 4, 0, out32,
                   None, L.F32)
    torch.cuda.synchronize()
    e32 = np.abs(decode_rows(out32, L.F32, n, sp.c, sp.d_r) - exact).max()
    report("compress bf16->f32", max_abs=e32)
    assert e32 <= 2e-3


# =================================================================== indexer
def _decode_small(name, B, lengths, seed):
    sp = I.CONFIGS[name].replace(B=B)
    return I.decode_inputs(sp, seed=seed, lengths=lengths)


@pytest.mark.parametrize("lengths", [[4100, 2051, 8191], [64, 3, 4099]])
def test_indexer_bf16_mfma(lengths):
    d = dev()
    inp = _decode_small("decode_64k", len(lengths), lengths, 200)
    g = G.upload_decode(inp, d)
    g.scores.fill_(float("nan"))
    G.decode_indexer(g)
    torch.cuda.synchronize()
    S = np64(g.scores)
    for b in range(len(lengths)):
        ref, nv = OP.decode_scores(inp, b)
        bound = score_error_bound(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv)
        err = np.abs(S[b, 0, :nv] - ref)
        report("indexer bf16", b=b, nv=nv, max_err=err.max() if nv else 0)
        assert np.all(err <= bound + 1e-30)
        assert np.all(np.isnan(S[b, 0, nv:]))          # invisible entries untouched


def test_indexer_mxfp4_matches_quantized_oracle():
    d = dev()
    inp = _decode_small("decode_1m_fp4", 2, [4 * 3000 + 3, 4 * 777], 201)
    g = G.upload_decode(inp, d)
    G.decode_indexer(g)
    torch.cuda.synchronize()
    S = np64(g.scores)
    # the encoded keys are byte-identical to the oracle's quantiser
    packed, scales = F.mxfp4_quantize(inp["kI"].astype(np.float64))
    Nm = inp["Nmax"]
    np.testing.assert_array_equal(g.kI.cpu().numpy().reshape(2, Nm, 64), packed)
    np.testing.assert_array_equal(g.kI_scale.cpu().numpy().reshape(2, Nm, 4), scales)
    for b in range(2):
        ref, nv = OP.decode_scores(inp, b)          # quantised fp64 scores, rounded to bf16
        err = np.abs(S[b, 0, :nv] - ref)
        ulp = bf16_ulp(ref)
        report("indexer mxfp4", b=b, nv=nv, ulps=float((err / ulp).max()) if nv else 0.0,
               exact=float(np.mean(err == 0)) if nv else 1.0)
        assert np.all(err <= mx_score_bound(inp, b, ref, nv) + 1e-30)


@pytest.mark.parametrize("name", ["decode_64k", "decode_1m_fp4"])
def test_indexer_decode_step_boundaries(name):
    """Visible counts on both sides of the decode kernel's step boundaries (bf16
    steps of 128 entries per block of 4 waves, MXFP4 256; whole triples of steps,
    then a last one or two): every row is scored to the oracle's bound and the
    entries past its count stay untouched."""
    d = dev()
    nvs = [1, 15, 16, 17, 127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 512, 640, 767,
           768, 769, 1023, 1024, 1025, 1537, 2049]
    inp = _decode_small(name, len(nvs), [4 * n for n in nvs], 202)
    g = G.upload_decode(inp, d)
    g.scores.fill_(float("nan"))
    G.decode_indexer(g)
    torch.cuda.synchronize()
    S = np64(g.scores)
    for b, n in enumerate(nvs):
        ref, nv = OP.decode_scores(inp, b)
        assert nv == n
        err = np.abs(S[b, 0, :nv] - ref)
        if name == "decode_64k":
            bound = score_error_bound(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv)
        else:
            bound = mx_score_bound(inp, b, ref, nv)
        assert np.all(err <= bound + 1e-30), (name, nv)
        assert np.all(np.isnan(S[b, 0, nv:])), (name, nv)   # invisible entries untouched
    report("indexer step boundaries", cfg=name, rows=len(nvs))


@pytest.mark.parametrize("Tq,offset", [(1031, 0), (37, 4093), (9, 4093)])
def test_indexer_bf16_query_rows(Tq, offset):
    """Many query rows per sequence (the prefill kernel: a block of rows shares
    the keys through LDS): two sequences of different lengths, causal
    positions starting at ``offset``, a ragged last row group; every visible
    score within the fp32 bound, everything beyond N(q) untouched."""
    d = dev()
    rng = np.random.default_rng(Tq + offset)
    B, nI, cI, m = 2, 64, 128, 4
    N = (offset + Tq) // m + 3
    kI = I.cast(rng.standard_normal((B, N, cI)).astype(np.float32), "bf16")
    qI = I.cast(rng.standard_normal((B, Tq, nI, cI)).astype(np.float32), "bf16")
    w = rng.standard_normal((B, Tq, nI)).astype(np.float32)
    q_pos = (offset + np.arange(Tq, dtype=np.int32))[None].repeat(B, 0)
    n_ent = np.array([N, N - 5], np.int32)
    scores = torch.full((B, Tq, N), float("nan"), device=d)
    L.indexer_score(torch.from_numpy(qI).to(d).to(torch.bfloat16), None, L.BF16,
                    torch.from_numpy(w).to(d), torch.from_numpy(kI).to(d).to(torch.bfloat16), None,
                    L.BF16, torch.from_numpy(q_pos).to(d), torch.from_numpy(n_ent).to(d), B, Tq,
                    nI, cI, N, m, scores, L.F32)
    torch.cuda.synchronize()
    S = np64(scores)
    worst = 0.0
    for b in range(B):
        for t in list(range(0, Tq, 5)) + [Tq - 1]:
            nv = int(O.n_visible(int(q_pos[b, t]), m, int(n_ent[b])))
            want = O.index_scores(qI[b, t].astype(np.float64), w[b, t].astype(np.float64),
                                  kI[b].astype(np.float64), nv)
            bound = score_error_bound(qI[b, t].astype(np.float64), w[b, t].astype(np.float64),
                                      kI[b].astype(np.float64), nv)
            assert np.all(np.abs(S[b, t, :nv] - want) <= bound + 1e-6), (b, t)
            assert np.all(np.isnan(S[b, t, nv:])), (b, t)
            if nv:
                worst = max(worst, float(np.abs(S[b, t, :nv] - want).max()))
    report("indexer bf16 query rows", Tq=Tq, max_err=worst)


@pytest.mark.parametrize("Tq,offset", [(1031, 0), (37, 4093)])
def test_indexer_mxfp4_query_rows(Tq, offset):
    """MXFP4 keys and queries with many query rows per sequence (the prefill
    form of the block-scaled fp4 indexer): every visible bf16 score within one
    bf16 step plus the fp32 accumulation bound of the quantised oracle (same
    E2M1 values and scales in fp64, then bf16); beyond N(q) untouched."""
    d = dev()
    rng = np.random.default_rng(3 * Tq + offset)
    B, nI, cI, m = 2, 64, 128, 4
    N = (offset + Tq) // m + 3
    kraw = rng.standard_normal((B, N, cI)).astype(np.float32)
    qraw = rng.standard_normal((B, Tq, nI, cI)).astype(np.float32)
    w = rng.standard_normal((B, Tq, nI)).astype(np.float32)
    q_pos = (offset + np.arange(Tq, dtype=np.int32))[None].repeat(B, 0)
    n_ent = np.array([N, N - 5], np.int32)
    kI, kS = G.encode_rows(torch.from_numpy(kraw).to(d), L.MXFP4, B * N, cI)
    qI, qS = G.encode_rows(torch.from_numpy(qraw).to(d), L.MXFP4, B * Tq * nI, cI)
    scores = torch.full((B, Tq, N), float("nan"), dtype=torch.bfloat16, device=d)
    L.indexer_score(qI, qS, L.MXFP4, torch.from_numpy(w).to(d), kI, kS, L.MXFP4,
                    torch.from_numpy(q_pos).to(d), torch.from_numpy(n_ent).to(d), B, Tq, nI, cI,
                    N, m, scores, L.BF16)
    torch.cuda.synchronize()
    S = np64(scores)
    worst_ulps = 0.0
    for b in range(B):
        kq, _, _ = OP.mxfp4_values(kraw[b].astype(np.float64))
        for t in list(range(0, Tq, 7)) + [Tq - 1]:
            nv = int(O.n_visible(int(q_pos[b, t]), m, int(n_ent[b])))
            qq, _, _ = OP.mxfp4_values(qraw[b, t].astype(np.float64))
            ref = F.bf16_round(O.index_scores(qq, w[b, t].astype(np.float64), kq, nv))
            err = np.abs(S[b, t, :nv] - ref)
            # fp32 accumulation error of the exact E2M1 products, plus one bf16
            # step (the two sides may round to neighbouring bf16 values)
            e = score_error_bound(qq, w[b, t].astype(np.float64), kq, nv)
            assert np.all(err <= bf16_ulp(np.abs(ref) + e) + e + 1e-30), (b, t)
            assert np.all(np.isnan(S[b, t, nv:])), (b, t)
            if nv:
                worst_ulps = max(worst_ulps, float((err / bf16_ulp(ref)).max()))
    report("indexer mxfp4 query rows", Tq=Tq, max_ulps=worst_ulps)


def test_indexer_generic_f32_and_causal_prefill():
    d = dev()
    sp = I.CONFIGS["tiny_csa"]
    inp = I.prefill_inputs(sp)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    n = sp.T // 4
    scores = torch.full((1, sp.T, n), float("nan"), device=d)
    L.indexer_score(p.qI, None, L.F32, p.w, p.kI, None, L.F32, p.q_pos, p.n_entries, 1, sp.T,
                    sp.nI, sp.cI, n, 4, scores, L.F32)
    torch.cuda.synchronize()
    S = np64(scores)[0]
    ref = OP.prefill_caches(inp)
    worst = 0.0
    for t in range(0, sp.T, 7):
        nv = (t + 1) // 4
        want = O.index_scores(inp["qI"][t], inp["w"][t], ref["kI"], nv)
        bound = score_error_bound(inp["qI"][t], inp["w"][t], ref["kI"], nv, rel=1e-4)
        assert np.all(np.abs(S[t, :nv] - want) <= bound + 1e-5)
        assert np.all(np.isnan(S[t, nv:]))
        if nv:
            worst = max(worst, float(np.abs(S[t, :nv] - want).max()))
    report("indexer f32 causal", max_err=worst)


# =================================================================== top-k
def _score_rows(rng, kind, rows, N):
    if kind == "ties":
        return rng.integers(-4, 5, size=(rows, N)).astype(np.float32)
    if kind == "ties81":  # a few hundred tied candidates per row
        return rng.integers(-40, 41, size=(rows, N)).astype(np.float32)
    if kind == "ties5":   # thousands of candidates: past the compaction buffer
        return rng.integers(-2, 3, size=(rows, N)).astype(np.float32)
    if kind == "bf16":
        return I.cast(rng.standard_normal((rows, N)).astype(np.float32) * 0.5, "bf16")
    if kind == "bf16ties":  # integers, exact in bf16: equal keys across many slices
        return rng.integers(-40, 41, size=(rows, N)).astype(np.float32)
    if kind == "bf16ties5":  # tens of thousands of equal keys in one row
        return rng.integers(-2, 3, size=(rows, N)).astype(np.float32)
    if kind == "bf16wide":  # magnitudes 2^-120 .. 2^120, both signs: thousands of distinct keys
        mag = np.exp2(rng.uniform(-120, 120, size=(rows, N)))
        return I.cast((np.where(rng.random((rows, N)) < 0.5, -mag, mag)).astype(np.float32), "bf16")
    return rng.standard_normal((rows, N)).astype(np.float32)


@pytest.mark.parametrize("kind", ["ties", "ties81", "ties5", "bf16", "bf16ties", "bf16ties5", "bf16wide",
                                  "normal"])
@pytest.mark.parametrize("N,k,m", [(16384, 1024, 4), (3000, 1024, 4), (700, 32, 4),
                                   (1025, 1024, 4), (40000, 512, 4), (20001, 100, 4),
                                   (262144, 1024, 4)])
def test_topk_bit_exact(kind, N, k, m):
    """Same score arrays (from the seeded generator) on both sides: the index
    sets are integer results and must be identical, ties included."""
    d = dev()
    rng = np.random.default_rng(N + k)
    rows = 6
    S = _score_rows(rng, kind, rows, N)
    # query positions: full, ragged, tiny (N(q) <= k), empty
    qpos = np.array([4 * N - 1, 4 * N - 3, 4 * (N // 3) + 2, 4 * k + 1, 4 * k + 7, 2], np.int32)
    n_ent = np.full(rows, N, np.int32)
    fmt = L.BF16 if kind.startswith("bf16") else L.F32
    dt = torch.bfloat16 if fmt == L.BF16 else torch.float32
    st = torch.from_numpy(S).to(d).to(dt).reshape(rows, 1, N)
    idx = torch.empty(rows, 1, k, dtype=torch.int32, device=d)
    # rows over 16384 entries take the multi-block path (workspace); the odd
    # length exercises the unaligned key loads
    L.topk_select(st, fmt, torch.from_numpy(qpos).reshape(rows, 1).to(d),
                  torch.from_numpy(n_ent).to(d), rows, 1, N, m, k, idx)
    got = idx.cpu().numpy()[:, 0]
    for r in range(rows):
        nv = int(O.n_visible(int(qpos[r]), m, N))
        want = O.topk(S[r].astype(np.float64), nv, k)
        np.testing.assert_array_equal(got[r], want, err_msg=f"row {r} nv {nv}")


@pytest.mark.parametrize("N,k,rows", [(262144, 1024, 70),    # more rows than one launch pair takes
                                       (40000, 20000, 3)])     # k above a slice: the per-digit path
def test_topk_long_bf16_rows_bit_exact(N, k, rows):
    d = dev()
    rng = np.random.default_rng(N + k + rows)
    S = _score_rows(rng, "bf16", rows, N)
    m = 4
    qpos = (4 * N - 1 - 4 * rng.integers(0, N, size=rows)).astype(np.int32)
    qpos[:3] = [4 * N - 1, 4 * k - 1, 4 * k + 3]   # full, exactly k, k + 1 visible
    n_ent = np.full(rows, N, np.int32)
    st = torch.from_numpy(S).to(d).to(torch.bfloat16).reshape(rows, 1, N)
    idx = torch.empty(rows, 1, k, dtype=torch.int32, device=d)
    L.topk_select(st, L.BF16, torch.from_numpy(qpos).reshape(rows, 1).to(d),
                  torch.from_numpy(n_ent).to(d), rows, 1, N, m, k, idx)
    got = idx.cpu().numpy()[:, 0]
    for r in range(rows):
        nv = int(O.n_visible(int(qpos[r]), m, N))
        want = O.topk(S[r].astype(np.float64), nv, k)
        np.testing.assert_array_equal(got[r], want, err_msg=f"row {r} nv {nv}")


@pytest.mark.parametrize("kind", ["ties", "ties5", "normal"])
@pytest.mark.parametrize("N,k", [(3000, 1024), (9000, 1024), (700, 32)])
def test_topk_many_rows_bit_exact(kind, N, k):
    """More rows than compute units take the fp32 kernel with a 12-bit first
    digit (four blocks per CU); the index sets must still match the oracle
    exactly, ties and the candidate-buffer overflow included."""
    d = dev()
    m, rows = 4, 300
    rng = np.random.default_rng(7 * N + k)
    S = _score_rows(rng, kind, rows, N)
    qpos = rng.integers(0, 4 * N + 8, size=rows).astype(np.int32)   # ragged, some short
    qpos[:3] = [4 * N - 1, 2, 4 * k + 1]
    n_ent = np.full(rows, N, np.int32)
    st = torch.from_numpy(S).to(d).reshape(rows, 1, N)
    idx = torch.empty(rows, 1, k, dtype=torch.int32, device=d)
    L.topk_select(st, L.F32, torch.from_numpy(qpos).reshape(rows, 1).to(d),
                  torch.from_numpy(n_ent).to(d), rows, 1, N, m, k, idx)
    got = idx.cpu().numpy()[:, 0]
    for r in range(rows):
        nv = int(O.n_visible(int(qpos[r]), m, N))
        want = O.topk(S[r].astype(np.float64), nv, k)
        np.testing.assert_array_equal(got[r], want, err_msg=f"row {r} nv {nv}")


# =================================================================== attention
def _attend_case(name, lengths, seed, holes=0.1, n_win=None):
    sp = I.CONFIGS[name].replace(B=len(lengths))
    if n_win is not None:
        sp = sp.replace(n_win=n_win)
    inp = I.decode_inputs(sp, seed=seed, lengths=lengths)
    rng = np.random.default_rng(seed + 1)
    nv = np.array([O.n_visible(int(inp["q_pos"][b, 0]), sp.m, int(inp["n_entries"][b]))
                   for b in range(sp.B)])
    idx = I.random_index_sets(rng, nv, sp.k, holes=holes) if sp.kind == "decode" else None
    return sp, inp, idx


@pytest.mark.parametrize("name,lengths", [
    ("decode_64k", [4100, 9000, 300]),           # bf16 KV, 64 heads, split path
    ("decode_1m_fp4", [8192 + 5, 5000]),          # FP8/BF16 KV, 128 heads (two head groups)
    ("hca_decode_1m", [128 * 300 + 5, 128 * 40, 100]),  # dense HCA, bf16
])
def test_attend_decode_vs_oracle(name, lengths):
    d = dev()
    sp, inp, idx = _attend_case(name, lengths, 300)
    g = G.upload_decode(inp, d)
    idx_t = torch.from_numpy(idx).reshape(sp.B, 1, sp.k).to(d) if idx is not None else None
    G.decode_attend(g, idx=idx_t)
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend", g, inp, b, idx[b] if idx is not None else None, out[b, 0],
                               cfg=name, b=b)


@pytest.mark.parametrize("k,lengths,holes,qf32", [
    (64, [4100, 9000, 300], 0.1, False),   # 192 slots: one block per row, no split
    (128, [1, 5, 130, 4096], 0.5, False),  # window crossing position 0, half-empty selections
    (100, [4100, 777], 0.0, False),        # k not a multiple of the 32-slot tile
    (100, [4100, 777], 0.0, True),         # fp32 queries: the single-block kernel, unsplit
])
def test_attend_unsplit_rows_vs_oracle(k, lengths, holes, qf32):
    """Slot lists short enough to stay whole (at most 256 slots with one query
    per sequence, or any list of a prefill) take, with bf16 queries, the kernel
    that runs two blocks per compute unit and loads rows straight into shared
    memory."""
    d = dev()
    sp = I.CONFIGS["decode_64k"].replace(B=len(lengths), k=k)
    inp = I.decode_inputs(sp, seed=340 + k, lengths=lengths)
    rng = np.random.default_rng(341 + k)
    nv = np.array([O.n_visible(int(inp["q_pos"][b, 0]), sp.m, int(inp["n_entries"][b]))
                   for b in range(sp.B)])
    idx = I.random_index_sets(rng, nv, k, holes=holes)
    if holes >= 0.5:
        idx[1, :] = -1                      # one sequence with the window only
    g = G.upload_decode(inp, d)
    if qf32:
        g.q = torch.from_numpy(np.ascontiguousarray(inp["q"], dtype=np.float32)).reshape(g.q.shape).to(d)
    G.decode_attend(g, idx=torch.from_numpy(idx).reshape(sp.B, 1, k).to(d))
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend unsplit", g, inp, b, idx[b], out[b, 0], k=k, b=b)


@pytest.mark.parametrize("total", [900, 950, 980, 1000, 1100, 1300, 1700, 2000, 2300, 2700, 3000])
def test_attend_split_tile_counts_vs_oracle(total):
    """Split slot lists (k + 128 window slots = total) whose splits hold 4 to 12
    tiles of 32 slots and whose last split holds 1 to 10: every way through
    the loader ring (phases in pairs while both stages are real tiles, then the
    last phases with their conditions).  The second sequence sees only half of
    k entries, so its selections are half empty."""
    d = dev()
    k = total - 128
    sp = I.CONFIGS["decode_64k"].replace(B=2, k=k)
    inp = I.decode_inputs(sp, seed=360 + total % 97, lengths=[4 * k + 400, 2 * k])
    rng = np.random.default_rng(361 + total)
    nv = np.array([O.n_visible(int(inp["q_pos"][b, 0]), sp.m, int(inp["n_entries"][b]))
                   for b in range(sp.B)])
    idx = I.random_index_sets(rng, nv, k, holes=0.05)
    g = G.upload_decode(inp, d)
    G.decode_attend(g, idx=torch.from_numpy(idx).reshape(sp.B, 1, k).to(d))
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend split tiles", g, inp, b, idx[b], out[b, 0], total=total, b=b)


@pytest.mark.parametrize("k", [8, 40, 72, 104, 136, 168, 200, 232])
def test_attend_fp8_unsplit_tile_counts_vs_oracle(k):
    """FP8 rows with unsplit lists of 1 to 8 tiles (k + 16 window slots): the
    single-block kernel's loader ring from its shortest lists up."""
    d = dev()
    sp = I.CONFIGS["decode_1m_fp4"].replace(B=2, k=k, n_win=16)
    inp = I.decode_inputs(sp, seed=370 + k, lengths=[4 * k + 100, 300])
    rng = np.random.default_rng(371 + k)
    nv = np.array([O.n_visible(int(inp["q_pos"][b, 0]), sp.m, int(inp["n_entries"][b]))
                   for b in range(sp.B)])
    idx = I.random_index_sets(rng, nv, k, holes=0.1)
    g = G.upload_decode(inp, d)
    G.decode_attend(g, idx=torch.from_numpy(idx).reshape(sp.B, 1, k).to(d))
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend fp8 unsplit tiles", g, inp, b, idx[b], out[b, 0], k=k, b=b)


def test_attend_window_edges_and_empty_selection():
    """Window crossing position 0, all-empty selections (window only), one row."""
    d = dev()
    sp, inp, _ = _attend_case("decode_64k", [1, 5, 130, 4096], 310)
    idx = np.full((sp.B, sp.k), -1, np.int32)
    idx[3, :7] = np.arange(7) * 100
    g = G.upload_decode(inp, d)
    G.decode_attend(g, idx=torch.from_numpy(idx).reshape(sp.B, 1, sp.k).to(d))
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend window edges", g, inp, b, idx[b], out[b, 0], b=b)


def test_attend_unaligned_output_takes_generic_kernel():
    """An output pointer off 16-byte alignment cannot take the matrix-core
    kernels (their stores are 16 bytes wide): the call falls back to the
    generic kernel and still matches the oracle."""
    d = dev()
    sp, inp, idx = _attend_case("decode_64k", [4100, 300], 330)
    g = G.upload_decode(inp, d)
    buf = torch.zeros(g.out.numel() + 8, dtype=g.out.dtype, device=d)
    g.out = buf[1:1 + g.out.numel()].view(g.out.shape)    # 2 bytes past a 16-byte boundary
    assert g.out.data_ptr() % 16 == 2
    G.decode_attend(g, idx=torch.from_numpy(idx).reshape(sp.B, 1, sp.k).to(d))
    torch.cuda.synchronize()
    out = np64(g.out)
    for b in range(sp.B):
        check_decode_attention("attend unaligned out", g, inp, b, idx[b], out[b, 0], b=b)


def test_attend_deterministic_and_batch_invariant():
    d = dev()
    sp, inp, idx = _attend_case("decode_64k", [4100, 9000, 300], 320)
    g = G.upload_decode(inp, d)
    it = torch.from_numpy(idx).reshape(sp.B, 1, sp.k).to(d)
    G.decode_attend(g, idx=it)
    a = g.out.clone()
    G.decode_attend(g, idx=it)
    assert torch.equal(a, g.out)
    # sequence 1 alone gives the same bits as inside the batch
    one = {k: (v[1:2] if isinstance(v, np.ndarray) and v.ndim and v.shape[0] == sp.B else v)
           for k, v in inp.items()}
    one["spec"] = sp.replace(B=1)
    one["Nmax"] = inp["Nmax"]
    g1 = G.upload_decode(one, d)
    G.decode_attend(g1, idx=it[1:2].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(g1.out[0], a[1])


@pytest.mark.parametrize("k,slot", [(32, 5), (4096, 3000)])
def test_attend_fp8_rows_decode_every_code(k, slot):
    """FP8/BF16 rows whose e4m3 bodies hold every non-NaN code.  One selected
    entry, no window and a sink of -1e30: the output is that row exactly, so
    dims 0..447 must equal the oracle's decode of the codes bit for bit (e4m3
    values are exact in bf16).  k = 4096 also runs the split / bf16-partial
    path (one split carries the row, the others are empty)."""
    d = dev()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 codes
    B, N, nh, c, d_r = 2, 8, 64, 512, 64
    body = np.stack([np.resize(codes, 448), np.resize(codes[::-1], 448)])        # [2, 448]
    rng = np.random.default_rng(77)
    rope = F.bf16_encode(rng.standard_normal((B, d_r))).view(np.uint8).reshape(B, 2 * d_r)
    rows = np.zeros((B, N, 576), np.uint8)
    rows[:, 2, :448], rows[:, 2, 448:] = body, rope                               # entry 2 carries it
    kv = torch.from_numpy(rows).to(d)
    idx = np.full((B, 1, k), -1, np.int32)
    idx[:, 0, slot] = 2
    q = torch.from_numpy(I.cast(rng.standard_normal((B, 1, nh, c)).astype(np.float32), "bf16")).to(d).to(torch.bfloat16)
    q_pos = torch.full((B, 1), 4 * N - 1, dtype=torch.int32, device=d)
    sink = torch.full((nh,), -1e30, dtype=torch.float32, device=d)
    win = torch.zeros(B, 1, 576, dtype=torch.uint8, device=d)
    out = torch.empty(B, 1, nh, c, dtype=torch.bfloat16, device=d)
    L.sparse_mqa_attend(q, L.BF16, None, 1e-6, d_r, 1e4, q_pos, kv, L.FP8MIX, N,
                        torch.from_numpy(idx).to(d), k, win, 1, 0, sink, 1 / math.sqrt(c),
                        B, 1, nh, c, out, L.BF16)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[:, 0, :, :448]
    want = F.e4m3_decode(body)                                                    # [2, 448]
    report("attend fp8 codes", k=k, exact=bool(np.array_equal(got, np.broadcast_to(want[:, None], got.shape))))
    np.testing.assert_array_equal(got, np.broadcast_to(want[:, None, :], got.shape))


# =================================================================== decode-time compression
def _append_case(p, inp, sp, which, entries, out_t, Nmax):
    """Run csa_compress_append for sequences completing ``entries`` (all
    cut from the one prefill sequence) and return (cache, scales, full rows)."""
    d_ = p.H.device
    m = sp.m
    overlap = m == 4
    H = p.H.float() if p.H.dtype == torch.float32 else p.H
    Tt = 2 * m if overlap else m
    tails = []
    for i in entries:
        lo = m * i + m - Tt
        t = torch.zeros(Tt, sp.d, dtype=H.dtype, device=d_)
        src = H[max(lo, 0): m * i + m]
        t[Tt - src.shape[0]:] = src
        tails.append(t)
    Ht = torch.stack(tails)
    W = p.W
    if which == "main":
        Ws = (W["W_kv_a"], W["W_z_a"], W.get("W_kv_b"), W.get("W_z_b"), W["bias_a"], W.get("bias_b"))
        c, d_r, norm = sp.c, sp.d_r, p.gamma
    else:
        Ws = (W["WI_kv_a"], W["WI_z_a"], W["WI_kv_b"], W["WI_z_b"], W["biasI_a"], W["biasI_b"])
        c, d_r, norm = sp.cI, 0, None
    B = len(entries)
    rb = L.row_bytes(out_t, c, d_r)
    cache = torch.full((B * Nmax * rb,), 0xAB, dtype=torch.uint8, device=d_)
    scales = torch.full((B * Nmax * (c // 32),), 0xCD, dtype=torch.uint8, device=d_) if out_t == L.MXFP4 else None
    entry = torch.tensor(entries, dtype=torch.int32, device=d_)
    ht = L.F32 if Ht.dtype == torch.float32 else L.BF16
    L.csa_compress_append(Ht, ht, B, sp.d, Ws[0], Ws[1], Ws[2] if overlap else None,
                          Ws[3] if overlap else None, Ws[4], Ws[5] if overlap else None, m,
                          int(overlap), c, norm, 1e-6, d_r, 1e4, m, 0, entry, cache, scales, out_t,
                          Nmax)
    torch.cuda.synchronize()
    return cache.view(B, Nmax, rb), None if scales is None else scales.view(B, Nmax, c // 32), rb


@pytest.mark.parametrize("name", ["tiny_csa", "tiny_hca"])
def test_compress_append_tiny_f32(name):
    """Appending entry i from the tail of hidden states reproduces the full
    compressor's row i bit for bit and the oracle's entry within 1e-5; no
    other cache row is touched."""
    d = dev()
    sp = I.CONFIGS[name]
    inp = I.prefill_inputs(sp)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    torch.cuda.synchronize()
    n = sp.T // sp.m
    ref = OP.prefill_caches(inp)
    entries = [0, 1, min(137, n - 1), n - 1]
    cache, _, rb = _append_case(p, inp, sp, "main", entries, L.F32, n)
    full = p.kv.view(n, rb)
    worst = 0.0
    for b, i in enumerate(entries):
        assert torch.equal(cache[b, i], full[i]), (b, i)
        got = cache[b, i].view(torch.float32).double().cpu().numpy()
        worst = max(worst, float(np.abs(got - ref["kv"][i]).max()))
        others = torch.cat([cache[b, :i], cache[b, i + 1:]])
        assert bool((others == 0xAB).all()), (b, i)
    report("compress append", cfg=name, max_abs_vs_oracle=worst)
    assert worst <= 1e-5


def test_compress_append_bf16_and_mxfp4_index_keys():
    """bf16 hidden states and weights (the prefill shape, 4,096 tokens):
    main entries in bf16 and MXFP4 index keys appended from tails equal the full
    compressor's rows and scales bit for bit."""
    d = dev()
    sp = I.CONFIGS["prefill_32k_mxfp4"]
    inp = I.prefill_inputs(sp, T=4096)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    torch.cuda.synchronize()
    n = 4096 // sp.m
    entries = [0, 1, 500, n - 1]
    cache, _, rb = _append_case(p, inp, sp, "main", entries, L.BF16, n)
    full = p.kv.view(n, rb)
    for b, i in enumerate(entries):
        assert torch.equal(cache[b, i], full[i]), ("main", b, i)
    cI, sI, rbI = _append_case(p, inp, sp, "index", entries, L.MXFP4, n)
    fullI, fullS = p.kI.view(n, rbI), p.kI_scale.view(n, sp.cI // 32)
    for b, i in enumerate(entries):
        assert torch.equal(cI[b, i], fullI[i]) and torch.equal(sI[b, i], fullS[i]), ("index", b, i)
    report("compress append bf16 / mxfp4", entries=entries, bit_exact=True)
