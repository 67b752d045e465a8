"""Full-size parity: the workloads ``bench.py`` times, in the same launch
configuration, checked on sampled sequences / query rows the oracle computes
one by one.  Top-k sets must be bit-exact wherever the oracle's k-th and
(k+1)-th scores are further apart than the fp32 error bound; elsewhere the GPU
set must be a valid top-k of the oracle's scores within that bound."""
import numpy as np
import pytest
import torch

import csa_inputs as I
from long_context_sparse_10_amd import pipeline as G
from oracle import csa as O
from oracle import pipeline as OP
import long_context_sparse_10_amd as L
from tests.gpu_util import (bf16_ulp, check_attention, check_decode_attention, decode_rows, dev,
                            kernel_rows, mx_score_bound, np64, report, score_error_bound)

pytestmark = pytest.mark.gpu


def check_topk(got, scores, nv, k, bound):
    """Returns True when the set is bit-exact; asserts validity otherwise."""
    want = O.topk(scores, nv, k)
    if np.array_equal(got, want):
        return True
    sel = got[got >= 0]
    assert sel.size == min(k, nv) and np.all(np.diff(sel) > 0) and np.all(got[sel.size:] == -1)
    assert not OP.tie_free(scores, nv, k, 2 * bound), "tie-free query selected a different set"
    mask = np.zeros(nv, bool)
    mask[sel] = True
    assert scores[mask].min() >= scores[~mask].max() - 2 * bound
    return False


def _decode_full(name, seqs):
    d = dev()
    sp = I.CONFIGS[name]
    inp = I.decode_inputs(sp)
    print(f"[full] {name}: inputs ready", flush=True)
    g = G.upload_decode(inp, d)
    G.decode_step(g)
    torch.cuda.synchronize()
    print(f"[full] {name}: GPU step done", flush=True)
    return sp, inp, g


def test_decode_64k_full():
    sp, inp, g = _decode_full("decode_64k", None)
    S, idx, out = np64(g.scores), g.idx.cpu().numpy(), np64(g.out)
    exact = 0
    for b in (0, 13, 31):
        ref = OP.decode_reference(inp, b)
        nv = ref["n_vis"]
        bound = score_error_bound(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv)
        assert np.all(np.abs(S[b, 0, :nv] - ref["scores"]) <= bound)
        same = check_topk(idx[b, 0], ref["scores"], nv, sp.k, bound.max())
        exact += same
        check_decode_attention("decode_64k", g, inp, b, idx[b, 0], out[b, 0], b=b, idx_exact=same)
    assert exact >= 1


def test_hca_decode_1m_full():
    sp, inp, g = _decode_full("hca_decode_1m", None)
    out = np64(g.out)
    for b in (0, 15):
        check_decode_attention("hca_decode_1m", g, inp, b, None, out[b, 0], b=b)


def test_decode_1m_fp4_full():
    """MXFP4 index keys + FP8/BF16 KV at 262,144 entries: scores within one
    bf16 step of the quantised oracle, top-k valid against it (bit-exact where
    tie-free), attention within 2e-2; recall against the unquantised fp64
    oracle is reported (parity unpinned: the pages' 99.7% is a trained-model
    figure)."""
    sp, inp, g = _decode_full("decode_1m_fp4", None)
    S, idx, out = np64(g.scores), g.idx.cpu().numpy(), np64(g.out)
    for b in (0, 7):
        ref = OP.decode_reference(inp, b)
        nv = ref["n_vis"]
        bound = mx_score_bound(inp, b, ref["scores"], nv)
        assert np.all(np.abs(S[b, 0, :nv] - ref["scores"]) <= bound)
        same = check_topk(idx[b, 0], ref["scores"], nv, sp.k, float(bound.max()))
        exact_scores = O.index_scores(inp["qI"][b, 0], inp["w"][b, 0], inp["kI"][b], nv)
        ref_set = set(O.topk(exact_scores, nv, sp.k).tolist())
        recall = len(ref_set & set(idx[b, 0].tolist())) / sp.k
        check_decode_attention("decode_1m_fp4", g, inp, b, idx[b, 0], out[b, 0], b=b,
                               idx_exact_vs_quantised=same, recall_vs_fp64=recall)
        # regression floor: N(0,1) keys leave small score gaps at rank k, so
        # MXFP4 recall against the unquantised set is ~0.77 here (the pages'
        # 99.7% is a trained-model figure and is not compared)
        assert recall >= 0.70, recall


def _check_prefill_attention(tag, p, inp, caches, sp, r, got_idx, same, ref_out):
    """One prefill query row: 2e-2 against the oracle (its own caches, the
    GPU's index set) and the kernel bound against the GPU's stored rows."""
    pos = int(inp["q_pos"][r])
    T = inp["T"]
    n = T // sp.m
    got_idx = np.asarray(got_idx)
    if same:
        want = ref_out
    else:
        X = O.gather_rows(caches["kv"], got_idx, caches["win"], pos, sp.n_win, T)
        want = O.attend_query(inp["q"][r], None, 1e-6, sp.d_r, 1e4, pos, X, inp["sink"],
                              1 / np.sqrt(sp.c))
    sel_slots = [v for v, s_ in enumerate(got_idx) if s_ >= 0]
    Xk = kernel_rows(p.kv, p.win, L.BF16, sp.c, sp.d_r, max(n, 1), T, 0, got_idx[sel_slots], pos,
                     sp.n_win)
    return check_attention(tag, p.out[0, r].double().cpu().numpy(), inp["q"][r], Xk, inp["sink"],
                           1 / np.sqrt(sp.c), sp.d_r, pos, sel_slots, sp.k, sp.n_win, want, Tq=T,
                           row=r, idx_exact=same)


def _check_compressed_entries(p, inp, sp, entries):
    """Entries of the GPU's compressed cache at a full-length prefill against
    the oracle's compressor run on just the tokens each entry pools (blocks
    i-1 and i; RoPE at position m*i)."""
    m = sp.m
    n = inp["T"] // m
    kv = p.kv.view(n, -1)
    for i in entries:
        t0 = max(0, m * (i - 1))
        Hs = inp["H"][t0:m * (i + 1)]
        E = O.compress(Hs, inp["W_kv_a"], inp["W_z_a"], inp["bias_a"], m, inp["W_kv_b"],
                       inp["W_z_b"], inp["bias_b"], None, 1e-6, sp.d_r, 1e4, m, t0)
        want = E[-1]                                # the entry of block i
        got = decode_rows(kv[i:i + 1].contiguous(), L.BF16, 1, sp.c, sp.d_r)[0]
        err = float(np.abs(got - want).max())
        assert err <= 2e-2 and np.all(np.abs(got - want) <= bf16_ulp(want) + 1e-6), (i, err)
        Ei = O.compress(Hs, inp["WI_kv_a"], inp["WI_z_a"], inp["biasI_a"], m, inp["WI_kv_b"],
                        inp["WI_z_b"], inp["biasI_b"], normalize=False)[-1]
        if p.kI_scale is None:
            gi = decode_rows(p.kI.view(n, -1)[i:i + 1].contiguous(), L.BF16, 1, sp.cI, 0)[0]
            assert np.all(np.abs(gi - Ei) <= bf16_ulp(Ei) + 1e-6), i
        else:
            from oracle import formats as F
            gi = F.mxfp4_dequantize(p.kI.view(n, 64)[i].cpu().numpy()[None],
                                    p.kI_scale.view(n, 4)[i].cpu().numpy()[None])[0]
            # E2M1 codes of the GPU's fp32 entry: within one code step of the exact entry
            step = 2.0 ** (np.floor(np.log2(np.abs(Ei).reshape(4, 32).max(1))) - 2)
            assert np.all(np.abs(gi - Ei).reshape(4, 32) <= 2 * step[:, None] + 1e-6), i
    report("compressed entries", entries=len(entries), T=inp["T"])


def test_prefill_32k_full():
    """The whole prefill on the GPU (compression included), oracle on sampled
    query rows: causal boundaries, first window, middle and the last query."""
    d = dev()
    sp = I.CONFIGS["prefill_32k"]
    inp = I.prefill_inputs(sp)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    G.prefill_attention_path(p)
    torch.cuda.synchronize()
    print("[full] prefill_32k: GPU done", flush=True)
    _check_compressed_entries(p, inp, sp, [0, 1, 2, 1023, 1024, 4095, 8190, 8191])
    caches = OP.prefill_caches(inp)
    print("[full] prefill_32k: oracle caches done", flush=True)
    rows = [0, 3, 4, 7, 8, 127, 128, 4095, 4096, 4099, 16383, 20000, 32766, 32767]
    refs = OP.prefill_reference(inp, caches, rows)
    S = p.scores[0]
    exact = 0
    for r, ref in zip(rows, refs):
        nv = ref["n_vis"]
        got_idx = p.idx[0, r].cpu().numpy()
        srow = S[r, :nv].double().cpu().numpy()
        bound = score_error_bound(inp["qI"][r], inp["w"][r], caches["kI"], nv)
        # the GPU scores use the GPU's own bf16 index keys; compare within the
        # bf16 storage of the keys plus fp32 accumulation
        kb = score_error_bound(inp["qI"][r], inp["w"][r], caches["kI_exact"], nv, rel=2 ** -8)
        assert np.all(np.abs(srow - ref["scores"]) <= bound + kb + 1e-6)
        same = check_topk(got_idx, ref["scores"], nv, sp.k, float((bound + kb).max()) if nv else 0)
        exact += same
        _check_prefill_attention("prefill_32k", p, inp, caches, sp, r, got_idx, same, ref["out"])
    report("prefill_32k", rows=len(rows), idx_exact=exact)


def _mx_prefill_rows(p, inp, caches, sp, rows, tag):
    """MXFP4 prefill rows: scores in the quantised-oracle mode against the GPU's
    own stored E2M1 codes and scales (fp64 products, bf16 scores), top-k
    against those scores (bit-exact where tie-free), attention checked."""
    from oracle import formats as F
    T = inp["T"]
    n = T // sp.m
    kq = F.mxfp4_dequantize(p.kI.cpu().numpy().reshape(n, 64), p.kI_scale.cpu().numpy().reshape(n, 4))
    qI = p.qI.view(T, sp.nI, 64)
    qs = p.qI_scale.view(T, sp.nI, 4)
    S = p.scores[0]
    exact = 0
    for r in rows:
        pos = int(inp["q_pos"][r])
        nv = int(O.n_visible(pos, sp.m, n))
        qq = F.mxfp4_dequantize(qI[r].cpu().numpy(), qs[r].cpu().numpy())
        ref = F.bf16_round(O.index_scores(qq, inp["w"][r], kq, nv))
        e = score_error_bound(qq, inp["w"][r], kq, nv)
        srow = S[r, :nv].double().cpu().numpy()
        assert np.all(np.abs(srow - ref) <= bf16_ulp(np.abs(ref) + e) + e + 1e-30), r
        got = p.idx[0, r].cpu().numpy()
        bound = float((bf16_ulp(np.abs(ref) + e) + e).max()) if nv else 0.0
        same = check_topk(got, ref, nv, sp.k, bound)
        exact += same
        _check_prefill_attention(tag, p, inp, caches, sp, r, got, False, None)
    report(tag, rows=len(rows), idx_exact=exact)
    return exact


def test_prefill_mxfp4_indexer_4k():
    """The prefill with MXFP4 index keys and queries at 4,096 tokens
    (compression on the GPU)."""
    d = dev()
    sp = I.CONFIGS["prefill_32k_mxfp4"]
    inp = I.prefill_inputs(sp, T=4096)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    G.prefill_attention_path(p)
    torch.cuda.synchronize()
    caches = OP.prefill_caches(inp)
    _mx_prefill_rows(p, inp, caches, sp, [0, 3, 4, 7, 8, 127, 1000, 1023, 1024, 2049, 4095],
                     "prefill mxfp4 4k")


def test_prefill_32k_mxfp4_full():
    """The benched MXFP4 prefill at its full 32,768 tokens (32 key chunks per
    row group of the many-row indexer), in the launch configuration the
    benchmark times: sampled compressed entries against the oracle's
    compressor, and sampled query rows (causal boundaries, chunk edges, the
    middle and the last row) through scores, top-k and attention."""
    d = dev()
    sp = I.CONFIGS["prefill_32k_mxfp4"]
    inp = I.prefill_inputs(sp)
    p = G.upload_prefill(inp, d)
    G.prefill_compress(p)
    G.prefill_attention_path(p)
    torch.cuda.synchronize()
    print("[full] prefill_32k_mxfp4: GPU done", flush=True)
    _check_compressed_entries(p, inp, sp, [0, 1, 255, 256, 4095, 8191])
    caches = OP.prefill_caches(inp)
    print("[full] prefill_32k_mxfp4: oracle caches done", flush=True)
    rows = [0, 3, 4, 7, 8, 1023, 1024, 4099, 8191, 16384, 24577, 32766, 32767]
    _mx_prefill_rows(p, inp, caches, sp, rows, "prefill_32k_mxfp4")
