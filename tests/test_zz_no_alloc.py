"""sparse_mqa_attend_noalloc -- attention that allocates nothing, its split
partials in the library's fixed per-GPU scratch -- against sparse_mqa_attend
with a caller workspace.  Both run the same kernels on the same split plan,
so the outputs must be identical bit for bit: two calls in a row, the second
on a smaller input, both on the split path that uses the scratch.  A call
needing more than the scratch is refused before any launch."""
import math

import numpy as np
import pytest
import torch

import csa_inputs as I
import long_context_sparse_10_amd as L
from long_context_sparse_10_amd import pipeline as G
from oracle import csa as O
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _decode_case(name, lengths, seed):
    sp = I.CONFIGS[name].replace(B=len(lengths))
    inp = I.decode_inputs(sp, seed=seed, lengths=lengths)
    rng = np.random.default_rng(seed + 1)
    nv = np.array([O.n_visible(int(inp["q_pos"][b, 0]), sp.m, int(inp["n_entries"][b]))
                   for b in range(sp.B)])
    idx = I.random_index_sets(rng, nv, sp.k, holes=0.1)
    return sp, inp, idx


def _noalloc(g, sp, it, out):
    qt = L.BF16 if g.q.dtype == torch.bfloat16 else L.F32
    L.sparse_mqa_attend_noalloc(g.q, qt, g.gamma, G.EPS, sp.d_r, G.ROPE_THETA, g.q_pos, g.kv,
                                g.kv_fmt, g.Nmax, it, sp.k, g.win, g.win_len, sp.n_win, g.sink,
                                1.0 / math.sqrt(sp.c), g.B, 1, sp.nh, sp.c, out, L.BF16)


def test_noalloc_attend_equals_workspace_attend():
    d = dev()
    # FP8/BF16 rows and 128 heads, then a smaller call: bf16 rows, 64 heads
    cases = [("decode_1m_fp4", [8192 + 5, 5000, 3000], 31), ("decode_64k", [4100, 300], 32)]
    used = []
    for name, lengths, seed in cases:
        print(f"[noalloc] {name} lengths={lengths}", flush=True)
        sp, inp, idx = _decode_case(name, lengths, seed)
        g = G.upload_decode(inp, d)
        it = torch.from_numpy(idx).reshape(sp.B, 1, sp.k).to(d)
        G.decode_attend(g, idx=it)                       # caller workspace
        assert g.ws is not None and g.ws.numel() > 0     # the split path
        used.append(g.ws.numel())
        out = torch.full_like(g.out, 7.0)
        _noalloc(g, sp, it, out)
        torch.cuda.synchronize()
        assert torch.equal(out, g.out), name
        assert used[-1] <= L.NOALLOC_SCRATCH_BYTES
    assert used[1] < used[0]                             # the second call is smaller


def test_noalloc_attend_refuses_more_than_its_scratch():
    d = dev()
    B, nh, c, d_r, k, N = 64, 128, 512, 64, 1024, 2048
    # 1152 slots per row, 8 splits: bf16 O / l and fp32 (m, l) per split and head
    need = B * 8 * nh * (2 * c + 8)
    assert need > L.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, 1, nh, c, dtype=torch.bfloat16, device=d)
    kv = torch.zeros(B, N, c, dtype=torch.bfloat16, device=d)
    win = torch.zeros(B, 128, c, dtype=torch.bfloat16, device=d)
    idx = torch.zeros(B, 1, k, dtype=torch.int32, device=d)
    q_pos = torch.full((B, 1), 4 * N - 1, dtype=torch.int32, device=d)
    sink = torch.zeros(nh, dtype=torch.float32, device=d)
    out = torch.full((B, 1, nh, c), 7.0, dtype=torch.bfloat16, device=d)
    with pytest.raises(L.CsaError) as e:
        L.sparse_mqa_attend_noalloc(q, L.BF16, None, 1e-6, d_r, 1e4, q_pos, kv, L.BF16, N, idx, k,
                                    win, 128, 128, sink, 1 / math.sqrt(c), B, 1, nh, c, out,
                                    L.BF16)
    assert e.value.status == L.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                      # nothing was launched
    # an empty call only sets up the scratch address
    L.sparse_mqa_attend_noalloc(q, L.BF16, None, 1e-6, d_r, 1e4, q_pos, kv, L.BF16, N, idx, k,
                                win, 128, 128, sink, 1 / math.sqrt(c), 0, 1, nh, c, out, L.BF16)
