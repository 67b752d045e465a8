"""The decode step captured in a HIP graph (as ``bench.py`` replays it): every
replay must reproduce the eager step bit for bit, with eager work, output
clobbering and synchronisations between the replays.  The library records no
memset and allocates nothing, so the captured launches are the whole step."""
import numpy as np
import pytest
import torch

import csa_inputs as I
from long_context_sparse_10_amd import pipeline as G
from tests.gpu_util import dev, report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,lengths", [
    ("decode_64k", [65536, 40003, 7000]),        # single-block top-k, split attention
    ("decode_1m_fp4", [4 * 20000 + 3, 4 * 17000]),  # multi-block top-k (workspace)
    ("hca_decode_1m", [1 << 20, 300000]),        # dense HCA
])
def test_decode_step_graph_replays_match_eager(name, lengths):
    d = dev()
    sp = I.CONFIGS[name].replace(B=len(lengths))
    inp = I.decode_inputs(sp, seed=404, lengths=lengths)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = G.upload_decode(inp, d, stream)
        G.decode_step(g, stream)                 # eager: sizes every workspace
    torch.cuda.synchronize()
    want_out = g.out.clone()
    want_idx = g.idx.clone() if g.idx is not None else None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        G.decode_step(g, stream)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work and clobbered outputs between replays
        g.out.fill_(float("nan"))
        if g.idx is not None:
            g.idx.fill_(-7)
            g.scores.fill_(0)
        junk = torch.randn(1 << 20, device=d).sum()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        same_out = torch.equal(g.out, want_out)
        same_idx = want_idx is None or torch.equal(g.idx, want_idx)
        report("graph replay", cfg=name, rep=rep, out_equal=same_out, idx_equal=same_idx)
        assert same_idx and same_out


@pytest.mark.parametrize("name,lengths,chunks", [
    ("decode_64k", [65536, 40003, 7000, 65536, 12345], 2),
    ("decode_1m_fp4", [4 * 20000 + 3, 4 * 17000, 4 * 18000], 3),
    ("hca_decode_1m", [1 << 20, 300000, 5000], 2),
])
def test_overlapped_step_matches_plain_step(name, lengths, chunks):
    """Batch cut into groups whose chains run on two streams (eagerly and as a
    captured graph): bit-identical to the one-stream step."""
    d = dev()
    sp = I.CONFIGS[name].replace(B=len(lengths))
    inp = I.decode_inputs(sp, seed=405, lengths=lengths)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(main):
        g = G.upload_decode(inp, d, main)
        G.decode_step(g, main)
    torch.cuda.synchronize()
    want_out = g.out.clone()
    want_idx = g.idx.clone() if g.idx is not None else None
    g.out.fill_(float("nan"))
    with torch.cuda.stream(main):
        G.decode_step_overlapped(g, [main, side], chunks)
    torch.cuda.synchronize()
    assert torch.equal(g.out, want_out)
    assert want_idx is None or torch.equal(g.idx, want_idx)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=main):
        G.decode_step_overlapped(g, [main, side], chunks)
    torch.cuda.synchronize()
    for rep in range(3):
        g.out.fill_(float("nan"))
        if g.idx is not None:
            g.idx.fill_(-7)
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(g.out, want_out) and (want_idx is None or torch.equal(g.idx, want_idx))
        report("overlapped graph replay", cfg=name, chunks=chunks, rep=rep, equal=same)
        assert same
