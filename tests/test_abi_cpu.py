"""Host-side checks of libcsa's C ABI (CPU only: nothing here launches a kernel).

The library must load, export every entry point include/csa.h declares, and
reject bad arguments on the host before any launch.  Pointers passed below are
dummies that are never dereferenced: every call either fails validation or is a
pure workspace-size query."""
import ctypes
import os
import re

import pytest

import long_context_sparse_10_amd as L
from long_context_sparse_10_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")
D = 4096          # dummy non-null "device pointer", never dereferenced


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"^(?:csa_status|const char\*)\s+(\w+)\(", src, flags=re.M)


def test_library_loads_and_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert set(names) == {"csa_version", "csa_status_string", "csa_prep_rows", "csa_compress",
                          "csa_compress_append", "indexer_score", "topk_select",
                          "sparse_mqa_attend", "hca_attend", "csa_compress_paged",
                          "csa_compress_append_paged", "indexer_score_paged",
                          "sparse_mqa_attend_paged", "hca_attend_paged", "grouped_out_proj",
                          "sparse_mqa_attend_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)
    assert "gfx950" in L.version()


def _prep(**kw):
    a = dict(x=D, x_t=L.F32, rows=10, c=64, norm_w=None, eps=1e-6, rope_dims=16, theta=1e4,
             pos=None, rps=1, ps=1, po=0, out=D, out_scale=None, out_t=L.BF16)
    a.update(kw)
    return L.lib().csa_prep_rows(a["x"], a["x_t"], a["rows"], a["c"], a["norm_w"], a["eps"],
                                 a["rope_dims"], a["theta"], a["pos"], a["rps"], a["ps"], a["po"],
                                 a["out"], a["out_scale"], a["out_t"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x_t=L.MXFP4), _lib.ERR_UNSUPPORTED),
    (dict(out_t=7), _lib.ERR_UNSUPPORTED),
    (dict(c=63), _lib.ERR_INVALID),
    (dict(rope_dims=66), _lib.ERR_INVALID),
    (dict(rope_dims=15), _lib.ERR_INVALID),
    (dict(x=None), _lib.ERR_INVALID),
    (dict(out=None), _lib.ERR_INVALID),
    (dict(rows=-1), _lib.ERR_INVALID),
    (dict(rps=0), _lib.ERR_INVALID),
    (dict(out_t=L.MXFP4, c=48, out_scale=D), _lib.ERR_INVALID),
    (dict(out_t=L.MXFP4, out_scale=None), _lib.ERR_INVALID),
    (dict(out_t=L.FP8MIX, rope_dims=0), _lib.ERR_INVALID),
    (dict(theta=0.0), _lib.ERR_INVALID),
    (dict(eps=-1.0), _lib.ERR_INVALID),
    (dict(rows=0), _lib.OK),            # nothing to do: no launch
])
def test_prep_rows_validation(kw, want):
    assert _prep(**kw) == want


def _compress(ws=None, ws_bytes=None, **kw):
    a = dict(H=D, h_t=L.BF16, B=1, T=64, d=32, kva=D, za=D, kvb=D, zb=D, ba=D, bb=D, m=4, ov=1,
             c=64, norm=None, eps=1e-6, rd=16, th=1e4, ps=4, po=0, out=D, osc=None, out_t=L.BF16)
    a.update(kw)
    return L.lib().csa_compress(a["H"], a["h_t"], a["B"], a["T"], a["d"], a["kva"], a["za"],
                                a["kvb"], a["zb"], a["ba"], a["bb"], a["m"], a["ov"], a["c"],
                                a["norm"], a["eps"], a["rd"], a["th"], a["ps"], a["po"], a["out"],
                                a["osc"], a["out_t"], ws, ws_bytes, None)


def test_compress_validation_and_workspace():
    need = ctypes.c_size_t(0)
    assert _compress(ws_bytes=ctypes.byref(need)) == _lib.OK
    assert need.value == 64 * 64 * 4 * 4           # four fp32 [T, c] projections
    need1 = ctypes.c_size_t(0)
    assert _compress(ws_bytes=ctypes.byref(need1), za=None, kvb=None, zb=None, ba=None, bb=None,
                     m=1, ov=0) == _lib.OK
    assert need1.value == 64 * 64 * 4
    small = ctypes.c_size_t(16)
    assert _compress(ws=D, ws_bytes=ctypes.byref(small)) == _lib.ERR_WORKSPACE
    assert _compress(ws=D, ws_bytes=None) == _lib.ERR_WORKSPACE
    assert _compress(za=None) == _lib.ERR_INVALID                      # m = 4 needs gates
    assert _compress(kvb=None) == _lib.ERR_INVALID                     # overlap needs b-series
    assert _compress(ov=0) == _lib.ERR_INVALID                         # b-series without overlap
    assert _compress(h_t=L.FP8MIX) == _lib.ERR_UNSUPPORTED
    assert _compress(T=0) == _lib.ERR_INVALID


def _indexer(**kw):
    a = dict(qI=D, qs=None, qt=L.BF16, w=D, kI=D, ks=None, kt=L.BF16, qp=D, ne=D, B=2, Tq=1, nI=64,
             cI=128, N=100, m=4, sc=D, st=L.F32)
    a.update(kw)
    return L.lib().indexer_score(a["qI"], a["qs"], a["qt"], a["w"], a["kI"], a["ks"], a["kt"],
                                 a["qp"], a["ne"], a["B"], a["Tq"], a["nI"], a["cI"], a["N"],
                                 a["m"], a["sc"], a["st"], None)


def test_indexer_validation():
    assert _indexer(kt=L.F32) == _lib.ERR_UNSUPPORTED
    assert _indexer(qt=L.FP8MIX, kt=L.FP8MIX) == _lib.ERR_UNSUPPORTED
    assert _indexer(st=L.MXFP4) == _lib.ERR_UNSUPPORTED
    assert _indexer(qt=L.MXFP4, kt=L.MXFP4) == _lib.ERR_INVALID          # scales missing
    assert _indexer(qt=L.MXFP4, kt=L.MXFP4, qs=D, ks=D, cI=48) == _lib.ERR_INVALID
    assert _indexer(w=None) == _lib.ERR_INVALID
    assert _indexer(m=0) == _lib.ERR_INVALID
    assert _indexer(N=0) == _lib.ERR_INVALID
    assert _indexer(B=0) == _lib.OK                                         # empty batch


def test_topk_validation_and_workspace():
    f = L.lib().topk_select
    need = ctypes.c_size_t(99)
    assert f(D, L.F32, D, D, 2, 1, 100, 4, 8, D, None, ctypes.byref(need), None) == _lib.OK
    assert need.value == 0
    # rows longer than 16384 entries run multi-block and need a workspace
    assert f(D, L.BF16, D, D, 8, 1, 262144, 4, 1024, D, None, ctypes.byref(need), None) == _lib.OK
    assert need.value >= 8 * 64 * 2048 * 4
    assert f(D, L.BF16, D, D, 8, 1, 262144, 4, 1024, D, None, None, None) == _lib.ERR_WORKSPACE
    assert f(D, L.F32, D, D, 2, 1, 100, 4, 0, D, None, None, None) == _lib.ERR_INVALID
    assert f(D, L.FP8MIX, D, D, 2, 1, 100, 4, 8, D, None, None, None) == _lib.ERR_UNSUPPORTED
    assert f(None, L.F32, D, D, 2, 1, 100, 4, 8, D, None, None, None) == _lib.ERR_INVALID
    assert f(D, L.F32, D, D, 0, 1, 100, 4, 8, D, None, None, None) == _lib.OK


def _attend(sparse=True, ws=None, ws_bytes=None, **kw):
    a = dict(q=D, qt=L.BF16, qn=None, eps=1e-6, rd=64, th=1e4, qp=D, kv=D, kvt=L.BF16, N=16384,
             idx=D, k=1024, ne=D, mp=128, win=D, wl=128, nw=128, sink=D, scale=0.044, B=32, Tq=1,
             nh=64, c=512, out=D, ot=L.BF16)
    a.update(kw)
    if sparse:
        return L.lib().sparse_mqa_attend(a["q"], a["qt"], a["qn"], a["eps"], a["rd"], a["th"],
                                         a["qp"], a["kv"], a["kvt"], a["N"], a["idx"], a["k"],
                                         a["win"], a["wl"], a["nw"], a["sink"], a["scale"], a["B"],
                                         a["Tq"], a["nh"], a["c"], a["out"], a["ot"], ws, ws_bytes,
                                         None)
    return L.lib().hca_attend(a["q"], a["qt"], a["qn"], a["eps"], a["rd"], a["th"], a["qp"],
                              a["kv"], a["kvt"], a["N"], a["ne"], a["mp"], a["win"], a["wl"],
                              a["nw"], a["sink"], a["scale"], a["B"], a["Tq"], a["nh"], a["c"],
                              a["out"], a["ot"], ws, ws_bytes, None)


def test_attend_validation():
    assert _attend(win=None) == _lib.ERR_INVALID
    assert _attend(wl=64) == _lib.ERR_INVALID                 # ring shorter than the window
    assert _attend(idx=None) == _lib.ERR_INVALID
    assert _attend(k=0) == _lib.ERR_INVALID
    assert _attend(kvt=L.FP8MIX, rd=0) == _lib.ERR_INVALID
    assert _attend(kvt=L.MXFP4) == _lib.ERR_UNSUPPORTED
    assert _attend(qt=L.FP8MIX) == _lib.ERR_UNSUPPORTED
    assert _attend(sparse=False, ne=None) == _lib.ERR_INVALID
    assert _attend(sparse=False, mp=0) == _lib.ERR_INVALID
    assert _attend(rd=63) == _lib.ERR_INVALID
    assert _attend(sink=None) == _lib.ERR_INVALID


def _noalloc(**kw):
    a = dict(q=D, qt=L.BF16, qn=None, eps=1e-6, rd=64, th=1e4, qp=D, kv=D, kvt=L.BF16, N=16384,
             idx=D, k=1024, win=D, wl=128, nw=128, sink=D, scale=0.044, B=32, Tq=1, nh=64, c=512,
             out=D, ot=L.BF16)
    a.update(kw)
    return L.lib().sparse_mqa_attend_noalloc(a["q"], a["qt"], a["qn"], a["eps"], a["rd"], a["th"],
                                             a["qp"], a["kv"], a["kvt"], a["N"], a["idx"], a["k"],
                                             a["win"], a["wl"], a["nw"], a["sink"], a["scale"],
                                             a["B"], a["Tq"], a["nh"], a["c"], a["out"], a["ot"],
                                             None)


def test_noalloc_attend_host_checks():
    """The no-allocation attention checks its arguments like sparse_mqa_attend
    and refuses, before touching the GPU, a call whose split partials exceed
    its fixed scratch (32 MiB)."""
    assert _noalloc(idx=None) == _lib.ERR_INVALID
    assert _noalloc(win=None) == _lib.ERR_INVALID
    assert _noalloc(kvt=L.MXFP4) == _lib.ERR_UNSUPPORTED
    # partials of 64 rows x 128 heads x 8 splits = 67.6 MB > 32 MiB
    need = ctypes.c_size_t(0)
    assert _attend(B=64, nh=128, ws=None, ws_bytes=ctypes.byref(need)) == _lib.OK
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(B=64, nh=128) == _lib.ERR_WORKSPACE
    # 32 rows x 64 heads (the 64K decode batch) fit
    assert _attend(B=32, nh=64, ws=None, ws_bytes=ctypes.byref(need)) == _lib.OK
    assert 0 < need.value <= _lib.NOALLOC_SCRATCH_BYTES


def test_attend_workspace_depends_on_slots_not_batch():
    """Split partials are sized per query row; the split plan is a function of
    the slot count only, so the per-row size is the same at any batch size."""
    sizes = []
    for B in (1, 8, 32):
        need = ctypes.c_size_t(0)
        assert _attend(B=B, ws_bytes=ctypes.byref(need)) == _lib.OK
        sizes.append(need.value / B)
    assert sizes[0] == sizes[1] == sizes[2] > 0
    need = ctypes.c_size_t(0)
    assert _attend(Tq=4096, B=1, ws_bytes=ctypes.byref(need)) == _lib.OK
    assert need.value == 0                                    # many query rows: no split
    small = ctypes.c_size_t(1)
    assert _attend(ws=D, ws_bytes=ctypes.byref(small)) == _lib.ERR_WORKSPACE


def test_compress_append_validation_and_workspace():
    f = L.lib().csa_compress_append

    def call(H=D, W_z_a=D, Wb=D, bias_b=D, overlap=1, B=4, m=4, entry=D, cache=D, Nmax=100,
             ws=None, szp=None, out_t=L.BF16):
        return f(H, L.BF16, B, 256, D, W_z_a, Wb, Wb, D, bias_b, m, overlap, 64, None, 1e-6, 16,
                 1e4, m, 0, entry, cache, None, out_t, Nmax, ws, szp, None)
    need = ctypes.c_size_t(0)
    assert call(szp=ctypes.byref(need)) == _lib.OK
    assert need.value == 4 * 4 * (2 * 4) * 64 * 4          # 4 projections of B * 2m rows, fp32
    assert call(overlap=0, Wb=None, bias_b=None, szp=ctypes.byref(need)) == _lib.OK
    assert need.value == 2 * 4 * 4 * 64 * 4                # 2 projections of B * m rows
    assert call(entry=None) == _lib.ERR_INVALID
    assert call(W_z_a=None) == _lib.ERR_INVALID
    assert call(Nmax=0) == _lib.ERR_INVALID
    assert call(overlap=0) == _lib.ERR_INVALID              # b-series weights without overlap
    assert call(out_t=L.MXFP4) == _lib.ERR_INVALID          # MXFP4 needs a scale array
    assert call() == _lib.ERR_WORKSPACE                     # workspace needed, none given


def _pages(max_blocks=64, log2=5, page_bytes=41984, table=D):
    return ctypes.byref(_lib.CsaPages(table, max_blocks, log2, page_bytes))


# a hybrid page of 32 bf16 main rows (1 KiB), 32 bf16 index keys (256 B) and one
# HCA row: 41,984 bytes
BAD_PAGES = [
    dict(table=None),                        # no block table
    dict(max_blocks=0),
    dict(log2=17),                           # entries per page out of range
    dict(page_bytes=41985),                  # not a multiple of 16
    dict(page_bytes=4096),                   # 32 rows of 1 KiB (or 256 B) do not fit
    dict(max_blocks=2),                      # 2 blocks x 32 < Nmax
]


@pytest.mark.parametrize("bad", BAD_PAGES)
def test_paged_calls_check_the_page_descriptor(bad):
    """Every paged entry point validates the descriptor on the host; a good one
    passes (workspace queries, or empty batches that launch nothing)."""
    lib = L.lib()
    Nmax = 1024

    def attend(pages, kv=D):
        need = ctypes.c_size_t(0)
        return lib.sparse_mqa_attend_paged(D, L.BF16, None, 1e-6, 64, 1e4, D, kv, L.BF16, Nmax,
                                           pages, D, 512, D, 128, 128, D, 0.04, 4, 1, 64, 512, D,
                                           L.BF16, None, ctypes.byref(need), None)

    def hca(pages):
        need = ctypes.c_size_t(0)
        return lib.hca_attend_paged(D, L.BF16, None, 1e-6, 64, 1e4, D, D, L.BF16, Nmax, pages, D,
                                    128, D, 128, 128, D, 0.04, 4, 1, 64, 512, D, L.BF16, None,
                                    ctypes.byref(need), None)

    def index(pages, kI=D):
        return lib.indexer_score_paged(D, None, L.BF16, D, kI, None, L.BF16, pages, D, D, 0, 1,
                                       64, 128, Nmax, 4, D, L.F32, None)

    def compress(pages):
        need = ctypes.c_size_t(0)
        return lib.csa_compress_paged(D, L.BF16, 1, 4 * Nmax, 256, D, D, D, D, D, D, 4, 1, 512,
                                      D, 1e-6, 64, 1e4, 4, 0, D, None, L.BF16, pages, None,
                                      ctypes.byref(need), None)

    def append(pages):
        need = ctypes.c_size_t(0)
        return lib.csa_compress_append_paged(D, L.BF16, 4, 256, D, D, D, D, D, D, 4, 1, 512, D,
                                             1e-6, 64, 1e4, 4, 0, D, D, None, L.BF16, Nmax, pages,
                                             None, ctypes.byref(need), None)

    calls = [attend, index, compress, append]
    for f in calls:
        assert f(_pages()) == _lib.OK, f.__name__
        assert f(None) == _lib.ERR_INVALID, f.__name__
        assert f(_pages(**bad)) == _lib.ERR_INVALID, (f.__name__, bad)
    # HCA rows: one entry per page
    assert hca(_pages(log2=0, max_blocks=Nmax)) == _lib.OK
    assert hca(_pages(log2=0, max_blocks=Nmax - 1)) == _lib.ERR_INVALID
    # series bases must be 16-byte aligned
    assert attend(_pages(), kv=D + 8) == _lib.ERR_INVALID
    assert index(_pages(), kI=D + 4) == _lib.ERR_INVALID


def test_paged_compress_needs_the_same_workspace_as_dense():
    lib = L.lib()
    dense, paged = ctypes.c_size_t(0), ctypes.c_size_t(0)
    args = (D, L.BF16, 2, 4096, 256, D, D, D, D, D, D, 4, 1, 512, D, 1e-6, 64, 1e4, 4, 0, D, None,
            L.BF16)
    assert lib.csa_compress(*args, None, ctypes.byref(dense), None) == _lib.OK
    assert lib.csa_compress_paged(*args, _pages(max_blocks=32), None, ctypes.byref(paged),
                                  None) == _lib.OK
    assert dense.value == paged.value > 0


def test_grouped_out_proj_validation_and_workspace():
    f = L.lib().grouped_out_proj

    def call(o=D, t=L.BF16, R=32, nh=64, c=512, g=8, d_g=1024, Wa=D, Wb=D, d=4096, y=D,
             y_t=L.BF16, ws=None, szp=None):
        return f(o, t, R, nh, c, g, d_g, Wa, Wb, d, y, y_t, ws, szp, None)
    need = ctypes.c_size_t(0)
    assert call(szp=ctypes.byref(need)) == _lib.OK
    # u in bf16, then fp32 K-slice partials (4 slices x 32 x 8192, or 8 x 32 x 4096)
    assert need.value == 32 * 8 * 1024 * 2 + 8 * 32 * 4096 * 4
    assert call(t=L.F32, szp=ctypes.byref(need)) == _lib.OK
    assert need.value == 32 * 8 * 1024 * 4                      # u in fp32 only
    assert call(nh=60) == _lib.ERR_INVALID                      # heads not a multiple of g
    assert call(c=6, szp=ctypes.byref(need)) == _lib.ERR_INVALID    # bf16 K1 = 48, not a multiple of 32
    assert call(Wa=None) == _lib.ERR_INVALID
    assert call(y=D + 8) == _lib.ERR_INVALID                    # 16-byte alignment
    assert call(t=L.MXFP4) == _lib.ERR_UNSUPPORTED
    assert call(R=0, szp=ctypes.byref(need)) == _lib.OK and need.value == 0
    assert call() == _lib.ERR_WORKSPACE
