"""ctypes binding of libcsa.so: the C entry points under the same names, taking
torch device tensors instead of raw pointers.  Argument marshalling only --
every step runs in the library's HIP kernels.  If the library is missing the
first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

# csa_dtype
F32, BF16, FP8MIX, MXFP4 = 0, 1, 2, 3
# csa_status
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, 1, 2, 3, 4

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_psz = ctypes.POINTER(ctypes.c_size_t)


class CsaPages(ctypes.Structure):
    """struct csa_pages of include/csa.h."""
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int),
                ("entries_log2", ctypes.c_int), ("page_bytes", ctypes.c_int64)]


_pp = ctypes.POINTER(CsaPages)

# name -> argument types, in the order of include/csa.h
SIGNATURES = {
    "csa_version": [],
    "csa_status_string": [_i32],
    "csa_prep_rows": [_vp, _i32, _i64, _i32, _vp, _f32, _i32, _f32, _vp, _i32, _i32, _i32,
                      _vp, _vp, _i32, _vp],
    "csa_compress": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                     _vp, _f32, _i32, _f32, _i32, _i32, _vp, _vp, _i32, _vp, _psz, _vp],
    "csa_compress_append": [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                            _vp, _f32, _i32, _f32, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _vp,
                            _psz, _vp],
    "indexer_score": [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                      _i32, _i32, _vp, _i32, _vp],
    "topk_select": [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _psz, _vp],
    "sparse_mqa_attend": [_vp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _i32, _i32, _vp, _i32,
                          _vp, _i32, _i32, _vp, _f32, _i32, _i32, _i32, _i32, _vp, _i32, _vp,
                          _psz, _vp],
    "hca_attend": [_vp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32,
                   _i32, _vp, _f32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _psz, _vp],
    "grouped_out_proj": [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i32, _vp,
                         _psz, _vp],
    "csa_compress_paged": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                           _i32, _vp, _f32, _i32, _f32, _i32, _i32, _vp, _vp, _i32, _pp, _vp,
                           _psz, _vp],
    "csa_compress_append_paged": [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                  _i32, _i32, _vp, _f32, _i32, _f32, _i32, _i32, _vp, _vp, _vp,
                                  _i32, _i32, _pp, _vp, _psz, _vp],
    "indexer_score_paged": [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _pp, _vp, _vp, _i32, _i32, _i32,
                            _i32, _i32, _i32, _vp, _i32, _vp],
    "sparse_mqa_attend_paged": [_vp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _i32, _i32, _pp, _vp,
                                _i32, _vp, _i32, _i32, _vp, _f32, _i32, _i32, _i32, _i32, _vp,
                                _i32, _vp, _psz, _vp],
    "hca_attend_paged": [_vp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _i32, _i32, _pp, _vp, _i32,
                         _vp, _i32, _i32, _vp, _f32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _psz,
                         _vp],
    "sparse_mqa_attend_noalloc": [_vp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _i32, _i32, _vp,
                                  _i32, _vp, _i32, _i32, _vp, _f32, _i32, _i32, _i32, _i32, _vp,
                                  _i32, _vp],
}

# bytes of the fixed scratch of sparse_mqa_attend_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20


class Pages:
    """A cache series held in pages: ``table`` is the device int32 block table
    [B, max_blocks]; each page holds ``2**entries_log2`` entries of the series
    and pages are ``page_bytes`` apart.  The series base (the address of slot 0
    of page 0) is passed where the dense call takes the cache tensor."""

    def __init__(self, table, entries_log2, page_bytes):
        self.table, self.entries_log2, self.page_bytes = table, int(entries_log2), int(page_bytes)

    def struct(self):
        return CsaPages(_p(self.table), int(self.table.shape[-1]), self.entries_log2,
                        self.page_bytes)

_lib = None


class CsaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load libcsa.so once (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with long_context_sparse_10_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name in ("csa_version", "csa_status_string") else ctypes.c_int
        _lib = L
    return _lib


def version() -> str:
    return lib().csa_version().decode()


def status_string(status: int) -> str:
    return lib().csa_status_string(int(status)).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn, st):
    if st != OK:
        raise CsaError(fn, st)


def _workspace(call, device, ws):
    """Run ``call(ws_ptr, size_ptr)``: size query first, then the real call with
    ``ws`` (a byte tensor) or a freshly allocated one."""
    need = ctypes.c_size_t(0)
    st = call(None, ctypes.byref(need))
    if st != OK:
        return st, None
    if need.value == 0:
        return call(None, None), None
    if ws is None:
        ws = torch.empty(need.value, dtype=torch.uint8, device=device)
    size = ctypes.c_size_t(ws.numel() * ws.element_size())
    return call(_p(ws), ctypes.byref(size)), ws


def workspace_bytes(fn_name, *args):
    """Workspace size an entry point reports for these arguments (no launch)."""
    need = ctypes.c_size_t(0)
    st = getattr(lib(), fn_name)(*args, None, ctypes.byref(need), None)
    _check(fn_name, st)
    return need.value


# ---------------------------------------------------------------- entry points
def csa_prep_rows(x, x_t, rows, c, norm_w, eps, rope_dims, rope_theta, pos, rows_per_seq,
                  pos_stride, pos_offset, out, out_scale, out_t, stream=None):
    st = lib().csa_prep_rows(_p(x), x_t, rows, c, _p(norm_w), eps, rope_dims, rope_theta, _p(pos),
                             rows_per_seq, pos_stride, pos_offset, _p(out), _p(out_scale), out_t,
                             _s(stream))
    _check("csa_prep_rows", st)


def csa_compress(H, h_t, B, T, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m, overlap, c,
                 norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset, out, out_scale, out_t,
                 ws=None, stream=None, pages=None):
    L = lib()
    sid = _s(stream)
    head = (_p(H), h_t, B, T, d, _p(W_kv_a), _p(W_z_a), _p(W_kv_b), _p(W_z_b), _p(bias_a),
            _p(bias_b), m, overlap, c, _p(norm_w), eps, rope_dims, rope_theta, pos_stride,
            pos_offset, _p(out), _p(out_scale), out_t)
    ps = pages.struct() if pages is not None else None

    def call(wp, szp):
        if ps is not None:
            return L.csa_compress_paged(*head, ctypes.byref(ps), wp, szp, sid)
        return L.csa_compress(*head, wp, szp, sid)
    st, ws = _workspace(call, H.device, ws)
    _check("csa_compress_paged" if ps is not None else "csa_compress", st)
    return ws


def csa_compress_append(H, h_t, B, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m, overlap, c,
                        norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset, entry, cache,
                        cache_scale, out_t, Nmax, ws=None, stream=None, pages=None):
    L = lib()
    sid = _s(stream)
    head = (_p(H), h_t, B, d, _p(W_kv_a), _p(W_z_a), _p(W_kv_b), _p(W_z_b), _p(bias_a),
            _p(bias_b), m, overlap, c, _p(norm_w), eps, rope_dims, rope_theta, pos_stride,
            pos_offset, _p(entry), _p(cache), _p(cache_scale), out_t, Nmax)
    ps = pages.struct() if pages is not None else None

    def call(wp, szp):
        if ps is not None:
            return L.csa_compress_append_paged(*head, ctypes.byref(ps), wp, szp, sid)
        return L.csa_compress_append(*head, wp, szp, sid)
    st, ws = _workspace(call, H.device, ws)
    _check("csa_compress_append_paged" if ps is not None else "csa_compress_append", st)
    return ws


def indexer_score(qI, qI_scale, qI_t, w, kI, kI_scale, kI_t, q_pos, n_entries, B, Tq, nI, cI,
                  Nmax, m, scores, score_t, stream=None, pages=None):
    k = (_p(qI), _p(qI_scale), qI_t, _p(w), _p(kI), _p(kI_scale), kI_t)
    tail = (_p(q_pos), _p(n_entries), B, Tq, nI, cI, Nmax, m, _p(scores), score_t, _s(stream))
    if pages is not None:
        ps = pages.struct()
        _check("indexer_score_paged", lib().indexer_score_paged(*k, ctypes.byref(ps), *tail))
    else:
        _check("indexer_score", lib().indexer_score(*k, *tail))


def topk_select(scores, score_t, q_pos, n_entries, B, Tq, Nmax, m, k, idx, ws=None, stream=None):
    L = lib()
    sid = _s(stream)

    def call(wp, szp):
        return L.topk_select(_p(scores), score_t, _p(q_pos), _p(n_entries), B, Tq, Nmax, m, k,
                             _p(idx), wp, szp, sid)
    st, ws = _workspace(call, scores.device, ws)
    _check("topk_select", st)
    return ws


def sparse_mqa_attend(q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, idx, k,
                      win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t, ws=None,
                      stream=None, pages=None):
    L = lib()
    sid = _s(stream)
    head = (_p(q), q_t, _p(q_norm_w), eps, rope_dims, rope_theta, _p(q_pos), _p(kv), kv_t, Nmax)
    tail = (_p(idx), k, _p(win), win_len, n_win, _p(sink), scale, B, Tq, nh, c, _p(out), out_t)
    ps = pages.struct() if pages is not None else None

    def call(wp, szp):
        if ps is not None:
            return L.sparse_mqa_attend_paged(*head, ctypes.byref(ps), *tail, wp, szp, sid)
        return L.sparse_mqa_attend(*head, *tail, wp, szp, sid)
    st, ws = _workspace(call, q.device, ws)
    _check("sparse_mqa_attend_paged" if ps is not None else "sparse_mqa_attend", st)
    return ws


def sparse_mqa_attend_noalloc(q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax,
                              idx, k, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t,
                              stream=None):
    """sparse_mqa_attend with the library's fixed per-GPU scratch: no
    workspace, no allocation."""
    st = lib().sparse_mqa_attend_noalloc(
        _p(q), q_t, _p(q_norm_w), eps, rope_dims, rope_theta, _p(q_pos), _p(kv), kv_t, Nmax,
        _p(idx), k, _p(win), win_len, n_win, _p(sink), scale, B, Tq, nh, c, _p(out), out_t,
        _s(stream))
    _check("sparse_mqa_attend_noalloc", st)


def hca_attend(q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, n_entries,
               m_prime, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t, ws=None,
               stream=None, pages=None):
    L = lib()
    sid = _s(stream)
    head = (_p(q), q_t, _p(q_norm_w), eps, rope_dims, rope_theta, _p(q_pos), _p(kv), kv_t, Nmax)
    tail = (_p(n_entries), m_prime, _p(win), win_len, n_win, _p(sink), scale, B, Tq, nh, c,
            _p(out), out_t)
    ps = pages.struct() if pages is not None else None

    def call(wp, szp):
        if ps is not None:
            return L.hca_attend_paged(*head, ctypes.byref(ps), *tail, wp, szp, sid)
        return L.hca_attend(*head, *tail, wp, szp, sid)
    st, ws = _workspace(call, q.device, ws)
    _check("hca_attend_paged" if ps is not None else "hca_attend", st)
    return ws


def grouped_out_proj(o, t, R, nh, c, g, d_g, W_a, W_b, d, y, y_t, ws=None, stream=None):
    L = lib()
    sid = _s(stream)

    def call(wp, szp):
        return L.grouped_out_proj(_p(o), t, R, nh, c, g, d_g, _p(W_a), _p(W_b), d, _p(y), y_t, wp,
                                  szp, sid)
    st, ws = _workspace(call, o.device, ws)
    _check("grouped_out_proj", st)
    return ws
