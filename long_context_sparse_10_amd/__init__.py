"""MI355X (gfx950) Compressed Sparse Attention: a C-ABI HIP library (libcsa.so)
and its thin Python binding.

The five calls of the path -- ``csa_compress``, ``indexer_score``,
``topk_select``, ``sparse_mqa_attend``, ``hca_attend`` -- plus the row encoder
``csa_prep_rows``, the decode-time ``csa_compress_append`` and the
``grouped_out_proj`` that follows attention, and
``sparse_mqa_attend_noalloc`` (attention on a fixed per-GPU scratch, for
callers that cannot allocate) are re-exported
from :mod:`._lib` with torch tensors in place of device pointers.  The cache
calls take ``pages=Pages(...)`` for caches held in a paged pool (the
``*_paged`` entry points).  See ``include/csa.h`` for the contract of each call.
"""
from ._lib import (  # noqa: F401
    BF16, ERR_WORKSPACE, F32, FP8MIX, MXFP4, NOALLOC_SCRATCH_BYTES, CsaError, LIB_PATH, Pages,
    csa_compress, csa_compress_append, csa_prep_rows, grouped_out_proj, hca_attend,
    indexer_score, lib, sparse_mqa_attend, sparse_mqa_attend_noalloc, status_string, topk_select,
    version,
)


def row_bytes(fmt: int, c: int, rope_dims: int = 0) -> int:
    """Bytes of one stored row in format ``fmt`` (scales of MXFP4 excluded)."""
    return {F32: 4 * c, BF16: 2 * c, FP8MIX: (c - rope_dims) + 2 * rope_dims, MXFP4: c // 2}[fmt]
