"""Helpers shared by the GPU parity tests: device handle, decoding of the
library's stored rows with torch's own dtype views (independent of the oracle),
and the tolerance rules."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_10_amd as L


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def decode_rows(buf: torch.Tensor, fmt: int, rows: int, c: int, d_r: int) -> np.ndarray:
    """fp64 values of ``rows`` stored rows (torch dtype views do the decoding)."""
    b = buf.reshape(rows, -1)
    if fmt == L.F32:
        return b.view(torch.float32).double().cpu().numpy()
    if fmt == L.BF16:
        return b.view(torch.bfloat16).double().cpu().numpy()
    if fmt == L.FP8MIX:
        body = b[:, : c - d_r].contiguous().view(torch.float8_e4m3fn).double()
        rope = b[:, c - d_r:].contiguous().view(torch.bfloat16).double()
        return torch.cat([body, rope], 1).cpu().numpy()
    raise ValueError(fmt)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (for tolerances)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def e4m3_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -6)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 3)


def score_error_bound(qI, w, kI, nv, rel=1e-5):
    """A posteriori bound on |fp32 score - exact score| per entry:
    rel * sum_h |w_h| sum_j |qI_hj kI_sj|."""
    if nv == 0:
        return np.zeros(0)
    return rel * (np.abs(kI[:nv]) @ np.abs(qI).T) @ np.abs(w)


def mx_score_bound(inp, b, ref, nv):
    """Bound on |GPU bf16 score - quantised-oracle bf16 score| for MXFP4 keys:
    the fp32 accumulation error of the exact E2M1 products plus one bf16 step
    (the two sides may round to neighbouring bf16 values)."""
    from oracle import pipeline as OP
    kI, _, _ = OP.mxfp4_values(inp["kI"][b][:nv])
    qI, _, _ = OP.mxfp4_values(inp["qI"][b, 0])
    e = score_error_bound(qI, inp["w"][b, 0], kI, nv)
    return bf16_ulp(np.abs(ref) + e) + e


def report(name, **kv):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)
