"""Grouped output projection on the GPU against the fp64 oracle.

Tolerance (derived from the arithmetic, not fitted): u is accumulated in fp32
over K1 terms and rounded to bf16 (8 significant bits), y is accumulated in
fp32 over g*d_g terms (and rounded to bf16 when y_t is bf16):
  |u_gpu - u| <= 2^-8 |u| + K1 2^-24 (|o| . |W_a|^T)
  |y_gpu - y| <= |W_b| . e_u + Ku 2^-24 ((|u| + e_u) . |W_b|^T) [+ 2^-8 |y|]
"""
import numpy as np
import pytest
import torch

import csa_inputs as I
import long_context_sparse_10_amd as L
from oracle import csa as O
from tests.gpu_util import dev, report

pytestmark = pytest.mark.gpu


def _case(rng, R, nh, c, g, d_g, d, dtype):
    K1, Ku = nh // g * c, g * d_g
    o = rng.standard_normal((R, nh, c)).astype(np.float32)
    W_a = (rng.standard_normal((g, d_g, K1)) / np.sqrt(K1)).astype(np.float32)
    W_b = (rng.standard_normal((d, Ku)) / np.sqrt(Ku)).astype(np.float32)
    if dtype == "bf16":
        o, W_a, W_b = I.cast(o, "bf16"), I.cast(W_a, "bf16"), I.cast(W_b, "bf16")
    return o, W_a, W_b


def _run(o, W_a, W_b, dtype, y_t, reps=1):
    d_ = dev()
    R, nh, c = o.shape
    g, d_g, _ = W_a.shape
    d = W_b.shape[0]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(d_).to(tdt)
    To, Ta, Tb = to(o), to(W_a), to(W_b)
    ydt = torch.bfloat16 if y_t == L.BF16 else torch.float32
    outs = []
    ws = None
    for _ in range(reps):
        y = torch.full((R, d), float("nan"), dtype=ydt, device=d_)
        ws = L.grouped_out_proj(To, L.BF16 if dtype == "bf16" else L.F32, R, nh, c, g, d_g, Ta, Tb,
                                d, y, y_t, ws)
        torch.cuda.synchronize()
        outs.append(y)
    return outs


def _bound(o, W_a, W_b, u, y, bf16_u, bf16_y):
    R, nh, c = o.shape
    g, d_g, K1 = W_a.shape
    Ku = g * d_g
    au = np.abs(O.grouped_out_proj(np.abs(o), np.abs(W_a), np.eye(Ku))[1])  # |o| . |W_a|^T
    e_u = (2.0 ** -8 * np.abs(u) if bf16_u else 0.0) + K1 * 2.0 ** -24 * au
    aW = np.abs(W_b)
    e_y = e_u @ aW.T + Ku * 2.0 ** -24 * ((np.abs(u) + e_u) @ aW.T)
    if bf16_y:
        e_y = e_y + 2.0 ** -8 * np.abs(y)
    return e_y


@pytest.mark.parametrize("R,nh,c,g,d_g,d,y_t", [
    (32, 64, 512, 8, 1024, 4096, L.BF16),     # Flash decode batch: skinny kernel, 2 m-tiles
    (37, 64, 512, 8, 1024, 4096, L.F32),      # ragged rows: 4 m-tiles, 27 rows unused
    (1, 64, 512, 8, 1024, 4096, L.BF16),      # one row
    (4, 128, 512, 16, 1024, 7168, L.BF16),    # Pro: 16 groups, d = 7168
    (300, 64, 512, 8, 1024, 4096, L.BF16),    # many rows: tiled kernel, ragged tiles
    (130, 16, 64, 2, 96, 200, L.F32),         # tiled kernel, N not a multiple of 128
])
def test_grouped_out_proj_bf16_vs_oracle(R, nh, c, g, d_g, d, y_t):
    rng = np.random.default_rng(R * 7 + d)
    o, W_a, W_b = _case(rng, R, nh, c, g, d_g, d, "bf16")
    y1, y2 = _run(o, W_a, W_b, "bf16", y_t, reps=2)
    assert torch.equal(y1, y2)                                   # run-to-run bitwise
    y_ref, u_ref = O.grouped_out_proj(o, W_a, W_b)
    got = y1.double().cpu().numpy()
    bound = _bound(o, W_a, W_b, u_ref, y_ref, True, y_t == L.BF16)
    err = np.abs(got - y_ref)
    report("grouped out proj", R=R, nh=nh, g=g, d_g=d_g, d=d, max_abs=float(err.max()),
           max_err_over_bound=float((err / bound).max()))
    assert np.all(err <= bound)


def test_grouped_out_proj_f32():
    rng = np.random.default_rng(5)
    o, W_a, W_b = _case(rng, 5, 8, 16, 4, 8, 12, "f32")
    (y,) = _run(o, W_a, W_b, "f32", L.F32)
    y_ref, u_ref = O.grouped_out_proj(o, W_a, W_b)
    bound = _bound(o, W_a, W_b, u_ref, y_ref, False, False)
    err = np.abs(y.double().cpu().numpy() - y_ref)
    report("grouped out proj f32", max_abs=float(err.max()))
    assert np.all(err <= bound + 1e-12)
