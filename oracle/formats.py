"""Exact numpy emulation of the storage formats the compressed caches use.

TEST INFRASTRUCTURE ONLY. This module is part of the fp64 CPU oracle. Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the product path never does.

Formats (all rounding is round-to-nearest, ties-to-even):

* bf16 -- 8 significant bits, IEEE-style exponent range of fp32.  The pages put
  the RoPE dimensions of the KV cache and the index scores in BF16
  (Evidence Ledger page, "Shared attention details" / Section 2.3.4 and
  Section 5.2.1).
* e4m3 -- OCP FP8 "E4M3FN": bias 7, three mantissa bits, no infinities, largest
  finite value 448; values beyond are saturated to +-448 (our reading: the pages
  give FP8 storage with no scale bytes, 576 B per entry: "DeepSeek V4 study"
  (shuhuayu), section 06 "What grows with context").
* E2M1 / MXFP4 -- OCP MX FP4 elements {0, 0.5, 1, 1.5, 2, 3, 4, 6} in blocks of
  32 sharing one e8m0 power-of-two scale 2^(floor(log2 amax) - 2) (Evidence
  Ledger page, Section 5.2.1: MXFP4 (E2M1) in 1x32 tiles).  Elements saturate
  at +-6.  Packing: two codes per byte, the even element in the low nibble.

The value-level functions return float64 arrays holding exactly representable
values of the format; the code-level functions produce the stored bytes.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# generic binary floating-point rounding
# --------------------------------------------------------------------------


def _round_binary(x, mant_bits: int, emin: int, max_finite: float, saturate: bool):
    """Round float64 ``x`` to a binary format with ``mant_bits`` stored mantissa
    bits and smallest normal exponent ``emin`` (subnormals below), RNE."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)            # ax = f * 2**e, f in [0.5, 1)
    e = np.maximum(e - 1, emin)     # exponent of the leading bit, clamped for subnormals
    ulp = np.ldexp(1.0, e - mant_bits)
    q = np.rint(ax / ulp) * ulp     # np.rint rounds half to even
    if saturate:
        q = np.minimum(q, max_finite)
    else:
        q = np.where(q > max_finite, np.inf, q)
    q = np.where(np.isnan(x), np.nan, q)
    return np.copysign(q, x)


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x):
    """Nearest bf16 value (RNE, overflow to inf) of float64 ``x``."""
    return _round_binary(x, 7, -126, BF16_MAX, saturate=False)


def bf16_encode(x):
    """uint16 bf16 codes of ``x`` (rounded RNE first)."""
    v = bf16_round(x).astype(np.float32)     # exact: bf16 values are fp32 values
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_decode(codes):
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << 16
    return c.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# OCP e4m3 (FN variant, as on gfx950), saturating
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_round(x):
    return _round_binary(x, 3, -6, E4M3_MAX, saturate=True)


def e4m3_encode(x):
    """uint8 e4m3 codes: sign | exponent(4, bias 7) | mantissa(3)."""
    v = e4m3_round(x)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    normal = a >= 2.0 ** -6
    _, e = np.frexp(np.where(normal, a, 1.0))
    e = e - 1
    mant_n = np.rint(a / np.ldexp(1.0, e) * 8.0 - 8.0)
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, mant_n, np.rint(a / 2.0 ** -9))
    return (sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 0xF) & (mf == 0x7), np.nan, val)
    return s * val


# --------------------------------------------------------------------------
# E2M1 (FP4) and MXFP4 blocks
# --------------------------------------------------------------------------
E2M1_MAX = 6.0
MX_BLOCK = 32


def e2m1_round(x):
    return _round_binary(x, 1, 0, E2M1_MAX, saturate=True)


def e2m1_encode(x):
    """4-bit codes (uint8 0..15): sign | exponent(2, bias 1) | mantissa(1)."""
    v = e2m1_round(x)
    sign = (np.signbit(v)).astype(np.uint8) << 3
    a = np.abs(v)
    normal = a >= 1.0
    _, e = np.frexp(np.where(normal, a, 1.0))
    e = e - 1
    mant_n = np.rint(a / np.ldexp(1.0, e) * 2.0 - 2.0)
    exp_field = np.where(normal, e + 1, 0)
    mant = np.where(normal, mant_n, np.rint(a / 0.5))
    return (sign | (exp_field.astype(np.uint8) << 1) | mant.astype(np.uint8)).astype(np.uint8)


def e2m1_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    ef = (c >> 1) & 0x3
    mf = c & 0x1
    val = np.where(ef == 0, mf * 0.5, (1.0 + mf / 2.0) * np.ldexp(1.0, ef - 1))
    return s * val


def mx_scale_exponent(block_amax):
    """Shared exponent of an MX block: floor(log2(amax)) - 2 (E2M1 emax is 2);
    an all-zero block gets the smallest scale 2^-127.  Clamped to e8m0 range."""
    a = np.asarray(block_amax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    ex = np.where(a > 0, (e - 1) - 2, -127)
    return np.clip(ex, -127, 127).astype(np.int64)


def mxfp4_quantize(x):
    """Quantize rows of ``x`` (last dim a multiple of 32) to MXFP4.

    Returns ``(packed, scales)``: packed uint8 [..., c/2] with the even element in
    the low nibble, and e8m0 scale bytes uint8 [..., c/32] (byte = exponent + 127).
    """
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    assert c % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (c // MX_BLOCK, MX_BLOCK))
    ex = mx_scale_exponent(np.max(np.abs(blocks), axis=-1))
    scaled = blocks / np.ldexp(1.0, ex)[..., None]
    codes = e2m1_encode(scaled).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (ex + 127).astype(np.uint8)


def mxfp4_dequantize(packed, scales):
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0xF
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    vals = e2m1_decode(codes)
    c = vals.shape[-1]
    ex = np.asarray(scales, dtype=np.int64) - 127
    blocks = vals.reshape(vals.shape[:-1] + (c // MX_BLOCK, MX_BLOCK))
    return (blocks * np.ldexp(1.0, ex)[..., None]).reshape(vals.shape)


# --------------------------------------------------------------------------
# mixed FP8 / BF16 KV row: [c - d_r e4m3 bytes | d_r bf16]
# --------------------------------------------------------------------------


def fp8mix_encode(x, d_r):
    """Encode KV rows as (c-d_r) e4m3 bytes followed by d_r little-endian bf16."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    body = e4m3_encode(x[..., : c - d_r])
    rope = bf16_encode(x[..., c - d_r:]).view(np.uint8).reshape(x.shape[:-1] + (2 * d_r,))
    return np.concatenate([body, rope], axis=-1)


def fp8mix_decode(rows, c, d_r):
    rows = np.asarray(rows, dtype=np.uint8)
    body = e4m3_decode(rows[..., : c - d_r])
    rope = bf16_decode(np.ascontiguousarray(rows[..., c - d_r:]).view(np.uint16))
    return np.concatenate([body, rope], axis=-1)


def fp8mix_round(x, d_r):
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    return np.concatenate([e4m3_round(x[..., : c - d_r]), bf16_round(x[..., c - d_r:])], axis=-1)
