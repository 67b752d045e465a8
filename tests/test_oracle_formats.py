"""Pins of the oracle's storage formats against the format definitions and
independent library conversions (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import formats as F


# ----------------------------------------------------------------- bf16
def test_bf16_matches_torch_conversion():
    """torch's fp32 -> bfloat16 cast (RNE) is an independent implementation."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),    # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        # exact ties: bf16 value + half an ulp
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    codes = F.bf16_encode(x.astype(np.float64))
    ref_codes = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(codes, ref_codes)
    np.testing.assert_array_equal(F.bf16_decode(codes), ref)


def test_bf16_overflow_to_inf():
    assert F.bf16_round(np.array([3.5e38]))[0] == np.inf
    assert F.bf16_round(np.array([-3.5e38]))[0] == -np.inf


# ----------------------------------------------------------------- e4m3
def test_e4m3_named_values():
    """OCP FP8 E4M3 spec constants: max normal 448 = S.1111.110, min normal 2^-6
    = S.0001.000, min subnormal 2^-9 = S.0000.001, 1.0 = S.0111.000; S.1111.111
    is NaN."""
    assert F.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert F.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert F.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert F.e4m3_decode(np.uint8(0x38)) == 1.0
    assert F.e4m3_decode(np.uint8(0xB8)) == -1.0
    assert np.isnan(F.e4m3_decode(np.uint8(0x7F)))
    assert np.isnan(F.e4m3_decode(np.uint8(0xFF)))
    assert F.e4m3_encode(np.array([448.0]))[0] == 0x7E
    assert F.e4m3_encode(np.array([1.0]))[0] == 0x38


def test_e4m3_round_trip_all_codes_and_monotone():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    np.testing.assert_array_equal(F.e4m3_encode(vals), codes)
    pos = np.sort(F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    assert np.all(np.diff(pos) > 0) and pos.size == 127


def test_e4m3_matches_torch_in_range():
    """torch.float8_e4m3fn conversion (RNE) is independent; compare within the
    finite range (torch does not saturate above 448)."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.uniform(-448, 448, 5000),
                        rng.standard_normal(2000) * 1e-3]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.e4m3_round(x.astype(np.float64)), ref)
    ref_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e4m3_encode(x.astype(np.float64)), ref_codes)


def test_e4m3_ties_and_saturation():
    # spacing in [1, 2) is 1/8: 1 + 1/16 ties to 1 (even mantissa), 1 + 3/16 to 1.25
    assert F.e4m3_round(np.array([1.0625]))[0] == 1.0
    assert F.e4m3_round(np.array([1.1875]))[0] == 1.25
    assert F.e4m3_round(np.array([1000.0, -1e9]))[0] == 448.0
    assert F.e4m3_round(np.array([-1e9]))[0] == -448.0
    assert F.e4m3_round(np.array([2.0 ** -10]))[0] == 0.0          # tie with 0 -> even
    assert F.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8  # 1.5 ulps -> 2


# ----------------------------------------------------------------- E2M1 / MXFP4
E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX spec, FP4 E2M1 values


def test_e2m1_grid_and_codes():
    np.testing.assert_array_equal(F.e2m1_decode(np.arange(8, dtype=np.uint8)), E2M1_GRID)
    np.testing.assert_array_equal(F.e2m1_decode(np.arange(8, 16, dtype=np.uint8)),
                                  [-v for v in E2M1_GRID])
    np.testing.assert_array_equal(F.e2m1_encode(np.array(E2M1_GRID)), np.arange(8))


@pytest.mark.parametrize("x,want", [
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),
    (5.01, 6.0), (7.0, 6.0), (100.0, 6.0), (0.26, 0.5), (-2.6, -3.0),
])
def test_e2m1_rne_ties_and_saturation(x, want):
    assert F.e2m1_round(np.array([x]))[0] == want


def test_mxfp4_scale_rule_and_packing():
    """Scale 2^(floor(log2 amax) - 2) per 32-block; even element in the low nibble."""
    blk = np.zeros((1, 64))
    blk[0, 0] = 1.0          # block 0: amax 1 -> exponent -2 -> 1.0 / 0.25 = 4 -> code 6
    blk[0, 1] = -0.25        # -> -1.0 -> code 0b1010
    blk[0, 32] = 6.0         # block 1: amax 6 -> exponent 0 -> 6 -> code 7
    blk[0, 33] = 7.9         # same block, saturates to 6 -> code 7
    packed, scales = F.mxfp4_quantize(blk)
    assert scales.tolist() == [[127 - 2, 127 + 0]]
    assert packed[0, 0] == (6 | (0b1010 << 4))
    assert packed[0, 16] == (7 | (7 << 4))
    deq = F.mxfp4_dequantize(packed, scales)
    assert deq[0, 0] == 1.0 and deq[0, 1] == -0.25 and deq[0, 32] == 6.0 and deq[0, 33] == 6.0


def test_mxfp4_zero_block_and_idempotence():
    packed, scales = F.mxfp4_quantize(np.zeros((2, 32)))
    assert np.all(packed == 0) and np.all(scales == 0)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128))
    p1, s1 = F.mxfp4_quantize(x)
    d1 = F.mxfp4_dequantize(p1, s1)
    p2, s2 = F.mxfp4_quantize(d1)
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)
    # error bound: half a grid step (at most 1 scale unit, between 4 and 6);
    # scaled magnitudes in (6, 8) saturate to 6, an error below 2 scale units
    scale = np.repeat(np.ldexp(1.0, s1.astype(np.int64) - 127), 32, axis=-1)
    err = np.abs(x - d1)
    sat = np.abs(x) > 6 * scale
    assert np.all(err[~sat] <= 1.0 * scale[~sat])
    assert np.all(err[sat] < 2.0 * scale[sat]) and sat.any()


def test_fp8mix_row_bytes_and_round_trip():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 512))
    rows = F.fp8mix_encode(x, 64)
    assert rows.shape == (4, 576)
    np.testing.assert_array_equal(F.fp8mix_decode(rows, 512, 64), F.fp8mix_round(x, 64))
