"""Pins for the oracle's element formats (E2M1, E4M3FN, bf16 rounding)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4 as O
from tests import exact as X


def test_e2m1_grid_is_the_e2m1_format():
    # OCP E2M1: the eight magnitudes of a float with 2 exponent bits (bias 1)
    # and 1 mantissa bit.
    assert [Fraction(v) for v in O.E2M1_GRID] == X.E2M1
    assert list(O.E2M1_GRID) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_decode_matches_torch_for_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], ours[~nan])
    assert O.E4M3_FINITE[-1] == 448.0 and O.E4M3_FINITE[1] == 2.0 ** -9
    assert np.all(np.diff(O.E4M3_FINITE) > 0)


def test_e4m3_widens_to_bf16_exactly_like_torch():
    # FP8 K/V enter the encoder as bf16; torch's float8_e4m3fn -> bfloat16
    # cast is an independent implementation of that widening
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.bfloat16)
    ours = O.e4m3_codes_to_bf16_bits(codes)
    assert np.array_equal(ref.view(torch.int16).numpy().view(np.uint16), ours)
    # -0, 2**-9 (smallest subnormal) and -448
    assert O.e4m3_codes_to_bf16_bits(np.array([0x80, 0x01, 0xFE], np.uint8)).tolist() == \
        [0x8000, 0x3B00, 0xC3E0]
    with pytest.raises(ValueError):
        O.e4m3_codes_to_bf16_bits(np.array([0x7F], np.uint8))


def test_e4m3_rounding_of_exact_values_matches_torch():
    # every exact product e2m1 * e4m3 * gs for a few gs whose products fit
    # fp32 exactly (so torch's fp32 -> float8_e4m3fn cast sees the value
    # itself); torch gives NaN past 464, where the oracle saturates to 448
    for gs in (1.0, 0.375, 2.0 ** -5, 3.0, 1.25):
        v = np.outer(O.E2M1_GRID, O.E4M3_FINITE).reshape(-1) * gs
        v = np.concatenate([v, -v])
        keep = np.abs(v) < 464.0
        ref = torch.from_numpy(v[keep].astype(np.float32)).to(torch.float8_e4m3fn)
        ours = O.f64_to_e4m3_rne(v[keep])
        assert np.array_equal(ref.view(torch.uint8).numpy(), ours), gs
    # saturation, signed zeros, and the subnormal ties: 2^-10 lies halfway
    # between 0 and 2^-9 (code 0 is even), 3 * 2^-10 between codes 1 and 2
    assert O.f64_to_e4m3_rne(np.array([464.0, 1e30, -1e30, -0.0, 0.0, 2.0 ** -10,
                                       3 * 2.0 ** -11, 3 * 2.0 ** -10])).tolist() == \
        [0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x01, 0x02]


def test_e4m3_encode_matches_torch_on_every_bf16_value():
    # every non-negative finite bf16 value up to 464 (above that torch gives
    # NaN, the oracle saturates); torch's fp32 -> e4m3fn cast rounds to
    # nearest even
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    keep = vals <= 464.0
    vals = vals[keep]
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    ours = O.round_half_even_to_grid(vals, O.E4M3_FINITE)
    assert np.array_equal(ref.numpy().astype(np.int64), ours)


def test_e4m3_saturates_above_448():
    q = np.array([448.0, 464.0, 465.0, 1e6, 3e38])
    assert list(O.round_half_even_to_grid(q, O.E4M3_FINITE)) == [126] * 5


def test_e2m1_rounding_ties_and_brute_force():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, code in ties.items():
        assert O.round_half_even_to_grid(np.array([y]), O.E2M1_GRID)[0] == code
    rng = np.random.default_rng(0)
    ys = np.concatenate([rng.uniform(0, 8, 4000), np.arange(0, 8.01, 0.125),
                         np.nextafter(np.array(list(ties)), 0),
                         np.nextafter(np.array(list(ties)), 10), [1e30]])
    ours = O.round_half_even_to_grid(ys, O.E2M1_GRID)
    ref = [X.nearest_even(Fraction(float(y)), X.E2M1) for y in ys]
    assert list(ours) == ref


def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # fp32 subnormals
        np.array([0.0, -0.0, 1.00390625, 1.01171875, 3.3e38, -3.39e38,
                  np.float32(3.3961e38)], dtype=np.float32),
    ]).astype(np.float32)
    ours = O.f64_to_bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_exact_on_wide_products():
    # products of up to 30 significant bits (the dequantizer's case), rounded
    # once: compare with exhaustive exact-rational rounding
    rng = np.random.default_rng(2)
    gs = rng.uniform(0.5, 2.0, 300).astype(np.float32).astype(np.float64) * \
        2.0 ** rng.integers(-140, 120, 300)
    gs = gs.astype(np.float32).astype(np.float64)
    gs = gs[gs > 0]
    c = rng.choice(O.E2M1_GRID[1:], gs.shape[0])
    s = rng.choice(O.E4M3_FINITE[1:], gs.shape[0])
    sign = rng.choice([-1.0, 1.0], gs.shape[0])
    v = sign * c * s * gs  # exact in fp64
    ours = O.f64_to_bf16_rne(v)
    ref = [X.bf16_round_exact(Fraction(float(a))) for a in v]
    assert list(ours.astype(np.int64)) == ref


def test_bf16_rne_overflow_and_signed_zero():
    # largest bf16 is 2**128 - 2**120; the midpoint to 2**128 is 2**128 - 2**119
    big = np.array([2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100, 2.0 ** 128 - 2.0 ** 119,
                    3.4e38, -3.4e38])
    out = O.f64_to_bf16_rne(big)
    assert out[0] == 0x7F7F  # below the midpoint
    assert out[1] == 0x7F80  # the midpoint: ties to even (odd mantissa 0x7F) -> inf
    assert out[2] == 0x7F80 and out[3] == 0xFF80
    assert O.f64_to_bf16_rne(np.array([-0.0]))[0] == 0x8000
