"""Pins for the oracle's number formats (E4M3 codec, BF16 rounding)."""

from fractions import Fraction

import numpy as np
import torch

import oracle
from tests.exact import round_binary, to_bf16_bits

ALL = np.arange(256, dtype=np.uint8)


def test_e4m3_decode_named_values():
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0                      # largest finite, the pages' 448
    assert d(0xFE) == -448.0
    assert d(0x38) == 1.0                        # exponent field 7 = bias
    assert d(0x01) == 2.0 ** -9                  # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9              # largest subnormal
    assert d(0x08) == 2.0 ** -6                  # smallest normal
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0x44) == 3.0 and d(0xC2) == -2.5


def test_e4m3_decode_matches_torch_for_all_codes():
    ours = oracle.e4m3_decode(ALL)
    lib = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ours)
    assert np.array_equal(nan, np.isnan(lib))
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_e4m3_positive_codes_strictly_increasing():
    v = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_e4m3_roundtrip_every_finite_code():
    finite = ALL[~np.isnan(oracle.e4m3_decode(ALL))]
    back = oracle.e4m3_encode(oracle.e4m3_decode(finite).astype(np.float32))
    assert np.array_equal(back, finite)


def _neighbour_midpoints():
    v = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2  # exactly representable in float32
    return v, mids


def test_e4m3_ties_go_to_even_code():
    v, mids = _neighbour_midpoints()
    got = oracle.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect.astype(np.uint8))
    got_neg = oracle.e4m3_encode(-mids.astype(np.float32))
    assert np.array_equal(got_neg, (expect | 0x80).astype(np.uint8))


def test_e4m3_one_ulp_off_midpoint_goes_to_nearest():
    v, mids = _neighbour_midpoints()
    m32 = mids.astype(np.float32)
    below = np.nextafter(m32, np.float32(0))
    above = np.nextafter(m32, np.float32(np.inf))
    lo = np.arange(126)
    assert np.array_equal(oracle.e4m3_encode(below), lo.astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode(above), (lo + 1).astype(np.uint8))


def test_e4m3_saturates_and_keeps_sign_of_zero():
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3e38], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    tiny = np.array([0.0, 1e-30, 2.0 ** -10, 2.0 ** -11], np.float32)
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.uniform(-448, 448, 200000),
        g.standard_normal(200000) * 10,
        g.standard_normal(50000) * 1e-3,
        g.standard_normal(50000) * 1e-6,
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), lib)


def test_bf16_from_f64_matches_torch_on_float32_values():
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(100000) * s for s in (1e-40, 1e-3, 1.0, 1e5, 1e30)])
    x = x.astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f64(x.astype(np.float64)), lib)


def test_bf16_from_f64_rounds_once_from_fp64():
    # Values just off a BF16 midpoint by less than half a float32 ulp: going
    # through float32 first would land on the midpoint and round to even.
    g = np.random.default_rng(3)
    base = oracle.bf16_bits_to_f64(g.integers(0x3000, 0x4F00, 2000).astype(np.uint16))
    ulp = np.array([float(round_binary(Fraction(b), 7, -126)) for b in base])  # == base
    assert np.array_equal(ulp, base)
    step = np.ldexp(1.0, np.frexp(base)[1] - 8)   # BF16 ulp of base
    mid = base + step / 2
    eps = np.ldexp(1.0, np.frexp(base)[1] - 40)
    vals = np.concatenate([mid, mid + eps, mid - eps, -(mid + eps), base + step * 0.3])
    got = oracle.bf16_from_f64(vals)
    want = np.array([to_bf16_bits(Fraction(float(v))) | (0x8000 if v < 0 else 0)
                     for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_from_f64_random_fp64_exact():
    g = np.random.default_rng(4)
    vals = np.concatenate([g.standard_normal(3000) * 10.0 ** g.integers(-45, 30, 3000)])
    got = oracle.bf16_from_f64(vals)
    want = np.array([to_bf16_bits(Fraction(float(v))) | (0x8000 if v < 0 else 0)
                     for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_subnormal_and_zero():
    vals = np.array([0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -127])
    got = oracle.bf16_from_f64(vals)
    assert list(got) == [0x0000, 0x8000, 0x0001, 0x0000, 0x0002, 0x0040]
