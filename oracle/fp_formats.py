"""Number formats used by the layer: OCP FP8 E4M3 (the "FN" variant), BF16,
and the MXFP4 weight format (E2M1 elements with E8M0 block scales).

TEST INFRASTRUCTURE ONLY (see the package docstring).

E4M3: the pages fix the format through its largest finite value, 448
(TensorRT-LLM PR #21250, review comment on the quantizer constants, which
takes it from ``float8_e4m3fn``). That is the OCP E4M3 encoding: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2**-9, no
infinities, and S.1111.111 as the only NaN. The pages say nothing about ties,
saturation or negative zero; the reading taken here is round to nearest with
ties to the even code, saturation to +-448, and a sign-preserving zero.

BF16 is held as uint16 bit patterns because numpy has no bfloat16 type.

MXFP4: the pages name FP4 weights only (vLLM PR #59128, description: prefix
sums for FP4 weights on SM10.x) and give no encoding. The reading taken is
the OCP Microscaling (MX) v1.0 format: E2M1 elements (1 sign bit, 2 exponent
bits with bias 1, 1 mantissa bit; exponent 0 holds the subnormal m * 0.5;
magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN) sharing one
E8M0 scale (2**(b - 127), byte 255 = NaN) per 32 consecutive elements along
K. Two elements share a byte, the even-K element in the low nibble.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode E4M3 byte codes to float64, straight from the field layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    subnormal = man * 2.0 ** -9
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# The 127 finite non-negative codes 0x00..0x7E decode to strictly increasing
# values, so encoding is a nearest-neighbour search in this table.
_POS_CODES = np.arange(0, 127, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES.astype(np.uint8))


def e4m3_encode(x):
    """Round float32 values to E4M3 codes (nearest, ties to even code).

    Works by table search rather than bit manipulation: for |x| the two
    neighbouring representable magnitudes are found, the nearer one wins, and
    an exact tie goes to the code whose mantissa LSB (= code LSB) is zero.
    Magnitudes at or above 448 saturate to 448 (code 0x7E). The sign bit is
    kept even when the magnitude rounds to zero. Differences are formed in
    float64, where they are exact for float32 inputs of this range.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    neg = np.signbit(x).astype(np.int64)
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a >= E4M3_MAX, 126, code)
    return (code | (neg << 7)).astype(np.uint8)


def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_from_f64(x):
    """Round float64 values to BF16 (nearest, ties to even), as uint16 bits.

    The rounding is done once, directly on the float64 significand, so there
    is no double rounding through float32. Normal BF16 magnitudes keep 7 of
    the 52 stored fraction bits; below 2**-126 the BF16 grid is the fixed
    subnormal quantum 2**-133. Results past the largest finite BF16 become
    infinity, as IEEE rounding prescribes. NaN input is outside the contract.
    """
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint32)
    mag = bits & np.uint64(0x7FFFFFFFFFFFFFFF)
    drop = np.uint64(45)
    lsb = (mag >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)
    rounded = ((mag + half_minus_one + lsb) >> drop) << drop
    y = rounded.view(np.float64)
    ax = np.abs(x)
    tiny = ax < 2.0 ** -126
    y_tiny = np.rint(ax * 2.0 ** 133) * 2.0 ** -133
    y = np.where(tiny, y_tiny, y)
    y = np.where(y >= 2.0 ** 128, np.inf, y)
    f = y.astype(np.float32)  # exact: y is on the BF16 grid (or inf)
    top = (f.view(np.uint32) >> 16).astype(np.uint32)
    return (top | (sign << 15)).astype(np.uint16)


def e2m1_decode(nibbles):
    """Decode E2M1 4-bit codes (0..15) to float64, straight from the field layout."""
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 0xF
    sign = (c >> 3) & 1
    exp = (c >> 1) & 0x3
    man = c & 0x1
    subnormal = man * 0.5
    normal = (1.0 + man / 2.0) * np.exp2(exp.astype(np.float64) - 1.0)
    mag = np.where(exp == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag)


def e8m0_decode(codes):
    """Decode E8M0 scale bytes to float64: 2**(b - 127); 255 is NaN."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def fp4_unpack(packed):
    """[..., K/2] bytes -> [..., K] E2M1 codes; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
