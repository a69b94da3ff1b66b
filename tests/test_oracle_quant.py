"""Pins for the oracle's 1x128 activation quantization rule."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact import f32_bits_of, round_binary

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_rule_cases.json")


def _bf16_bits(values):
    t = torch.tensor(values, dtype=torch.float32)
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), t), "golden inputs must be exact in BF16"
    return b.view(torch.int16).numpy().view(np.uint16)


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
def test_hand_derived_cases(case, fmt):
    x = np.zeros(128, np.float32)
    for i, v in case["x"].items():
        x[int(i)] = v
    xb = oracle.bf16_bits_to_f64(_bf16_bits(x.tolist())).astype(np.float32)
    q, s = oracle.quantize_groups(xb[None, :], fmt)
    exp = case[fmt]
    if fmt == "ue8m0":
        assert s.dtype == np.uint8 and int(s[0, 0]) == exp["byte"]
    else:
        assert s.dtype == np.float32 and f32_bits_of(float(s[0, 0])) == int(exp["scale_bits"], 16)
    want = np.zeros(128, np.uint8)
    for i, c in exp["codes"].items():
        want[int(i)] = int(c, 16)
    assert np.array_equal(q[0], want)


def _random_groups(rows, seed, scale=1.0):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((rows, 512)) * scale).astype(np.float32)
    return oracle.bf16_bits_to_f64(
        torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ).astype(np.float32)


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
def test_codes_are_nearest_to_exact_quotient_of_stored_scale(fmt):
    """Each code is the E4M3 value nearest the float32 quotient x/s, where s
    is checked against its exact definition with rational arithmetic."""
    x = _random_groups(6, 11, scale=3.0)
    q, stored = oracle.quantize_groups(x, fmt)
    s = oracle.scales_to_f64(stored, fmt)  # [G, rows]
    for r in range(x.shape[0]):
        for gi in range(x.shape[1] // 128):
            grp = x[r, gi * 128:(gi + 1) * 128]
            amax = Fraction(float(np.max(np.abs(grp))))
            s_exact = max(round_binary(amax / 448, 23, -126),
                          round_binary(Fraction(1, 229376), 23, -126))
            if fmt != "fp32":
                p = Fraction(1)
                while p < s_exact:
                    p *= 2
                while p / 2 >= s_exact:
                    p /= 2
                s_exact = p
            assert Fraction(float(s[gi, r])) == s_exact
            for j in range(0, 128, 7):
                quot = round_binary(Fraction(float(grp[j])) / s_exact, 23, -126)
                code = int(q[r, gi * 128 + j])
                val = Fraction(float(oracle.e4m3_decode(code)))
                # no representable E4M3 magnitude is strictly nearer
                table = [Fraction(float(v)) for v in oracle.e4m3_decode(np.arange(127, dtype=np.uint8))]
                best = min(abs(abs(quot) - t) for t in table)
                assert abs(abs(quot) - abs(val)) == best
                assert (code >> 7) == (1 if float(grp[j]) < 0 or (grp[j] == 0 and np.signbit(grp[j])) else 0)


@pytest.mark.parametrize("fmt", ["pow2", "ue8m0"])
def test_pow2_invariants(fmt):
    x = _random_groups(64, 12, scale=7.0)
    _, s32 = oracle.quantize_groups(x, "fp32")
    q, sp = oracle.quantize_groups(x, fmt)
    s = s32.astype(np.float64)
    p = oracle.scales_to_f64(sp, fmt)
    assert np.all(p >= s) and np.all(p < 2 * s)
    m, _ = np.frexp(p)
    assert np.all(m == 0.5)  # exact powers of two
    # nothing saturates: every code decodes to at most 448 and no group
    # reaches 448 unless amax/scale is exactly 448
    assert np.all(np.abs(oracle.e4m3_decode(q)) <= 448)


def test_ue8m0_and_pow2_give_identical_codes():
    x = _random_groups(32, 13)
    q1, s1 = oracle.quantize_groups(x, "pow2")
    q2, s2 = oracle.quantize_groups(x, "ue8m0")
    assert np.array_equal(q1, q2)
    assert np.array_equal(np.ldexp(1.0, s2.astype(np.int64) - 127), s1.astype(np.float64))


def test_floor_binds_only_below_amax_one_over_512():
    # amax/448 <= 1/229376  <=>  amax <= 1/512 (at equality both sides agree)
    for amax, floored in [(2.0 ** -10, True), (2.0 ** -9 * 0.99, True), (2.0 ** -9, True), (2.0 ** -9 * 1.01, False), (1.0, False)]:
        s, _ = oracle.group_scales(np.float32(amax), "fp32")
        assert (float(s) == float(np.float32(1) / np.float32(229376))) == floored


def test_scale_layout_is_group_major():
    x = _random_groups(5, 14)
    q, s = oracle.quantize_groups(x, "fp32")
    assert s.shape == (4, 5)
    for r in range(5):
        q_r, s_r = oracle.quantize_groups(x[r:r + 1], "fp32")
        assert np.array_equal(q_r[0], q[r])
        assert np.array_equal(s_r[:, 0], s[:, r])
