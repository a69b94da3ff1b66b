"""Pins for the oracle's reciprocal rounding convention (TensorRT-LLM PR
#21250, rounding-fix commit message: the fused CUTLASS op's quantizers
multiply by a correctly rounded 448 / amax and store its reciprocal, the
SwiGLU output is rounded to BF16 before quantization; review comment on the
block-scale order: the two scales are multiplied first)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact import f32_bits_of, round_binary, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_reciprocal_cases.json")


def _bf16_exact(values):
    t = torch.tensor(values, dtype=torch.float32)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t), "inputs must be BF16 values"
    return t.numpy()


def _cases():
    with open(GOLDEN) as f:
        return [(c, r, fmt) for c in json.load(f)["cases"] for r in ("reciprocal", "divide")
                for fmt in c[r]]


@pytest.mark.parametrize("case,rounding,fmt", _cases(),
                         ids=lambda v: v["name"] if isinstance(v, dict) else str(v))
def test_hand_derived_cases(case, rounding, fmt):
    x = np.zeros(128, np.float32)
    for i, v in case["x"].items():
        x[int(i)] = v
    x = _bf16_exact(x.tolist())
    q, s = oracle.quantize_groups(x[None, :], fmt, rounding)
    exp = case[rounding][fmt]
    if fmt == "ue8m0":
        assert int(s[0, 0]) == exp["byte"]
    else:
        assert f32_bits_of(float(s[0, 0])) == int(exp["scale_bits"], 16)
    want = np.zeros(128, np.uint8)
    for i, c in exp["codes"].items():
        want[int(i)] = int(c, 16)
    assert np.array_equal(q[0], want)


_TABLE = [Fraction(float(v)) for v in oracle.e4m3_decode(np.arange(127, dtype=np.uint8))]


def _nearest_code_ok(quot, code, x_is_negative):
    val = Fraction(float(oracle.e4m3_decode(code)))
    best = min(abs(abs(quot) - t) for t in _TABLE)
    if abs(quot) >= 448:
        return abs(val) == 448
    return abs(abs(quot) - abs(val)) == best and (code >> 7) == (1 if x_is_negative else 0)


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
def test_reciprocal_codes_follow_the_exact_definition(fmt):
    """Scale and codes against the convention's definition in exact rational
    arithmetic: inv = RN(448 / max(amax, 2^-9)), stored RN(1 / inv) (rounded up
    to a power of two for pow2/UE8M0), each code the E4M3 value nearest to
    RN(x * inv) (or x / s_pow2). Independent of numpy's float32 operations."""
    g = np.random.default_rng(21)
    x = (g.standard_normal((4, 512)) * 2.5).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    x[1, :128] *= 2.0 ** -12  # a group below the floor
    q, stored = oracle.quantize_groups(x, fmt, "reciprocal")
    s = oracle.scales_to_f64(stored, fmt)
    for r in range(x.shape[0]):
        for gi in range(4):
            grp = x[r, gi * 128:(gi + 1) * 128]
            amax = max(Fraction(float(np.max(np.abs(grp)))), Fraction(1, 512))
            inv = round_binary(Fraction(448) / amax, 23, -126)
            s_exact = round_binary(1 / inv, 23, -126)
            if fmt != "fp32":
                p = Fraction(1)
                while p < s_exact:
                    p *= 2
                while p / 2 >= s_exact:
                    p /= 2
                s_exact = p
            assert Fraction(float(s[gi, r])) == s_exact
            for j in range(0, 128, 5):
                xv = Fraction(float(grp[j]))
                quot = round_binary(xv * inv if fmt == "fp32" else xv / s_exact, 23, -126)
                assert _nearest_code_ok(quot, int(q[r, gi * 128 + j]), bool(np.signbit(grp[j])))


def test_reciprocal_and_divide_share_floor_and_pow2_scales_but_not_codes():
    g = np.random.default_rng(22)
    x = torch.from_numpy((g.standard_normal((64, 1024)) * 3).astype(np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()
    _, sd = oracle.quantize_groups(x, "fp32", "divide")
    _, sr = oracle.quantize_groups(x, "fp32", "reciprocal")
    # the two fp32 scales differ by at most one float32 ulp
    ratio = sr.astype(np.float64) / sd.astype(np.float64)
    assert np.all(np.abs(ratio - 1) <= 2.0 ** -23)
    qd, _ = oracle.quantize_groups(x, "fp32", "divide")
    qr, _ = oracle.quantize_groups(x, "fp32", "reciprocal")
    assert (qd != qr).sum() > 0 and (qd != qr).mean() < 1e-2


def test_reciprocal_swiglu_is_the_bf16_rounding_of_the_float32_value():
    """The convention's SwiGLU output is the float32 value of the divide
    convention, rounded to BF16 (checked against torch's BF16 cast, a library
    routine, and against exact rounding)."""
    g = np.random.default_rng(23)
    gate = torch.from_numpy(g.standard_normal(4096).astype(np.float32) * 3).to(torch.bfloat16).to(torch.float32).numpy()
    up = torch.from_numpy(g.standard_normal(4096).astype(np.float32) * 3).to(torch.bfloat16).to(torch.float32).numpy()
    for act, lim in (("swiglu", np.inf), ("swiglu_clamp", 2.0), ("swiglu_clamp_after_silu", 1.5)):
        y32 = oracle.swiglu(gate, up, act, lim, "divide")
        yr = oracle.swiglu(gate, up, act, lim, "reciprocal")
        ref = torch.from_numpy(y32).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(yr.view(np.uint32), ref.view(np.uint32))
        for i in range(0, 4096, 97):
            assert (yr.view(np.uint32)[i] >> 16) == to_bf16_bits(Fraction(float(y32[i])))


def test_reciprocal_gemm_forms_the_scale_product_in_float32():
    """C = bf16(sum_kb RN32(sa * sw) * P_kb), evaluated with exact rationals."""
    g = np.random.default_rng(24)
    m, n, kd = 3, 128, 384
    a = g.integers(0, 126, (m, kd)).astype(np.uint8)
    w = g.integers(0, 126, (n, kd)).astype(np.uint8) | (g.integers(0, 2, (n, kd)) << 7).astype(np.uint8)
    sa = (g.uniform(0.5, 2, (kd // 128, m)) * 1e-2).astype(np.float32)
    sw = (g.uniform(0.5, 2, (1, kd // 128)) * 1e-3).astype(np.float32)
    got = oracle.moe.gemm_rows(a, sa.astype(np.float64), w, sw, "reciprocal")
    da = [[Fraction(float(v)) for v in row] for row in oracle.e4m3_decode(a)]
    dw = [[Fraction(float(v)) for v in row] for row in oracle.e4m3_decode(w)]
    for i in range(m):
        for j in range(0, n, 9):
            acc = Fraction(0)
            for kb in range(kd // 128):
                part = sum(da[i][k] * dw[j][k] for k in range(kb * 128, kb * 128 + 128))
                acc += round_binary(Fraction(float(sa[kb, i])) * Fraction(float(sw[0, kb])), 23, -126) * part
            assert int(got[i, j]) == to_bf16_bits(acc)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_reciprocal_layer_equals_per_token_brute_force(fmt):
    g = np.random.default_rng(25)
    e, h, inter, k, t = 5, 256, 128, 2, 7
    from synth.gen import quantize_weight_blocks
    w1 = [quantize_weight_blocks((g.standard_normal((2 * inter, h)) * 0.05).astype(np.float32)) for _ in range(e)]
    w2 = [quantize_weight_blocks((g.standard_normal((h, inter)) * 0.05).astype(np.float32)) for _ in range(e)]
    W1 = (np.stack([a for a, _ in w1]), np.stack([b for _, b in w1]))
    W2 = (np.stack([a for a, _ in w2]), np.stack([b for _, b in w2]))
    x = oracle.bf16_from_f64(g.standard_normal((t, h)))
    ids = g.integers(0, e, (t, k)).astype(np.int32)
    wt = g.uniform(0.1, 1, (t, k)).astype(np.float32)
    full = oracle.forward(x, ids, wt, W1, W2, t, 16, fmt, rounding="reciprocal")["out"]
    brute = oracle.token_forward(x, ids, wt, W1, W2, e, t, fmt, rounding="reciprocal")
    assert np.array_equal(full, brute)
    plain = oracle.forward(x, ids, wt, W1, W2, t, 16, fmt)["out"]
    assert not np.array_equal(full, plain)  # the BF16 rounding of SwiGLU alone changes codes


def test_scale_product_rounding_decides_a_bf16_tie():
    """Hand-derived: one product of codes 1.0 x 1.0 (P = 1), sa = 1 + 2^-8 -
    2^-20 and sw = 1 + 2^-20 (both float32 values). The exact product is
    1 + 2^-8 + 2^-28 - 2^-40, just above the BF16 midpoint 1 + 2^-8 between
    1.0 and 1 + 2^-7, so it rounds up to 1 + 2^-7 (0x3F81). Formed in float32
    first it rounds to 1 + 2^-8 exactly (the rest is below half a float32
    ulp), a tie that BF16 resolves to the even 1.0 (0x3F80)."""
    a = np.zeros((1, 128), np.uint8)
    w = np.zeros((128, 128), np.uint8)
    a[0, 5] = 0x38  # 1.0
    w[0, 5] = 0x38
    sa = np.array([[1 + 2.0 ** -8 - 2.0 ** -20]], np.float64)
    sw = np.array([[1 + 2.0 ** -20]], np.float32)
    assert float(np.float32(sa[0, 0])) == sa[0, 0]
    assert int(oracle.moe.gemm_rows(a, sa, w, sw, "reciprocal")[0, 0]) == 0x3F80
    assert int(oracle.moe.gemm_rows(a, sa, w, sw, "divide")[0, 0]) == 0x3F81
