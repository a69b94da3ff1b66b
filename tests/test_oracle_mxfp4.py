"""Pins of the oracle's MXFP4 weight path (FP4 E2M1 codes, E8M0 block scales).

The pages name FP4 weights only (vLLM PR #59128, description); the format is
read as OCP MXFP4. The pins tie the oracle to things other than its own
code: the format's value table, torch's E8M0 cast, a hand-packed byte, the
already-pinned FP8 GEMM (to which an MXFP4 GEMM reduces when the weight
scales are constant over 128x128 blocks), exact rational brute force, and the
dense per-token layer.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# OCP Microscaling Formats v1.0, FP4 (E2M1): the eight magnitudes of codes
# 0..7; codes 8..15 are the same magnitudes with the sign bit set.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_format_table():
    got = oracle.e2m1_decode(np.arange(16))
    assert list(got[:8]) == E2M1_TABLE
    assert list(-got[8:]) == E2M1_TABLE
    assert np.signbit(got[8]) and not np.signbit(got[0])
    assert oracle.e2m1_decode(np.array([0x1F])) == oracle.e2m1_decode(np.array([0xF]))  # low nibble only


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_fp4_unpack_puts_the_even_element_in_the_low_nibble():
    got = oracle.fp4_unpack(np.array([[0x21, 0xF7]], np.uint8))
    assert got.tolist() == [[1, 2, 7, 15]]
    # decoded: 0.5, 1.0, 6.0, -6.0
    assert oracle.e2m1_decode(got).tolist() == [[0.5, 1.0, 6.0, -6.0]]


def _random_mx(rng, n, k, scale_lo=117, scale_hi=122):
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(n, k // 32)).astype(np.uint8)
    return packed, scales


def _random_act(rng, m, k, fmt="fp32"):
    x = rng.standard_normal((m, k)).astype(np.float32)
    return oracle.quantize_groups(x, fmt)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_mxfp4_gemm_reduces_to_the_fp8_gemm(fmt):
    # Every E2M1 value is an E4M3 value, and with the E8M0 byte constant over
    # each 128x128 block the weight is code * 2**(b-127) with a 128x128 block
    # scale: the FP8 GEMM's own input. The two must agree bit for bit.
    rng = np.random.default_rng(11)
    m, n, k = 5, 256, 384
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    blk = rng.integers(116, 124, size=(n // 128, k // 128)).astype(np.uint8)
    scales = np.repeat(np.repeat(blk, 128, axis=0), 4, axis=1)  # [n, k/32]
    aq, asc = _random_act(rng, m, k, fmt)
    sa = oracle.scales_to_f64(asc, fmt)
    got = oracle.gemm_rows_mxfp4(aq, sa, packed, scales)
    w_vals = oracle.e2m1_decode(oracle.fp4_unpack(packed))
    w_e4m3 = oracle.e4m3_encode(w_vals.astype(np.float32))
    assert np.array_equal(oracle.e4m3_decode(w_e4m3), w_vals)  # exactly representable
    w_scales = np.exp2(blk.astype(np.float64) - 127.0).astype(np.float32)
    from oracle.moe import gemm_rows
    ref = gemm_rows(aq, sa, w_e4m3, w_scales)
    assert np.array_equal(got, ref)


def _bf16_of_fraction(q):
    f = float(q)  # exact here: every sum below is a dyadic rational of < 53 bits
    assert Fraction(f) == q
    return oracle.bf16_from_f64(np.array([f]))[0]


def test_mxfp4_gemm_against_exact_rationals():
    # Tiny case with per-32 scales varying inside each 128-wide block.
    rng = np.random.default_rng(5)
    m, n, k = 3, 4, 256
    packed, scales = _random_mx(rng, n, k, 118, 126)
    aq, asc = _random_act(rng, m, k)
    got = oracle.gemm_rows_mxfp4(aq, oracle.scales_to_f64(asc, "fp32"), packed, scales)
    nib = oracle.fp4_unpack(packed)
    mags = [Fraction(v).limit_denominator(2) for v in E2M1_TABLE]

    def w_val(i, j):
        c = int(nib[i, j])
        v = mags[c & 7] * Fraction(2) ** (int(scales[i, j // 32]) - 127)
        return -v if c & 8 else v

    def a_val(r, j):
        return Fraction(float(oracle.e4m3_decode(np.array([aq[r, j]]))[0]))

    for r in range(m):
        for i in range(n):
            total = Fraction(0)
            for kb in range(k // 128):
                part = sum((a_val(r, j) * w_val(i, j) for j in range(kb * 128, kb * 128 + 128)),
                           Fraction(0))
                total += Fraction(float(asc[kb, r])) * part
            assert got[r, i] == _bf16_of_fraction(total), (r, i)


@pytest.mark.parametrize("fmt,rounding", [("fp32", "divide"), ("ue8m0", "divide"),
                                          ("fp32", "reciprocal")])
def test_mxfp4_layer_equals_dense_per_token_brute_force(fmt, rounding):
    cfg = synth.get("tiny")
    x, ids, w = synth.make_workload(cfg, 8)
    ws = synth.ExpertWeightsMxfp4(cfg)
    w1, w2 = ws.stacked()
    res = oracle.forward(x, ids, w, w1, w2, 8, cfg.align_rows, fmt, rounding=rounding,
                         weight_fmt="mxfp4")
    ref = oracle.token_forward(x, ids, w, w1, w2, cfg.num_experts, 8, fmt, rounding=rounding,
                               weight_fmt="mxfp4")
    assert np.array_equal(res["out"][:8], ref)
    # and the batched masked-M layout gives the same output
    bat = oracle.forward(x, ids, w, w1, w2, 8, cfg.align_rows, fmt, rounding=rounding,
                         expert_cap=16, weight_fmt="mxfp4")
    assert np.array_equal(bat["out"][:8], ref)


def test_mxfp4_layer_tracks_the_unquantized_weights():
    # Sanity against the weights' real values: the quantized layer with MXFP4
    # weights stays close to the same layer with no activation quantization
    # and fp64 intermediates (only the activation path is quantized here).
    cfg = synth.get("tiny")
    x, ids, w = synth.make_workload(cfg, 8)
    (w1p, w1s), (w2p, w2s) = synth.ExpertWeightsMxfp4(cfg).stacked()
    res = oracle.forward(x, ids, w, (w1p, w1s), (w2p, w2s), 8, cfg.align_rows, "fp32",
                         weight_fmt="mxfp4")
    xf = oracle.bf16_bits_to_f64(x[:8])
    out = np.zeros_like(xf)
    for t in range(8):
        for kk in range(cfg.topk):
            e = int(ids[t, kk])
            W1 = oracle.mxfp4_dequant(w1p[e], w1s[e])
            W2 = oracle.mxfp4_dequant(w2p[e], w2s[e])
            h = W1 @ xf[t]
            g, u = h[:cfg.inter], h[cfg.inter:]
            out[t] += w[t, kk] * (W2 @ (g / (1 + np.exp(-g)) * u))
    got = oracle.bf16_bits_to_f64(res["out"][:8])
    rel = np.linalg.norm(got - out) / np.linalg.norm(out)
    assert rel < 0.1, rel
