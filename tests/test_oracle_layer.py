"""Pins for the oracle's GEMM, SwiGLU, combine and whole-layer functions."""

from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
import synth
from tests.exact import near_tie, round_binary, to_bf16_bits

DEC = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))


def _finite_codes(g, shape):
    c = g.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, 0x7E, c).astype(np.uint8)


# ---------------------------------------------------------------- GEMM


@pytest.mark.parametrize("m,n,kd,seed", [(3, 384, 256, 0), (1, 128, 384, 1), (5, 256, 128, 2)])
def test_gemm_rows_equals_exact_rational(m, n, kd, seed):
    g = np.random.default_rng(seed)
    a = _finite_codes(g, (m, kd))
    w = _finite_codes(g, (n, kd))
    sa = g.uniform(1e-3, 2.0, (kd // 128, m)).astype(np.float32).astype(np.float64)
    sw = g.uniform(1e-4, 1e-2, (n // 128, kd // 128)).astype(np.float32)
    got = oracle.moe.gemm_rows(a, sa, w, sw)
    ai = np.round(DEC[a] * 512).astype(np.int64)   # every E4M3 value is k * 2**-9
    wi = np.round(DEC[w] * 512).astype(np.int64)
    ties = 0
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            for kb in range(kd // 128):
                sl = slice(kb * 128, (kb + 1) * 128)
                p = int(np.dot(ai[i, sl], wi[j, sl]))
                exact += Fraction(float(sa[kb, i])) * Fraction(float(sw[j // 128, kb])) * Fraction(p, 1 << 18)
            if near_tie(exact, 7, -126):
                ties += 1
                continue
            assert int(got[i, j]) == to_bf16_bits(exact), (i, j)
    assert ties < 3


def test_gemm_scale_indexing_is_per_block():
    """A scale change in one (row-block, K-block) moves only that block's sums."""
    g = np.random.default_rng(3)
    a = _finite_codes(g, (2, 256))
    w = _finite_codes(g, (256, 256))
    sa = np.ones((2, 2))
    sw = np.ones((2, 2), np.float32)
    base = oracle.bf16_bits_to_f64(oracle.moe.gemm_rows(a, sa, w, sw))
    sw2 = sw.copy()
    sw2[1, 0] = 2.0  # output columns 128..255, K block 0
    moved = oracle.bf16_bits_to_f64(oracle.moe.gemm_rows(a, sa, w, sw2))
    assert np.array_equal(moved[:, :128], base[:, :128])
    ai, wi = DEC[a], DEC[w]
    want = (ai[:, :128] @ wi[128:, :128].T) * 2 + ai[:, 128:] @ wi[128:, 128:].T
    assert np.array_equal(moved[:, 128:], oracle.bf16_bits_to_f64(oracle.bf16_from_f64(want)))
    sa2 = sa.copy()
    sa2[1, 1] = 4.0  # row 1, K block 1
    moved = oracle.bf16_bits_to_f64(oracle.moe.gemm_rows(a, sa2, w, sw))
    assert np.array_equal(moved[0], base[0])
    want = ai[1, :128] @ wi[:, :128].T + 4 * (ai[1, 128:] @ wi[:, 128:].T)
    assert np.array_equal(moved[1], oracle.bf16_bits_to_f64(oracle.bf16_from_f64(want)))


# ---------------------------------------------------------------- SwiGLU

mpmath.mp.dps = 60


def _mp_swiglu(g, u, act, lim):
    g = mpmath.mpf(g)
    u = mpmath.mpf(u)
    if act == "swiglu_clamp":
        g = min(g, mpmath.mpf(lim))
        u = max(min(u, mpmath.mpf(lim)), -mpmath.mpf(lim))
        return g / (1 + mpmath.exp(-g)) * u
    s = g / (1 + mpmath.exp(-g))
    if act == "swiglu_clamp_after_silu":
        s = min(s, mpmath.mpf(lim))
        u = max(min(u, mpmath.mpf(lim)), -mpmath.mpf(lim))
    return s * u


def _bf16_values(g, n, scale):
    x = (g.standard_normal(n) * scale).astype(np.float32)
    return oracle.bf16_bits_to_f64(oracle.bf16_from_f64(x.astype(np.float64)))


@pytest.mark.parametrize("act,lim", [("swiglu", np.inf), ("swiglu_clamp", 7.0),
                                     ("swiglu_clamp_after_silu", 7.0), ("swiglu_clamp", 0.5)])
def test_swiglu_is_correctly_rounded_float32(act, lim):
    g = np.random.default_rng(4)
    gate = np.concatenate([_bf16_values(g, 1500, 3.0), _bf16_values(g, 300, 30.0), [0.0, -0.0, 1e-30]])
    up = np.concatenate([_bf16_values(g, 1800, 3.0), [1.0, 2.0, 3.0]])
    got = oracle.swiglu(gate, up, act, lim)
    skipped = 0
    for gv, uv, yv in zip(gate, up, got):
        y = _mp_swiglu(gv, uv, act, lim)
        if y == 0:
            assert float(yv) == 0.0
            continue
        sign, man, exp, _ = mpmath.mpf(y)._mpf_
        exact = (-1) ** sign * Fraction(int(man)) * Fraction(2) ** int(exp)
        if near_tie(exact, 23, -126, rel=2.0 ** -45):
            skipped += 1
            continue
        assert Fraction(float(yv)) == round_binary(exact, 23, -126), (gv, uv)
    assert skipped <= 2


def test_swiglu_special_values():
    assert oracle.swiglu([0.0], [5.0])[0] == 0.0
    g = np.array([20.0, 40.0, 80.0])
    assert np.array_equal(oracle.swiglu(g, [1.0, 1.0, 1.0]), g.astype(np.float32))  # silu(g) -> g
    g = np.random.default_rng(5).standard_normal(100) * 4
    u = np.random.default_rng(6).standard_normal(100) * 4
    plain = oracle.swiglu(g, u)
    assert np.array_equal(oracle.swiglu(g, u, "swiglu_clamp", np.inf), plain)
    assert np.array_equal(oracle.swiglu(g, u, "swiglu_clamp_after_silu", np.inf), plain)
    # clamping is idempotent: pre-clamped inputs give the same result
    lim = 1.5
    gc, uc = np.minimum(g, lim), np.clip(u, -lim, lim)
    assert np.array_equal(oracle.swiglu(gc, uc, "swiglu_clamp", lim), oracle.swiglu(g, u, "swiglu_clamp", lim))
    assert np.all(np.abs(oracle.swiglu(g, u, "swiglu_clamp_after_silu", lim)) <= lim * lim)


# ---------------------------------------------------------------- combine


def test_combine_equals_exact_weighted_sum():
    g = np.random.default_rng(7)
    t, k, h, rows = 6, 3, 64, 20
    y = oracle.bf16_from_f64(g.standard_normal((rows, h)))
    w = g.uniform(0, 1, (t, k)).astype(np.float32)
    p2r = g.integers(-1, rows, t * k).astype(np.int32)
    p2r[3 * k:4 * k] = -1  # token 3 has no valid pair
    out = oracle.combine(y, p2r, w, t)
    yv = oracle.bf16_bits_to_f64(y)
    for ti in range(t):
        for c in range(h):
            exact = sum((Fraction(float(w[ti, kk])) * Fraction(float(yv[p2r[ti * k + kk], c]))
                         for kk in range(k) if p2r[ti * k + kk] >= 0), Fraction(0))
            if near_tie(exact, 7, -126):
                continue
            assert int(out[ti, c]) == to_bf16_bits(exact)
    assert np.all(out[3] == 0)


def test_combine_single_unit_weight_is_identity():
    g = np.random.default_rng(8)
    y = oracle.bf16_from_f64(g.standard_normal((5, 32)))
    out = oracle.combine(y, np.array([4, 2, 0], np.int32), np.ones((3, 1), np.float32), 3)
    assert np.array_equal(out, y[[4, 2, 0]])


# ---------------------------------------------------------------- layer


def _tiny_layer(e, h, i, k, t_cap, seed, id_lo=0, id_hi=None):
    g = np.random.default_rng(seed)
    id_hi = e if id_hi is None else id_hi
    ids = g.integers(id_lo, id_hi, (t_cap, k)).astype(np.int32)
    w = g.uniform(0.1, 1.0, (t_cap, k)).astype(np.float32)
    x = oracle.bf16_from_f64(g.standard_normal((t_cap, h)))
    w1 = [synth.quantize_weight_blocks((g.standard_normal((2 * i, h)) * 0.02).astype(np.float32)) for _ in range(e)]
    w2 = [synth.quantize_weight_blocks((g.standard_normal((h, i)) * 0.02).astype(np.float32)) for _ in range(e)]
    w1 = (np.stack([a for a, _ in w1]), np.stack([b for _, b in w1]))
    w2 = (np.stack([a for a, _ in w2]), np.stack([b for _, b in w2]))
    return x, ids, w, w1, w2


LAYER_CASES = [
    # E, H, I, K, t_cap, t_live, seed, id range
    (1, 128, 128, 1, 3, 3, 0, (0, 1)),
    (3, 256, 128, 2, 8, 7, 1, (0, 3)),
    (4, 256, 128, 3, 8, 8, 2, (0, 4)),
    (5, 128, 256, 2, 2, 1, 3, (-1, 6)),     # invalid ids dropped
    (72, 128, 128, 3, 8, 8, 4, (0, 72)),
    (4, 128, 128, 2, 4, 0, 5, (0, 4)),      # empty routing
    (3, 128, 128, 3, 6, 6, 6, (1, 2)),      # everything on one expert, duplicates
]


@pytest.mark.parametrize("fmt", oracle.SCALE_FMTS)
@pytest.mark.parametrize("e,h,i,k,t_cap,t_live,seed,rng", LAYER_CASES)
def test_aligned_layer_equals_per_token_brute_force(e, h, i, k, t_cap, t_live, seed, rng, fmt):
    x, ids, w, w1, w2 = _tiny_layer(e, h, i, k, t_cap, seed, *rng)
    r = oracle.forward(x, ids, w, w1, w2, t_live, 4, fmt)
    ref = oracle.token_forward(x, ids, w, w1, w2, e, t_live, fmt)
    assert np.array_equal(r["out"], ref)


@pytest.mark.parametrize("act,lim", [("swiglu_clamp", 0.05), ("swiglu_clamp_after_silu", 0.05)])
def test_aligned_layer_equals_brute_force_with_clamp(act, lim):
    x, ids, w, w1, w2 = _tiny_layer(4, 256, 128, 2, 8, 9)
    r = oracle.forward(x, ids, w, w1, w2, 8, 16, "fp32", act, lim)
    ref = oracle.token_forward(x, ids, w, w1, w2, 4, 8, "fp32", act, lim)
    assert np.array_equal(r["out"], ref)
    plain = oracle.forward(x, ids, w, w1, w2, 8, 16, "fp32")
    assert not np.array_equal(r["out"], plain["out"])  # the limit does bind


def test_layer_is_independent_of_alignment_and_token_order():
    x, ids, w, w1, w2 = _tiny_layer(5, 256, 128, 3, 9, 10)
    outs = [oracle.forward(x, ids, w, w1, w2, 9, a, "fp32")["out"] for a in (1, 4, 16, 64)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    perm = np.random.default_rng(11).permutation(9)
    o = oracle.forward(x[perm], ids[perm], w[perm], w1, w2, 9, 16, "fp32")["out"]
    assert np.array_equal(o, outs[0][perm])


def test_quantized_layer_tracks_unquantized_layer():
    """vLLM PR #65794, Claims: ~0.06 relative error against a BF16 reference."""
    cfg = synth.get("tiny")
    x, ids, w = synth.make_workload(cfg, 8)
    (w1q, w1s), (w2q, w2s) = synth.ExpertWeights(cfg).stacked()
    r = oracle.forward(x, ids, w, (w1q, w1s), (w2q, w2s), 8, 16, "fp32")
    ref = oracle.unquantized_reference(x, ids, w, (w1q, w1s), (w2q, w2s), 4, 8)
    got = oracle.bf16_bits_to_f64(r["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.005 < rel < 0.15
    # a wrong scale (e.g. dividing instead of multiplying) is far off
    assert np.linalg.norm(ref) > 0
