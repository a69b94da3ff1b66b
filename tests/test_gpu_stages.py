"""Stage-isolated parity of the HIP kernels against the CPU oracle.

Bit-exact: alignment indices and endpoints, FP8 codes and scales (act_quant,
silu_mul_quant fed identical BF16 inputs), GEMM outputs on the exactly
representable special case. Tolerance (|err| <= 1e-2 * max|ref| + 2 BF16
ulp): general GEMM and combine outputs. Every test also checks that rows the
layer must leave alone keep their poison.
"""

import numpy as np
import pytest
import torch

import block_fp8_mixture_amd as moe
import oracle
import synth
from tests.gpu_helpers import (POISON_BF16, POISON_I32, POISON_U8, assert_bf16_close, dev, down,
                               say, up)

pytestmark = pytest.mark.gpu


def _full(shape, value, dtype):
    return torch.full(shape, value, dtype=dtype, device=dev())


def _t_live(n):
    return up(np.array([n], np.int32))


def _f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# ------------------------------------------------------------------ align

ALIGN_CASES = [
    # t_cap, t_live, K, E, A, seed, id_lo, id_hi
    (8, 8, 2, 4, 16, 0, 0, 4),
    (8, 5, 2, 4, 1, 1, 0, 4),
    (16, 16, 8, 72, 16, 2, 0, 72),     # 128 pairs
    (24, 24, 8, 72, 16, 3, 0, 72),     # 192 pairs
    (7, 7, 3, 5, 4, 4, -2, 7),         # invalid ids dropped
    (9, 9, 3, 3, 2, 5, 0, 2),          # an empty expert, duplicate ids
    (4, 0, 8, 288, 16, 6, 0, 288),     # empty routing
    (512, 16, 8, 32, 16, 7, 0, 32),
    (4096, 4096, 8, 32, 16, 8, 0, 32),
    (1000, 999, 8, 1024, 7, 9, 0, 1024),
    (4096, 4096, 8, 256, 16, 10, 0, 3),  # three experts own every pair
    (1500, 1500, 1, 1, 1, 11, 0, 1),
    (2048, 2000, 8, 256, 16, 12, -3, 259),  # the most experts ranked by lane masks
    (300, 300, 8, 257, 16, 13, 0, 257),     # the fewest ranked by the ballot loop
]


def _check_align(ids, t_cap, t_live, k, e, a):
    ref = oracle.align(ids, t_live, e, a)
    row_cap = moe.moe_min_row_cap(t_cap, k, e, a) + 5
    out = {
        "counts": _full((e,), POISON_I32, torch.int32),
        "offsets": _full((e + 1,), POISON_I32, torch.int32),
        "row_to_pair": _full((row_cap,), POISON_I32, torch.int32),
        "pair_to_row": _full((max(t_cap * k, 1),), POISON_I32, torch.int32),
    }
    moe.moe_align(up(ids), e, a, row_cap, t_live=_t_live(t_live), out=out)
    torch.cuda.synchronize()
    got = {key: down(v) for key, v in out.items()}
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    total = int(ref["offsets"][-1])
    assert np.array_equal(got["row_to_pair"][:total], ref["row_to_pair"])
    assert np.all(got["row_to_pair"][total:] == POISON_I32)
    p = t_live * k
    assert np.array_equal(got["pair_to_row"][:p], ref["pair_to_row"])
    assert np.all(got["pair_to_row"][p:] == POISON_I32)


@pytest.mark.parametrize("t_cap,t_live,k,e,a,seed,lo,hi", ALIGN_CASES)
def test_align_bit_exact(t_cap, t_live, k, e, a, seed, lo, hi):
    say(f"align t_cap={t_cap} t_live={t_live} K={k} E={e} A={a}")
    ids = np.random.default_rng(seed).integers(lo, hi, (t_cap, k)).astype(np.int32)
    _check_align(ids, t_cap, t_live, k, e, a)


@pytest.mark.parametrize("name,t_cap,t_live", [("tiny", 8, 8), ("decode", 1, 1), ("decode", 4, 4),
                                               ("padded", 512, 16), ("full", 4096, 4096),
                                               ("sweep", 64, 64), ("sweep", 4096, 4096)])
def test_align_workload_routing(name, t_cap, t_live):
    say(f"align workload {name} t_cap={t_cap} t_live={t_live}")
    cfg = synth.get(name)
    ids, _ = synth.make_routing(cfg, t_cap)
    _check_align(ids, t_cap, t_live, cfg.topk, cfg.num_experts, cfg.align_rows)


# ------------------------------------------------------------------ act_quant


def _tokens(kind, t_cap, h, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((t_cap, h))
    if kind == "mixed":
        groups = x.reshape(t_cap, h // 128, 128)
        groups *= 10.0 ** g.uniform(-8, 3, (t_cap, h // 128, 1))
        groups[:, ::7, :] = 0.0                                   # all-zero groups
        groups[:, 1::11, :] *= 1e-4                               # floor active
        # groups with amax 448 and values on E4M3 midpoints (scale exactly 1)
        mids = oracle.e4m3_decode(np.arange(126, dtype=np.uint8))
        mids = (mids + oracle.e4m3_decode(np.arange(1, 127, dtype=np.uint8))) / 2
        sel = groups[:, 2::9, :]
        sel[...] = g.choice(np.concatenate([mids, -mids]), sel.shape)
        sel[..., 0] = 448.0
        groups[:, 2::9, :] = sel
        # groups where the two rounding conventions round midpoints apart:
        # amax 1.625 with 39/32 and 39/64 (exact quotients 336 and 168), at
        # random powers of two
        split = groups[:, 4::10, :]
        split[...] = g.choice([1.21875, 0.609375, -1.21875, 0.0], split.shape)
        split[..., 0] = 1.625
        split *= np.exp2(g.integers(-20, 8, split.shape[:2] + (1,)))
        groups[:, 4::10, :] = split
        x = groups.reshape(t_cap, h)
    bits = oracle.bf16_from_f64(x)
    if kind == "mixed":
        bits[:, 5::13] = 0x8000  # negative zeros
    return bits


@pytest.mark.parametrize("rounding", ["divide", "reciprocal"])
@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
@pytest.mark.parametrize("t_cap,t_live,h,seed,kind", [
    (8, 8, 256, 0, "normal"), (37, 30, 4096, 1, "mixed"), (512, 16, 7168, 2, "normal"),
    (300, 300, 6144, 3, "mixed"), (5, 0, 128, 4, "normal")])
def test_act_quant_bit_exact(fmt, t_cap, t_live, h, seed, kind, rounding):
    say(f"act_quant fmt={fmt} {rounding} t_cap={t_cap} t_live={t_live} H={h} {kind}")
    x = _tokens(kind, t_cap, h, seed)
    sdt = torch.uint8 if fmt == "ue8m0" else torch.float32
    xq = _full((t_cap, h), POISON_U8, torch.uint8)
    xs = _full((h // 128, t_cap), POISON_U8 if fmt == "ue8m0" else float("nan"), sdt)
    moe.moe_act_quant(up(x), fmt, t_live=_t_live(t_live), xq=xq, xs=xs, rounding=rounding)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_groups(oracle.bf16_bits_to_f64(x[:t_live]).astype(np.float32), fmt,
                                    rounding)
    gq, gs = down(xq), down(xs)
    assert np.array_equal(gq[:t_live], rq)
    assert np.all(gq[t_live:] == POISON_U8)
    if fmt == "ue8m0":
        assert np.array_equal(gs[:, :t_live], rs)
        assert np.all(gs[:, t_live:] == POISON_U8)
    else:
        assert np.array_equal(_f32_bits(gs[:, :t_live]), _f32_bits(rs))
        assert np.all(np.isnan(gs[:, t_live:]))


# ------------------------------------------------------------------ silu_mul_quant


def _segments(g, e, max_rows, align, zero_frac=0.3):
    counts = g.integers(1, max_rows + 1, e)
    counts[g.random(e) < zero_frac] = 0
    offsets = np.concatenate([[0], np.cumsum(-(-counts // align) * align)]).astype(np.int32)
    return counts.astype(np.int32), offsets


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
@pytest.mark.parametrize("act,lim,amp", [("swiglu", float("inf"), 2.0), ("swiglu_clamp", 7.0, 8.0),
                                         ("swiglu_clamp_after_silu", 7.0, 8.0),
                                         ("swiglu_clamp", 0.5, 1.0),
                                         ("swiglu_clamp_after_silu", 0.5, 1.0)])
@pytest.mark.parametrize("inter,e,seed,rounding", [(128, 4, 0, "divide"), (512, 288, 1, "divide"),
                                                   (2048, 32, 2, "divide"),
                                                   (128, 4, 3, "reciprocal"),
                                                   (2048, 32, 4, "reciprocal")])
def test_silu_mul_quant_bit_exact(fmt, act, lim, amp, inter, e, seed, rounding):
    say(f"silu_mul_quant fmt={fmt} {rounding} act={act} lim={lim} I={inter} E={e}")
    g = np.random.default_rng(seed)
    counts, offsets = _segments(g, e, 40, 16)
    row_cap = int(offsets[-1]) + 16
    gu = oracle.bf16_from_f64(g.standard_normal((row_cap, 2 * inter)) * amp)
    live = np.zeros(row_cap, bool)
    for i in range(e):
        live[offsets[i]:offsets[i] + counts[i]] = True
    gu[~live] = POISON_BF16  # never read
    sdt = torch.uint8 if fmt == "ue8m0" else torch.float32
    hq = _full((row_cap, inter), POISON_U8, torch.uint8)
    hs = _full((inter // 128, row_cap), POISON_U8 if fmt == "ue8m0" else float("nan"), sdt)
    lim32 = float(np.float32(lim))
    moe.moe_silu_mul_quant(up(gu), up(counts), up(offsets), act, lim32, fmt, hq=hq, hs=hs,
                           rounding=rounding)
    torch.cuda.synchronize()
    rq, rs = oracle.silu_mul_quant(gu[live], fmt, act, lim32, rounding)
    gq, gs = down(hq), down(hs)
    assert np.array_equal(gq[live], rq)
    assert np.all(gq[~live] == POISON_U8)
    if fmt == "ue8m0":
        assert np.array_equal(gs[:, live], rs)
        assert np.all(gs[:, ~live] == POISON_U8)
    else:
        assert np.array_equal(_f32_bits(gs[:, live]), _f32_bits(rs))
        assert np.all(np.isnan(gs[:, ~live]))


def _gate_specials(g, shape):
    """BF16 gate bits around and outside the SiLU table's range [2^-12, 2^4):
    zeros of both signs, tiny and huge magnitudes, the range's end points and
    their BF16 neighbours."""
    edges = np.array([2.0 ** -12, 2.0 ** 4], np.float32).view(np.uint32) >> 16
    pool = np.concatenate([edges - 1, edges, edges + 1, [0, 1, 0x7F, 0x80]]).astype(np.uint16)
    mags = (np.exp2(g.uniform(-24.0, 7.0, shape)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pick = g.random(shape) < 0.2
    bits = np.where(pick, g.choice(pool, shape), mags)
    return (bits | (g.integers(0, 2, shape, dtype=np.uint16) << 15)).astype(np.uint16)


@pytest.mark.parametrize("fmt,act,lim,rounding", [("fp32", "swiglu", float("inf"), "divide"),
                                                   ("ue8m0", "swiglu_clamp", 7.0, "divide"),
                                                   ("pow2", "swiglu_clamp", 0.3, "divide"),
                                                   ("ue8m0", "swiglu_clamp_after_silu", 7.0, "divide"),
                                                   ("fp32", "swiglu", float("inf"), "reciprocal"),
                                                   ("pow2", "swiglu_clamp", 0.3, "reciprocal")])
def test_silu_mul_quant_table_path(fmt, act, lim, rounding):
    """Launches large enough that every workgroup takes SiLU from its table of
    BF16 gates (at least 128 groups each with two workgroups per CU): codes
    and scales bit-exact, including gates outside the table's range and a
    clamp limit that is not a BF16 value."""
    cus = torch.cuda.get_device_properties(dev()).multi_processor_count
    inter, e = 2048, 32
    rows_needed = 128 * 2 * cus * 128 // inter
    say(f"silu_mul_quant table path fmt={fmt} act={act} lim={lim} rows>={rows_needed}")
    g = np.random.default_rng(7)
    per = -(-rows_needed // e) + 24
    counts = g.integers(per - 16, per + 16, e).astype(np.int32)
    counts[3] = 0
    offsets = np.concatenate([[0], np.cumsum(-(-counts // 16) * 16)]).astype(np.int32)
    assert offsets[-1] >= rows_needed
    row_cap = int(offsets[-1]) + 16
    # Truncated float32 normals as BF16 inputs; a tenth of the gates special.
    gu = (np.float32(3.0) * g.standard_normal((row_cap, 2 * inter), np.float32)).view(np.uint32)
    gu = (gu >> 16).astype(np.uint16)
    sp = g.random((row_cap, inter)) < 0.1
    gu[:, :inter] = np.where(sp, _gate_specials(g, (row_cap, inter)), gu[:, :inter])
    live = np.zeros(row_cap, bool)
    for i in range(e):
        live[offsets[i]:offsets[i] + counts[i]] = True
    gu[~live] = POISON_BF16
    sdt = torch.uint8 if fmt == "ue8m0" else torch.float32
    hq = _full((row_cap, inter), POISON_U8, torch.uint8)
    hs = _full((inter // 128, row_cap), POISON_U8 if fmt == "ue8m0" else float("nan"), sdt)
    lim32 = float(np.float32(lim))
    moe.moe_silu_mul_quant(up(gu), up(counts), up(offsets), act, lim32, fmt, hq=hq, hs=hs,
                           rounding=rounding)
    torch.cuda.synchronize()
    rq, rs = oracle.silu_mul_quant(gu[live], fmt, act, lim32, rounding)
    gq, gs = down(hq), down(hs)
    bad = np.argwhere(gq[live] != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"
    assert np.all(gq[~live] == POISON_U8)
    if fmt == "ue8m0":
        assert np.array_equal(gs[:, live], rs)
    else:
        assert np.array_equal(_f32_bits(gs[:, live]), _f32_bits(rs))


# ------------------------------------------------------------------ grouped GEMM

EXACT_CODES = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)  # 0, +-.5, +-1, +-2


def _gemm_case(seed, e, n, k, counts, exact, fmt, gather_k=0):
    g = np.random.default_rng(seed)
    counts = np.asarray(counts, np.int32)
    offsets = np.concatenate([[0], np.cumsum(-(-counts // 16) * 16)]).astype(np.int32)
    row_cap = int(offsets[-1]) + 32
    kb = k // 128
    if exact:
        w = EXACT_CODES[g.integers(0, len(EXACT_CODES), (e, n, k), dtype=np.uint8)]
        ws = g.choice(np.array([0.5, 1.0, 2.0], np.float32), (e, n // 128, kb))
    else:
        w = np.empty((e, n, k), np.uint8)
        ws = np.empty((e, n // 128, kb), np.float32)
        for i in range(e):
            w[i], ws[i] = synth.quantize_weight_blocks((g.standard_normal((n, k)) * 0.02).astype(np.float32))
    if gather_k:
        a_rows = max(int(counts.sum()) // gather_k + 3, 4)
        row_map = np.full(row_cap, POISON_I32, np.int32)
        for i in range(e):
            row_map[offsets[i]:offsets[i] + counts[i]] = g.integers(0, a_rows * gather_k, counts[i])
        div = gather_k
    else:
        a_rows, row_map, div = row_cap, None, 1
    if exact:
        a = g.choice(EXACT_CODES, (a_rows, k))
        p2 = g.integers(-1, 2, (kb, a_rows))
        a_sc = np.ldexp(1.0, p2).astype(np.float32)
        if fmt == "ue8m0":
            a_sc = (p2 + 127).astype(np.uint8)
    else:
        x = g.standard_normal((a_rows, k)).astype(np.float32)
        a, a_sc = oracle.quantize_groups(x, fmt)
    return dict(w=w, ws=ws, a=a, a_sc=a_sc, counts=counts, offsets=offsets, row_cap=row_cap,
                row_map=row_map, div=div, n=n, k=k, fmt=fmt)


def _run_gemm(c):
    out = _full((c["row_cap"], c["n"]), POISON_BF16, torch.int16)
    tiles = torch.zeros(1, dtype=torch.int32, device=dev())
    moe.moe_grouped_gemm_fp8(up(c["a"]), up(c["a_sc"]), c["fmt"], up(c["w"]), up(c["ws"]),
                             up(c["counts"]), up(c["offsets"]), c["row_cap"],
                             a_row_map=None if c["row_map"] is None else up(c["row_map"]),
                             a_row_div=c["div"], out=out, tiles_visited=tiles)
    torch.cuda.synchronize()
    return down(out), int(tiles.item())


def _expected_tiles(counts, n):
    t = 0
    for cnt in counts:
        if 0 < cnt <= moe.GEMM_TILES["stream_max_rows"]:
            t += -(-cnt // moe.GEMM_TILES["stream_tile_m"])
        elif cnt > 0:
            t += -(-cnt // moe.GEMM_TILES["tiled_tile_m"])
    return t * (n // moe.GEMM_TILES["col_tile"])


def _ref_gemm(c):
    idx = None if c["row_map"] is None else np.where(c["row_map"] >= 0, c["row_map"] // c["div"], 0)
    ref, live = oracle.grouped_gemm(c["a"], c["a_sc"], c["fmt"], (c["w"], c["ws"]), c["counts"],
                                    c["offsets"], idx)
    return ref, live


# Counts of 32 streaming-sized experts (1..41 rows): enough (expert, 64-row)
# tasks that the streaming kernel takes its 64-row task shape; the smaller
# cases take the 16-row shape with K blocks split over the waves.
_MANY = [(i * 7) % 41 + 1 for i in range(32)]

GEMM_SHAPES = [
    # seed, E, N, K, counts, gather_k
    (0, 4, 256, 256, [3, 0, 17, 100], 0),           # streaming and tiled experts
    (1, 3, 384, 1024, [64, 65, 1], 0),              # either side of the 64-row limit
    (2, 5, 512, 2048, [16, 0, 300, 7, 129], 0),
    (3, 6, 256, 512, [9, 33, 0, 200, 2, 64], 8),    # gathered A rows (FC1 layout)
    (4, 2, 1024, 7168, [5, 140], 8),
    (5, 3, 256, 640, [5, 20, 1], 0),                # K/128 = 5: waves idle in the last stage
    (6, 3, 256, 384, [40, 3, 16], 8),               # K/128 = 3, gathered
    (7, 32, 1024, 256, _MANY, 0),                   # 64-row streaming tasks
    (8, 32, 1024, 384, _MANY, 8),                   # the same, gathered, K/128 = 3
    (9, 8, 8192, 256, [300] * 8, 0),                # enough tiles for 256-wide weight tiles
    (10, 8, 2048, 256, [300] * 8, 0),               # 128-wide weight tiles
    (11, 12, 1024, 512, [400] * 12, 8),             # 128-wide, gathered
    (12, 8, 8320, 256, [300] * 7 + [211], 8),       # 256-wide, output staged in LDS; N % 256 = 128
    (13, 8, 8192, 2048, [300] * 7 + [271], 0),      # 256-wide at K = 2048 (the full layer's FC2)
]

# The 256-wide staged-output kernel at the full layer's FC1 depth, K = 7168
# (56 scale blocks of accumulator rescaling), gathered: 16 experts of about
# 300 rows on N = 4096 give 35 x 16 tiles, past the 2 x CU bound of the
# narrow kernels.
LONG_K_SHAPE = (14, 16, 4096, 7168, [300] * 15 + [270], 8)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("seed,e,n,k,counts,gk", GEMM_SHAPES)
def test_gemm_exact_special_case_bitwise(fmt, seed, e, n, k, counts, gk):
    """Codes in {0, +-0.5, +-1, +-2} and power-of-two scales: every partial sum
    is exact in fp32, so the HIP result must equal the oracle bit for bit."""
    say(f"gemm exact fmt={fmt} E={e} N={n} K={k} counts={counts} gather={gk}")
    c = _gemm_case(seed, e, n, k, counts, True, fmt, gk)
    got, tiles = _run_gemm(c)
    ref, live = _ref_gemm(c)
    total = int(c["offsets"][-1])
    assert np.array_equal(got[:total][live], ref[live])
    assert np.all(got[:total][~live] == POISON_BF16)
    assert np.all(got[total:] == POISON_BF16)
    assert tiles == _expected_tiles(c["counts"], n)


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
@pytest.mark.parametrize("seed,e,n,k,counts,gk", GEMM_SHAPES)
def test_gemm_tolerance(fmt, seed, e, n, k, counts, gk):
    say(f"gemm tol fmt={fmt} E={e} N={n} K={k} counts={counts} gather={gk}")
    c = _gemm_case(seed + 100, e, n, k, counts, False, fmt, gk)
    got, _ = _run_gemm(c)
    ref, live = _ref_gemm(c)
    total = int(c["offsets"][-1])
    assert_bf16_close(got[:total][live], ref[live], "gemm")
    assert np.all(got[:total][~live] == POISON_BF16)
    assert np.all(got[total:] == POISON_BF16)


@pytest.mark.parametrize("fmt,exact", [("fp32", True), ("ue8m0", True), ("fp32", False),
                                       ("pow2", False)])
def test_gemm_wide_tiles_at_long_k(fmt, exact):
    seed, e, n, k, counts, gk = LONG_K_SHAPE
    say(f"gemm 256-wide K={k} fmt={fmt} exact={exact}")
    c = _gemm_case(seed + (0 if exact else 100), e, n, k, counts, exact, fmt, gk)
    got, tiles = _run_gemm(c)
    ref, live = _ref_gemm(c)
    total = int(c["offsets"][-1])
    if exact:
        assert np.array_equal(got[:total][live], ref[live])
    else:
        assert_bf16_close(got[:total][live], ref[live], "gemm K=7168")
    assert np.all(got[:total][~live] == POISON_BF16)
    assert np.all(got[total:] == POISON_BF16)
    assert tiles == _expected_tiles(c["counts"], n)


def test_gemm_empty_experts_write_nothing():
    c = _gemm_case(7, 3, 256, 256, [0, 0, 0], False, "fp32")
    got, tiles = _run_gemm(c)
    assert tiles == 0 and np.all(got == POISON_BF16)


# ------------------------------------------------------------------ combine


@pytest.mark.parametrize("t_cap,t_live,k,h,seed", [(8, 8, 2, 256, 0), (37, 30, 8, 4096, 1),
                                                   (4, 4, 8, 7168, 2), (64, 0, 8, 128, 3)])
def test_combine_tolerance(t_cap, t_live, k, h, seed):
    say(f"combine t_cap={t_cap} t_live={t_live} K={k} H={h}")
    g = np.random.default_rng(seed)
    rows = 200
    y = oracle.bf16_from_f64(g.standard_normal((rows, h)))
    p2r = g.integers(-1, rows, t_cap * k).astype(np.int32)
    w = g.uniform(0, 1, (t_cap, k)).astype(np.float32)
    out = _full((t_cap, h), POISON_BF16, torch.int16)
    moe.moe_topk_combine(up(y), up(p2r), up(w), t_live=_t_live(t_live), out=out)
    torch.cuda.synchronize()
    got = down(out)
    ref = oracle.combine(y, p2r, w, t_live, h)
    assert_bf16_close(got[:t_live], ref, "combine")
    assert np.all(got[t_live:] == POISON_BF16)


def test_combine_unit_weight_is_identity():
    g = np.random.default_rng(5)
    y = oracle.bf16_from_f64(g.standard_normal((50, 512)))
    p2r = g.permutation(50)[:20].astype(np.int32)
    out = moe.moe_topk_combine(up(y), up(p2r), up(np.ones((20, 1), np.float32)))
    torch.cuda.synchronize()
    assert np.array_equal(down(out), y[p2r])
