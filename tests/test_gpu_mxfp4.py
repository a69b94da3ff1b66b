"""Parity of the MXFP4-weight path (FP4 E2M1 weights with E8M0 scales per 32
along K, FP8 activations) against the oracle: the grouped GEMM on its own
(aligned and batched layouts, gathered and plain A rows, every activation
scale format, ragged token tiles, several K splits), an exact case compared
bit for bit, and the whole layer through moe_forward."""

import numpy as np
import pytest
import torch

import block_fp8_mixture_amd as moe
import oracle
import synth
from tests.gpu_helpers import POISON_BF16, POISON_U8, assert_bf16_close, dev, down, say, up

pytestmark = pytest.mark.gpu

INF = float("inf")


def _routing_layout(counts, align=16):
    counts = np.asarray(counts, np.int64)
    seg = (counts + align - 1) // align * align
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    return counts.astype(np.int32), offsets


def _gemm_case(seed, counts, n, k, fmt, gather, a_rows=None):
    g = np.random.default_rng(seed)
    e_n = len(counts)
    counts, offsets = _routing_layout(counts)
    row_cap = int(offsets[-1]) + 16
    a_rows = a_rows or (row_cap if not gather else 40)
    x = g.standard_normal((a_rows, k)).astype(np.float32)
    aq, asc = oracle.quantize_groups(x, fmt)
    wp = g.integers(0, 256, size=(e_n, n, k // 2), dtype=np.uint8)
    ws = g.integers(116, 124, size=(e_n, n, k // 32)).astype(np.uint8)
    row_map = None
    if gather:
        row_map = np.full(row_cap, -1, np.int32)
        for e in range(e_n):
            row_map[offsets[e]:offsets[e] + counts[e]] = g.integers(0, a_rows * 4, counts[e])
    return dict(aq=aq, asc=asc, wp=wp, ws=ws, counts=counts, offsets=offsets, row_cap=row_cap,
                row_map=row_map, a_rows=a_rows)


def _ref(case, fmt):
    ri = None if case["row_map"] is None else np.where(case["row_map"] >= 0, case["row_map"] // 4, 0)
    c, live = oracle.grouped_gemm(case["aq"], case["asc"], fmt, (case["wp"], case["ws"]),
                                  case["counts"], case["offsets"], ri, weight_fmt="mxfp4")
    return c, live


GEMM_CASES = [
    # (counts per expert, N, K)
    ([1, 0, 3, 2], 256, 256),          # decode-sized: many K splits
    ([33, 0, 70, 1, 5], 128, 512),     # ragged 32-row token tiles
    ([64, 64], 512, 1024),
    ([130, 7, 0, 31, 32], 384, 384),   # 3 K steps: an odd count through the 3-deep pipeline
    ([0, 0, 0], 128, 128),             # nothing live
]


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("ci", range(len(GEMM_CASES)))
def test_mxfp4_gemm_matches_oracle(ci, gather, fmt):
    counts, n, k = GEMM_CASES[ci]
    case = _gemm_case(100 + ci, counts, n, k, fmt, gather)
    say(f"mxfp4 gemm case {ci} counts={counts} n={n} k={k} fmt={fmt} gather={gather}")
    out = torch.full((case["row_cap"], n), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_grouped_gemm_mxfp4(up(case["aq"]), up(case["asc"]), fmt, up(case["wp"]), up(case["ws"]),
                               up(case["counts"]), up(case["offsets"]), case["row_cap"],
                               a_row_map=None if case["row_map"] is None else up(case["row_map"]),
                               a_row_div=4, out=out)
    torch.cuda.synchronize()
    got = down(out)
    ref, live = _ref(case, fmt)
    if live.any():
        assert_bf16_close(got[:len(live)][live], ref[live], "mxfp4 gemm")
    assert np.all(got[:len(live)][~live] == POISON_BF16), "rows that are not live were written"
    assert np.all(got[len(live):] == POISON_BF16)


def test_mxfp4_gemm_exact_case_is_bit_exact():
    # Small integers everywhere (E2M1 codes of 0, 1, 2, 3, 4, 6; E4M3 codes of
    # integers up to 16; unit scales): every partial sum is an exact fp32
    # integer, so the BF16 result is the oracle's bit for bit.
    g = np.random.default_rng(3)
    e_n, n, k = 3, 256, 512
    counts, offsets = _routing_layout([5, 40, 17])
    row_cap = int(offsets[-1])
    int_codes = np.array([0, 2, 4, 5, 6, 7, 8 | 2, 8 | 4, 8 | 5, 8 | 6, 8 | 7], np.uint8)
    nib = int_codes[g.integers(0, len(int_codes), size=(e_n, n, k))]
    wp = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    ws = np.full((e_n, n, k // 32), 127, np.uint8)
    vals = g.integers(-16, 17, size=(row_cap, k)).astype(np.float32)
    aq = oracle.e4m3_encode(vals)
    assert np.array_equal(oracle.e4m3_decode(aq), vals)
    asc = np.ones((k // 128, row_cap), np.float32)
    out = torch.full((row_cap, n), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_grouped_gemm_mxfp4(up(aq), up(asc), "fp32", up(wp), up(ws), up(counts), up(offsets),
                               row_cap, out=out)
    torch.cuda.synchronize()
    ref, live = oracle.grouped_gemm(aq, asc, "fp32", (wp, ws), counts, offsets, weight_fmt="mxfp4")
    assert np.array_equal(down(out)[live], ref[live])


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_mxfp4_gemm_batched_layout(fmt):
    g = np.random.default_rng(9)
    e_n, cap, n, k = 4, 48, 256, 256
    masked = np.array([0, 48, 13, 33], np.int32)
    rows = e_n * cap
    x = g.standard_normal((rows, k)).astype(np.float32)
    aq, asc = oracle.quantize_groups(x, fmt)
    wp = g.integers(0, 256, size=(e_n, n, k // 2), dtype=np.uint8)
    ws = g.integers(118, 124, size=(e_n, n, k // 32)).astype(np.uint8)
    out = torch.full((rows, n), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_grouped_gemm_mxfp4(up(aq), up(asc), fmt, up(wp), up(ws), up(masked), expert_cap=cap,
                               out=out)
    torch.cuda.synchronize()
    got = down(out)
    offsets = (np.arange(e_n + 1) * cap).astype(np.int32)
    ref, live = oracle.grouped_gemm(aq, asc, fmt, (wp, ws), masked, offsets, weight_fmt="mxfp4")
    assert_bf16_close(got[live], ref[live], "batched mxfp4 gemm")
    assert np.all(got[~live] == POISON_BF16)


LAYER_RUNS = [
    ("tiny", 8, 8, "fp32", "divide", 0),    # general schedule (I = 128)
    ("tiny", 8, 6, "ue8m0", "reciprocal", 0),
    ("decode", 1, 1, "fp32", "divide", 0),  # the one-launch layer from here to sweep 8
    ("decode", 4, 4, "fp32", "divide", 0),
    ("decode", 1, 1, "ue8m0", "reciprocal", 0),
    ("decode", 4, 3, "pow2", "divide", 0),
    ("sweep", 1, 1, "fp32", "divide", 0),   # H 6144 (1.5 column blocks per CU), I 256 (one stage)
    ("sweep", 8, 8, "fp32", "divide", 0),   # 4-deep ring for the wider token codes
    ("sweep", 8, 5, "ue8m0", "divide", 0),
    ("sweep", 64, 64, "pow2", "divide", 0),
    ("tiny", 8, 8, "fp32", "divide", 16),   # batched masked-M layout
]


@pytest.mark.parametrize("run", LAYER_RUNS, ids=[f"{r[0]}-{r[2]}-{r[3]}-{r[4]}-cap{r[5]}" for r in LAYER_RUNS])
def test_mxfp4_layer_matches_oracle(run):
    name, t_cap, t_live, fmt, rounding, cap = run
    cfg = synth.get(name)
    E, H, I, K, A = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cfg.align_rows
    say(f"mxfp4 layer {name} t_cap={t_cap} t_live={t_live} {fmt} {rounding} cap={cap}")
    x, ids, w = synth.make_workload(cfg, t_cap)
    (w1p, w1s), (w2p, w2s) = synth.ExpertWeightsMxfp4(cfg).stacked(threads=16)
    lay = moe.moe_workspace_plan(E, H, I, K, t_cap, A, 0, fmt, "swiglu", INF, rounding,
                                 expert_cap=cap, weight_fmt="mxfp4")
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((t_cap, H), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(up(x), up(ids), up(w), up(w1p), up(w1s), up(w2p), up(w2s), fmt, "swiglu", INF,
                    A, 0, t_live=up(np.array([t_live], np.int32)), out=out, workspace=ws,
                    rounding=rounding, expert_cap=cap, weight_fmt="mxfp4")
    torch.cuda.synchronize()
    got = down(out)
    assert np.all(got[t_live:] == POISON_BF16)
    R = lay["row_cap"]
    one_launch = lay["act"] < lay["status"]  # the plan lays out act rows for the one-launch layer only
    assert one_launch == (name in ("decode", "sweep") and t_cap <= 8 and cap == 0), (name, t_cap)
    if one_launch:  # it ran: the first live row's fp32 act values were written
        act0 = ws[lay["act"]:lay["act"] + 4 * I].cpu().numpy().view(np.uint32)
        assert not np.all(act0 == np.uint32(POISON_U8 * 0x01010101))
    # stage by stage on the GPU's own inputs: FC1 rows, the FC2 input codes
    # (bit-exact), FC2 rows
    sdt = np.uint8 if fmt == "ue8m0" else np.float32

    def view(name_, dtype, shape):
        nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return ws[lay[name_]:lay[name_] + nbytes].cpu().numpy().view(dtype).reshape(shape)
    counts = view("expert_counts", np.int32, (E,))
    offsets = view("expert_offsets", np.int32, (E + 1,))
    r2p = view("row_to_pair", np.int32, (R,))
    xq = view("xq", np.uint8, (t_cap, H))
    xs = view("xs", sdt, (H // 128, t_cap))
    c1 = view("c1", np.uint16, (R, 2 * I))
    hq = view("hq", np.uint8, (R, I))
    hs = view("hs", sdt, (I // 128, R))
    y = view("y", np.uint16, (R, H))
    tok = np.where(r2p >= 0, r2p // K, 0)
    ref_c1, live = oracle.grouped_gemm(xq, xs, fmt, (w1p, w1s), counts, offsets, tok, rounding,
                                       weight_fmt="mxfp4")
    assert_bf16_close(c1[:len(live)][live], ref_c1[live], "FC1")
    rhq, rhs = oracle.silu_mul_quant(c1[:len(live)][live], fmt, "swiglu", INF, rounding)
    assert np.array_equal(hq[:len(live)][live], rhq)
    assert np.array_equal(np.ascontiguousarray(hs[:, :len(live)][:, live]).view(np.uint8),
                          np.ascontiguousarray(rhs).view(np.uint8))
    ref_y, _ = oracle.grouped_gemm(hq, hs, fmt, (w2p, w2s), counts, offsets, rounding=rounding,
                                   weight_fmt="mxfp4")
    assert_bf16_close(y[:len(live)][live], ref_y[live], "FC2")
    # the whole layer against the dense per-token oracle (8 sampled tokens)
    toks = np.arange(t_live) if t_live <= 8 else np.unique(
        np.concatenate([[0, t_live - 1], np.random.default_rng(2).choice(t_live, 6, replace=False)]))
    ref = oracle.token_forward(x, ids, w, (w1p, w1s), (w2p, w2s), E, t_live, fmt, tokens=toks,
                               rounding=rounding, weight_fmt="mxfp4")
    err = assert_bf16_close(got[toks], ref, "layer")
    say(f"  layer max err / max|ref| = {err:.3e}")


FULL_SIZE = [(4096, 7168, False), (4096, 7168, True), (7168, 2048, False)]


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("shape", FULL_SIZE, ids=[f"n{n}-k{k}-gather{g}" for n, k, g in FULL_SIZE])
def test_mxfp4_gemm_full_size_sampled(shape, fmt):
    # The 4096-token layer's FC1 (N 4096, K 7168, gathered and plain) and FC2
    # (N 7168, K 2048) shapes with 32 experts of about 1024 rows: enough tiles
    # for the 256 x 256 ping-pong kernel with E2M1 weight slabs. Checked on
    # whole 64 x 128 blocks of several experts, row and column positions (the
    # first, a middle and the last, ragged, ones) against the oracle.
    n, k, gather = shape
    g = np.random.default_rng(21)
    e_n = 32
    cnt = g.integers(900, 1150, e_n)
    counts, offsets = _routing_layout(cnt)
    row_cap = int(offsets[-1])
    a_rows = 4096 if gather else row_cap
    x = g.standard_normal((a_rows, k)).astype(np.float32)
    aq, asc = oracle.quantize_groups(x, fmt)
    wp = g.integers(0, 256, size=(e_n, n, k // 2), dtype=np.uint8)
    ws = g.integers(117, 122, size=(e_n, n, k // 32)).astype(np.uint8)
    row_map = None
    if gather:
        row_map = np.full(row_cap, -1, np.int32)
        for e in range(e_n):
            row_map[offsets[e]:offsets[e] + counts[e]] = g.integers(0, a_rows * 8, counts[e])
    say(f"mxfp4 gemm full size n={n} k={k} gather={gather} {fmt} row_cap={row_cap}")
    out = torch.full((row_cap, n), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_grouped_gemm_mxfp4(up(aq), up(asc), fmt, up(wp), up(ws), up(counts), up(offsets),
                               row_cap, a_row_map=None if row_map is None else up(row_map),
                               a_row_div=8, out=out)
    torch.cuda.synchronize()
    got = down(out)
    for e in (0, 13, e_n - 1):
        c = int(counts[e])
        for mt in sorted({0, (c - 1) // 64, c // 128}):
            r0 = int(offsets[e]) + 64 * mt
            rows = np.arange(r0, min(r0 + 64, int(offsets[e]) + c))
            src = rows if row_map is None else row_map[rows] // 8
            for n0 in (0, n // 256 * 128, n - 128):
                ref = oracle.gemm_rows_mxfp4(aq[src], oracle.scales_to_f64(asc[:, src], fmt),
                                             wp[e, n0:n0 + 128], ws[e, n0:n0 + 128])
                assert_bf16_close(got[rows, n0:n0 + 128], ref, f"expert {e} rows {r0} cols {n0}")
    # rows past each expert's count stay untouched
    for e in (0, e_n - 1):
        pad = np.arange(int(offsets[e]) + int(counts[e]), int(offsets[e + 1]))
        assert np.all(got[pad] == POISON_BF16)



def test_mxfp4_gemm_ue8m0_equals_fp32_powers_of_two():
    # With UE8M0 activation scales the 256 x 256 kernel passes each token's
    # byte to the matrix cores as B's scale and never rescales the
    # accumulator; with fp32 scales it rescales by the ratio of consecutive
    # blocks' scales. For the same powers of two every factor is exact, so
    # both must give the same bits on every live row (FC2's shape at 4096
    # tokens: enough tiles for that kernel).
    n, k = 7168, 2048
    g = np.random.default_rng(22)
    e_n = 32
    counts, offsets = _routing_layout(g.integers(900, 1150, e_n))
    row_cap = int(offsets[-1])
    codes = g.integers(0, 0x7F, size=(row_cap, k), dtype=np.uint8)  # E4M3 codes without NaN
    codes |= (g.integers(0, 2, size=(row_cap, k)) << 7).astype(np.uint8)
    sb = g.integers(110, 135, size=(k // 128, row_cap)).astype(np.uint8)
    sf = np.ldexp(np.float32(1.0), sb.astype(np.int32) - 127).astype(np.float32)
    wp = g.integers(0, 256, size=(e_n, n, k // 2), dtype=np.uint8)
    ws = g.integers(117, 122, size=(e_n, n, k // 32)).astype(np.uint8)
    say(f"mxfp4 gemm ue8m0 vs fp32 powers of two n={n} k={k} row_cap={row_cap}")
    outs = {}
    for fmt, sc in (("ue8m0", sb), ("fp32", sf)):
        out = torch.full((row_cap, n), POISON_BF16, dtype=torch.int16, device=dev())
        moe.moe_grouped_gemm_mxfp4(up(codes), up(sc), fmt, up(wp), up(ws), up(counts), up(offsets),
                                   row_cap, out=out)
        torch.cuda.synchronize()
        outs[fmt] = down(out)
    live = np.zeros(row_cap, bool)
    for e in range(e_n):
        live[offsets[e]:offsets[e] + counts[e]] = True
    diff = int((outs["ue8m0"][live] != outs["fp32"][live]).sum())
    assert diff == 0, f"{diff} outputs differ"
    assert np.all(outs["ue8m0"][~live] == POISON_BF16)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_mxfp4_layer_full_size_complete(fmt):
    """The 4096-token layer with MXFP4 weights through moe_forward (FC1 and
    FC2 on the 256 x 256 kernel with E2M1 slabs; with UE8M0 activations the
    matrix cores apply both scales), compared in full: alignment and
    activation codes bit-exact; C1 of every live row within tolerance of the
    oracle's fp64 FC1 from the same codes; the FC2 input codes and scales of
    every live row bit-exact against SiLU+quant of the GPU's own C1; Y of
    every live row within tolerance of the oracle's FC2 of the GPU's own FC2
    input; every output token within tolerance of the combine of the GPU's
    own Y and of the oracle's chain from the GPU's FC2-input codes; nothing
    written outside the live rows."""
    cfg = synth.get("full")
    E, H, I, K, A = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cfg.align_rows
    T = 4096
    say(f"mxfp4 layer full size complete T={T} fmt={fmt}")
    x, ids, w = synth.make_workload(cfg, T)
    (w1p, w1s), (w2p, w2s) = synth.ExpertWeightsMxfp4(cfg).stacked(threads=16)
    lay = moe.moe_workspace_plan(E, H, I, K, T, A, 0, fmt, weight_fmt="mxfp4")
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((T, H), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(up(x), up(ids), up(w), up(w1p), up(w1s), up(w2p), up(w2s), fmt, align_rows=A,
                    out=out, workspace=ws, weight_fmt="mxfp4")
    torch.cuda.synchronize()
    R = lay["row_cap"]
    sdt = np.uint8 if fmt == "ue8m0" else np.float32

    def view(name_, dtype, shape):
        nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return ws[lay[name_]:lay[name_] + nbytes].cpu().numpy().view(dtype).reshape(shape)

    def raw(a):
        return np.ascontiguousarray(a).view(np.uint8)

    # The oracle's steps up to FC1 (its own SiLU, FC2 and combine are not
    # needed: FC2 and the combine are checked from the GPU's own inputs).
    ref = dict(oracle.align(ids, T, E, A))
    ref["xq"], ref["xs"] = oracle.quantize_groups(oracle.bf16_bits_to_f64(x).astype(np.float32), fmt)
    token_of_row = np.where(ref["row_to_pair"] >= 0, ref["row_to_pair"] // K, 0)
    ref["c1"], ref["live"] = oracle.grouped_gemm(ref["xq"], ref["xs"], fmt, (w1p, w1s), ref["counts"],
                                                 ref["offsets"], token_of_row, weight_fmt="mxfp4")
    total = int(ref["offsets"][-1])
    assert np.array_equal(view("expert_counts", np.int32, (E,)), ref["counts"])
    assert np.array_equal(view("expert_offsets", np.int32, (E + 1,)), ref["offsets"])
    assert np.array_equal(view("row_to_pair", np.int32, (R,))[:total], ref["row_to_pair"])
    assert np.array_equal(view("pair_to_row", np.int32, (T * K,)), ref["pair_to_row"])
    assert np.array_equal(view("xq", np.uint8, (T, H)), ref["xq"])
    assert np.array_equal(raw(view("xs", sdt, (H // 128, T))), raw(ref["xs"]))
    live = ref["live"]
    c1 = view("c1", np.uint16, (R, 2 * I))
    err = assert_bf16_close(c1[:total][live], ref["c1"][live], "FC1, every live row")
    say(f"  FC1 max err / max|ref| = {err:.3e}")
    assert np.all(c1[:total][~live] == (POISON_U8 << 8 | POISON_U8))
    hq = view("hq", np.uint8, (R, I))
    hs = view("hs", sdt, (I // 128, R))
    rhq, rhs = oracle.silu_mul_quant(c1[:total][live], fmt)
    assert np.array_equal(hq[:total][live], rhq)
    assert np.array_equal(raw(hs[:, :total][:, live]), raw(rhs))
    y = view("y", np.uint16, (R, H))
    ref_y, _ = oracle.grouped_gemm(hq[:total], hs[:, :total], fmt, (w2p, w2s), ref["counts"],
                                   ref["offsets"], weight_fmt="mxfp4")
    err = assert_bf16_close(y[:total][live], ref_y[live], "FC2, every live row")
    say(f"  FC2 max err / max|ref| = {err:.3e}")
    got = down(out)
    assert_bf16_close(got, oracle.combine(y, ref["pair_to_row"], w, T, H), "combine, every token")
    err = assert_bf16_close(got, oracle.combine(ref_y, ref["pair_to_row"], w, T, H), "layer, every token")
    say(f"  layer max err / max|ref| = {err:.3e} (oracle chain from the GPU's FC2-input codes)")
