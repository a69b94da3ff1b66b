"""The batched masked-M layout (vLLM PR #65794, Details, batched experts) and
expert-parallel local ids (TensorRT-LLM PR #21250, For MoE owners; review
comment: drop other ranks' pairs) on the GPU, against the CPU oracle:
alignment bit-exact, SiLU+quant codes bit-exact, GEMM outputs bit-exact on
the exactly representable case and within tolerance otherwise, the whole
layer within tolerance, rows past each expert's mask untouched."""

import numpy as np
import pytest
import torch

import block_fp8_mixture_amd as moe
import oracle
import synth
from tests.gpu_helpers import (POISON_BF16, POISON_I32, POISON_U8, assert_bf16_close, dev,
                               device_weights, down, host_weights, say, up)
from tests.test_gpu_stages import EXACT_CODES, _f32_bits, _full, _t_live

pytestmark = pytest.mark.gpu

INF = float("inf")

ALIGN_CASES = [
    # t_cap, t_live, K, E, cap, start, seed, id range
    (8, 8, 2, 4, 16, 0, 0, (0, 4)),
    (8, 5, 2, 4, 3, 0, 1, (0, 4)),          # overflow
    (24, 24, 8, 16, 40, 32, 5, (0, 96)),    # a rank owning experts [32, 48)
    (4096, 4096, 8, 32, 1100, 0, 2, (0, 32)),
    (4096, 4000, 8, 32, 700, 0, 3, (0, 32)),  # overflow at scale
    (2048, 2048, 8, 300, 80, 100, 4, (0, 512)),  # ballot-loop ranking, EP slice
]


@pytest.mark.parametrize("t_cap,t_live,k,e,cap,start,seed,rng", ALIGN_CASES)
def test_align_batched_bit_exact(t_cap, t_live, k, e, cap, start, seed, rng):
    say(f"align batched t_cap={t_cap} t_live={t_live} E={e} cap={cap} start={start}")
    g = np.random.default_rng(seed)
    ids = g.integers(rng[0], rng[1], (t_cap, k)).astype(np.int32)
    ref = oracle.align_batched(ids, t_live, e, cap, start)
    out = {"masked_m": _full((e,), POISON_I32, torch.int32),
           "row_to_pair": _full((e * cap,), POISON_I32, torch.int32),
           "pair_to_row": _full((t_cap * k,), POISON_I32, torch.int32),
           "overflow": _full((1,), POISON_I32, torch.int32)}
    moe.moe_align_batched(up(ids), e, cap, t_live=_t_live(t_live), out=out, expert_start=start)
    torch.cuda.synchronize()
    got = {key: down(v) for key, v in out.items()}
    assert np.array_equal(got["masked_m"], ref["masked_m"])
    assert int(got["overflow"][0]) == ref["overflow"]
    live = ref["row_to_pair"] >= 0
    assert np.array_equal(got["row_to_pair"][live], ref["row_to_pair"][live])
    assert np.all(got["row_to_pair"][~live] == POISON_I32)  # rows past the mask untouched
    p = t_live * k
    assert np.array_equal(got["pair_to_row"][:p], ref["pair_to_row"])
    assert np.all(got["pair_to_row"][p:] == POISON_I32)


@pytest.mark.parametrize("start", [0, 7, 40])
def test_align_local_ids(start):
    g = np.random.default_rng(11 + start)
    t_cap, k, e = 300, 8, 32
    ids = g.integers(0, 80, (t_cap, k)).astype(np.int32)
    ref = oracle.align(ids, t_cap, e, 16, start)
    rc = moe.moe_min_row_cap(t_cap, k, e, 16)
    got = moe.moe_align(up(ids), e, 16, rc, expert_start=start)
    torch.cuda.synchronize()
    assert np.array_equal(down(got["counts"]), ref["counts"])
    assert np.array_equal(down(got["offsets"]), ref["offsets"])
    total = int(ref["offsets"][-1])
    assert np.array_equal(down(got["row_to_pair"])[:total], ref["row_to_pair"])
    assert np.array_equal(down(got["pair_to_row"])[:t_cap * k], ref["pair_to_row"])


def _masked_gemm_case(seed, e, cap, n, k, masked, exact, fmt, gather_k=0):
    g = np.random.default_rng(seed)
    masked = np.asarray(masked, np.int32)
    rows = e * cap
    kb = k // 128
    if exact:
        w = g.choice(EXACT_CODES, (e, n, k))
        ws = g.choice(np.array([0.5, 1.0, 2.0], np.float32), (e, n // 128, kb))
    else:
        w = np.empty((e, n, k), np.uint8)
        ws = np.empty((e, n // 128, kb), np.float32)
        for i in range(e):
            w[i], ws[i] = synth.quantize_weight_blocks((g.standard_normal((n, k)) * 0.02).astype(np.float32))
    if gather_k:
        a_rows = max(rows // gather_k + 3, 4)
        row_map = np.full(rows, POISON_I32, np.int32)
        for i in range(e):
            m = min(int(masked[i]), cap)
            row_map[i * cap:i * cap + m] = g.integers(0, a_rows * gather_k, m)
    else:
        a_rows, row_map = rows, None
    if exact:
        a = g.choice(EXACT_CODES, (a_rows, k))
        p2 = g.integers(-1, 2, (kb, a_rows))
        a_sc = np.ldexp(1.0, p2).astype(np.float32)
        if fmt == "ue8m0":
            a_sc = (p2 + 127).astype(np.uint8)
    else:
        x = g.standard_normal((a_rows, k)).astype(np.float32)
        a, a_sc = oracle.quantize_groups(x, fmt)
    return dict(w=w, ws=ws, a=a, a_sc=a_sc, masked=masked, cap=cap, rows=rows, row_map=row_map,
                div=gather_k or 1, n=n, k=k, fmt=fmt, e=e)


def _run_masked(c):
    out = _full((c["rows"], c["n"]), POISON_BF16, torch.int16)
    moe.moe_grouped_gemm_fp8_masked(up(c["a"]), up(c["a_sc"]), c["fmt"], up(c["w"]), up(c["ws"]),
                                    up(c["masked"]), c["cap"],
                                    a_row_map=None if c["row_map"] is None else up(c["row_map"]),
                                    a_row_div=c["div"], out=out)
    torch.cuda.synchronize()
    return down(out)


def _ref_masked(c):
    counts = np.minimum(c["masked"], c["cap"])
    offsets = (np.arange(c["e"] + 1) * c["cap"]).astype(np.int32)
    idx = None if c["row_map"] is None else np.where(c["row_map"] >= 0, c["row_map"] // c["div"], 0)
    return oracle.grouped_gemm(c["a"], c["a_sc"], c["fmt"], (c["w"], c["ws"]), counts, offsets, idx)


MASKED_SHAPES = [
    # seed, E, cap, N, K, masked_m, gather_k
    (0, 4, 64, 256, 256, [3, 0, 17, 64], 0),
    (1, 3, 400, 512, 1024, [300, 65, 1], 0),       # tiled and streaming experts
    (2, 6, 200, 256, 512, [9, 200, 0, 150, 2, 64], 8),  # gathered (FC1)
    (3, 8, 320, 4096, 256, [300] * 8, 0),           # 256-wide tiles
    (4, 5, 40, 384, 384, [41, 40, 100, 7, 0], 0),   # masks beyond the capacity are capped
]


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("seed,e,cap,n,k,masked,gk", MASKED_SHAPES)
def test_masked_gemm_exact_special_case_bitwise(fmt, seed, e, cap, n, k, masked, gk):
    say(f"masked gemm exact fmt={fmt} E={e} cap={cap} N={n} K={k} masked={masked}")
    c = _masked_gemm_case(seed, e, cap, n, k, masked, True, fmt, gk)
    got = _run_masked(c)
    ref, live = _ref_masked(c)
    assert np.array_equal(got[live], ref[live])
    assert np.all(got[~live] == POISON_BF16)


@pytest.mark.parametrize("fmt", ["fp32", "pow2"])
@pytest.mark.parametrize("seed,e,cap,n,k,masked,gk", MASKED_SHAPES)
def test_masked_gemm_tolerance(fmt, seed, e, cap, n, k, masked, gk):
    say(f"masked gemm tol fmt={fmt} E={e} cap={cap} N={n} K={k}")
    c = _masked_gemm_case(seed + 50, e, cap, n, k, masked, False, fmt, gk)
    got = _run_masked(c)
    ref, live = _ref_masked(c)
    assert_bf16_close(got[live], ref[live], "masked gemm")
    assert np.all(got[~live] == POISON_BF16)


@pytest.mark.parametrize("fmt,act,lim,rounding", [("fp32", "swiglu", INF, "divide"),
                                                   ("ue8m0", "swiglu_clamp", 0.5, "divide"),
                                                   ("pow2", "swiglu", INF, "reciprocal")])
@pytest.mark.parametrize("inter,e,cap", [(256, 5, 48), (2048, 32, 96)])
def test_masked_silu_mul_quant_bit_exact(fmt, act, lim, rounding, inter, e, cap):
    say(f"masked silu_mul_quant fmt={fmt} {act} {rounding} I={inter} E={e} cap={cap}")
    g = np.random.default_rng(inter + e)
    masked = g.integers(0, cap + 8, e).astype(np.int32)
    masked[1] = 0
    rows = e * cap
    gu = oracle.bf16_from_f64(g.standard_normal((rows, 2 * inter)) * 2)
    live = np.zeros(rows, bool)
    for i in range(e):
        live[i * cap:i * cap + min(int(masked[i]), cap)] = True
    gu[~live] = POISON_BF16  # never read
    sdt = torch.uint8 if fmt == "ue8m0" else torch.float32
    hq = _full((rows, inter), POISON_U8, torch.uint8)
    hs = _full((inter // 128, rows), POISON_U8 if fmt == "ue8m0" else float("nan"), sdt)
    lim32 = float(np.float32(lim))
    moe.moe_silu_mul_quant_masked(up(gu), up(masked), cap, act, lim32, fmt, hq=hq, hs=hs,
                                  rounding=rounding)
    torch.cuda.synchronize()
    rq, rs = oracle.silu_mul_quant(gu[live], fmt, act, lim32, rounding)
    gq, gs = down(hq), down(hs)
    assert np.array_equal(gq[live], rq)
    assert np.all(gq[~live] == POISON_U8)
    if fmt == "ue8m0":
        assert np.array_equal(gs[:, live], rs)
    else:
        assert np.array_equal(_f32_bits(gs[:, live]), _f32_bits(rs))


def _ws_view(ws, lay, name, dtype, shape):
    nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
    return ws[lay[name]:lay[name] + nbytes].cpu().numpy().view(dtype).reshape(shape)


LAYER_RUNS = [
    # workload, t_cap, t_live, fmt, expert_cap, rounding
    ("tiny", 8, 8, "fp32", 8, "divide"),
    ("tiny", 8, 6, "ue8m0", 3, "divide"),          # overflow: pairs dropped
    ("decode", 4, 4, "fp32", 4, "reciprocal"),     # decode-sized, general path
    ("padded", 512, 16, "fp32", 64, "divide"),     # 512-token capacity, 16 live
    ("sweep", 256, 256, "pow2", 160, "divide"),
    ("full", 4096, 4096, "ue8m0", 1152, "divide"),
]


@pytest.mark.parametrize("name,t_cap,t_live,fmt,cap,rounding", LAYER_RUNS)
def test_batched_layer_matches_oracle(name, t_cap, t_live, fmt, cap, rounding):
    """The whole layer on the batched layout: alignment and codes bit-exact,
    output within tolerance of the oracle (batched layout, same overflow), and
    equal bit for bit to the aligned layout's output when nothing overflows
    (every row is computed by the same kernels in the same order)."""
    cfg = synth.get(name)
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk
    say(f"batched layer {name} t_cap={t_cap} t_live={t_live} {fmt} cap={cap} {rounding}")
    x, ids, w = synth.make_workload(cfg, t_cap, 4)
    (w1q, w1s), (w2q, w2s) = host_weights(name)
    d = device_weights(name)
    lay = moe.moe_workspace_plan(E, H, I, K, t_cap, 16, 0, fmt, rounding=rounding, expert_cap=cap)
    assert lay["row_cap"] == E * cap
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((t_cap, H), POISON_BF16, dtype=torch.int16, device=dev())
    live_t = up(np.array([t_live], np.int32))
    moe.moe_forward(up(x), up(ids), up(w), *d, fmt, t_live=live_t, out=out, workspace=ws,
                    rounding=rounding, expert_cap=cap)
    torch.cuda.synchronize()
    al = oracle.align_batched(ids, t_live, E, cap)
    assert np.array_equal(_ws_view(ws, lay, "expert_counts", np.int32, (E,)), al["masked_m"])
    assert int(_ws_view(ws, lay, "overflow", np.int32, (1,))[0]) == al["overflow"]
    r2p = _ws_view(ws, lay, "row_to_pair", np.int32, (E * cap,))
    live_rows = al["row_to_pair"] >= 0
    assert np.array_equal(r2p[live_rows], al["row_to_pair"][live_rows])
    assert np.array_equal(_ws_view(ws, lay, "pair_to_row", np.int32, (t_cap * K,))[:t_live * K],
                          al["pair_to_row"])
    got = down(out)
    assert np.all(got[t_live:] == POISON_BF16)
    n_tok = 16 if H * I < 4096 * 1024 else 6  # the per-token oracle decodes whole experts
    toks = np.arange(t_live) if t_live <= n_tok else np.unique(
        np.concatenate([[0, t_live - 1], np.random.default_rng(5).choice(t_live, n_tok - 2,
                                                                          replace=False)]))
    # the oracle with the overflowed pairs dropped, token by token
    kept = np.full_like(ids, -1)
    rows = al["pair_to_row"].reshape(t_live, K)
    kept[:t_live] = np.where(rows >= 0, ids[:t_live], -1)
    ref = oracle.token_forward(x, kept, w, (w1q, w1s), (w2q, w2s), E, t_live, fmt,
                               tokens=toks, rounding=rounding)
    err = assert_bf16_close(got[toks], ref, "batched layer")
    say(f"  layer max err / max|ref| = {err:.3e}")
    if al["overflow"] == 0:
        aligned, _ = moe.moe_forward(up(x), up(ids), up(w), *d, fmt, t_live=live_t,
                                     rounding=rounding)
        torch.cuda.synchronize()
        assert np.array_equal(down(aligned)[:t_live], got[:t_live])


EP_RUNS = [
    # workload, t_cap, experts per rank, rank start, fmt, expert_cap
    ("decode", 4, 72, 144, "fp32", 0),     # the one-launch decode layer on a rank's slice
    ("decode", 4, 72, 0, "fp32", 8),       # the same slice on the batched layout
    ("sweep", 64, 64, 64, "pow2", 0),      # general path
    ("full", 512, 8, 24, "fp32", 0),       # tiled GEMMs
]


@pytest.mark.parametrize("name,t_cap,e_loc,start,fmt,cap", EP_RUNS)
def test_expert_parallel_rank(name, t_cap, e_loc, start, fmt, cap):
    """A rank owning experts [start, start + e_loc) with its slice of the
    weights: equal (within tolerance) to the oracle's layer over the owned
    pairs only."""
    cfg = synth.get(name)
    H, I, K = cfg.hidden, cfg.inter, cfg.topk
    say(f"EP rank {name} t_cap={t_cap} experts [{start}, {start + e_loc}) {fmt} cap={cap}")
    x, ids, w = synth.make_workload(cfg, t_cap, 6)
    (w1q, w1s), (w2q, w2s) = host_weights(name)
    d = device_weights(name)
    sl = [t[start:start + e_loc].contiguous() for t in d]
    gave_up = moe.moe_barrier_timeouts()
    out, _ = moe.moe_forward(up(x), up(ids), up(w), *sl, fmt, expert_start=start, expert_cap=cap)
    torch.cuda.synchronize()
    assert moe.moe_barrier_timeouts() == gave_up
    owned = np.where((ids >= start) & (ids < start + e_loc), ids, -1).astype(np.int32)
    toks = np.arange(t_cap) if t_cap <= 16 else np.arange(0, t_cap, t_cap // 6)
    ref = oracle.token_forward(x, owned, w, (w1q, w1s), (w2q, w2s), cfg.num_experts, t_cap, fmt,
                               tokens=toks)
    assert_bf16_close(down(out)[toks], ref, "EP rank")
