"""End-to-end parity of moe_forward on the five workloads, plus the layer's
invariants: graph replay with changing routing and live count, poisoned
workspaces, untouched capacity, and independence from alignment/capacity.

Checks per run:
* alignment and per-token FP8 codes/scales read back from the workspace are
  bit-exact against the oracle on every live pair/token;
* each later stage is checked on sampled live rows against the oracle applied
  to the GPU's own inputs to that stage (bit-exact for silu_mul_quant,
  tolerance for the GEMMs and the combine);
* the final output of sampled tokens is within tolerance of the oracle's
  dense per-token evaluation of the whole layer.
"""

import numpy as np
import pytest
import torch

import block_fp8_mixture_amd as moe
import oracle
import synth
from tests.gpu_helpers import (POISON_BF16, POISON_U8, assert_bf16_close, dev, device_weights,
                               down, host_weights, say, up)

pytestmark = pytest.mark.gpu

INF = float("inf")


def _ws_view(ws, lay, name, dtype, shape):
    nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
    raw = ws[lay[name]:lay[name] + nbytes].cpu().numpy()
    return raw.view(dtype).reshape(shape)


def _sample(n, k, seed):
    if n <= k:
        return np.arange(n)
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], g.choice(n, k - 2, replace=False)]))


def run_and_check(name, t_cap, t_live, fmt, act="swiglu", lim=INF, variant=0, n_tok=8,
                  n_rows=16, rounding="divide"):
    cfg = synth.get(name)
    say(f"forward {name} t_cap={t_cap} t_live={t_live} fmt={fmt} act={act} lim={lim} {rounding}")
    E, H, I, K, A = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cfg.align_rows
    x, ids, w = synth.make_workload(cfg, t_cap, variant)
    (w1q, w1s), (w2q, w2s) = host_weights(name)
    d_w1q, d_w1s, d_w2q, d_w2s = device_weights(name)
    lim32 = float(np.float32(lim))
    out = torch.full((t_cap, H), POISON_BF16, dtype=torch.int16, device=dev())
    row_cap = cfg.row_cap or 0
    lay = moe.moe_workspace_plan(E, H, I, K, t_cap, A, row_cap, fmt, act, lim32, rounding)
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    gave_up = moe.moe_barrier_timeouts()
    moe.moe_forward(up(x), up(ids), up(w), d_w1q, d_w1s, d_w2q, d_w2s, fmt, act, lim32, A,
                    row_cap, t_live=up(np.array([t_live], np.int32)), out=out, workspace=ws,
                    rounding=rounding)
    torch.cuda.synchronize()
    assert moe.moe_barrier_timeouts() == gave_up, "a wait at the decode layer's grid barrier gave up"
    if moe.decode_layer_applies(t_cap, K, H, I):  # the one-launch layer reports per workgroup
        grid = torch.cuda.get_device_properties(0).multi_processor_count
        assert np.all(_ws_view(ws, lay, "status", np.int32, (grid,)) == 0)
    R = lay["row_cap"]
    sdt = np.uint8 if fmt == "ue8m0" else np.float32

    # alignment: bit-exact
    al = oracle.align(ids, t_live, E, A)
    counts = _ws_view(ws, lay, "expert_counts", np.int32, (E,))
    offsets = _ws_view(ws, lay, "expert_offsets", np.int32, (E + 1,))
    r2p = _ws_view(ws, lay, "row_to_pair", np.int32, (R,))
    p2r = _ws_view(ws, lay, "pair_to_row", np.int32, (t_cap * K,))
    assert np.array_equal(counts, al["counts"]) and np.array_equal(offsets, al["offsets"])
    total = int(offsets[-1])
    assert np.array_equal(r2p[:total], al["row_to_pair"])
    assert np.array_equal(p2r[:t_live * K], al["pair_to_row"])

    # per-token activation quantization: bit-exact
    xq = _ws_view(ws, lay, "xq", np.uint8, (t_cap, H))
    xs = _ws_view(ws, lay, "xs", sdt, (H // 128, t_cap))
    rq, rs = oracle.quantize_groups(oracle.bf16_bits_to_f64(x[:t_live]).astype(np.float32), fmt,
                                    rounding)
    assert np.array_equal(xq[:t_live], rq)
    assert np.array_equal(np.ascontiguousarray(xs[:, :t_live]).view(np.uint8),
                          np.ascontiguousarray(rs).view(np.uint8))

    c1 = _ws_view(ws, lay, "c1", np.uint16, (R, 2 * I))
    hq = _ws_view(ws, lay, "hq", np.uint8, (R, I))
    hs = _ws_view(ws, lay, "hs", sdt, (I // 128, R))
    y = _ws_view(ws, lay, "y", np.uint16, (R, H))
    sa_x = oracle.scales_to_f64(xs, fmt)
    sa_h = oracle.scales_to_f64(hs, fmt)
    g = np.random.default_rng(1)
    live_experts = np.flatnonzero(al["counts"] > 0)
    for e in g.permutation(live_experts)[:3]:
        seg = np.arange(al["offsets"][e], al["offsets"][e] + al["counts"][e])
        rows = seg[_sample(len(seg), n_rows, int(e))]
        tok = al["row_to_pair"][rows] // K
        ref_c1 = oracle.moe.gemm_rows(xq[tok], sa_x[:, tok], w1q[e], w1s[e], rounding)
        assert_bf16_close(c1[rows], ref_c1, f"FC1 expert {e}")
        rhq, rhs = oracle.silu_mul_quant(c1[rows], fmt, act, lim32, rounding)
        assert np.array_equal(hq[rows], rhq)
        assert np.array_equal(np.ascontiguousarray(hs[:, rows]).view(np.uint8),
                              np.ascontiguousarray(rhs).view(np.uint8))
        ref_y = oracle.moe.gemm_rows(hq[rows], sa_h[:, rows], w2q[e], w2s[e], rounding)
        assert_bf16_close(y[rows], ref_y, f"FC2 expert {e}")

    got = down(out)
    assert np.all(got[t_live:] == POISON_BF16), "rows of tokens past the live count were written"
    toks = _sample(t_live, n_tok, 2)
    if len(toks):
        # combine of the GPU's own expert outputs
        p2r_s = p2r[:t_live * K].reshape(t_live, K)[toks].reshape(-1)
        ref_comb = oracle.combine(y, p2r_s, w[toks], len(toks), H)
        assert_bf16_close(got[toks], ref_comb, "combine")
        # whole layer against the dense per-token oracle
        ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), E, t_live, fmt, act, lim32,
                                   tokens=toks, rounding=rounding)
        err = assert_bf16_close(got[toks], ref, "layer")
        say(f"  layer max err / max|ref| = {err:.3e}")
    return got, ws, lay


CONFIG_RUNS = [
    ("tiny", 8, 8, "fp32", "swiglu", INF),
    ("tiny", 8, 5, "ue8m0", "swiglu", INF),
    ("tiny", 8, 8, "pow2", "swiglu_clamp", 0.25),
    ("decode", 1, 1, "fp32", "swiglu", INF),
    ("decode", 4, 4, "fp32", "swiglu", INF),
    ("decode", 4, 4, "fp32", "swiglu_clamp", 7.0),
    ("decode", 4, 4, "fp32", "swiglu_clamp_after_silu", 7.0),
    ("padded", 512, 16, "ue8m0", "swiglu", INF),
    ("padded", 512, 16, "fp32", "swiglu", INF),
    ("sweep", 1, 1, "fp32", "swiglu", INF),
    ("sweep", 8, 8, "pow2", "swiglu", INF),
    ("sweep", 64, 64, "fp32", "swiglu", INF),
    ("sweep", 256, 256, "pow2", "swiglu", INF),
    ("sweep", 1024, 1024, "fp32", "swiglu", INF),
]

# The reciprocal rounding convention on every schedule: the one-launch layer
# (tiny, decode, sweep at 8 tokens with the 4-deep ring), the general path.
RECIPROCAL_RUNS = [
    ("tiny", 8, 8, "fp32", "swiglu", INF),
    ("decode", 4, 4, "fp32", "swiglu", INF),
    ("decode", 1, 1, "ue8m0", "swiglu_clamp", 7.0),
    ("sweep", 8, 8, "pow2", "swiglu", INF),
    ("padded", 512, 16, "fp32", "swiglu", INF),
    ("sweep", 1024, 1024, "fp32", "swiglu", INF),
]


@pytest.mark.parametrize("name,t_cap,t_live,fmt,act,lim", CONFIG_RUNS)
def test_forward_matches_oracle(name, t_cap, t_live, fmt, act, lim):
    run_and_check(name, t_cap, t_live, fmt, act, lim)


@pytest.mark.parametrize("name,t_cap,t_live,fmt,act,lim", RECIPROCAL_RUNS)
def test_forward_reciprocal_rounding_matches_oracle(name, t_cap, t_live, fmt, act, lim):
    run_and_check(name, t_cap, t_live, fmt, act, lim, rounding="reciprocal")


# The 4096-token layers, compared element by element in full (below) rather
# than on samples.
FULL_SIZE_RUNS = [("full", "fp32"), ("full", "ue8m0"), ("sweep", "fp32"), ("sweep", "pow2")]


@pytest.mark.parametrize("name,fmt", FULL_SIZE_RUNS)
def test_full_size_parity_complete(name, fmt):
    """Every live row and every token of the 4096-token layers: alignment and
    activation codes bit-exact; C1 of every live row within tolerance of the
    oracle's fp64 FC1 (from the same codes); the FC2 input codes and scales
    of every live row bit-exact against SiLU+quant of the GPU's own C1; Y of
    every live row within tolerance of the oracle's FC2 of the GPU's own FC2
    input; every output token within tolerance of the oracle's whole layer
    (oracle.forward, whole-expert fp64 GEMMs) and of the combine of the GPU's
    own Y; nothing written outside the live rows."""
    cfg = synth.get(name)
    E, H, I, K, A = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cfg.align_rows
    T = 4096
    say(f"full-size complete parity {name} T={T} fmt={fmt}")
    x, ids, w = synth.make_workload(cfg, T)
    (w1q, w1s), (w2q, w2s) = host_weights(name)
    d = device_weights(name)
    lay = moe.moe_workspace_plan(E, H, I, K, T, A, 0, fmt)
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((T, H), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(up(x), up(ids), up(w), *d, fmt, align_rows=A, out=out, workspace=ws)
    torch.cuda.synchronize()
    R = lay["row_cap"]
    sdt = np.uint8 if fmt == "ue8m0" else np.float32
    ref = oracle.forward(x, ids, w, (w1q, w1s), (w2q, w2s), T, A, fmt)
    total = int(ref["offsets"][-1])
    assert np.array_equal(_ws_view(ws, lay, "expert_counts", np.int32, (E,)), ref["counts"])
    assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, (E + 1,)), ref["offsets"])
    assert np.array_equal(_ws_view(ws, lay, "row_to_pair", np.int32, (R,))[:total], ref["row_to_pair"])
    assert np.array_equal(_ws_view(ws, lay, "pair_to_row", np.int32, (T * K,)), ref["pair_to_row"])
    xq = _ws_view(ws, lay, "xq", np.uint8, (T, H))
    xs = _ws_view(ws, lay, "xs", sdt, (H // 128, T))
    assert np.array_equal(xq, ref["xq"])
    assert np.array_equal(np.ascontiguousarray(xs).view(np.uint8),
                          np.ascontiguousarray(ref["xs"]).view(np.uint8))
    live = ref["live"]
    c1 = _ws_view(ws, lay, "c1", np.uint16, (R, 2 * I))
    err = assert_bf16_close(c1[:total][live], ref["c1"][live], "FC1, every live row")
    say(f"  FC1 max err / max|ref| = {err:.3e}")
    assert np.all(c1[:total][~live] == (POISON_U8 << 8 | POISON_U8))
    hq = _ws_view(ws, lay, "hq", np.uint8, (R, I))
    hs = _ws_view(ws, lay, "hs", sdt, (I // 128, R))
    rhq, rhs = oracle.silu_mul_quant(c1[:total][live], fmt)
    assert np.array_equal(hq[:total][live], rhq)
    assert np.array_equal(np.ascontiguousarray(hs[:, :total][:, live]).view(np.uint8),
                          np.ascontiguousarray(rhs).view(np.uint8))
    y = _ws_view(ws, lay, "y", np.uint16, (R, H))
    ref_y, _ = oracle.grouped_gemm(hq[:total], hs[:, :total], fmt, (w2q, w2s), ref["counts"],
                                   ref["offsets"])
    err = assert_bf16_close(y[:total][live], ref_y[live], "FC2, every live row")
    say(f"  FC2 max err / max|ref| = {err:.3e}")
    got = down(out)
    assert np.all(got[T:] == POISON_BF16)
    assert_bf16_close(got, oracle.combine(y, ref["pair_to_row"], w, T, H), "combine, every token")
    # End to end, every token, against the oracle's chain with each FP8 code
    # decision taken from the same values the GPU took it from: the FC2 input
    # codes are a function of C1, which two correct accumulation orders round
    # to BF16 values one ulp apart here and there, so both sides requantize the
    # GPU's C1 (checked bit for bit above) and the oracle carries its own FC2
    # (fp64) and combine from there.
    anchored = oracle.combine(ref_y, ref["pair_to_row"], w, T, H)
    err = assert_bf16_close(got, anchored, "layer, every token")
    # For the record: against the oracle's chain from its own C1.
    same_row = (np.all(hq[:total] == ref["hq"], axis=1) & np.all(hs[:, :total] == ref["hs"], axis=0)
                & live)
    g64, r64 = oracle.bf16_bits_to_f64(got), oracle.bf16_bits_to_f64(ref["out"])
    worst = float(np.max(np.abs(g64 - r64)) / np.max(np.abs(r64)))
    say(f"  layer max err / max|ref| = {err:.3e} (oracle chain anchored at the FC2-input codes); "
        f"{int((live & ~same_row).sum())} of {int(live.sum())} live rows hold an FC2-input code "
        f"that the oracle's own C1 rounds differently; against that chain {worst:.3e}")


def test_forward_forced_clamp_on_decode_shape():
    """Inputs scaled so that the FC1 outputs exceed the limit of 7.0."""
    cfg = synth.get("decode")
    x = synth.make_tokens(cfg, 4, scale=8.0)
    ids, w = synth.make_routing(cfg, 4)
    (w1q, w1s), (w2q, w2s) = host_weights("decode")
    d = device_weights("decode")
    out, _ = moe.moe_forward(up(x), up(ids), up(w), *d, "fp32", "swiglu_clamp", 7.0, 16)
    torch.cuda.synchronize()
    ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), cfg.num_experts, 4, "fp32",
                               "swiglu_clamp", 7.0)
    plain = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), cfg.num_experts, 4, "fp32")
    assert not np.array_equal(ref, plain)
    assert_bf16_close(down(out), ref, "forced clamp")


def _forward(x, ids, w, name, fmt="fp32", align=16, row_cap=0, t_live=None, ws_fill=None):
    cfg = synth.get(name)
    d = device_weights(name)
    ws = None
    if ws_fill is not None:
        n = moe.moe_workspace_bytes(cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, x.shape[0],
                                    align, row_cap, fmt)
        ws = torch.full((n,), ws_fill, dtype=torch.uint8, device=dev())
    out, _ = moe.moe_forward(up(x), up(ids), up(w), *d, fmt, "swiglu", INF, align, row_cap,
                             t_live=None if t_live is None else up(np.array([t_live], np.int32)),
                             workspace=ws)
    torch.cuda.synchronize()
    return down(out)


def test_output_independent_of_alignment_capacity_and_poison():
    cfg = synth.get("padded")
    x, ids, w = synth.make_workload(cfg, 512, 3)
    base = _forward(x, ids, w, "padded", t_live=16)[:16]
    for align, extra in [(1, 0), (64, 0), (16, 4000)]:
        rc = moe.moe_min_row_cap(512, 8, 32, align) + extra
        got = _forward(x, ids, w, "padded", align=align, row_cap=rc, t_live=16)[:16]
        assert np.array_equal(got, base), (align, extra)
    for fill in (0x00, 0xFF, 0x7F):
        assert np.array_equal(_forward(x, ids, w, "padded", t_live=16, ws_fill=fill)[:16], base)


def test_output_independent_of_token_order():
    cfg = synth.get("decode")
    x, ids, w = synth.make_workload(cfg, 4, 5)
    base = _forward(x, ids, w, "decode")
    perm = np.array([2, 0, 3, 1])
    got = _forward(x[perm], ids[perm], w[perm], "decode")
    assert np.array_equal(got, base[perm])


def test_dropped_ids_and_empty_routing():
    cfg = synth.get("tiny")
    x, ids, w = synth.make_workload(cfg, 8, 6)
    ids2 = ids.copy()
    ids2[::2, 0] = -1
    ids2[1, :] = cfg.num_experts  # every pair of token 1 dropped
    (w1q, w1s), (w2q, w2s) = host_weights("tiny")
    got = _forward(x, ids2, w, "tiny")
    ref = oracle.token_forward(x, ids2, w, (w1q, w1s), (w2q, w2s), 4, 8, "fp32")
    assert np.all(got[1] == 0)
    assert_bf16_close(got, ref, "dropped ids")
    out = torch.full((8, cfg.hidden), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(up(x), up(ids), up(w), *device_weights("tiny"), t_live=up(np.array([0], np.int32)),
                    out=out)
    torch.cuda.synchronize()
    assert np.all(down(out) == POISON_BF16)


REPLAYS = {
    32: [(11, 32), (12, 7), (13, 1), (14, 0), (15, 20)],  # the general schedule
    4: [(11, 4), (12, 3), (13, 1), (14, 0), (15, 2), (16, 4)],  # the one-launch decode layer
}


@pytest.mark.parametrize("t_cap", sorted(REPLAYS))
def test_graph_replay_with_changing_routing_and_live_count(t_cap):
    """Capture the layer once; replay it with new routing, tokens and live
    counts written into the captured buffers (vLLM PR #59128, SM100 on B200:
    graph replay with changing routing, one live row, empty routing and a
    device token count)."""
    gave_up = moe.moe_barrier_timeouts()
    name = "decode"
    cfg = synth.get(name)
    (w1q, w1s), (w2q, w2s) = host_weights(name)
    d = device_weights(name)
    x0, ids0, w0 = synth.make_workload(cfg, t_cap, 10)
    sx, sids, sw = up(x0), up(ids0), up(w0)
    st = up(np.array([t_cap], np.int32))
    out = torch.zeros((t_cap, cfg.hidden), dtype=torch.int16, device=dev())
    nbytes = moe.moe_workspace_bytes(cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, t_cap, 16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture
        moe.moe_forward(sx, sids, sw, *d, t_live=st, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_forward(sx, sids, sw, *d, t_live=st, out=out, workspace=ws)
    torch.cuda.synchronize()
    for variant, t_live in REPLAYS[t_cap]:
        say(f"  replay variant={variant} t_live={t_live}")
        x, ids, w = synth.make_workload(cfg, t_cap, variant)
        sx.copy_(up(x))
        sids.copy_(up(ids))
        sw.copy_(up(w))
        st.fill_(t_live)
        out.fill_(POISON_BF16)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = down(out)
        assert np.all(got[t_live:] == POISON_BF16)
        if t_live:
            ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), cfg.num_experts,
                                       t_live, "fp32")
            assert_bf16_close(got[:t_live], ref, f"replay {variant}")
            eager = _forward(x, ids, w, name, t_live=t_live)
            assert np.array_equal(eager[:t_live], got[:t_live])
    assert moe.moe_barrier_timeouts() == gave_up


# A shape outside the five workloads, for the one-launch decode layer's
# limits: ids of 10 bits (1000 experts) and top-16, so all 64 pair slots of
# the layer's LDS tables are live at 4 tokens.
WIDE = synth.Workload(name="wide", index=9, num_experts=1000, hidden=512, inter=256, topk=16,
                      tokens=(4,), t_cap=4, align_rows=16, row_cap=0, scale_fmts=("fp32",))


@pytest.mark.parametrize("t_live,fmt", [(4, "fp32"), (3, "ue8m0")])
def test_one_launch_layer_wide_routing(t_live, fmt):
    gave_up = moe.moe_barrier_timeouts()
    cfg = WIDE
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk
    say(f"wide routing E={E} top-{K} t_live={t_live} fmt={fmt}")
    x, ids, w = synth.make_workload(cfg, 4)
    ew = synth.ExpertWeights(cfg)
    w1q = np.zeros((E, 2 * I, H), np.uint8)
    w1s = np.zeros((E, 2 * I // 128, H // 128), np.float32)
    w2q = np.zeros((E, H, I), np.uint8)
    w2s = np.zeros((E, H // 128, I // 128), np.float32)
    for e in np.unique(ids):  # only routed experts are ever read
        (w1q[e], w1s[e]), (w2q[e], w2s[e]) = ew.fc1(e), ew.fc2(e)
    lay = moe.moe_workspace_plan(E, H, I, K, 4, cfg.align_rows, 0, fmt)
    assert lay["act"] < lay["status"]  # the decode path
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((4, H), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(up(x), up(ids), up(w), up(w1q), up(w1s), up(w2q), up(w2s), fmt,
                    align_rows=cfg.align_rows, t_live=up(np.array([t_live], np.int32)), out=out,
                    workspace=ws)
    torch.cuda.synchronize()
    assert moe.moe_barrier_timeouts() == gave_up
    al = oracle.align(ids, t_live, E, cfg.align_rows)
    assert np.array_equal(_ws_view(ws, lay, "expert_counts", np.int32, (E,)), al["counts"])
    assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, (E + 1,)), al["offsets"])
    got = down(out)
    assert np.all(got[t_live:] == POISON_BF16)
    ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), E, t_live, fmt)
    err = assert_bf16_close(got[:t_live], ref, "wide layer")
    say(f"  layer max err / max|ref| = {err:.3e}")


# The one-launch layer's variant with a 4-deep weight ring, for token codes
# beyond the 6-deep layout's 24 KB of LDS (up to 60 KB and 512 scales).
MANY_TOKENS = [
    # t_cap, t_live, E, H, I, topk, fmt, act, limit
    (8, 8, 256, 6144, 256, 8, "fp32", "swiglu", float("inf")),      # the sweep shape at 8 tokens
    (8, 7, 64, 7168, 256, 8, "ue8m0", "swiglu_clamp", 7.0),         # 56 KB of codes, 448 scales
    (16, 13, 96, 3584, 256, 4, "pow2", "swiglu_clamp_after_silu", 7.0),  # 16 tokens
]


@pytest.mark.parametrize("t_cap,t_live,E,H,I,K,fmt,act,lim", MANY_TOKENS)
def test_one_launch_layer_many_token_bytes(t_cap, t_live, E, H, I, K, fmt, act, lim):
    gave_up = moe.moe_barrier_timeouts()
    assert t_cap * (H + 16) > 24576 and t_cap * (H + 16) <= 61440 and t_cap * (H // 128) <= 512
    cfg = synth.Workload(name="many", index=10 + t_cap + H % 1000, num_experts=E, hidden=H, inter=I,
                         topk=K, tokens=(t_cap,), t_cap=t_cap, align_rows=16, row_cap=0,
                         scale_fmts=(fmt,))
    say(f"one-launch layer, wide ring: t_cap={t_cap} t_live={t_live} E={E} H={H} I={I} top-{K} {fmt} {act}")
    x, ids, w = synth.make_workload(cfg, t_cap)
    ew = synth.ExpertWeights(cfg)
    w1q = np.zeros((E, 2 * I, H), np.uint8)
    w1s = np.zeros((E, 2 * I // 128, H // 128), np.float32)
    w2q = np.zeros((E, H, I), np.uint8)
    w2s = np.zeros((E, H // 128, I // 128), np.float32)
    for e in np.unique(ids):  # only routed experts are ever read
        (w1q[e], w1s[e]), (w2q[e], w2s[e]) = ew.fc1(e), ew.fc2(e)
    lay = moe.moe_workspace_plan(E, H, I, K, t_cap, cfg.align_rows, 0, fmt)
    assert lay["act"] < lay["status"]  # the decode path
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((t_cap, H), POISON_BF16, dtype=torch.int16, device=dev())
    lim32 = float(np.float32(lim))
    for rep in range(2):  # the barrier's epochs advance per launch
        moe.moe_forward(up(x), up(ids), up(w), up(w1q), up(w1s), up(w2q), up(w2s), fmt, act=act,
                        clamp_limit=lim32, align_rows=cfg.align_rows,
                        t_live=up(np.array([t_live], np.int32)), out=out, workspace=ws)
        torch.cuda.synchronize()
        assert moe.moe_barrier_timeouts() == gave_up
    al = oracle.align(ids, t_live, E, cfg.align_rows)
    assert np.array_equal(_ws_view(ws, lay, "expert_counts", np.int32, (E,)), al["counts"])
    assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, (E + 1,)), al["offsets"])
    got = down(out)
    assert np.all(got[t_live:] == POISON_BF16)
    ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), E, t_live, fmt, act=act,
                               clamp_limit=lim32)
    err = assert_bf16_close(got[:t_live], ref, "wide-ring layer")
    say(f"  layer max err / max|ref| = {err:.3e}")


def test_one_launch_variants_alternate():
    """The 6-deep and 4-deep ring variants of the one-launch layer share the
    grid barrier's epochs: launches alternating between them (and repeated)
    stay correct and no barrier wait gives up."""
    gave_up = moe.moe_barrier_timeouts()
    cases = []
    for t_cap, H, idx in [(2, 1024, 30), (8, 4096, 31)]:  # 2 x 1040 B / 8 x 4112 B of codes
        cfg = synth.Workload(name="alt", index=idx, num_experts=16, hidden=H, inter=256, topk=8,
                             tokens=(t_cap,), t_cap=t_cap, align_rows=16, row_cap=0,
                             scale_fmts=("fp32",))
        x, ids, w = synth.make_workload(cfg, t_cap)
        ew = synth.ExpertWeights(cfg)
        (w1q, w1s), (w2q, w2s) = ew.stacked()
        lay = moe.moe_workspace_plan(16, H, 256, 8, t_cap)
        assert moe.decode_layer_applies(t_cap, 8, H, 256)
        ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), 16, t_cap, "fp32")
        dev_in = [up(a) for a in (x, ids, w, w1q, w1s, w2q, w2s)]
        ws = torch.empty((lay["total"],), dtype=torch.uint8, device=dev())
        cases.append((t_cap, H, dev_in, ws, ref))
    say("one-launch layer: 6-deep and 4-deep ring launches alternating")
    for order in (0, 1, 0, 0, 1, 1, 0):
        t_cap, H, dev_in, ws, ref = cases[order]
        out = torch.full((t_cap, H), POISON_BF16, dtype=torch.int16, device=dev())
        moe.moe_forward(*dev_in, "fp32", out=out, workspace=ws)
        torch.cuda.synchronize()
        assert moe.moe_barrier_timeouts() == gave_up
        assert_bf16_close(down(out), ref, f"one-launch layer t_cap={t_cap} H={H}")


def test_padded_tiles_are_skipped():
    """On the 512-capacity / 16-live workload the FC1 GEMM visits exactly the
    tiles that hold live rows, far fewer than the capacity holds."""
    name = "padded"
    cfg = synth.get(name)
    x, ids, w = synth.make_workload(cfg, 512)
    _, ws, lay = run_and_check(name, 512, 16, "fp32", n_tok=4, n_rows=8)
    R, E, H, I = lay["row_cap"], cfg.num_experts, cfg.hidden, cfg.inter
    d_w1q, d_w1s, _, _ = device_weights(name)

    def view(nm, dt, n):
        return ws[lay[nm]:lay[nm] + n * np.dtype(dt).itemsize].view(
            torch.int32 if dt == np.int32 else torch.uint8)
    counts = view("expert_counts", np.int32, E)
    offsets = view("expert_offsets", np.int32, E + 1)
    r2p = view("row_to_pair", np.int32, R)
    xq = ws[lay["xq"]:lay["xq"] + 512 * H].view(512, H)
    xs = ws[lay["xs"]:lay["xs"] + (H // 128) * 512 * 4].view(torch.float32).view(H // 128, 512)
    c = torch.empty((R, 2 * I), dtype=torch.int16, device=dev())
    tiles = torch.zeros(1, dtype=torch.int32, device=dev())
    moe.moe_grouped_gemm_fp8(xq, xs, "fp32", d_w1q, d_w1s, counts, offsets, R, a_row_map=r2p,
                             a_row_div=cfg.topk, out=c, tiles_visited=tiles)
    torch.cuda.synchronize()
    cnt = down(counts)
    live_tiles = sum(-(-int(v) // 16) for v in cnt if v > 0) * (2 * I // 128)
    capacity_tiles = -(-R // 16) * (2 * I // 128)
    assert int(tiles.item()) == live_tiles
    assert live_tiles * 4 < capacity_tiles


FC1_DECODE_RUNS = [
    ("decode", 4, 4, "fp32", "swiglu", INF, "divide"),
    ("decode", 4, 4, "fp32", "swiglu", INF, "reciprocal"),
    ("decode", 4, 3, "ue8m0", "swiglu_clamp", 7.0, "divide"),
    ("decode", 1, 1, "pow2", "swiglu_clamp_after_silu", 7.0, "divide"),
    ("decode", 1, 1, "pow2", "swiglu_clamp_after_silu", 7.0, "reciprocal"),
    ("tiny", 8, 5, "fp32", "swiglu", INF, "divide"),
    ("sweep", 1, 1, "fp32", "swiglu", INF, "divide"),
]


@pytest.mark.parametrize("name,t_cap,t_live,fmt,act,lim,rounding", FC1_DECODE_RUNS)
def test_fc1_decode_alone(name, t_cap, t_live, fmt, act, lim, rounding):
    """The decode path's first launch on its own: alignment and activation codes
    bit-exact, C1 rows within the GEMM tolerance, act = SiLU(gate)*up of the GPU's
    own C1 rows bit for bit, and nothing written outside the live rows."""
    cfg = synth.get(name)
    say(f"fc1_decode {name} t_cap={t_cap} t_live={t_live} fmt={fmt} act={act} {rounding}")
    E, H, I, K, A = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cfg.align_rows
    x, ids, w = synth.make_workload(cfg, t_cap)
    (w1q, w1s), _ = host_weights(name)
    d_w1q, d_w1s, _, _ = device_weights(name)
    lim32 = float(np.float32(lim))
    row_cap = cfg.row_cap or 0
    lay = moe.moe_workspace_plan(E, H, I, K, t_cap, A, row_cap, fmt, act, lim32, rounding)
    assert lay["act"] < lay["status"]
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    moe.moe_fc1_decode(up(x), up(ids), d_w1q, d_w1s, I, fmt, act, lim32, A, row_cap,
                       t_live=up(np.array([t_live], np.int32)), workspace=ws, rounding=rounding)
    torch.cuda.synchronize()
    R = lay["row_cap"]
    sdt = np.uint8 if fmt == "ue8m0" else np.float32
    al = oracle.align(ids, t_live, E, A)
    assert np.array_equal(_ws_view(ws, lay, "expert_counts", np.int32, (E,)), al["counts"])
    assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, (E + 1,)), al["offsets"])
    total = int(al["offsets"][-1])
    r2p = _ws_view(ws, lay, "row_to_pair", np.int32, (R,))
    assert np.array_equal(r2p[:total], al["row_to_pair"])
    assert np.all(r2p[total:].view(np.uint32) == np.uint32(POISON_U8 * 0x01010101))
    p2r = _ws_view(ws, lay, "pair_to_row", np.int32, (t_cap * K,))
    assert np.array_equal(p2r[:t_live * K], al["pair_to_row"])
    xq = _ws_view(ws, lay, "xq", np.uint8, (t_cap, H))
    xs = _ws_view(ws, lay, "xs", sdt, (H // 128, t_cap))
    rq, rs = oracle.quantize_groups(oracle.bf16_bits_to_f64(x[:t_live]).astype(np.float32), fmt,
                                    rounding)
    assert np.array_equal(xq[:t_live], rq)
    assert np.all(xq[t_live:] == POISON_U8)
    assert np.array_equal(np.ascontiguousarray(xs[:, :t_live]).view(np.uint8),
                          np.ascontiguousarray(rs).view(np.uint8))
    c1 = _ws_view(ws, lay, "c1", np.uint16, (R, 2 * I))
    act_rows = _ws_view(ws, lay, "act", np.float32, (R, I))
    sa_x = oracle.scales_to_f64(xs, fmt)
    live_rows = np.flatnonzero(np.isin(np.arange(R), al["pair_to_row"][al["pair_to_row"] >= 0]))
    for e in np.flatnonzero(al["counts"] > 0):
        seg = np.arange(al["offsets"][e], al["offsets"][e] + al["counts"][e])
        tok = al["row_to_pair"][seg] // K
        ref_c1 = oracle.moe.gemm_rows(xq[tok], sa_x[:, tok], w1q[e], w1s[e], rounding)
        assert_bf16_close(c1[seg], ref_c1, f"FC1 expert {e}")
        g = oracle.bf16_bits_to_f64(c1[seg][:, :I])
        u = oracle.bf16_bits_to_f64(c1[seg][:, I:])
        ref_act = oracle.moe.swiglu(g, u, act, lim32, rounding)
        assert np.array_equal(act_rows[seg].view(np.uint32), ref_act.view(np.uint32)), e
    dead = np.setdiff1d(np.arange(R), live_rows)
    assert np.all(c1[dead] == (POISON_U8 << 8 | POISON_U8))


@pytest.mark.parametrize("weights", ["e4m3", "mxfp4"])
def test_barrier_timeout_is_reported_in_the_launch_outputs(weights):
    """A grid-barrier wait of the one-launch layer that gives up (forced from
    the host: a negative spin limit makes every wait give up at once, and every
    kernel still exits normally) shows in that launch's own outputs: each
    workgroup's status slot says so and its output columns of the live tokens
    are NaN. With the limit restored the next launch is correct again and all
    slots read 0. Both weight formats' kernels."""
    name = "decode"
    cfg = synth.get(name)
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk
    x, ids, w = synth.make_workload(cfg, 4, 7)
    if weights == "mxfp4":
        (w1q, w1s), (w2q, w2s) = synth.ExpertWeightsMxfp4(cfg).stacked(threads=16)
        d = (up(w1q), up(w1s), up(w2q), up(w2s))
    else:
        (w1q, w1s), (w2q, w2s) = host_weights(name)
        d = device_weights(name)
    assert moe.decode_layer_applies(4, K, H, I, weights)
    lay = moe.moe_workspace_plan(E, H, I, K, 4, weight_fmt=weights)
    ws = torch.full((lay["total"],), POISON_U8, dtype=torch.uint8, device=dev())
    out = torch.full((4, H), POISON_BF16, dtype=torch.int16, device=dev())
    live = up(np.array([3], np.int32))
    before = moe.moe_barrier_timeouts()
    old = moe.moe_barrier_spin_limit(-1)
    try:
        say(f"one-launch layer ({weights} weights) with every barrier wait forced to give up")
        moe.moe_forward(up(x), up(ids), up(w), *d, t_live=live, out=out, workspace=ws, weight_fmt=weights)
        torch.cuda.synchronize()
    finally:
        moe.moe_barrier_spin_limit(old)
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    status = _ws_view(ws, lay, "status", np.int32, (1024,))
    assert np.all(status[:grid] == 1)
    assert np.all(status[grid:].view(np.uint32) == np.uint32(POISON_U8 * 0x01010101))
    got = down(out)
    assert np.all(got[:3] == 0x7FC0), "output columns of a failed workgroup must be NaN"
    assert np.all(got[3:] == POISON_BF16)
    assert moe.moe_barrier_timeouts() >= before + grid
    # the next launch, with the default limit, is whole again
    say("one-launch layer with the default spin limit")
    moe.moe_forward(up(x), up(ids), up(w), *d, t_live=live, out=out, workspace=ws, weight_fmt=weights)
    torch.cuda.synchronize()
    assert np.all(_ws_view(ws, lay, "status", np.int32, (1024,))[:grid] == 0)
    ref = oracle.token_forward(x, ids, w, (w1q, w1s), (w2q, w2s), E, 3, "fp32", weight_fmt=weights)
    assert_bf16_close(down(out)[:3], ref, "after a forced timeout")


@pytest.mark.parametrize("name,t_cap", [("decode", 4), ("tiny", 8), ("sweep", 64)])
def test_missing_routing_weights_mean_ones(name, t_cap):
    cfg = synth.get(name)
    x, ids, _ = synth.make_workload(cfg, t_cap, 8)
    d = device_weights(name)
    ones = np.ones(ids.shape, np.float32)
    a, _ = moe.moe_forward(up(x), up(ids), None, *d, align_rows=cfg.align_rows)
    b, _ = moe.moe_forward(up(x), up(ids), up(ones), *d, align_rows=cfg.align_rows)
    torch.cuda.synchronize()
    assert np.array_equal(down(a), down(b))
