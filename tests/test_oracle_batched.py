"""Pins for the oracle's batched masked-M layout (vLLM PR #65794, Details,
"Batched experts") and expert-parallel local ids (TensorRT-LLM PR #21250, For
MoE owners; review comment: drop pairs of other ranks' experts)."""

import numpy as np
import pytest

import oracle
from synth.gen import quantize_weight_blocks


def brute_force_batched(ids, t_live, num_experts, cap, start=0):
    """Per-expert lists in (t, k) order, cut at the capacity."""
    k = ids.shape[1]
    lists = {e: [] for e in range(num_experts)}
    for t in range(t_live):
        for kk in range(k):
            e = int(ids[t, kk]) - start
            if e in lists:
                lists[e].append(t * k + kk)
    rows = [-1] * (num_experts * cap)
    p2r = [-1] * (t_live * k)
    over = 0
    for e, seg in lists.items():
        for i, p in enumerate(seg):
            if i < cap:
                rows[e * cap + i] = p
                p2r[p] = e * cap + i
            else:
                over += 1
    return [min(len(lists[e]), cap) for e in range(num_experts)], rows, p2r, over


CASES = [
    # t_cap, t_live, K, E, cap, start, seed, id range
    (8, 8, 2, 4, 16, 0, 0, (0, 4)),
    (8, 5, 2, 4, 3, 0, 1, (0, 4)),          # capacity overflows
    (16, 16, 8, 72, 4, 0, 2, (0, 72)),
    (7, 7, 3, 5, 8, 0, 3, (-2, 7)),         # invalid ids
    (4, 0, 8, 288, 2, 0, 4, (0, 288)),      # empty routing
    (24, 24, 8, 16, 40, 32, 5, (0, 96)),    # rank owning experts [32, 48)
    (30, 28, 4, 8, 5, 100, 6, (90, 120)),   # ids below and above the rank's range
]


@pytest.mark.parametrize("t_cap,t_live,k,e,cap,start,seed,rng", CASES)
def test_batched_align_matches_brute_force(t_cap, t_live, k, e, cap, start, seed, rng):
    g = np.random.default_rng(seed)
    ids = g.integers(rng[0], rng[1], (t_cap, k)).astype(np.int32)
    got = oracle.align_batched(ids, t_live, e, cap, start)
    masked, rows, p2r, over = brute_force_batched(ids, t_live, e, cap, start)
    assert got["masked_m"].tolist() == masked
    assert got["row_to_pair"].tolist() == rows
    assert got["pair_to_row"].tolist() == p2r
    assert got["overflow"] == over
    assert got["offsets"].tolist() == [i * cap for i in range(e + 1)]


@pytest.mark.parametrize("t_cap,t_live,k,e,cap,start,seed,rng", CASES)
def test_local_ids_drop_other_ranks_pairs(t_cap, t_live, k, e, cap, start, seed, rng):
    """align with expert_start equals align of the ids with every pair of
    another rank's expert replaced by an invalid id, shifted to local ids."""
    g = np.random.default_rng(seed)
    ids = g.integers(rng[0], rng[1], (t_cap, k)).astype(np.int32)
    owned = (ids >= start) & (ids < start + e)
    local = np.where(owned, ids - start, -1).astype(np.int32)
    a = oracle.align(ids, t_live, e, 16, start)
    b = oracle.align(local, t_live, e, 16)
    for key in a:
        assert np.array_equal(a[key], b[key])


def _layer(g, e, h, inter):
    w1 = [quantize_weight_blocks((g.standard_normal((2 * inter, h)) * 0.05).astype(np.float32)) for _ in range(e)]
    w2 = [quantize_weight_blocks((g.standard_normal((h, inter)) * 0.05).astype(np.float32)) for _ in range(e)]
    return ((np.stack([a for a, _ in w1]), np.stack([b for _, b in w1])),
            (np.stack([a for a, _ in w2]), np.stack([b for _, b in w2])))


@pytest.mark.parametrize("fmt,rounding", [("fp32", "divide"), ("ue8m0", "reciprocal")])
def test_batched_layer_equals_aligned_layer_and_brute_force(fmt, rounding):
    g = np.random.default_rng(31)
    e, h, inter, k, t = 5, 256, 128, 3, 9
    W1, W2 = _layer(g, e, h, inter)
    x = oracle.bf16_from_f64(g.standard_normal((t, h)))
    ids = g.integers(0, e, (t, k)).astype(np.int32)
    w = g.uniform(0.1, 1, (t, k)).astype(np.float32)
    cap = int(max(np.bincount(ids.reshape(-1), minlength=e)))
    batched = oracle.forward(x, ids, w, W1, W2, t, 16, fmt, rounding=rounding, expert_cap=cap + 3)
    aligned = oracle.forward(x, ids, w, W1, W2, t, 16, fmt, rounding=rounding)
    assert np.array_equal(batched["out"], aligned["out"])
    brute = oracle.token_forward(x, ids, w, W1, W2, e, t, fmt, rounding=rounding)
    assert np.array_equal(batched["out"], brute)


def test_batched_layer_with_overflow_drops_the_late_pairs():
    g = np.random.default_rng(32)
    e, h, inter, k, t = 3, 128, 128, 2, 12
    W1, W2 = _layer(g, e, h, inter)
    x = oracle.bf16_from_f64(g.standard_normal((t, h)))
    ids = g.integers(0, e, (t, k)).astype(np.int32)
    w = g.uniform(0.1, 1, (t, k)).astype(np.float32)
    cap = 4
    res = oracle.forward(x, ids, w, W1, W2, t, 16, "fp32", expert_cap=cap)
    assert res["overflow"] > 0
    kept = ids.copy()
    seen = np.zeros(e, int)
    for tt in range(t):
        for kk in range(k):
            ex = ids[tt, kk]
            if seen[ex] >= cap:
                kept[tt, kk] = -1
            seen[ex] += 1
    brute = oracle.token_forward(x, kept, w, W1, W2, e, t, "fp32")
    assert np.array_equal(res["out"], brute)


@pytest.mark.parametrize("expert_cap", [0, 24])
def test_expert_parallel_rank_equals_layer_restricted_to_owned_pairs(expert_cap):
    """A rank owning experts [start, start + E) with the local slice of the
    weights computes exactly the layer over its owned pairs only."""
    g = np.random.default_rng(33)
    e_total, e, start, h, inter, k, t = 12, 4, 4, 256, 128, 4, 10
    W1, W2 = _layer(g, e_total, h, inter)
    x = oracle.bf16_from_f64(g.standard_normal((t, h)))
    ids = g.integers(0, e_total, (t, k)).astype(np.int32)
    w = g.uniform(0.1, 1, (t, k)).astype(np.float32)
    L1 = (W1[0][start:start + e], W1[1][start:start + e])
    L2 = (W2[0][start:start + e], W2[1][start:start + e])
    rank = oracle.forward(x, ids, w, L1, L2, t, 16, "fp32", expert_start=start,
                          expert_cap=expert_cap)["out"]
    owned_only = np.where((ids >= start) & (ids < start + e), ids, -1).astype(np.int32)
    ref = oracle.token_forward(x, owned_only, w, W1, W2, e_total, t, "fp32")
    assert np.array_equal(rank, ref)
