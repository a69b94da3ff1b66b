"""Pins for the oracle's routing alignment: brute force and invariants."""

import numpy as np
import pytest

import oracle


def brute_force(ids, t_live, num_experts, a):
    """Lists per expert, appended in (t, k) order, then laid out end to end."""
    k = ids.shape[1]
    lists = {e: [] for e in range(num_experts)}
    for t in range(t_live):
        for kk in range(k):
            e = int(ids[t, kk])
            if e in lists:
                lists[e].append(t * k + kk)
    rows, p2r, counts, offsets = [], {}, [], [0]
    for e in range(num_experts):
        seg = lists[e]
        counts.append(len(seg))
        pad = (-len(seg)) % a
        for p in seg:
            p2r[p] = len(rows)
            rows.append(p)
        rows.extend([-1] * pad)
        offsets.append(len(rows))
    pair_to_row = [p2r.get(p, -1) for p in range(t_live * k)]
    return counts, offsets, rows, pair_to_row


CASES = [
    # (t_cap, t_live, K, E, A, seed, id range)
    (8, 8, 2, 4, 16, 0, (0, 4)),
    (8, 5, 2, 4, 1, 1, (0, 4)),
    (16, 16, 8, 72, 16, 2, (0, 72)),      # 128 pairs, non-power-of-two E
    (24, 24, 8, 72, 16, 3, (0, 72)),      # 192 pairs
    (7, 7, 3, 5, 4, 4, (-2, 7)),          # invalid ids on both sides
    (9, 9, 3, 3, 2, 5, (0, 2)),           # expert 2 empty, duplicates
    (4, 0, 8, 288, 16, 6, (0, 288)),      # empty routing
    (64, 40, 8, 256, 16, 7, (0, 256)),
    (300, 300, 8, 32, 16, 8, (0, 32)),
]


@pytest.mark.parametrize("t_cap,t_live,k,e,a,seed,rng", CASES)
def test_align_matches_brute_force(t_cap, t_live, k, e, a, seed, rng):
    g = np.random.default_rng(seed)
    ids = g.integers(rng[0], rng[1], (t_cap, k)).astype(np.int32)
    got = oracle.align(ids, t_live, e, a)
    counts, offsets, rows, p2r = brute_force(ids, t_live, e, a)
    assert got["counts"].tolist() == counts
    assert got["offsets"].tolist() == offsets
    assert got["row_to_pair"].tolist() == rows
    assert got["pair_to_row"].tolist() == p2r


@pytest.mark.parametrize("t_cap,t_live,k,e,a,seed,rng", CASES)
def test_align_invariants(t_cap, t_live, k, e, a, seed, rng):
    g = np.random.default_rng(seed)
    ids = g.integers(rng[0], rng[1], (t_cap, k)).astype(np.int32)
    r = oracle.align(ids, t_live, e, a)
    flat = ids.reshape(-1)[:t_live * k]
    valid = (flat >= 0) & (flat < e)
    assert r["counts"].sum() == valid.sum()
    off = r["offsets"]
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and np.all(off % a == 0)
    assert np.all(np.diff(off) == -(-r["counts"] // a) * a)
    # every valid pair exactly once, in its expert's segment, ascending
    p2r = r["pair_to_row"]
    assert np.all((p2r >= 0) == valid)
    assert len(set(p2r[valid].tolist())) == valid.sum()
    for ex in range(e):
        seg = r["row_to_pair"][off[ex]:off[ex + 1]]
        live = seg[:r["counts"][ex]]
        assert np.all(np.diff(live) > 0)
        assert np.all(flat[live] == ex)
        assert np.all(seg[r["counts"][ex]:] == -1)
        assert np.all(p2r[live] == np.arange(off[ex], off[ex] + len(live)))


def test_align_ignores_tokens_past_live_count():
    g = np.random.default_rng(9)
    ids = g.integers(0, 8, (10, 4)).astype(np.int32)
    a = oracle.align(ids, 6, 8, 4)
    ids2 = ids.copy()
    ids2[6:] = g.integers(0, 8, (4, 4))
    b = oracle.align(ids2, 6, 8, 4)
    for key in a:
        assert np.array_equal(a[key], b[key])
