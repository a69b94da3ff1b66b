"""Top-k routing alignment into per-expert contiguous rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (vLLM PR #59128, Purpose: a shared permutation helper
produces expert endpoints that both grouped GEMMs and the fused activation
quantization consume; an alignment scope pads each expert's rows; TensorRT-LLM
PR #21250, description and sequence diagram: alignment produces padded expert
blocks and sorted token ids; review comment on expert parallelism: ids outside
the local range should be dropped rather than clamped):

* every (token, k) pair p = t*K + k with a valid expert id gets one row in
  that expert's segment;
* segment e starts at the prefix sum of the earlier experts' row counts, each
  rounded up to the alignment;
* ids outside [0, E) are dropped.

Readings where the pages are silent: within a segment, pairs are in
ascending p (a stable counting sort); pad rows inside a segment map to -1;
rows past the last endpoint, and pairs of tokens past the live count, are
not part of the result (the device leaves them untouched).

Expert parallelism (TensorRT-LLM PR #21250, For MoE owners and the review
comment that asks to drop non-owned pairs instead of clamping them): a rank
owns experts [expert_start, expert_start + E); its local id of a routed id is
id - expert_start, and pairs whose local id falls outside [0, E) are dropped
like invalid ids.

The batched masked-M layout (vLLM PR #65794, Details, "Batched experts":
persistent_masked_m_silu_mul_quant): a fixed capacity of ``cap`` rows per
expert, expert e owning rows [e*cap, (e+1)*cap), of which the first
masked_m[e] = min(count, cap) are live, in ascending pair order. The pages do
not say what happens to pairs beyond the capacity; the reading taken here
drops them (their pair maps to -1) and reports how many were dropped.
"""

import numpy as np


def align(topk_ids, t_live, num_experts, align_rows, expert_start=0):
    """Stable counting sort of the live (token, k) pairs by expert.

    ``topk_ids`` is [t_cap, K] int. Only tokens t < t_live take part; local
    ids are id - expert_start. Returns a dict with ``counts[E]``,
    ``offsets[E+1]``, ``row_to_pair[offsets[E]]`` and ``pair_to_row[t_live*K]``
    (int32).
    """
    ids = np.asarray(topk_ids, dtype=np.int64) - int(expert_start)
    k = ids.shape[1]
    n_pairs = t_live * k
    flat = ids.reshape(-1)[:n_pairs]

    counts = np.zeros(num_experts, dtype=np.int64)
    for p in range(n_pairs):
        e = int(flat[p])
        if 0 <= e < num_experts:
            counts[e] += 1

    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    for e in range(num_experts):
        padded = -(-int(counts[e]) // align_rows) * align_rows
        offsets[e + 1] = offsets[e] + padded

    row_to_pair = np.full(int(offsets[num_experts]), -1, dtype=np.int64)
    pair_to_row = np.full(n_pairs, -1, dtype=np.int64)
    fill = np.zeros(num_experts, dtype=np.int64)
    for p in range(n_pairs):
        e = int(flat[p])
        if 0 <= e < num_experts:
            row = int(offsets[e] + fill[e])
            fill[e] += 1
            row_to_pair[row] = p
            pair_to_row[p] = row

    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "row_to_pair": row_to_pair.astype(np.int32),
        "pair_to_row": pair_to_row.astype(np.int32),
    }


def align_batched(topk_ids, t_live, num_experts, cap, expert_start=0):
    """The batched masked-M layout: pairs of local expert e in rows
    [e*cap, e*cap + masked_m[e]), ascending pair order; pairs beyond the
    capacity dropped.

    Returns a dict with ``masked_m[E]`` (live rows per expert),
    ``offsets[E+1]`` (= e*cap, so the layout reads as segments),
    ``row_to_pair[E*cap]`` (-1 on rows that hold no pair),
    ``pair_to_row[t_live*K]`` and ``overflow`` (pairs dropped for capacity).
    """
    ids = np.asarray(topk_ids, dtype=np.int64) - int(expert_start)
    k = ids.shape[1]
    n_pairs = t_live * k
    flat = ids.reshape(-1)[:n_pairs]
    fill = np.zeros(num_experts, dtype=np.int64)
    row_to_pair = np.full(num_experts * cap, -1, dtype=np.int64)
    pair_to_row = np.full(n_pairs, -1, dtype=np.int64)
    overflow = 0
    for p in range(n_pairs):
        e = int(flat[p])
        if not 0 <= e < num_experts:
            continue
        if fill[e] < cap:
            row = e * cap + int(fill[e])
            row_to_pair[row] = p
            pair_to_row[p] = row
        else:
            overflow += 1
        fill[e] += 1
    return {
        "masked_m": np.minimum(fill, cap).astype(np.int32),
        "offsets": (np.arange(num_experts + 1, dtype=np.int64) * cap).astype(np.int32),
        "row_to_pair": row_to_pair.astype(np.int32),
        "pair_to_row": pair_to_row.astype(np.int32),
        "overflow": overflow,
    }
