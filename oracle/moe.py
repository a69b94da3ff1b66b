"""The expert layer, stage by stage, in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Stages and the passages they follow:

* ``grouped_gemm`` -- FP8 x FP8 products with 128x128 weight block scales
  and 1x128 activation scales (TensorRT-LLM PR #21250, description; vLLM PR
  #59128, Purpose: one grouped GEMM per projection over the live rows of each
  expert). Each 128-wide K block's partial dot product is formed exactly
  (every E4M3 value is a multiple of 2**-9, so a product is a multiple of
  2**-18 below 2**18 and a 128-term sum needs at most 43 bits), scaled by
  the exact product of its two scales, and accumulated over K blocks in
  ascending order in fp64. The block-scale order the TensorRT-LLM review
  discusses does not arise: sa*sb is exact in fp64. Outputs are rounded once
  to BF16.
* ``swiglu`` / ``silu_mul_quant`` -- SiLU(gate) * up without an intermediate
  BF16 rounding, then the 1x128 quantization rule (vLLM PR #65794, Details:
  the fused kernel's arithmetic). Gate is the first half of the FC1 output
  columns, up the second half (the pages leave the order open; the weight
  layout [E, 2I, H] puts gate rows first here). SiLU is evaluated in fp64 as
  g / (1 + exp(-g)), times u in fp64, and rounded once to float32.
* ``rounding="reciprocal"`` -- the convention of the fused CUTLASS op that
  TensorRT-LLM PR #21250 follows (rounding-fix commit message; review comment
  on the block-scale order): both quantizers multiply by fl32(448 / amax)
  (see ``quant``), the SwiGLU output is rounded to BF16 before its FP8
  quantization, and each K block's scale is the float32 product
  fl32(sa * sw), formed before it multiplies the block's dot product. The
  default ``divide`` is vLLM PR #65794's arithmetic described above.
* ``weight_fmt="mxfp4"`` -- FP4 weights (vLLM PR #59128, description, names
  FP4 weights only; the format read as OCP MXFP4, see ``fp_formats``): each
  weight is e2m1(code) * 2**(b - 127) with one E8M0 byte b per 32 weights
  along K, so the weight scale sits inside the 128-wide K block instead of
  multiplying it. Per 128-wide K block the partial dot product of the E4M3
  activations with the dequantized weights is formed in fp64 (exact when the
  block's four weight scales lie within 20 binades of each other, as in every
  test input), multiplied by the activation scale and accumulated; the
  rounding conventions only differ upstream, in the quantizers.
* ``combine`` -- the routing weights scale the BF16 expert outputs, in top-k
  order, not the FC2 accumulators (TensorRT-LLM PR #21250, rounding-fix
  commit message). Accumulated in fp64, rounded once to BF16. A token with
  no valid pair gets zeros.
* ``forward`` -- align, quantize, FC1, SiLU*up+quantize, FC2, combine in the
  order the pages' full-expert benchmark covers them (vLLM PR #59128, SM100
  on B200) and TensorRT-LLM PR #21250's sequence diagram shows.
* ``token_forward`` -- the same layer computed token by token with no
  alignment at all (dense per-token brute force); it must equal ``forward``
  bit for bit.
"""

import numpy as np

from .align import align, align_batched
from .fp_formats import (bf16_bits_to_f64, bf16_from_f64, e2m1_decode, e4m3_decode,
                         e8m0_decode, fp4_unpack)
from .quant import GROUP, ROUNDINGS, quantize_groups, scales_to_f64

ACTS = ("swiglu", "swiglu_clamp", "swiglu_clamp_after_silu")
WEIGHT_FMTS = ("e4m3", "mxfp4")
MX_BLOCK = 32  # weights per E8M0 scale along K

_DECODE_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))


def _dec(codes):
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def gemm_rows(a_codes, a_scales, w_codes, w_scales, rounding="divide"):
    """C[m, n] = bf16( sum_kb (sa[kb, m] * sw[n/128, kb]) * sum_{j<128} a*w ).

    ``a_codes`` [m, Kd] uint8, ``a_scales`` [Kd/128, m] float64 (decoded),
    ``w_codes`` [N, Kd] uint8, ``w_scales`` [N/128, Kd/128] float32.
    Under ``rounding="reciprocal"`` the block factor is fl32(sa * sw).
    Returns BF16 bits [m, N].
    """
    if rounding not in ROUNDINGS:
        raise ValueError(rounding)
    a = _dec(a_codes)
    w = _dec(w_codes)
    m, kd = a.shape
    n = w.shape[0]
    nkb = kd // GROUP
    sw = np.repeat(np.asarray(w_scales, dtype=np.float64), GROUP, axis=0)  # [N, nkb]
    acc = np.zeros((m, n), dtype=np.float64)
    for kb in range(nkb):
        cols = slice(kb * GROUP, (kb + 1) * GROUP)
        part = a[:, cols] @ w[:, cols].T  # exact (see module docstring)
        scale = a_scales[kb][:, None] * sw[:, kb][None, :]  # exact in fp64
        if rounding == "reciprocal":  # the float32 product of the two scales
            scale = (a_scales[kb].astype(np.float32)[:, None]
                     * sw[:, kb].astype(np.float32)[None, :]).astype(np.float64)
        acc = acc + scale * part
    return bf16_from_f64(acc)


def mxfp4_dequant(w_packed, w_scales):
    """[N, Kd/2] packed E2M1 codes and [N, Kd/32] E8M0 bytes -> float64 [N, Kd]."""
    w = e2m1_decode(fp4_unpack(w_packed))
    s = np.repeat(e8m0_decode(w_scales), MX_BLOCK, axis=1)
    return w * s


def gemm_rows_mxfp4(a_codes, a_scales, w_packed, w_scales):
    """C[m, n] = bf16( sum_kb sa[kb, m] * sum_{j<128} a * w ) with MXFP4 weights.

    ``a_codes`` [m, Kd] uint8 E4M3, ``a_scales`` [Kd/128, m] float64 (decoded),
    ``w_packed`` [N, Kd/2] uint8, ``w_scales`` [N, Kd/32] uint8 (E8M0).
    Returns BF16 bits [m, N].
    """
    a = _dec(a_codes)
    w = mxfp4_dequant(w_packed, w_scales)
    m, kd = a.shape
    acc = np.zeros((m, w.shape[0]), dtype=np.float64)
    for kb in range(kd // GROUP):
        cols = slice(kb * GROUP, (kb + 1) * GROUP)
        acc = acc + a_scales[kb][:, None] * (a[:, cols] @ w[:, cols].T)
    return bf16_from_f64(acc)


def _gemm(a_codes, a_scales, w, rounding, weight_fmt):
    if weight_fmt == "mxfp4":
        return gemm_rows_mxfp4(a_codes, a_scales, w[0], w[1])
    if weight_fmt != "e4m3":
        raise ValueError(weight_fmt)
    return gemm_rows(a_codes, a_scales, w[0], w[1], rounding)


def _expert(weights, e):
    return weights(e) if callable(weights) else (weights[0][e], weights[1][e])


def grouped_gemm(a_codes, a_scales, fmt, weights, counts, offsets, row_index=None,
                 rounding="divide", weight_fmt="e4m3"):
    """Grouped FP8 GEMM over the live rows of every expert segment.

    ``a_codes``/``a_scales`` are indexed by A row; row r of the output reads
    A row ``row_index[r]`` (or r itself when ``row_index`` is None).
    ``weights`` is ``(w_codes [E, N, Kd], w_scales [E, N/128, Kd/128])`` or a
    callable e -> (w_codes[e], w_scales[e]); under ``weight_fmt="mxfp4"``
    ``(w_packed [E, N, Kd/2], w_scales [E, N, Kd/32] E8M0 bytes)``.
    Returns ``(c bits [offsets[E], N], live mask [offsets[E]])``; pad rows are
    zero in ``c`` and False in the mask.
    """
    num_experts = len(counts)
    total = int(offsets[num_experts])
    sa_all = scales_to_f64(a_scales, fmt)
    c = None
    live = np.zeros(total, dtype=bool)
    for e in range(num_experts):
        cnt = int(counts[e])
        if cnt == 0:
            continue
        rows = np.arange(int(offsets[e]), int(offsets[e]) + cnt)
        src = rows if row_index is None else np.asarray(row_index)[rows]
        out = _gemm(a_codes[src], sa_all[:, src], _expert(weights, e), rounding, weight_fmt)
        if c is None:
            c = np.zeros((total, out.shape[1]), dtype=np.uint16)
        c[rows] = out
        live[rows] = True
    if c is None:
        c = np.zeros((total, 0), dtype=np.uint16)
    return c, live


def swiglu(g, u, act="swiglu", clamp_limit=np.inf, rounding="divide"):
    """SiLU(gate) * up in fp64, rounded once to float32 (and then to BF16,
    held in float32, under ``rounding="reciprocal"``).

    Clamp variants (TensorRT-LLM PR #21250, Test Coverage, names "clamp" and
    "clamp after SiLU"; vLLM PR #65794, Details, ``clamp_limit``). The pages
    give no formula; the reading taken here, with L the scalar limit:

    * ``swiglu_clamp``: gate clamped above at L, up clamped to [-L, L],
      then SiLU(gate) * up;
    * ``swiglu_clamp_after_silu``: SiLU(gate) clamped above at L, times up
      clamped to [-L, L].
    """
    if rounding not in ROUNDINGS:
        raise ValueError(rounding)
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    lim = np.float64(clamp_limit)
    if act == "swiglu":
        s = g / (1.0 + np.exp(-g))
    elif act == "swiglu_clamp":
        gc = np.minimum(g, lim)
        s = gc / (1.0 + np.exp(-gc))
        u = np.clip(u, -lim, lim)
    elif act == "swiglu_clamp_after_silu":
        s = np.minimum(g / (1.0 + np.exp(-g)), lim)
        u = np.clip(u, -lim, lim)
    else:
        raise ValueError(act)
    y = (s * u).astype(np.float32)
    if rounding == "reciprocal":  # the fused op's epilogue rounds to BF16 first
        y = bf16_bits_to_f64(bf16_from_f64(y.astype(np.float64))).astype(np.float32)
    return y


def silu_mul_quant(c1_bits, fmt, act="swiglu", clamp_limit=np.inf, rounding="divide"):
    """FC1 output rows [rows, 2I] (BF16 bits) -> (codes [rows, I], scales [I/128, rows])."""
    c1 = bf16_bits_to_f64(c1_bits)
    inter = c1.shape[1] // 2
    y = swiglu(c1[:, :inter], c1[:, inter:], act, clamp_limit, rounding)
    return quantize_groups(y, fmt, rounding)


def combine(y_bits, pair_to_row, topk_w, t_live, hidden=None):
    """out[t] = bf16( sum_k w[t, k] * Y[row(t, k)] ), k ascending, valid pairs only."""
    topk_w = np.asarray(topk_w, dtype=np.float32)
    k = topk_w.shape[1]
    if hidden is None:
        hidden = y_bits.shape[1]
    acc = np.zeros((t_live, hidden), dtype=np.float64)
    p2r = np.asarray(pair_to_row)
    for kk in range(k):
        rows = p2r[np.arange(t_live) * k + kk] if t_live else np.zeros(0, np.int64)
        valid = rows >= 0
        if not valid.any():
            continue
        contrib = np.zeros((t_live, hidden), dtype=np.float64)
        contrib[valid] = (topk_w[:t_live, kk][valid].astype(np.float64)[:, None]
                          * bf16_bits_to_f64(y_bits[rows[valid]]))
        acc = np.where(valid[:, None], acc + contrib, acc)
    return bf16_from_f64(acc)


def forward(x_bits, topk_ids, topk_w, w1, w2, t_live, align_rows, fmt,
            act="swiglu", clamp_limit=np.inf, num_experts=None, rounding="divide",
            expert_start=0, expert_cap=0, weight_fmt="e4m3"):
    """The whole layer on the aligned, per-expert-contiguous row layout.

    ``x_bits`` [t_cap, H] BF16 bits; ``topk_ids``/``topk_w`` [t_cap, K];
    ``w1``/``w2`` are (codes, scales) pairs or callables (see grouped_gemm),
    in which case ``num_experts`` must be given. Activations are quantized
    once per token; FC1 gathers its A rows through the alignment map.
    Returns every intermediate (live rows only matter).
    """
    if num_experts is None:
        num_experts = w1[0].shape[0]
    return forward_e(x_bits, topk_ids, topk_w, w1, w2, num_experts, t_live,
                     align_rows, fmt, act, clamp_limit, rounding, expert_start, expert_cap,
                     weight_fmt)


def forward_e(x_bits, topk_ids, topk_w, w1, w2, num_experts, t_live, align_rows,
              fmt, act="swiglu", clamp_limit=np.inf, rounding="divide", expert_start=0,
              expert_cap=0, weight_fmt="e4m3"):
    """``forward`` with an explicit expert count (for callable weights).

    ``expert_start``: the rank's first expert (local id = id - expert_start;
    pairs of other ranks' experts are dropped). ``expert_cap`` > 0: the
    batched masked-M layout with that many rows per expert (align_rows is
    then unused); 0: the aligned layout.
    """
    k = np.asarray(topk_ids).shape[1]
    if expert_cap > 0:
        al = align_batched(topk_ids, t_live, num_experts, expert_cap, expert_start)
        al["counts"] = al["masked_m"]
    else:
        al = align(topk_ids, t_live, num_experts, align_rows, expert_start)
    x = bf16_bits_to_f64(np.asarray(x_bits)[:t_live]).astype(np.float32)
    xq, xs = quantize_groups(x, fmt, rounding)
    token_of_row = np.where(al["row_to_pair"] >= 0, al["row_to_pair"] // k, 0)
    c1, live = grouped_gemm(xq, xs, fmt, w1, al["counts"], al["offsets"], token_of_row, rounding,
                            weight_fmt)
    hq, hs = silu_mul_quant(c1[live], fmt, act, clamp_limit, rounding)
    total = int(al["offsets"][-1])
    inter = c1.shape[1] // 2
    hq_full = np.zeros((total, inter), dtype=np.uint8)
    hq_full[live] = hq
    hs_full = np.zeros((inter // GROUP, total), dtype=hs.dtype)
    hs_full[:, live] = hs
    y, _ = grouped_gemm(hq_full, hs_full, fmt, w2, al["counts"], al["offsets"], rounding=rounding,
                        weight_fmt=weight_fmt)
    out = combine(y, al["pair_to_row"], topk_w, t_live, np.asarray(x_bits).shape[1])
    res = dict(al)
    res.setdefault("overflow", 0)
    res.update(xq=xq, xs=xs, c1=c1, live=live, hq=hq_full, hs=hs_full, y=y, out=out)
    return res


def token_forward(x_bits, topk_ids, topk_w, w1, w2, num_experts, t_live, fmt,
                  act="swiglu", clamp_limit=np.inf, tokens=None, rounding="divide",
                  expert_start=0, weight_fmt="e4m3"):
    """Dense per-token brute force: no alignment, no row maps, one token at a time.

    ``tokens`` selects which tokens to evaluate (default: all t < t_live);
    experts are the local ids id - expert_start in [0, num_experts).
    Returns BF16 bits [len(tokens), H].
    """
    ids = np.asarray(topk_ids).astype(np.int64) - int(expert_start)
    topk_w = np.asarray(topk_w, dtype=np.float32)
    tokens = range(t_live) if tokens is None else tokens
    rows = []
    for t in tokens:
        x = bf16_bits_to_f64(np.asarray(x_bits)[t:t + 1]).astype(np.float32)
        xq, xs = quantize_groups(x, fmt, rounding)
        hidden = np.asarray(x_bits).shape[1]
        acc = np.zeros(hidden, dtype=np.float64)
        for kk in range(ids.shape[1]):
            e = int(ids[t, kk])
            if not 0 <= e < num_experts:
                continue
            c1 = _gemm(xq, scales_to_f64(xs, fmt), _expert(w1, e), rounding, weight_fmt)
            hq, hs = silu_mul_quant(c1, fmt, act, clamp_limit, rounding)
            y = _gemm(hq, scales_to_f64(hs, fmt), _expert(w2, e), rounding, weight_fmt)
            acc = acc + np.float64(topk_w[t, kk]) * bf16_bits_to_f64(y[0])
        rows.append(bf16_from_f64(acc))
    hidden = np.asarray(x_bits).shape[1]
    return np.stack(rows) if rows else np.zeros((0, hidden), dtype=np.uint16)


def unquantized_reference(x_bits, topk_ids, topk_w, w1, w2, num_experts, t_live,
                          act="swiglu", clamp_limit=np.inf):
    """The same layer with no activation quantization and no BF16 roundings.

    Weights are dequantized exactly (code * block scale); activations and all
    intermediates stay fp64. vLLM PR #65794 (Claims) reports a relative error
    of about 0.06 for the quantized layer against a BF16 reference at the
    GLM-5.3 TP8 shape; the quantized oracle should sit at that order.
    """
    ids = np.asarray(topk_ids)
    topk_w = np.asarray(topk_w, dtype=np.float32)
    x = bf16_bits_to_f64(np.asarray(x_bits)[:t_live])
    out = np.zeros_like(x)
    for e in range(num_experts):
        sel = np.argwhere((ids[:t_live] == e))
        if len(sel) == 0:
            continue
        w1c, w1s = _expert(w1, e)
        w2c, w2s = _expert(w2, e)
        W1 = _dec(w1c) * np.repeat(np.repeat(np.asarray(w1s, np.float64), GROUP, 0), GROUP, 1)
        W2 = _dec(w2c) * np.repeat(np.repeat(np.asarray(w2s, np.float64), GROUP, 0), GROUP, 1)
        t_idx = sel[:, 0]
        h = x[t_idx] @ W1.T
        inter = h.shape[1] // 2
        g, u = h[:, :inter], h[:, inter:]
        if act == "swiglu":
            a = g / (1.0 + np.exp(-g)) * u
        elif act == "swiglu_clamp":
            gc = np.minimum(g, clamp_limit)
            a = gc / (1.0 + np.exp(-gc)) * np.clip(u, -clamp_limit, clamp_limit)
        else:
            a = np.minimum(g / (1.0 + np.exp(-g)), clamp_limit) * np.clip(u, -clamp_limit, clamp_limit)
        y = a @ W2.T
        wts = topk_w[t_idx, sel[:, 1]].astype(np.float64)
        np.add.at(out, t_idx, wts[:, None] * y)
    return out
