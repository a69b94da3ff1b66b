"""Seeded generators: tokens, routing and FP8 weight checkpoints.

Every stream is a numpy PCG64 generator keyed by (seed, ...), so each
expert's weights can be regenerated on their own and only the experts a test
touches need to exist on the host.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

WEIGHT_SEED = 0x5EED00
TOKEN_SEED = 0x5EED10
WEIGHT_STD = 0.02
BLOCK = 128


def _rng(*key):
    return np.random.Generator(np.random.PCG64([int(k) for k in key]))


def _to_bf16_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_tokens(cfg, t_cap, variant=0, scale=1.0):
    """BF16 activations ~ N(0, 1) (times ``scale``), as uint16 bits [t_cap, H]."""
    g = _rng(TOKEN_SEED + 16 * cfg.index + variant, t_cap, 1)
    x = g.standard_normal((t_cap, cfg.hidden), dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return _to_bf16_bits(x)


def make_routing(cfg, t_cap, variant=0):
    """Router: logits ~ N(0, 1) (+ a Zipf per-expert bias), softmax, top-k.

    Returns ``(ids int32 [t_cap, K], weights float32 [t_cap, K])``; weights
    are the top-k probabilities renormalised to sum to one. Ties in the top-k
    go to the lower expert id. The Zipf(s) bias of expert e is
    -s * ln(rank_e), rank a seeded permutation of 1..E: the log of a Zipf
    probability mass.
    """
    g = _rng(TOKEN_SEED + 16 * cfg.index + variant, t_cap, 2)
    logits = g.standard_normal((t_cap, cfg.num_experts))
    if cfg.routing == "zipf":
        rank = g.permutation(cfg.num_experts) + 1
        logits = logits - cfg.zipf_s * np.log(rank)[None, :]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :cfg.topk]
    ids = order.astype(np.int32)
    top = np.take_along_axis(p, order, axis=1)
    w = (top / top.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def quantize_weight_blocks(w):
    """Checkpoint-style 128x128 block FP8 weights from float32 [N, K].

    Per block: scale = max(amax / 448, 1 / (448 * 512)) in float32, the
    activation rule's scale and floor (vLLM PR #65794, Details) applied to a
    128x128 block (not a power of two); codes = torch's float8_e4m3fn cast of
    w / scale. Returns (codes uint8 [N, K], scales float32 [N/128, K/128]).
    """
    n, k = w.shape
    blocks = w.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    scale = np.maximum(amax / np.float32(448.0), np.float32(1.0) / np.float32(229376.0))
    ratio = blocks / scale[:, None, :, None]
    codes = torch.from_numpy(np.ascontiguousarray(ratio.reshape(n, k))).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


class ExpertWeights:
    """Lazily generated FP8 expert weights of one workload.

    FC1 (gate rows first, then up rows) is [2I, H]; FC2 is [H, I]. Scales are
    [rows/128, cols/128] float32. ``fc1(e)`` / ``fc2(e)`` return one expert's
    (codes, scales); ``stacked()`` builds [E, ...] arrays with a thread pool.
    """

    def __init__(self, cfg, variant=0, std=WEIGHT_STD):
        self.cfg = cfg
        self.variant = variant
        self.std = np.float32(std)
        self._cache = {}

    def _make(self, e, which):
        c = self.cfg
        shape = (2 * c.inter, c.hidden) if which == 1 else (c.hidden, c.inter)
        g = _rng(WEIGHT_SEED + c.index, self.variant, e, which)
        w = g.standard_normal(shape, dtype=np.float32) * self.std
        return quantize_weight_blocks(w)

    def fc1(self, e):
        key = (e, 1)
        if key not in self._cache:
            self._cache[key] = self._make(e, 1)
        return self._cache[key]

    def fc2(self, e):
        key = (e, 2)
        if key not in self._cache:
            self._cache[key] = self._make(e, 2)
        return self._cache[key]

    def stacked(self, threads=8):
        """All experts as ((w1q, w1s), (w2q, w2s)) with a leading E axis."""
        c = self.cfg
        e_n = c.num_experts
        w1q = np.empty((e_n, 2 * c.inter, c.hidden), np.uint8)
        w1s = np.empty((e_n, 2 * c.inter // BLOCK, c.hidden // BLOCK), np.float32)
        w2q = np.empty((e_n, c.hidden, c.inter), np.uint8)
        w2s = np.empty((e_n, c.hidden // BLOCK, c.inter // BLOCK), np.float32)

        def one(e):
            a, b = self._make(e, 1)
            w1q[e], w1s[e] = a, b
            a, b = self._make(e, 2)
            w2q[e], w2s[e] = a, b

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(e_n)))
        return (w1q, w1s), (w2q, w2s)


MX_BLOCK = 32
MX_SCALE_BYTES = (117, 118, 119, 120, 121)  # E8M0 scales 2**-10 .. 2**-6


class ExpertWeightsMxfp4:
    """Seeded MXFP4 expert weights: FC1 [2I, H] and FC2 [H, I] as packed
    E2M1 codes [rows, cols/2] (even column in the low nibble) and E8M0 scale
    bytes [rows, cols/32]. Codes are drawn uniformly from all 16 (both zeros
    included) and scale bytes uniformly from MX_SCALE_BYTES, which gives an
    RMS weight of about 0.02 like the FP8 checkpoints; there is nothing to
    quantize, the draws are the checkpoint."""

    def __init__(self, cfg, variant=0):
        self.cfg = cfg
        self.variant = variant

    def _make(self, e, which):
        c = self.cfg
        rows, cols = (2 * c.inter, c.hidden) if which == 1 else (c.hidden, c.inter)
        g = _rng(WEIGHT_SEED + c.index, self.variant, e, 10 + which)
        packed = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
        scales = np.asarray(MX_SCALE_BYTES, np.uint8)[g.integers(0, len(MX_SCALE_BYTES),
                                                                   size=(rows, cols // MX_BLOCK))]
        return packed, scales

    def fc1(self, e):
        return self._make(e, 1)

    def fc2(self, e):
        return self._make(e, 2)

    def stacked(self, threads=8):
        """All experts as ((w1p, w1s), (w2p, w2s)) with a leading E axis."""
        c = self.cfg
        e_n = c.num_experts
        w1p = np.empty((e_n, 2 * c.inter, c.hidden // 2), np.uint8)
        w1s = np.empty((e_n, 2 * c.inter, c.hidden // MX_BLOCK), np.uint8)
        w2p = np.empty((e_n, c.hidden, c.inter // 2), np.uint8)
        w2s = np.empty((e_n, c.hidden, c.inter // MX_BLOCK), np.uint8)

        def one(e):
            w1p[e], w1s[e] = self._make(e, 1)
            w2p[e], w2s[e] = self._make(e, 2)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(e_n)))
        return (w1p, w1s), (w2p, w2s)


def make_workload(cfg, t_cap, variant=0):
    """(x bits, ids, weights) for ``t_cap`` tokens of a workload."""
    x = make_tokens(cfg, t_cap, variant)
    ids, w = make_routing(cfg, t_cap, variant)
    return x, ids, w
