"""moe_forward_noalloc (the library's static per-device workspace) against
moe_forward (a caller workspace): the same outputs bit for bit, on two calls in
a row with the second one smaller, on the one-launch decode path and on the
general path. Both run the same kernels, and the layer is deterministic (every
sum has a fixed order), so the outputs must be identical."""

import numpy as np
import pytest
import torch

import block_fp8_mixture_amd as moe
import synth
from tests.gpu_helpers import POISON_BF16, dev, device_weights, down, say, up

pytestmark = pytest.mark.gpu


_mx_cache = {}


def _weights(name, weights):
    if weights == "e4m3":
        return device_weights(name)
    if name not in _mx_cache:
        _mx_cache.clear()
        (w1p, w1s), (w2p, w2s) = synth.ExpertWeightsMxfp4(synth.get(name)).stacked(threads=16)
        _mx_cache[name] = (up(w1p), up(w1s), up(w2p), up(w2s))
    return _mx_cache[name]


def _both(name, t_cap, t_live, fmt, variant, weights):
    cfg = synth.get(name)
    x, ids, w = synth.make_workload(cfg, t_cap, variant)
    d = _weights(name, weights)
    need = moe.moe_workspace_bytes(cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, t_cap,
                                   cfg.align_rows, 0, fmt, weight_fmt=weights)
    assert 0 < need <= moe.NOALLOC_SCRATCH_BYTES
    live = up(np.array([t_live], np.int32))
    args = (up(x), up(ids), up(w), *d)
    ref = torch.full((t_cap, cfg.hidden), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward(*args, fmt, align_rows=cfg.align_rows, t_live=live, out=ref, weight_fmt=weights)
    got = torch.full((t_cap, cfg.hidden), POISON_BF16, dtype=torch.int16, device=dev())
    moe.moe_forward_noalloc(*args, fmt, align_rows=cfg.align_rows, t_live=live, out=got,
                            weight_fmt=weights)
    torch.cuda.synchronize()
    return down(got), down(ref)


@pytest.mark.parametrize("name,calls,weights", [
    ("decode", [(4, 4, "fp32", 1), (1, 1, "fp32", 2)], "e4m3"),      # the one-launch layer
    ("sweep", [(64, 64, "pow2", 3), (32, 29, "pow2", 4)], "e4m3"),   # the general path
    ("tiny", [(8, 8, "ue8m0", 5), (8, 3, "ue8m0", 6)], "e4m3"),
    ("decode", [(4, 4, "fp32", 1), (1, 1, "ue8m0", 2)], "mxfp4"),    # the one-launch layer
    ("tiny", [(8, 8, "fp32", 5), (8, 3, "fp32", 6)], "mxfp4"),       # the general path
])
def test_noalloc_matches_forward_on_two_calls(name, calls, weights):
    gave_up = moe.moe_barrier_timeouts()  # sticky per process: compare, do not expect 0
    for t_cap, t_live, fmt, variant in calls:
        say(f"noalloc {name} t_cap={t_cap} t_live={t_live} {fmt} {weights}")
        got, ref = _both(name, t_cap, t_live, fmt, variant, weights)
        assert np.array_equal(got, ref)
        assert np.all(got[t_live:] == POISON_BF16)
        assert np.all(np.isfinite((got[:t_live].astype(np.uint32) << 16).view(np.float32)))
    assert moe.moe_barrier_timeouts() == gave_up
