"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""

import functools
import os
import sys

import numpy as np
import torch

import oracle
import synth

POISON_I32 = 0x5A5A5A5A
POISON_U8 = 0xA5
POISON_BF16 = 0x7FC1  # a NaN pattern


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def up(a):
    """numpy -> GPU tensor (uint16 BF16 bits become int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def down(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def bf16_ulp(v):
    """Spacing of BF16 numbers at |v| (normal binade of v; subnormal quantum below)."""
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_bf16_close(got_bits, ref_bits, what="", rel=1e-2, ulps=2):
    """Elementwise |got - ref| <= rel * max|ref| + ulps * ulp_bf16(ref)."""
    got = oracle.bf16_bits_to_f64(got_bits)
    ref = oracle.bf16_bits_to_f64(ref_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bound = rel * np.max(np.abs(ref)) + ulps * bf16_ulp(ref)
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)} got {got[tuple(i)]} ref {ref[tuple(i)]} bound {bound[tuple(i)]}")
    return float(np.max(err / np.maximum(np.max(np.abs(ref)), 1e-30)))


@functools.lru_cache(maxsize=4)
def host_weights(name, variant=0):
    cfg = synth.get(name)
    return synth.ExpertWeights(cfg, variant).stacked(threads=min(16, os.cpu_count() or 8))


_dev_cache = {}


def device_weights(name, variant=0):
    key = (name, variant)
    if key not in _dev_cache:
        _dev_cache.clear()
        torch.cuda.empty_cache()
        (w1q, w1s), (w2q, w2s) = host_weights(name, variant)
        _dev_cache[key] = (up(w1q), up(w1s), up(w2q), up(w2s))
    return _dev_cache[key]
