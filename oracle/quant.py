"""Per-1x128 block quantization of activations to FP8 E4M3.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The rule is the one vLLM PR #65794 states in its Details section (sorted-A
bullet): scale = max(amax / 448, 1 / (448 * 512)), then x / scale. Both
divisions are IEEE float32 divisions (correctly rounded, as the TensorRT-LLM
PR #21250 rounding-fix commit insists for its quantizers), followed by the
E4M3 rounding of ``fp_formats.e4m3_encode``.

Scale formats (vLLM PR #59128, Purpose; vLLM PR #65794, Overview):

* ``fp32``  -- the scale above, stored as float32;
* ``pow2``  -- the scale rounded up to a power of two, stored as float32;
* ``ue8m0`` -- the same power of two stored as its biased exponent byte.

The pages say "power-of-two-rounded" without a direction. Rounding up is the
reading taken here: it is the only direction that keeps |x / scale| <= 448,
so no element saturates. The floor 1/(448*512) is applied before the
power-of-two rounding.

Two rounding conventions (``rounding``):

* ``divide`` -- the rule above (vLLM PR #65794, Details): two roundings,
  fl32(amax / 448) for the scale and fl32(x / scale) for each element.
* ``reciprocal`` -- the convention of the fused CUTLASS op that TensorRT-LLM
  PR #21250 follows (its rounding-fix commit message): the quantizer
  multiplies by 448 / amax and stores the reciprocal, both correctly
  rounded, so inv = fl32(448 / amax), the stored scale is fl32(1 / inv) and
  each element is fl32(x * inv). The pages give this convention no floor for
  an all-zero group; the reading taken here floors amax at 2**-9 = 448 /
  (448 * 512), the amax at which the divide rule's floor starts to bind, so
  both conventions floor the same groups (and an all-zero group gets the
  same stored scale, fl32(1/229376), in both). With a power-of-two format the
  stored scale fl32(1 / inv) is rounded up to a power of two and each element
  is divided by it, which is exact.
"""

import numpy as np

from .fp_formats import e4m3_encode

SCALE_FMTS = ("fp32", "pow2", "ue8m0")
ROUNDINGS = ("divide", "reciprocal")
GROUP = 128

_F448 = np.float32(448.0)
# 1/(448*512) as a float32 division; 448*512 = 229376 is exact in float32.
_FLOOR = np.float32(1.0) / np.float32(229376.0)
# The reciprocal convention's floor on amax: 448 * (1/(448*512)) = 2**-9.
_AMAX_FLOOR = np.float32(2.0 ** -9)


def _pow2_ceil(s):
    """Smallest power of two >= s, for positive normal float32 s."""
    mant, ex = np.frexp(s.astype(np.float64))  # s = mant * 2**ex, mant in [0.5, 1)
    ex = np.where(mant == 0.5, ex - 1, ex)
    return np.ldexp(1.0, ex).astype(np.float32), ex


def _check(fmt, rounding):
    if fmt not in SCALE_FMTS:
        raise ValueError(fmt)
    if rounding not in ROUNDINGS:
        raise ValueError(rounding)


def reciprocal_multiplier(amax):
    """inv = fl32(448 / max(amax, 2**-9)) of the reciprocal convention."""
    return _F448 / np.maximum(np.asarray(amax, dtype=np.float32), _AMAX_FLOOR)


def group_scales(amax, fmt, rounding="divide"):
    """Scales for groups with the given float32 amax.

    Returns ``(scale_f32, stored)``: the float32 scale of the group (what the
    codes are divided by under ``divide``, the stored reciprocal under
    ``reciprocal``) and what is stored (float32 for fp32/pow2, uint8 for
    ue8m0).
    """
    _check(fmt, rounding)
    amax = np.asarray(amax, dtype=np.float32)
    if rounding == "divide":
        s = np.maximum(amax / _F448, _FLOOR)
    else:
        s = np.float32(1.0) / reciprocal_multiplier(amax)
    if fmt == "fp32":
        return s, s
    p2, ex = _pow2_ceil(s)
    if fmt == "pow2":
        return p2, p2
    return p2, (ex + 127).astype(np.uint8)


def scales_to_f64(stored, fmt):
    """Decode stored scales (float32 or UE8M0 bytes) to float64."""
    if fmt == "ue8m0":
        return np.ldexp(1.0, np.asarray(stored, dtype=np.int64) - 127)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


def quantize_groups(v, fmt, rounding="divide"):
    """Quantize rows of float32 values in groups of 128 along the last axis.

    ``v`` is [rows, D] float32 with D a multiple of 128. Returns
    ``(codes uint8 [rows, D], stored scales [D/128, rows])``: scales are laid
    out group-major ("column-major in rows").
    """
    _check(fmt, rounding)
    v = np.asarray(v, dtype=np.float32)
    rows, d = v.shape
    if d % GROUP:
        raise ValueError("last dimension must be a multiple of 128")
    g = v.reshape(rows, d // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2) if rows else np.zeros((0, d // GROUP), np.float32)
    s, stored = group_scales(amax, fmt, rounding)
    if rounding == "reciprocal" and fmt == "fp32":
        q = e4m3_encode(g * reciprocal_multiplier(amax)[:, :, None])  # float32 product (IEEE)
    else:
        q = e4m3_encode(g / s[:, :, None])  # float32 / float32 -> float32 (IEEE)
    return q.reshape(rows, d), np.ascontiguousarray(stored.T)
