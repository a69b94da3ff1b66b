"""The quantization kernels divide by a group's scale with one reciprocal per
group and Markstein's correction (P. Markstein, IBM J. Res. Dev. 34(1), 1990):
q0 = RN(x * y), r = RN(x - q0 * s) (exact, one FMA), q = RN(q0 + r * y), with
y = RN(1 / s) and the sign of x copied back. The activation rule (vLLM PR
#65794, Details) asks for RN(x / s) itself, so the codes stay bit-exact only
if q equals RN(x / s) for every input the rule produces. This checks that
identity in binary32 on scales made by the rule over its whole range, on
quotients placed next to E4M3 rounding points, and on scales with extreme
significands. Binary64 carries every step exactly except the last sum; sums
that land within 2^-50 of a binary32 rounding point are settled with exact
rationals.
"""

from fractions import Fraction

import numpy as np

F32 = np.float32


def _rn32(fr):
    """Correctly rounded binary32 of a Fraction (ties to even)."""
    f = F32(float(fr))
    cands = [np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(v.view(np.uint32)) & 1))


def _near_midpoint(v64):
    v32 = v64.astype(F32)
    up = np.nextafter(v32, F32(np.inf)).astype(np.float64)
    dn = np.nextafter(v32, F32(-np.inf)).astype(np.float64)
    tol = np.abs(v64) * 2.0 ** -50
    return (np.abs(v64 - (v32 + up) / 2) <= tol) | (np.abs(v64 - (v32 + dn) / 2) <= tol)


def _mismatches(x, s):
    x, s = x.astype(F32), s.astype(F32)
    y = (F32(1) / s).astype(F32)
    q0 = (x * y).astype(F32)
    r = (x.astype(np.float64) - q0.astype(np.float64) * s).astype(F32)  # exact, then RN32
    t = q0.astype(np.float64) + r.astype(np.float64) * y
    q = np.copysign(t.astype(F32), x)
    ref = (x.astype(np.float64) / s).astype(F32)
    amb = _near_midpoint(t) | _near_midpoint(x.astype(np.float64) / s)
    bad = int(((q.view(np.uint32) != ref.view(np.uint32)) & ~amb).sum())
    for i in np.flatnonzero(amb):
        fx, fs, fy, fq0 = (Fraction(float(v)) for v in (x[i], s[i], y[i], q0[i]))
        fr = Fraction(float(_rn32(fx - fq0 * fs)))
        if _rn32(fq0 + fr * fy) != _rn32(fx / fs):
            bad += 1
    return bad


def test_markstein_quotient_is_correctly_rounded():
    g = np.random.default_rng(7)
    n = 400_000
    amax = (10.0 ** g.uniform(-12, 6, n)).astype(F32)
    s = np.maximum((amax / F32(448)).astype(F32), F32(1) / F32(229376)).astype(F32)
    x = (g.uniform(-1, 1, n) * amax).astype(F32)
    # quotients next to E4M3 rounding points (k/16 + 1/32) * 2^j, and one ulp either side
    k, j = g.integers(16, 32, n), g.integers(-9, 9, n)
    x2 = (s.astype(np.float64) * (k / 16 + 1 / 32) * 2.0 ** j).astype(F32)
    x2 = np.where(np.abs(x2) <= amax, x2, x).astype(F32)
    bad = 0
    for xx in (x, x2, np.nextafter(x2, F32(np.inf)), np.nextafter(x2, F32(-np.inf))):
        bad += _mismatches(xx, s)
    # scales with extreme significands over the rule's exponent range
    sig = np.array([1.0, 2 - 2.0 ** -23, 1 + 2.0 ** -23, 1.5 - 2.0 ** -23], np.float64)
    for sv in (sig[:, None] * 2.0 ** np.arange(-18, 10)[None, :]).ravel().astype(F32):
        xs = (g.uniform(-448, 448, 5000) * sv).astype(F32)
        bad += _mismatches(xs, np.full_like(xs, sv))
    assert bad == 0


def test_signed_zero_keeps_its_sign():
    s = np.array([1.0 / 229376, 0.5, 3.0], F32)
    for z in (F32(0.0), F32(-0.0)):
        x = np.full(3, z, F32)
        y = (F32(1) / s).astype(F32)
        q0 = (x * y).astype(F32)
        r = (x.astype(np.float64) - q0.astype(np.float64) * s).astype(F32)
        q = np.copysign((q0.astype(np.float64) + r.astype(np.float64) * y).astype(F32), x)
        assert np.array_equal(q.view(np.uint32), (x / s).astype(F32).view(np.uint32))
