"""Host check of the argument behind the quantizers' division-free integer codes.

The kernels round y = fl(x * r), r a refined reciprocal of the group scale s,
and keep rne(y) only where |y - rne(y)| < 0.5 - M 2^-19, M a power of two
above every |x / s| the caller can form (2^bits for the codes, 32 for the
Oaken magnitudes); elsewhere they divide.  The claim: every accepted rne(y) equals rne(fl(x / s)), the code the
binary32 definition gives.  This test replays the acceptance rule in numpy
(binary64 products rounded once to binary32 stand in for the fused
multiply-adds) with reciprocals deliberately perturbed by up to 3 ulp before
the Newton step, over random quotients, exact integers and exact
half-integers, on the group scales the quantizers form from fp16 data.
"""
import numpy as np

f32 = np.float32


def _nudge(r, k):
    toward = np.where(k > 0, f32(np.inf), f32(0))
    out = r.copy()
    for _ in range(int(np.max(np.abs(k)))):
        step = np.abs(k) > 0
        out = np.where(step, np.nextafter(out, toward).astype(f32), out)
        k = k - np.sign(k)
    return out


def _accepted_and_codes(x, s, rng, M):
    r0 = (f32(1) / s).astype(f32)
    r0 = _nudge(r0, rng.integers(-3, 4, s.size))
    e = (f32(1) - s.astype(np.float64) * r0).astype(f32)       # fma(-s, r0, 1)
    r = (e.astype(np.float64) * r0 + r0).astype(f32)            # fma(e, r0, r0)
    y = (x * r).astype(f32)
    n = np.rint(y).astype(f32)
    assert np.all(np.abs(y) < M)  # the premise of the bound
    ok = np.abs(y - n) < f32(0.5 - M * 2.0 ** -19)
    return ok, n


def test_accepted_fast_codes_equal_the_divided_codes():
    rng = np.random.default_rng(2026)
    N = 400_000
    for case in ("random", "integers", "half-integers"):
        for qmax in (3, 15, 31, 127, 255):
            hi = np.abs(rng.standard_normal(N) * 4).astype(np.float16).astype(f32)
            lo = -np.abs(rng.standard_normal(N) * 4).astype(np.float16).astype(f32)
            s = ((hi - lo) / f32(qmax)).astype(f32)
            keep = s > 0
            hi, lo, s = hi[keep], lo[keep], s[keep]
            if case == "random":
                x = (lo + (hi - lo) * rng.random(s.size).astype(f32)).astype(np.float16).astype(f32)
            else:
                k = rng.integers(-qmax, qmax + 1, s.size).astype(f32)
                x = ((k + (f32(0.5) if case == "half-integers" else f32(0))) * s).astype(f32)
            ok, n = _accepted_and_codes(x, s, rng, qmax + 1)
            ref = np.rint((x / s).astype(f32))
            assert not np.any(ok & (n != ref)), (case, qmax)
            if case == "random":
                assert ok.mean() > 0.99  # the fast path is the common one
            if case == "half-integers":
                # an exact tie is never accepted: such quotients take the divide
                tie = (np.abs((x / s).astype(f32) - ref) == f32(0.5))
                assert not np.any(ok & tie)


def test_accepted_codes_with_the_zero_point_folded_in():
    """The asymmetric codes round t = fl(x r + z) (one fused multiply-add) and
    accept rne(t) under the same rule; the claim is rne(t) = rne(fl(x / s)) + z
    with z = clamp(rne(fl(-lo / s)), 0, qmax), before the final clamp."""
    rng = np.random.default_rng(2027)
    N = 400_000
    for case in ("random", "integers", "half-integers"):
        for qmax in (3, 15):
            hi = np.abs(rng.standard_normal(N) * 4).astype(np.float16).astype(f32)
            lo = -np.abs(rng.standard_normal(N) * 4).astype(np.float16).astype(f32)
            s = ((hi - lo) / f32(qmax)).astype(f32)
            keep = s > 0
            hi, lo, s = hi[keep], lo[keep], s[keep]
            z = np.clip(np.rint((-lo / s).astype(f32)), 0, qmax).astype(f32)
            if case == "random":
                x = (lo + (hi - lo) * rng.random(s.size).astype(f32)).astype(np.float16).astype(f32)
            else:
                k = rng.integers(-qmax, qmax + 1, s.size).astype(f32)
                x = ((k + (f32(0.5) if case == "half-integers" else f32(0))) * s).astype(f32)
                x = np.clip(x, lo, hi)
            r0 = (f32(1) / s).astype(f32)
            r0 = _nudge(r0, rng.integers(-3, 4, s.size))
            e = (f32(1) - s.astype(np.float64) * r0).astype(f32)
            r = (e.astype(np.float64) * r0 + r0).astype(f32)
            t = (x.astype(np.float64) * r + z).astype(f32)           # fma(x, r, z)
            M = qmax + 1
            assert np.all(np.abs(t) < M)
            n = np.rint(t).astype(f32)
            ok = np.abs(t - n) < f32(0.5 - M * 2.0 ** -19)
            ref = np.rint((x / s).astype(f32)) + z
            assert not np.any(ok & (n != ref)), (case, qmax)
            if case == "random":
                assert ok.mean() > 0.99
