"""Pins for the oracle's group quantizers (CPU only).

Each test fixes the oracle against something other than its own formula:
exact reconstruction of grid-aligned groups, the half-step error bound of
round-to-nearest, hand-worked half-to-even ties, brute force over every code
and the fp16 decoding of numpy.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f16bits(x):
    a = np.asarray(x, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.all(h.astype(np.float64) == a), "test value not fp16-exact"
    return h.view(np.uint16)


def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("k", [-3, -1, 0, 2])
def test_asym_grid_aligned_round_trip(bits, k):
    """Codes covering 0 and 2^b-1 with x = (c - z) * 2^k reproduce s, z and c exactly."""
    rng = np.random.default_rng(1000 + bits * 10 + k)
    qmax = (1 << bits) - 1
    for trial in range(40):
        g = int(rng.choice([8, 32, 64, 128]))
        z = int(rng.integers(0, qmax + 1))
        c = rng.integers(0, qmax + 1, size=g)
        c[rng.integers(g)] = 0
        c[(rng.integers(g - 1) + 1 + np.argmin(c)) % g] = qmax
        x = (c.astype(np.float64) - z) * 2.0 ** k
        s, zz, q = oracle.quant_group_asym(f16bits(x), bits)
        assert s == np.float32(2.0 ** k)
        assert zz == z
        assert np.array_equal(q, c.astype(np.uint8))
        xh = oracle.dequant_rows(q[None], np.array([[s]], np.float32), np.array([[zz]], np.uint8), g)
        assert np.array_equal(xh[0], x.astype(np.float32))


def test_asym_half_even_ties():
    """lo = -7, hi = 8 gives s = 1, z = 7; halves round to even before the zero-point is added."""
    vals = [-7.0, 8.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, 0.0, 4.0, 4.5, -2.5]
    s, z, q = oracle.quant_group_asym(f16bits(vals), 4)
    assert s == 1.0 and z == 7
    assert list(q) == [0, 15, 7, 9, 9, 7, 5, 11, 7, 11, 11, 5]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_asym_bound_ranges_and_nearest_code(bits):
    """|x - x_hat| <= s/2 (+ binary32 rounding), codes in range, and each code is a nearest level."""
    rng = np.random.default_rng(7 + bits)
    qmax = (1 << bits) - 1
    for trial in range(300):
        g = int(rng.choice([4, 32, 64]))
        x = rng.standard_normal(g) * float(rng.choice([1e-3, 1.0, 30.0]))
        if trial % 3 == 0:
            x[rng.integers(g)] *= 25.0
        if trial % 5 == 0:
            x = np.abs(x)
        xb = x.astype(np.float16).view(np.uint16)
        xv = xb.view(np.float16).astype(np.float64)
        s, z, q = oracle.quant_group_asym(xb, bits)
        assert q.min() >= 0 and q.max() <= qmax and 0 <= z <= qmax
        lo, hi = min(0.0, xv.min()), max(0.0, xv.max())
        assert abs(float(s) - (hi - lo) / qmax) <= 1e-6 * (hi - lo) / qmax
        xh = (q.astype(np.float64) - z) * float(s)
        tol = float(s) / 2 * (1 + 1e-5) + 4 * np.spacing(np.maximum(np.abs(xv), np.abs(xh)).astype(np.float32))
        assert np.all(np.abs(xv - xh) <= tol)
        levels = (np.arange(qmax + 1) - z) * float(s)
        best = np.min(np.abs(xv[:, None] - levels[None, :]), axis=1)
        # the quotient x / s is rounded to binary32 before the integer rounding,
        # so a near-tie may go to the other neighbour within one quotient ulp
        qulp = np.spacing(np.abs(xv / float(s)).astype(np.float32)).astype(np.float64) * float(s)
        assert np.all(np.abs(xv - xh) <= best + 2 * qulp + 1e-9 * float(s))


def test_asym_zero_constant_single_sign():
    s, z, q = oracle.quant_group_asym(np.zeros(64, np.uint16), 4)
    assert s == 0 and z == 0 and not q.any()
    # constant positive group: lo = 0, hi = c -> z = 0, every code the top level
    s, z, q = oracle.quant_group_asym(f16bits([3.0] * 32), 4)
    assert z == 0 and np.all(q == 15) and s == np.float32(3.0) / np.float32(15.0)
    # all-negative group: hi = 0 -> z = qmax
    s, z, q = oracle.quant_group_asym(f16bits(-np.arange(1, 33) / 8.0), 2)
    assert z == 3
    # all-positive group -> z = 0
    s, z, q = oracle.quant_group_asym(f16bits(np.arange(1, 33) / 8.0), 8)
    assert z == 0


def test_sym8_round_trip_ties_and_bound():
    rng = np.random.default_rng(3)
    for k in (-4, 0, 3):
        c = rng.integers(-128, 128, size=128)
        c[5] = 127
        c = np.clip(c, -127, 127)
        x = c * 2.0 ** k
        s, q = oracle.quant_group_sym8(f16bits(x))
        assert s == np.float32(2.0 ** k)
        assert np.array_equal(q.astype(np.int64), c)
    s, q = oracle.quant_group_sym8(f16bits([127.0, 0.5, 1.5, 2.5, -2.5, -0.5, -127.0]))
    assert s == 1.0 and list(q) == [127, 0, 2, 2, -2, 0, -127]
    s, q = oracle.quant_group_sym8(np.zeros(128, np.uint16))
    assert s == 0 and not q.any()
    for trial in range(200):
        x = rng.standard_normal(128) * 3
        x[rng.integers(128)] *= 15
        xb = x.astype(np.float16).view(np.uint16)
        xv = xb.view(np.float16).astype(np.float64)
        s, q = oracle.quant_group_sym8(xb)
        assert q.min() >= -128 and q.max() <= 127
        xh = q.astype(np.float64) * float(s)
        assert np.all(np.abs(xv - xh) <= float(s) / 2 * (1 + 1e-5) + 1e-6)
        levels = np.arange(-128, 128) * float(s)
        best = np.min(np.abs(xv[:, None] - levels[None, :]), axis=1)
        qulp = np.spacing(np.abs(xv / float(s)).astype(np.float32)).astype(np.float64) * float(s)
        assert np.all(np.abs(xv - xh) <= best + 2 * qulp + 1e-9 * float(s))


@pytest.mark.parametrize("g,bits", [(64, 4), (32, 2), (32, 4), (128, 8)])
def test_rows_geometry_grid_aligned(g, bits):
    """Every (row, group) gets its own power-of-two scale and zero-point; all reproduce exactly."""
    rng = np.random.default_rng(g * 7 + bits)
    qmax = (1 << bits) - 1
    R, D = 9, 128
    ng = D // g
    k = rng.integers(-3, 2, size=(R, ng))
    z = rng.integers(0, qmax + 1, size=(R, ng))
    c = rng.integers(0, qmax + 1, size=(R, D))
    for r in range(R):
        for j in range(ng):
            c[r, j * g] = 0
            c[r, j * g + 1] = qmax
    x = (c - np.repeat(z, g, axis=1)) * 2.0 ** np.repeat(k, g, axis=1)
    codes, scale, zero = oracle.quant_rows(f16bits(x).reshape(R, D), g, bits)
    assert np.array_equal(scale, (2.0 ** k).astype(np.float32))
    assert np.array_equal(zero, z.astype(np.uint8))
    assert np.array_equal(codes, c.astype(np.uint8))
    assert np.array_equal(oracle.dequant_rows(codes, scale, zero, g), x.astype(np.float32))


def test_rows_sym_geometry():
    rng = np.random.default_rng(11)
    R = 6
    k = rng.integers(-3, 3, size=R)
    c = np.clip(rng.integers(-127, 128, size=(R, 128)), -127, 127)
    c[:, 3] = -127
    x = c * 2.0 ** k[:, None]
    codes, scale, _ = oracle.quant_rows(f16bits(x), 128, 8, sym=True)
    assert np.array_equal(scale[:, 0], (2.0 ** k).astype(np.float32))
    assert np.array_equal(codes.astype(np.int64), c)
    assert np.array_equal(oracle.dequant_rows(codes, scale, None, 128, sym=True), x.astype(np.float32))


def test_channel_blocks_geometry_grid_aligned():
    """Groups are 16 consecutive tokens of one channel: per-(block, channel) scales reproduce exactly."""
    rng = np.random.default_rng(5)
    S, T, D, gt, bits = 2, 48, 128, 16, 4
    nb = T // gt
    k = rng.integers(-3, 2, size=(S, nb, D))
    z = rng.integers(0, 16, size=(S, nb, D))
    c = rng.integers(0, 16, size=(S, T, D))
    for s_ in range(S):
        for b in range(nb):
            c[s_, b * gt, :] = 0
            c[s_, b * gt + 1, :] = 15
    x = (c - np.repeat(z, gt, axis=1)) * 2.0 ** np.repeat(k, gt, axis=1)
    codes, scale, zero = oracle.quant_channel_blocks(f16bits(x), gt, bits)
    assert np.array_equal(scale, (2.0 ** k).astype(np.float32))
    assert np.array_equal(zero, z.astype(np.uint8))
    assert np.array_equal(codes, c.astype(np.uint8))
    assert np.array_equal(oracle.dequant_channel_blocks(codes, scale, zero, gt), x.astype(np.float32))
