"""Pins of the oracle's FP8 codecs, E4M3 and E5M2 (CPU).

The E4M3 value table and the rounding are checked against torch's own
float8_e4m3fn conversion (an independent library implementation of the
same OCP format), against closed-form values of the format, and against
the ties and saturation the oracle's reading fixes.  The group quantizer is
checked by properties: the group maximum lands on +-448, the round-trip error
stays within half a unit in the last place of the code, and x_hat equals
the library's cast of x / s times s.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(y):
    t = torch.from_numpy(np.asarray(y, np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_closed_forms():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals m * 2^-9
    assert v(0x08) == 2.0 ** -6  # smallest normal
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x3C) == 1.5
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    mags = v(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(mags) > 0)  # magnitudes increase with the code
    assert np.array_equal(v(np.arange(0x80, 0xFF, dtype=np.uint8)), -mags)


def test_e4m3_values_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours, lib = oracle.e4m3_value(codes), torch_decode(codes)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_e4m3_encode_matches_library():
    # every finite fp16 value within the format's range, the exact midpoints
    # between neighbouring codes (ties), and random binary32 values
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) <= 448)]
    mags = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[1:] + mags[:-1]) / 2)  # exact in binary32
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000))).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    y = np.concatenate([h, mids, -mids, rnd])
    assert np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def test_e4m3_ties_and_saturation():
    enc = oracle.e4m3_encode
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): even code; 1.1875 -> 0x3A
    assert list(enc(np.array([1.0625, 1.1875, -1.0625], np.float32))) == [0x38, 0x3A, 0xB8]
    # subnormal ties: 0.5 and 1.5 units of 2^-9
    assert list(enc(np.array([2.0 ** -10, 3 * 2.0 ** -10], np.float32))) == [0x00, 0x02]
    big = np.array([448.0, 449.0, 464.0, 1000.0, 3e38, np.inf, -np.inf, -1e30], np.float32)
    assert list(enc(big)) == [0x7E] * 6 + [0xFE] * 2
    assert enc(np.array([-0.0], np.float32))[0] == 0x80


def rows_f16(rng, shape, outliers=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        x[..., 5] *= 40.0
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quant_rows_e4m3_properties(g):
    rng = np.random.default_rng(11 + g)
    xb = rows_f16(rng, (37, 128))
    xb[3] = 0  # all-zero row
    xb[4, :g] = np.float16(-0.0).view(np.uint16)
    codes, scale = oracle.quant_rows_e4m3(xb, g)
    x = xb.view(np.float16).astype(np.float32)
    xg = x.reshape(37, 128 // g, g)
    amax = np.abs(xg).max(-1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    assert np.all(codes[3] == 0) and np.all(scale[3] == 0)
    cg = codes.reshape(37, 128 // g, g)
    live = amax > 0
    top = np.take_along_axis(cg, np.abs(xg).argmax(-1)[..., None], -1)[..., 0]
    assert np.all((top[live] & 0x7F) == 0x7E)
    xh = oracle.dequant_rows_e4m3(codes, scale, g)
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 s for subnormals
    s_full = np.repeat(scale, g, axis=-1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s_full * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(xh - x) <= bound)
    # the library's cast of x / s, scaled back, in binary32
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(s_full > 0, x / s_full, 0).astype(np.float32)
    ref = (torch_decode(torch_encode(q)).astype(np.float32) * s_full).astype(np.float32)
    assert np.array_equal(xh.view(np.uint32) & 0x7FFFFFFF, ref.view(np.uint32) & 0x7FFFFFFF)


# ---------------------------------------------------------------------------
# E5M2 (1 sign, 5 exponent bits with bias 15, 2 mantissa bits): checked the
# same way against torch's float8_e5m2 conversion and closed forms.

def torch_decode5(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e5m2)
    return t.to(torch.float64).numpy()


def torch_encode5(y):
    t = torch.from_numpy(np.asarray(y, np.float32).copy()).to(torch.float8_e5m2)
    return t.view(torch.uint8).numpy()


def test_e5m2_closed_forms():
    v = oracle.e5m2_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -16 and v(0x03) == 3 * 2.0 ** -16  # subnormals m * 2^-16
    assert v(0x04) == 2.0 ** -14  # smallest normal, that of fp16
    assert v(0x3C) == 1.0 and v(0x40) == 2.0 and v(0x3E) == 1.5
    assert v(0x7B) == 57344.0 and v(0xFB) == -57344.0
    assert v(0x7C) == np.inf and np.isnan(v(0x7D)) and np.isnan(v(0xFF))
    mags = v(np.arange(0x7C, dtype=np.uint8))
    assert np.all(np.diff(mags) > 0)
    assert np.array_equal(v(np.arange(0x80, 0xFC, dtype=np.uint8)), -mags)
    # an E5M2 code is the high byte of the fp16 number of the same value
    h = (np.arange(0x7C, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert np.array_equal(h, mags)


def test_e5m2_values_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours, lib = oracle.e5m2_value(codes), torch_decode5(codes)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_e5m2_encode_matches_library():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) <= 57344)]
    mags = oracle.e5m2_value(np.arange(0x7C, dtype=np.uint8))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[1:] + mags[:-1]) / 2)
    rng = np.random.default_rng(9)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-14, 10, 20000))).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 57344]
    y = np.concatenate([h, mids, -mids, rnd])
    assert np.array_equal(oracle.e5m2_encode(y), torch_encode5(y))


def test_e5m2_ties_and_saturation():
    enc = oracle.e5m2_encode
    # 1.125 lies between 1.0 (0x3C) and 1.25 (0x3D): even code; 1.375 -> 0x3E
    assert list(enc(np.array([1.125, 1.375, -1.125], np.float32))) == [0x3C, 0x3E, 0xBC]
    # subnormal ties: 0.5 and 1.5 units of 2^-16
    assert list(enc(np.array([2.0 ** -17, 3 * 2.0 ** -17], np.float32))) == [0x00, 0x02]
    big = np.array([57344.0, 60000.0, 61440.0, 1e6, 3e38, np.inf, -np.inf, -1e30], np.float32)
    assert list(enc(big)) == [0x7B] * 6 + [0xFB] * 2
    assert enc(np.array([-0.0], np.float32))[0] == 0x80


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quant_rows_e5m2_properties(g):
    rng = np.random.default_rng(21 + g)
    xb = rows_f16(rng, (37, 128))
    xb[3] = 0
    codes, scale = oracle.quant_rows_e5m2(xb, g)
    x = xb.view(np.float16).astype(np.float32)
    xg = x.reshape(37, 128 // g, g)
    amax = np.abs(xg).max(-1)
    assert np.array_equal(scale, (amax / np.float32(57344)).astype(np.float32))
    assert np.all(codes[3] == 0) and np.all(scale[3] == 0)
    cg = codes.reshape(37, 128 // g, g)
    live = amax > 0
    top = np.take_along_axis(cg, np.abs(xg).argmax(-1)[..., None], -1)[..., 0]
    assert np.all((top[live] & 0x7F) == 0x7B)
    xh = oracle.dequant_rows_e5m2(codes, scale, g)
    # half a unit in the last place: 2^-3 relative for normals, 2^-17 s for subnormals
    s_full = np.repeat(scale, g, axis=-1)
    bound = np.maximum(np.abs(x) * 2.0 ** -3, s_full * 2.0 ** -17) * (1 + 1e-6)
    assert np.all(np.abs(xh - x) <= bound)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(s_full > 0, x / s_full, 0).astype(np.float32)
    ref = (torch_decode5(torch_encode5(q)).astype(np.float32) * s_full).astype(np.float32)
    assert np.array_equal(xh.view(np.uint32) & 0x7FFFFFFF, ref.view(np.uint32) & 0x7FFFFFFF)
