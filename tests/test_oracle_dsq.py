"""Pins for the oracle's differential significant-token quantization (CPU only).

The KVO-LLM page (§3.1, DSQ) fixes: groups of 64 tokens, the top 20 % of
each group significant and marked in a 1-bit mask, significant tokens INT8
per channel, K of the others as an INT2 difference from the base, V of the
others as group-wise INT2.  The oracle is pinned here against numpy's
stable sort (selection), hand-worked orders (ties, signed zeros, monotone
scores), the half-step bound of round-to-nearest per code, exact round
trips of grid-aligned values, the fp64 mean (base) and the identity that
lets decode form q . base from the significant tokens' scores.
"""
import numpy as np
import pytest

import oracle

T = 64


def _inputs(seed, n_groups=2, scale=1.0, outliers=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_groups * T, 128)) * scale
    v = rng.standard_normal((n_groups * T, 128)) * scale
    if outliers:
        k[:, [7, 93]] *= 15.0
    sc = rng.lognormal(size=n_groups * T).astype(np.float32)
    return (k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16), sc)


def _sig_tokens(mask):
    return [t for t in range(T) if (int(mask) >> t) & 1]


def _f(bits):
    return bits.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("n_sig", [1, 8, 13, 16])
@pytest.mark.parametrize("ties", [False, True])
def test_selection_matches_stable_sort(n_sig, ties):
    """Significant = the first n_sig tokens of a stable descending sort by score."""
    rng = np.random.default_rng(11 + n_sig + 100 * ties)
    for trial in range(5):
        k, v, sc = _inputs(trial, 1, outliers=False)
        if ties:
            sc = rng.integers(0, 3, size=T).astype(np.float32)
        r = oracle.dsq_quant(k, v, sc, n_sig=n_sig)
        order = np.lexsort((np.arange(T), -sc.astype(np.float64)))
        assert _sig_tokens(r["mask"][0]) == sorted(order[:n_sig].tolist())
        assert bin(int(r["mask"][0])).count("1") == n_sig


def test_selection_hand_worked_orders():
    k, v, _ = _inputs(3, 1, outliers=False)
    # equal scores: the lowest indices win
    r = oracle.dsq_quant(k, v, np.full(T, 2.5, np.float32))
    assert _sig_tokens(r["mask"][0]) == list(range(13))
    # increasing scores: the last 13 tokens
    r = oracle.dsq_quant(k, v, np.arange(T, dtype=np.float32))
    assert _sig_tokens(r["mask"][0]) == list(range(T - 13, T))
    # -0 orders below +0 (bit-pattern total order), so +0 tokens are taken first
    sc = np.zeros(T, np.float32)
    sc[:20] = -0.0
    r = oracle.dsq_quant(k, v, sc)
    assert _sig_tokens(r["mask"][0]) == list(range(20, 33))
    # negative scores below positive ones, the largest magnitude negative last
    sc = -np.arange(T, dtype=np.float32)
    sc[40] = 0.5
    r = oracle.dsq_quant(k, v, sc)
    assert _sig_tokens(r["mask"][0]) == sorted([40] + list(range(12)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_significant_rows_int8_per_channel(seed):
    """Slot i holds the i-th significant token; per channel |x - s c| <= s / 2, |c| <= 127 and the
    channel's largest magnitude lands on +-127."""
    k, v, sc = _inputs(seed)
    r = oracle.dsq_quant(k, v, sc)
    for g in range(2):
        toks = [g * T + t for t in _sig_tokens(r["mask"][g])]
        for x, codes, s in ((k, r["ksig"][g], r["kscale"][g]), (v, r["vsig"][g], r["vscale"][g])):
            xs = _f(x[toks])
            s64 = s.astype(np.float64)
            assert np.all(np.abs(codes.astype(np.int64)) <= 127)
            assert np.all(np.abs(xs - s64 * codes) <= s64 / 2 * (1 + 1e-6))
            live = np.abs(xs).max(axis=0) > 0
            assert np.all(np.abs(codes[:, live]).max(axis=0) == 127)


def test_significant_rows_grid_aligned_round_trip():
    """Values c * 2^-7 with 127 present in every channel are reproduced exactly."""
    rng = np.random.default_rng(5)
    c = rng.integers(-127, 128, size=(T, 128))
    c[0] = 127
    k = (c * 2.0 ** -7).astype(np.float16).view(np.uint16)
    v = (-c * 2.0 ** -7).astype(np.float16).view(np.uint16)
    sc = np.zeros(T, np.float32)
    sc[:13] = 1.0  # tokens 0..12 significant
    r = oracle.dsq_quant(k, v, sc)
    assert _sig_tokens(r["mask"][0]) == list(range(13))
    # every channel's significant maximum is 127 * 2^-7 (token 0)
    assert np.all(r["kscale"][0] == np.float32(2.0 ** -7))
    assert np.array_equal(r["ksig"][0].astype(np.int64), c[:13])
    assert np.array_equal(r["vsig"][0].astype(np.int64), -c[:13])
    kh, vh = oracle.dsq_dequant(r)
    assert np.array_equal(kh[:13].astype(np.float64), c[:13] * 2.0 ** -7)


@pytest.mark.parametrize("seed", [0, 4])
def test_base_is_mean_of_dequantized_significant_rows(seed):
    k, v, sc = _inputs(seed)
    r = oracle.dsq_quant(k, v, sc)
    for g in range(2):
        deq = r["kscale"][g].astype(np.float64) * r["ksig"][g].astype(np.float64)
        mean = deq.mean(axis=0)
        tol = 16 * 2.0 ** -24 * np.abs(deq).max(axis=0)
        assert np.all(np.abs(r["base"][g] - mean) <= tol)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_other_tokens_int2_difference_and_v(seed):
    """Slot j holds the j-th non-significant token; K = base + (c - z) s within s / 2 of k,
    V = (c - z) s within s / 2 of v; codes in 0..3."""
    k, v, sc = _inputs(seed)
    r = oracle.dsq_quant(k, v, sc)
    for g in range(2):
        sig = set(_sig_tokens(r["mask"][g]))
        toks = [g * T + t for t in range(T) if t not in sig]
        assert len(toks) == T - 13
        base = r["base"][g].astype(np.float64)
        for x, codes, s, z, b in ((k, r["kc2"][g], r["ks2"][g], r["kz2"][g], base),
                                  (v, r["vc2"][g], r["vs2"][g], r["vz2"][g], 0.0 * base)):
            assert codes.max() <= 3
            s64 = np.repeat(s.astype(np.float64), 32, axis=1)
            z64 = np.repeat(z.astype(np.float64), 32, axis=1)
            xh = b + (codes - z64) * s64
            xs = _f(x[toks])
            tol = s64 / 2 + 4 * 2.0 ** -24 * (np.abs(xs) + np.abs(b) + s64 * 4)
            assert np.all(np.abs(xs - xh) <= tol)


def test_dequant_in_token_order():
    """dsq_dequant puts each class's slots back at their tokens (checked against the bounds)."""
    k, v, sc = _inputs(9)
    r = oracle.dsq_quant(k, v, sc)
    kh, vh = oracle.dsq_dequant(r)
    for g in range(2):
        sig = _sig_tokens(r["mask"][g])
        for i, t in enumerate(sig):
            assert np.array_equal(kh[g * T + t], r["kscale"][g] * r["ksig"][g][i].astype(np.float32))
        others = [t for t in range(T) if t not in sig]
        rows = [g * T + t for t in others]
        s = np.repeat(r["vs2"][g].astype(np.float64), 32, axis=1)
        err = np.abs(vh[rows] - _f(v[rows]))
        assert np.all(err <= s / 2 * (1 + 1e-6) + 1e-7)
        s = np.repeat(r["ks2"][g].astype(np.float64), 32, axis=1)
        kx = _f(k[rows])
        err = np.abs(kh[rows] - kx)
        assert np.all(err <= s / 2 * (1 + 1e-6) + 8 * 2.0 ** -24 * (np.abs(kx) + 4 * s + 1))


def test_query_dot_base_equals_mean_significant_score():
    """q . base equals the mean of q . k_hat over the significant tokens (up to binary32 rounding
    of base): the identity the decode kernel uses instead of reading base."""
    k, v, sc = _inputs(2)
    r = oracle.dsq_quant(k, v, sc)
    kh, _ = oracle.dsq_dequant(r)
    q = np.random.default_rng(3).standard_normal(128)
    for g in range(2):
        sig = [g * T + t for t in _sig_tokens(r["mask"][g])]
        lhs = float(q @ r["base"][g].astype(np.float64))
        rhs = float(np.mean(kh[sig].astype(np.float64) @ q))
        assert abs(lhs - rhs) <= 1e-5 * (np.abs(q) @ np.abs(r["base"][g]) + 1)


def test_attention_over_dsq_cache_brute_force():
    k, v, sc = _inputs(6, 2, outliers=False)
    r = oracle.dsq_quant(k, v, sc)
    kh, vh = oracle.dsq_dequant(r)
    q = np.random.default_rng(8).standard_normal((2, 128)).astype(np.float16).view(np.uint16)
    got = oracle.attention(q, kh[None], vh[None], 1 / np.sqrt(128))
    qf = _f(q)
    s = qf @ kh.astype(np.float64).T / np.sqrt(128)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ vh.astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mask_overhead_under_half_percent():
    """The page keeps the 1-bit mask's metadata under 0.5 % of the data: 8 bytes per 64-token
    group and head against the group's packed K and V."""
    n_sig, n = 13, T - 13
    packed = 2 * (n_sig * 128 + n * 128 // 4)  # INT8 and INT2 codes of K and V
    assert 8 / packed < 0.005
