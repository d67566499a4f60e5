"""Pins for the oracle's Oaken threshold grouping, group shift and calibration (CPU only).

Fixed against: closed-form Student-t(3) quantiles, the region shares the
page states (about 5 / 25 / 70 %), nearest-rank percentiles taken from a
sorted copy, exact reconstruction of grid-aligned rows, strict threshold ties
and the exact additive dense + sparse split.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth

THR = np.array([-1.5, -0.5, 0.5, 1.5], np.float32)


def f16bits(x):
    a = np.asarray(x, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.all(h.astype(np.float64) == a)
    return h.view(np.uint16)


def decode_entries(row_entries, count):
    e = row_entries[:count].astype(np.int64)
    return e & 127, (e >> 7) & 1, (e >> 8) & 31


def test_percentile_nearest_rank_brute_force():
    rng = np.random.default_rng(2)
    for n in (1, 7, 100, 1001, 4096):
        x = (rng.standard_normal(n) * 3).astype(np.float16)
        x[: n // 10] = 0.0
        x[n // 10: n // 5] = -0.0
        hist = oracle.hist_f16(x.view(np.uint16))
        srt = np.sort(x.astype(np.float64), kind="stable")
        for bp in (1, 250, 1500, 5000, 8500, 9750, 10000):
            rank = max(1, -(-n * bp // 10000))
            assert oracle.hist_percentile(hist, bp) == srt[rank - 1]


def test_thresholds_match_student_t_quantiles():
    """Calibration of 0.5 * t(3) samples lands on the closed-form quantiles."""
    w = synth.scaled(synth.WORKLOADS[5], kv_heads=4, seq=512)
    hist = np.zeros(65536, np.uint64)
    for sample in range(100):
        oracle.hist_f16(w.calibration(0, sample), hist)
    n = int(hist.sum())
    thr = oracle.thresholds_from_hist(hist)
    for p, t in zip((0.025, 0.15, 0.85, 0.975), thr):
        exact = 0.5 * stats.t.ppf(p, 3)
        dens = stats.t.pdf(exact / 0.5, 3) / 0.5
        sampling = 5 * np.sqrt(p * (1 - p) / n) / dens
        ulp = np.spacing(np.float16(abs(exact))).astype(np.float64)
        assert abs(t - exact) <= sampling + ulp, (p, t, exact)
    assert thr[0] < thr[1] < thr[2] < thr[3]


def test_region_shares_on_fresh_data():
    """Outer ~5 %, middle ~25 %, inner ~70 % ([Oaken] §3.2.1) on data not used for calibration."""
    w = synth.scaled(synth.WORKLOADS[5], kv_heads=4, seq=512)
    hist = np.zeros(65536, np.uint64)
    for sample in range(20):
        oracle.hist_f16(w.calibration(1, sample), hist)
    thr = oracle.thresholds_from_hist(hist)
    x = synth.f16_to_f32(w.kv(1, 0, 2)).astype(np.float64)
    outer = np.mean((x > thr[3]) | (x < thr[0]))
    inner = np.mean((x <= thr[2]) & (x >= thr[1]))
    middle = 1 - outer - inner
    assert abs(outer - 0.05) < 0.004
    assert abs(middle - 0.25) < 0.01
    assert abs(inner - 0.70) < 0.01


def test_oaken_round_trip_grid_aligned():
    """Dense codes on a 1/8 grid and outer values at T +- mag * 2^-4 (max mag 31) reproduce exactly."""
    rng = np.random.default_rng(9)
    for trial in range(30):
        D, g = 128, 64
        z = 8
        c = rng.integers(0, 16, size=D)
        c[0], c[1], c[64], c[65] = 0, 15, 0, 15
        x = (c - z) * 0.125  # in [-1, 0.875], strictly inside the outer thresholds
        outer_idx = rng.choice(np.arange(2, 64).tolist() + np.arange(66, 128).tolist(), size=10, replace=False)
        side = rng.integers(0, 2, size=10)
        mag = rng.integers(1, 32, size=10)
        # every group that has outer elements gets one with magnitude 31
        for grp in (0, 1):
            sel = np.where((outer_idx // 64) == grp)[0]
            if len(sel):
                mag[sel[0]] = 31
        s_out = 2.0 ** -4
        for i, sd, m in zip(outer_idx, side, mag):
            x[i] = THR[3] + m * s_out if sd else THR[0] - m * s_out
        codes, scale, zero, oscale, entries, counts = oracle.oaken_rows(f16bits(x)[None], THR)
        assert counts[0] == 10
        idx, sd, mg = decode_entries(entries[0], counts[0])
        order = np.argsort(outer_idx)
        assert np.array_equal(idx, np.sort(outer_idx))
        assert np.array_equal(sd, side[order]) and np.array_equal(mg, mag[order])
        for grp in (0, 1):
            has = np.any(outer_idx // 64 == grp)
            assert oscale[0, grp] == (np.float32(s_out) if has else 0.0)
        assert np.all(scale[0] == 0.125) and np.all(zero[0] == z)
        dense = np.array(c, np.uint8)
        dense[outer_idx] = z
        assert np.array_equal(codes[0], dense)
        xh = oracle.oaken_dequant_rows(codes, scale, zero, oscale, entries, counts, THR)
        assert np.array_equal(xh[0], x.astype(np.float32))


def test_oaken_ties_are_not_outer_and_split_is_additive():
    x = np.zeros(128)
    x[3] = 1.5     # == T_hi_outer: not outer (strict)
    x[4] = -1.5    # == T_lo_outer: not outer
    x[5] = 1.5009765625
    x[70] = -2.0
    x[71] = 0.25
    codes, scale, zero, oscale, entries, counts = oracle.oaken_rows(f16bits(x)[None], THR)
    idx, sd, mg = decode_entries(entries[0], counts[0])
    assert list(idx) == [5, 70] and list(sd) == [1, 0] and list(mg) == [31, 31]
    dense_only = oracle.oaken_dequant_rows(codes, scale, zero, oscale, entries, np.zeros(1, np.int32), THR)
    assert dense_only[0, 5] == 0.0 and dense_only[0, 70] == 0.0
    full = oracle.oaken_dequant_rows(codes, scale, zero, oscale, entries, counts, THR)
    # the tie values stay in the dense body: within half a dense step
    half = scale[0, 0] / 2 + 1e-6
    assert abs(full[0, 3] - 1.5) <= half and abs(full[0, 4] + 1.5) <= half
    assert full[0, 5] == np.float32(x[5]) and full[0, 70] == -2.0


def test_oaken_error_bounds_random():
    rng = np.random.default_rng(4)
    x = (rng.standard_t(3, size=(400, 128)) * 0.5).astype(np.float16)
    codes, scale, zero, oscale, entries, counts = oracle.oaken_rows(x.view(np.uint16), THR)
    xh = oracle.oaken_dequant_rows(codes, scale, zero, oscale, entries, counts, THR).astype(np.float64)
    xv = x.astype(np.float64)
    outer = (xv > THR[3]) | (xv < THR[0])
    assert counts.sum() == outer.sum()
    s_el = np.repeat(scale, 64, axis=1).astype(np.float64)
    so_el = np.repeat(oscale, 64, axis=1).astype(np.float64)
    err = np.abs(xv - xh)
    assert np.all(err[~outer] <= s_el[~outer] / 2 * (1 + 1e-5) + 1e-7)
    assert np.all(err[outer] <= so_el[outer] / 2 * (1 + 1e-5) + 1e-6)
    assert codes.max() <= 15
    for r in range(400):
        idx, _, mg = decode_entries(entries[r], counts[r])
        assert np.all(np.diff(idx) > 0) and np.all(mg <= 31)
        assert np.array_equal(idx, np.where(outer[r])[0])
