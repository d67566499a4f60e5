"""Pins for the oracle's decode attention and log-sum-exp merge (CPU only).

Fixed against: a library softmax (scipy) on tiny inputs, closed-form special
cases (one token, identical keys, two tokens -> logistic weight), joint
permutation invariance of the (k, v) rows, the GQA head mapping and the
equality of segment-wise merged attention with unsegmented attention.
"""
import numpy as np
from scipy.special import softmax

import oracle


def q16(rng, n, D, scale=1.0):
    return (rng.standard_normal((n, D)) * scale).astype(np.float16)


def test_brute_force_tiny_against_scipy_softmax():
    rng = np.random.default_rng(0)
    for S in (1, 2, 5, 8):
        for D in (4, 16, 128):
            q = q16(rng, 1, D)
            k = rng.standard_normal((1, S, D)).astype(np.float32) * 2
            v = rng.standard_normal((1, S, D)).astype(np.float32)
            sm = 1 / np.sqrt(D)
            got = oracle.attention(q.view(np.uint16), k, v, sm)
            w = softmax(q.astype(np.float64) @ k[0].astype(np.float64).T * sm, axis=-1)
            ref = w @ v[0].astype(np.float64)
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_special_cases():
    rng = np.random.default_rng(1)
    D = 128
    q = q16(rng, 1, D)
    v = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)
    out = oracle.attention(q.view(np.uint16), k, v, 0.1)
    assert np.array_equal(out[0], v[0, 0].astype(np.float64))
    # identical keys -> uniform weights -> mean of the values
    S = 37
    k = np.tile(rng.standard_normal((1, 1, D)).astype(np.float32), (1, S, 1))
    v = rng.standard_normal((1, S, D)).astype(np.float32)
    out = oracle.attention(q.view(np.uint16), k, v, 0.1)
    assert np.allclose(out[0], v[0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)
    # two tokens: weight of the first is the logistic function of the score gap
    k = rng.standard_normal((1, 2, D)).astype(np.float32)
    v = rng.standard_normal((1, 2, D)).astype(np.float32)
    sm = 1 / np.sqrt(D)
    out = oracle.attention(q.view(np.uint16), k, v, sm)
    qd = q[0].astype(np.float64)
    gap = (qd @ k[0, 0].astype(np.float64) - qd @ k[0, 1].astype(np.float64)) * sm
    w0 = 1 / (1 + np.exp(-gap))
    assert np.allclose(out[0], w0 * v[0, 0] + (1 - w0) * v[0, 1], rtol=1e-12, atol=1e-14)
    # a dominant key (huge score margin) -> that key's value
    k = np.zeros((1, 3, D), np.float32)
    k[0, 1] = qd.astype(np.float32) * 50
    v = rng.standard_normal((1, 3, D)).astype(np.float32)
    out = oracle.attention(q.view(np.uint16), k, v, 1.0)
    assert np.allclose(out[0], v[0, 1], rtol=1e-12, atol=1e-12)


def test_joint_permutation_invariance():
    rng = np.random.default_rng(2)
    D, S = 128, 300
    q = q16(rng, 2, D)
    k = rng.standard_normal((1, S, D)).astype(np.float32)
    v = rng.standard_normal((1, S, D)).astype(np.float32)
    p = rng.permutation(S)
    a = oracle.attention(q.view(np.uint16), k, v, 0.088)
    b = oracle.attention(q.view(np.uint16), k[:, p], v[:, p], 0.088)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_gqa_head_mapping():
    """Consecutive query heads share a KV head: query h reads KV head h // (Hq / Hkv)."""
    rng = np.random.default_rng(3)
    D, S, Hq, Hkv = 128, 20, 8, 2
    q = q16(rng, Hq, D)
    k = rng.standard_normal((Hkv, S, D)).astype(np.float32)
    v = np.zeros((Hkv, S, D), np.float32)
    for j in range(Hkv):
        v[j] = j + 1
    out = oracle.attention(q.view(np.uint16), k, v, 0.1)
    for h in range(Hq):
        assert np.allclose(out[h], h // (Hq // Hkv) + 1, rtol=1e-13)


def test_segment_merge_equals_unsegmented():
    """[Cocktail] §3.2.3: attention per block then merged equals ordinary attention."""
    rng = np.random.default_rng(4)
    D, S = 128, 1000
    q = q16(rng, 1, D)[0]
    k = (rng.standard_normal((S, D)) * 3).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32)
    sm = 1 / np.sqrt(D)
    m, l, o_full = oracle.attention_partial(q.view(np.uint16), k, v, 0, S, sm)
    ref = oracle.attention(q.view(np.uint16)[None], k[None], v[None], sm)[0]
    assert np.allclose(o_full, ref, rtol=1e-13, atol=1e-15)
    for cuts in ([0, 1000], [0, 1, 999, 1000], [0, 100, 100, 640, 1000], [0, 333, 334, 900, 1000]):
        parts = [oracle.attention_partial(q.view(np.uint16), k, v, a, b, sm) for a, b in zip(cuts[:-1], cuts[1:])]
        ms = np.array([p[0] for p in parts])
        ls = np.array([p[1] for p in parts])
        os_ = np.array([p[2] for p in parts])
        merged = oracle.lse_merge(ms, ls, os_)
        assert np.allclose(merged, ref, rtol=1e-12, atol=1e-14)
    # empty segment contributes nothing
    mm, ll, oo = oracle.attention_partial(q.view(np.uint16), k, v, 5, 5, sm)
    assert mm == -np.inf and ll == 0 and not oo.any()
