"""Pins for the oracle's Cocktail chunk precision search and reorder (CPU only).

Fixed against: embeddings built with known cosine similarities, the
invariances of cosine similarity, the class shares implied by Gaussian
order statistics, and a library stable sort for the reorder.
"""
import numpy as np

import oracle
import synth


def test_chunk_bits_constructed_similarities():
    """Chunk i at angle theta_i from the query has similarity cos(theta_i); classes follow T_low/T_high."""
    dim = 16
    sims = np.linspace(-0.9, 0.95, 38)
    q = np.zeros(dim)
    q[0] = 2.0
    ce = np.zeros((len(sims), dim))
    ce[:, 0] = sims * 3.0
    ce[:, 1] = np.sqrt(1 - sims ** 2) * 3.0
    bits, got = oracle.chunk_bits(q, ce, alpha=0.6, beta=0.1)
    assert np.allclose(got, sims, atol=1e-12)
    # s_min = -0.9, s_max = 0.95: T_low = -0.9 + 1.85 * 0.6 = 0.21, T_high = 0.95 - 0.185 = 0.765
    expect = np.where(sims > 0.765 + 1e-9, 16, np.where(sims > 0.21 + 1e-9, 4, 2))
    assert np.array_equal(bits, expect)
    assert bits[np.argmax(sims)] == 16 and bits[np.argmin(sims)] == 2


def test_chunk_bits_invariances():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64)
    ce = rng.standard_normal((200, 64))
    b0, s0 = oracle.chunk_bits(q, ce)
    b1, s1 = oracle.chunk_bits(q * 7.5, ce * rng.uniform(0.1, 9, size=(200, 1)))
    assert np.array_equal(b0, b1) and np.allclose(s0, s1, atol=1e-12)
    # all chunks alike -> s_max == s_min -> every chunk INT2
    b2, _ = oracle.chunk_bits(q, np.tile(ce[:1], (10, 1)))
    assert np.all(b2 == 2)
    # beta = 0: nothing above T_high = s_max; alpha = 1 as well: every chunk at or below T_low
    b3, _ = oracle.chunk_bits(q, ce, alpha=0.6, beta=0.0)
    assert not np.any(b3 == 16)
    b4, _ = oracle.chunk_bits(q, ce, alpha=1.0, beta=0.0)
    assert np.all(b4 == 2)


def test_chunk_bits_shares_gaussian():
    """768-d Gaussian vectors: sims ~ N(0, 1/768); with 1024 chunks about 0.5 % / 26 % / 74 %."""
    w = synth.WORKLOADS[4]
    counts = np.zeros(3)
    for b in range(w.batch):
        qe, ce = w.chunk_embeddings(b)
        bits, sims = oracle.chunk_bits(qe, ce)
        assert abs(np.std(sims) * np.sqrt(768) - 1) < 0.08
        counts += [np.sum(bits == 16), np.sum(bits == 4), np.sum(bits == 2)]
    frac = counts / counts.sum()
    assert 0.001 < frac[0] < 0.02
    assert 0.18 < frac[1] < 0.34
    assert 0.64 < frac[2] < 0.82


def test_reorder_against_stable_sort():
    rng = np.random.default_rng(3)
    for n in (1, 8, 33, 1024):
        bits = rng.choice(np.array([16, 4, 2], np.uint8), size=(3, n), p=[0.1, 0.3, 0.6])
        perm, seg = oracle.reorder(bits)
        for b in range(3):
            cls = np.select([bits[b] == 16, bits[b] == 4], [0, 1], 2)
            expect = sorted(range(n), key=lambda i: cls[i])  # Python's sort is stable
            assert list(perm[b]) == expect
            assert list(seg[b]) == [np.sum(cls == 0), np.sum(cls == 1), np.sum(cls == 2), n]
            assert sorted(perm[b]) == list(range(n))
            inv = np.empty(n, np.int64)
            inv[perm[b]] = np.arange(n)
            assert np.array_equal(np.arange(n)[perm[b]][inv], np.arange(n))


def test_reorder_brute_force_tiny():
    """Every 4-chunk assignment: slots hold FP16 ids, then INT4, then INT2, each in increasing id order."""
    import itertools
    for combo in itertools.product([16, 4, 2], repeat=4):
        bits = np.array([combo], np.uint8)
        perm, seg = oracle.reorder(bits)
        slots = list(perm[0])
        fp16 = [i for i in range(4) if combo[i] == 16]
        i4 = [i for i in range(4) if combo[i] == 4]
        i2 = [i for i in range(4) if combo[i] == 2]
        assert slots == fp16 + i4 + i2
        assert list(seg[0]) == [len(fp16), len(i4), len(i2), 4]
