"""Host check of the row-index division the token quantizers use instead of
64-bit divides: for a divisor d fixed per launch, s = ceil(log2 d),
m = floor(2^32 (2^s - d) / d) + 1, and q = (t + ((n - t) >> 1)) >> (s - 1)
with t = floor(n m / 2^32) (q = n for d = 1).  The construction (Granlund and
Montgomery's round-up multiplier) is exact for every n < 2^32; this replays it
in integer arithmetic for the divisors the quantizers see (token counts and
head counts, powers of two and not) at the ends of the range and at random
points, including every multiple boundary near the top."""
import numpy as np


def make(d):
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((1 << 32) * ((1 << s) - d)) // d + 1
    assert 0 <= m < (1 << 32)
    return m, s


def fdiv(n, m, s):
    if s == 0:
        return n
    t = (n * m) >> 32
    return (t + ((n - t) >> 1)) >> (s - 1)


def test_fast_division_matches_integer_division():
    rng = np.random.default_rng(7)
    divisors = list(range(1, 300)) + [1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 32768, 65535, 131071,
                                      131072, (1 << 31) - 1, 1 << 31]
    for d in divisors:
        m, s = make(d)
        ns = {0, 1, d - 1, d, d + 1, (1 << 31) - 1, (1 << 32) - 1, (1 << 32) - 2}
        top = ((1 << 32) - 1) // d * d
        ns |= {top - 1, top, min(top + d - 1, (1 << 32) - 1)}
        ns |= set(int(v) for v in rng.integers(0, 1 << 32, 2000, dtype=np.uint64))
        for n in ns:
            if 0 <= n < (1 << 32):
                assert fdiv(n, m, s) == n // d, (d, n)
