"""Integer identities the kernels rely on, checked exhaustively on the CPU.

The small-group kernel divides small non-negative integers by runtime
divisors with a multiply-high: q = (n * ceil(2^32 / d)) >> 32 for d >= 2 and
q = n for d = 1, valid for 0 <= n < 2^16 and 1 <= d < 2^16.
"""
import numpy as np


def magic_div(n, d):
    if d == 1:
        return n
    m = (2 ** 32 + d - 1) // d
    return (n * m) >> 32


def test_magic_division_exact_small_divisors():
    n = np.arange(0, 1 << 16, dtype=np.uint64)
    for d in range(1, 600):
        m = np.uint64((2 ** 32 + d - 1) // d) if d > 1 else None
        q = n if d == 1 else (n * m) >> np.uint64(32)
        assert np.array_equal(q, n // np.uint64(d)), d


def test_magic_division_exact_large_divisors():
    rng = np.random.default_rng(1)
    n = np.concatenate([np.arange(0, 4096), rng.integers(0, 1 << 16, 20000), [65535]]).astype(np.uint64)
    for d in list(range(600, 70000, 97)) + [65535, 32768, 4097, 40000]:
        if d >= 1 << 16:
            continue
        m = np.uint64((2 ** 32 + d - 1) // d)
        assert np.array_equal((n * m) >> np.uint64(32), n // np.uint64(d)), d
