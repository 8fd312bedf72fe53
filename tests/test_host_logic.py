"""Host-side facts the kernels rely on (no GPU needed)."""
import numpy as np


def test_multiply_high_division_is_exact_on_the_layout_domain():
    """The layout kernels divide by d = L, R or G (d <= 1024) with dividends
    n < 2^22 as q = (n * m) >> 32, m = ceil(2^32 / d).

    With e = m*d - 2^32 in [0, d): n*m / 2^32 = n/d + n*e / (d * 2^32), and
    n*e < 2^22 * 2^10 = 2^32 makes the excess below 1/d, which cannot carry
    n/d (whose fraction is at most (d-1)/d) past the next integer.  Check the
    premise for every d and the result exhaustively for a few d.
    """
    for d in range(1, 1025):
        m = -(-(1 << 32) // d)
        assert 0 <= m * d - (1 << 32) < d
    n = np.arange(0, 1 << 22, dtype=np.uint64)
    for d in (1, 2, 3, 7, 16, 255, 256, 1000, 1023, 1024):
        m = np.uint64(-(-(1 << 32) // d))
        assert np.array_equal((n * m) >> np.uint64(32), n // np.uint64(d)), d
