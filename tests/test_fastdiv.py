"""The division-free floor(n / d) the block-centric kernel uses to turn a list
entry (row * top_k + slot) back into its row: with l = ceil(log2 d) and
m = ceil(2^(31 + l) / d), floor(n m / 2^(31 + l)) = floor(n / d) for every
0 <= n < 2^31.  The formula (make_fastdiv / fastdiv in the kernels' device
header) is checked here in exact integer arithmetic for every top_k the
library accepts (1 .. 4096) at the worst-case dividends: multiples of d, one
below and d - 1 above them, and the largest n."""
import numpy as np


def params(d):
    if d <= 1:
        return 1, -1
    l = (d - 1).bit_length()   # ceil(log2 d)
    return -(-(1 << (31 + l)) // d), l - 1


def fastdiv(n, m, s):
    return n if s < 0 else ((n * m) >> 32) >> s


def test_fastdiv_exact_for_every_top_k():
    rng = np.random.default_rng(3)
    top = (1 << 31) - 1
    for d in range(1, 4097):
        m, s = params(d)
        assert s < 0 or m < (1 << 32)
        qmax = top // d
        qs = np.unique(np.concatenate([[0, 1, 2, qmax - 1, qmax], rng.integers(0, qmax + 1, 64)]))
        for q in qs.tolist():
            for n in (q * d, q * d + d - 1, q * d - 1):
                if 0 <= n <= top:
                    assert fastdiv(n, m, s) == n // d, (d, n)
        assert fastdiv(top, m, s) == top // d
