"""Host check of the multiply-high division the layout kernels use for divisors fixed per
call (div_magic / fast_div in combine_moe_get_amd/csrc/moe_internal.hpp): n / d equals
(n * ceil(2^32 / d)) >> 32 for every divisor the kernels use (L, K, E, the sub-chunk size:
1 ... 2048) and every numerator they divide (lanes, expert ids, slots and tokens of a chunk:
below 2^13).  d = 1 is passed through unchanged (magic 0)."""
import numpy as np


def magic(d):
    return 0 if d == 1 else ((1 << 32) + d - 1) // d


def test_multiply_high_division_is_exact_on_the_kernels_domain():
    n = np.arange(1 << 13, dtype=np.uint64)
    for d in range(1, 2049):
        m = magic(d)
        q = n if m == 0 else (n * np.uint64(m)) >> np.uint64(32)
        assert np.array_equal(q, n // np.uint64(d)), d
        assert m < (1 << 32)
