"""The sampler's draw compare, decided on the first Philox word.

A block is kept iff its 53-bit uniform u = w0 * 2^21 + (w1 >> 11) is below
pi * 2^53.  The GPU decides on w0 alone unless w0 equals
f = floor(min(pi * 2^32, 2^32 - 1)), and takes the exact compare only then.
This checks that rule against the exact rational comparison, including the
ties (probability 2^-32 per block, so the GPU tests never reach them), pi = 0,
pi = 1 and values of pi * 2^32 within one step of 2^32.
"""
from fractions import Fraction

import numpy as np


def exact_keep(pi: float, w0: int, w1: int) -> bool:
    u = (w0 << 21) | (w1 >> 11)
    return Fraction(u) < Fraction(pi) * 2 ** 53


def fast_keep(pi: float, w0: int, w1: int) -> bool:
    x = pi * 4294967296.0                       # exact: a power-of-two scale
    f = int(x) if x < 4294967295.0 else 0xFFFFFFFF
    if w0 != f:
        return w0 < f
    return float((w0 << 21) | (w1 >> 11)) < x * 2097152.0


def test_rule_matches_exact_compare():
    rng = np.random.default_rng(7)
    pis = [0.0, 1.0, 2.0 ** -32, 2.0 ** -33, 3 * 2.0 ** -34, 0.5, 0.1, 1 - 2.0 ** -33,
           1 - 2.0 ** -32, 1 - 2.0 ** -40, float(np.nextafter(1.0, 0.0)),
           (2 ** 32 - 1) / 2 ** 32, 12345 / 2 ** 32, 12345.5 / 2 ** 32]
    pis += [float(p) for p in rng.random(300)]
    pis += [float(p) for p in np.exp(rng.uniform(np.log(1e-12), 0.0, 200))]
    n = 0
    for pi in pis:
        f = int(pi * 2 ** 32) if pi < 1 else 0xFFFFFFFF
        w0s = {0, 0xFFFFFFFF, f, max(f - 1, 0), min(f + 1, 0xFFFFFFFF)}
        w0s |= set(int(v) for v in rng.integers(0, 2 ** 32, 4))
        for w0 in w0s:
            # low words around the tie's split point and at the ends
            x = Fraction(pi) * 2 ** 53 - (w0 << 21)
            mid = int(x) << 11 if 0 <= x < 2 ** 21 else 0
            for w1 in {0, 0xFFFFFFFF, mid, max(mid - 2048, 0), min(mid + 2048, 0xFFFFFFFF),
                       int(rng.integers(0, 2 ** 32))}:
                assert fast_keep(pi, w0, w1) == exact_keep(pi, w0, w1), (pi, w0, w1)
                n += 1
    assert n > 5000
