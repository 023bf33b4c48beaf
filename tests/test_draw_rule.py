"""The sampler's draw compare on the shipped code.

A block is kept iff its 32-bit uniform integer w (one Philox word) is below
pi * 2^32, so it enters with probability ceil(pi * 2^32) / 2^32.  The
kernel's own decision function (sip_keep in csrc/draw_rule.h, which the
sampler kernel calls) is compiled for the host into a small harness and
checked against the exact rational comparison: pi = 0 and 1, pi * 2^32 on
and next to an integer, the ends of the word range, and random cases.  The
oracle's rule is checked against the same exact comparison.
"""
import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle


def exact_keep(pi: float, w: int) -> bool:
    return Fraction(w) < Fraction(pi) * 2 ** 32


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    exe = str(tmp_path_factory.mktemp("draw") / "draw_rule_harness")
    src = os.path.join(os.path.dirname(__file__), "draw_rule_harness.cpp")
    r = subprocess.run([hipcc, "-O2", src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(cases):
        text = "".join(f"{struct.unpack('<Q', struct.pack('<d', pi * 4294967296.0))[0]:x} {w}\n"
                       for pi, w in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return [line == "1" for line in out.stdout.split()]
    return run


def draw_cases():
    rng = np.random.default_rng(7)
    pis = [0.0, 1.0, 2.0 ** -32, 2.0 ** -33, 3 * 2.0 ** -34, 0.5, 0.1, 1 - 2.0 ** -33,
           1 - 2.0 ** -32, 1 - 2.0 ** -40, float(np.nextafter(1.0, 0.0)),
           (2 ** 32 - 1) / 2 ** 32, 12345 / 2 ** 32, 12345.5 / 2 ** 32,
           float(np.nextafter(12345 / 2 ** 32, 1.0)), float(np.nextafter(12345 / 2 ** 32, 0.0))]
    pis += [float(p) for p in rng.random(300)]
    pis += [float(p) for p in np.exp(rng.uniform(np.log(1e-12), 0.0, 200))]
    cases = []
    for pi in pis:
        x = Fraction(pi) * 2 ** 32
        f = int(x)                       # floor(pi * 2^32)
        ws = {0, 1, 0xFFFFFFFE, 0xFFFFFFFF}
        ws |= {min(max(f + d, 0), 0xFFFFFFFF) for d in (-2, -1, 0, 1, 2)}
        ws |= set(int(v) for v in rng.integers(0, 2 ** 32, 6))
        cases += [(pi, w) for w in sorted(ws)]
    return cases


def test_rule_matches_exact_compare(harness):
    cases = draw_cases()
    got = harness(cases)
    assert len(got) == len(cases) > 5000
    boundary = 0
    for (pi, w), g in zip(cases, got):
        assert g == exact_keep(pi, w), (pi, w)
        boundary += abs(Fraction(pi) * 2 ** 32 - w) <= 1
    assert boundary > 1000            # cases on and next to the threshold


def test_rule_extremes(harness):
    # pi = 0 keeps nothing, pi = 1 keeps every word, pi = 2^-32 keeps w = 0 only
    cases = [(0.0, 0), (0.0, 0xFFFFFFFF), (1.0, 0), (1.0, 0xFFFFFFFF),
             (2.0 ** -32, 0), (2.0 ** -32, 1), (1 - 2.0 ** -32, 0xFFFFFFFE),
             (1 - 2.0 ** -32, 0xFFFFFFFF)]
    assert harness(cases) == [False, False, True, True, True, False, True, False]


def test_oracle_rule_is_the_same_compare():
    # sample_row keeps block j iff its word is below pi * 2^32: with scores
    # that make every pi equal, the kept set is exactly the words below it
    n, budget = 64, 0.25
    s = np.full(n, 1.0, dtype=np.float32)
    pi = oracle.inclusion_probabilities(s, budget)
    assert np.all(pi == 0.25)
    for seed in range(20):
        cols, _ = oracle.sample_row(s, budget, 1, 2, 3, seed)
        w = oracle.block_words(1, 2, 3, n, seed)
        want = [j for j in range(n) if exact_keep(0.25, int(w[j]))]
        assert cols.tolist() == want
