"""The sampler's draw compare, decided on the first Philox word.

A block is kept iff its 53-bit uniform u = w0 * 2^21 + (w1 >> 11) is below
pi * 2^53.  The GPU decides on w0 alone unless w0 equals
f = floor(min(pi * 2^32, 2^32 - 1)), and takes the exact compare only then.
The kernel's own decision function (sip_keep in csrc/draw_rule.h, which the
sampler kernel calls) is compiled for the host into a small harness and
checked against the exact rational comparison, including the ties
(probability 2^-32 per block, so the GPU tests never reach them), pi = 0,
pi = 1 and values of pi * 2^32 within one step of 2^32.
"""
import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest


def exact_keep(pi: float, w0: int, w1: int) -> bool:
    u = (w0 << 21) | (w1 >> 11)
    return Fraction(u) < Fraction(pi) * 2 ** 53


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
        text = "".join(f"{struct.unpack('<Q', struct.pack('<d', pi * 4294967296.0))[0]:x} {w0} {w1}\n"
                       for pi, w0, w1 in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return [line == "1" for line in out.stdout.split()]
    return run


def test_rule_matches_exact_compare(harness):
    rng = np.random.default_rng(7)
    pis = [0.0, 1.0, 2.0 ** -32, 2.0 ** -33, 3 * 2.0 ** -34, 0.5, 0.1, 1 - 2.0 ** -33,
           1 - 2.0 ** -32, 1 - 2.0 ** -40, float(np.nextafter(1.0, 0.0)),
           (2 ** 32 - 1) / 2 ** 32, 12345 / 2 ** 32, 12345.5 / 2 ** 32]
    pis += [float(p) for p in rng.random(300)]
    pis += [float(p) for p in np.exp(rng.uniform(np.log(1e-12), 0.0, 200))]
    cases = []
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
                cases.append((pi, w0, w1))
    got = harness(cases)
    assert len(got) == len(cases) > 5000
    ties = 0
    for (pi, w0, w1), g in zip(cases, got):
        assert g == exact_keep(pi, w0, w1), (pi, w0, w1)
        ties += w0 == (int(pi * 2 ** 32) if pi < 1 else 0xFFFFFFFF)
    assert ties > 1000          # the tie branch is exercised
