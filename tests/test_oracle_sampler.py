"""Pins of the oracle's SIP sampler: inclusion probabilities, Philox, draws, plan.

Pins: the pages' 25%-counts-as-four example, brute force over cut-offs,
the Random123 known answers for Philox4x32-10 and rocRAND's independent
implementation of it, the sampling law over many seeds, and the
Horvitz-Thompson expectation by exact enumeration.
"""
import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import Problem
from workloads import random_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_sip_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "sip_worked_example.json")))
    s = np.array(g["scores"], dtype=np.float32)
    pi = oracle.inclusion_probabilities(s, g["budget"])
    np.testing.assert_array_equal(pi, g["expected_pi"])
    assert 1.0 / pi[1] == g["expected_ht_weight_of_quarter_block"]
    # every seed keeps block 0 (pi = 1) and never keeps the zero-score blocks;
    # a kept quarter block carries log-weight ln 4
    seen = set()
    for seed in range(64):
        cols, lw = oracle.sample_row(s, g["budget"], 0, 0, 0, seed)
        assert cols[0] == 0 and lw[0] == 0.0
        assert np.all(cols < 5)
        for c, w in zip(cols[1:], lw[1:]):
            assert w == np.float32(g["expected_logw_of_quarter_block_f32"])
            seen.add(int(c))
    assert seen == {1, 2, 3, 4}


def _brute_force_pi(s, m):
    """Try every number k of certain blocks (the k largest scores)."""
    order = np.argsort(-s, kind="stable")
    pos = s > 0
    for k in range(0, int(pos.sum()) + 1):
        cert = order[:k]
        rest = order[k:]
        rest = rest[s[rest] > 0]
        tot = s[rest].sum()
        if tot == 0:
            continue
        c = (m - k) / tot
        ok_cert = all(c * s[j] >= 1.0 - 1e-12 for j in cert)
        ok_rest = all(c * s[j] < 1.0 + 1e-12 for j in rest)
        if ok_cert and ok_rest:
            pi = np.where(pos, np.minimum(1.0, c * s), 0.0)
            pi[cert] = 1.0
            return pi
    raise AssertionError("no consistent cut-off")


@pytest.mark.parametrize("seed", range(20))
def test_inclusion_probabilities_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 14))
    s = np.exp(2.5 * rng.standard_normal(n)).astype(np.float32)
    if seed % 4 == 0:
        s[rng.integers(0, n)] = 0.0
    budget = float(rng.uniform(0.05, 0.9))
    pi = oracle.inclusion_probabilities(s, budget)
    m = budget * n
    npos = int((s > 0).sum())
    if m >= npos:
        np.testing.assert_array_equal(pi, (s > 0).astype(float))
        return
    np.testing.assert_allclose(pi, _brute_force_pi(s.astype(np.float64), m), rtol=1e-12, atol=1e-15)


def test_inclusion_probabilities_invariants():
    S = random_scores(50, 700, seed=4, spread=3.0)
    for i, budget in enumerate(np.linspace(0.01, 0.6, 50)):
        s = S[i].astype(np.float64)
        pi = oracle.inclusion_probabilities(S[i], budget)
        m = budget * 700
        assert np.all((pi >= 0) & (pi <= 1))
        assert abs(pi.sum() - m) < 1e-9 * m
        unc = pi < 1
        ratio = pi[unc] / s[unc]
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
        if np.any(~unc):  # the certain set is a top set of the scores
            assert s[~unc].min() >= s[unc].max()


def test_inclusion_probabilities_special_cases():
    n = 40
    u = np.full(n, 1.0 / n, dtype=np.float32)
    np.testing.assert_allclose(oracle.inclusion_probabilities(u, 0.25), 0.25, rtol=1e-12)
    np.testing.assert_array_equal(oracle.inclusion_probabilities(u, 1.0), np.ones(n))
    z = np.zeros(n, dtype=np.float32)
    z[:3] = [0.5, 0.25, 0.25]
    np.testing.assert_array_equal(oracle.inclusion_probabilities(z, 1.0), np.ones(n))
    np.testing.assert_array_equal(oracle.inclusion_probabilities(z, 0.5), (z > 0).astype(float))
    # one dominant block is certain, the rest share the remaining budget
    d = np.full(n, 0.01, dtype=np.float32)
    d[7] = 0.61
    pi = oracle.inclusion_probabilities(d, 0.1)
    assert pi[7] == 1.0
    np.testing.assert_allclose(np.delete(pi, 7), 3.0 / 39, rtol=1e-6)


# Philox4x32-10 known answers from the Random123 distribution (the
# generator's authors): counter, key -> the four output words
R123_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def test_philox_known_answers():
    for ctr, key, want in R123_KAT:
        out = oracle.philox4x32_10(tuple(np.array([c], np.uint64) for c in ctr), key)
        assert tuple(int(w[0]) for w in out) == want


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    """Runs rocRAND's header-only Philox4x32-10 engine on the host."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    header = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not (os.path.exists(hipcc) and os.path.exists(header)):
        pytest.skip("hipcc or the rocRAND headers are not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    src = os.path.join(os.path.dirname(__file__), "philox_ref.cpp")
    r = subprocess.run([hipcc, "-O1", src, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("could not build the rocRAND reference: " + r.stderr[-500:])

    def run(queries):
        text = "".join(f"{s} {u} {o}\n" for s, u, o in queries)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return [tuple(int(x, 16) for x in line.split()) for line in out.stdout.splitlines()]
    return run


def test_philox_matches_rocrand(rocrand_philox):
    # the engine at (seed, subsequence, offset) = Philox4x32-10 with counter
    # (offset/4 low, offset/4 high, subsequence low, subsequence high) and key
    # (seed low, seed high)
    rng = np.random.default_rng(1)
    cases = [[int(x) for x in rng.integers(0, 2 ** 32, 6, dtype=np.uint64)] for _ in range(64)]
    for cs in cases:
        cs[1] >>= 2  # the engine's offset is 64-bit: 4 * counter must fit
    queries = [(k0 | (k1 << 32), c2 | (c3 << 32), 4 * (c0 | (c1 << 32)))
               for c0, c1, c2, c3, k0, k1 in cases]
    ref = rocrand_philox(queries)
    for (c0, c1, c2, c3, k0, k1), want in zip(cases, ref):
        out = oracle.philox4x32_10(tuple(np.array([c], np.uint64) for c in (c0, c1, c2, c3)),
                                   (k0, k1))
        assert tuple(int(w[0]) for w in out) == want


def test_block_words_layout(rocrand_philox):
    # block j of row (b,h,qb): word j%4 at counter (j//4, qb, h, b)
    for b, h, qb, seed in [(1, 3, 17, 12345), (0, 39, 590, (1 << 63) + 977)]:
        w = oracle.block_words(b, h, qb, 11, seed)
        words = rocrand_philox([(seed, h | (b << 32), 4 * (j // 4 + (qb << 32))) for j in range(11)])
        for j in range(11):
            assert int(w[j]) == words[j][j % 4]
            assert 0 <= int(w[j]) < 2 ** 32


def test_sampling_law():
    s = random_scores(1, 64, seed=8, spread=1.5)[0]
    budget = 0.2
    pi = oracle.inclusion_probabilities(s, budget)
    T = 6000
    hits = np.zeros(64)
    counts = []
    for seed in range(T):
        cols, _ = oracle.sample_row(s, budget, 0, 2, 5, seed)
        hits[cols] += 1
        counts.append(len(cols))
    se = np.sqrt(T * pi * (1 - pi))
    z = np.where(se > 0, (hits - T * pi) / np.maximum(se, 1e-300), hits - T * pi)
    assert np.all(np.abs(z) < 4.5), z
    m = budget * 64
    var = (pi * (1 - pi)).sum()
    assert abs(np.mean(counts) - m) < 4.5 * math.sqrt(var / T)
    # certain blocks are always drawn
    assert np.all(hits[pi == 1.0] == T)


def test_plan_structure_and_forced_blocks():
    prob = Problem(B=1, H=2, N=600, D=16, n_forced_tail=32, n_clusters=4)
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((1, 2, 600, 16))
    K = rng.standard_normal((1, 2, 600, 16))
    p = oracle.plan(Q, K, prob, 0.2, seed=3)
    assert p.row_ptr.shape == (prob.R + 1,) and p.row_ptr[0] == 0
    assert np.all(np.diff(p.row_ptr) >= 0)
    nf = prob.n_kb - prob.n_kbs
    assert nf == 8
    for r in range(prob.R):
        cols, lw = p.row(r)
        assert np.all(np.diff(cols) > 0)
        np.testing.assert_array_equal(cols[-nf:], np.arange(prob.n_kbs, prob.n_kb))
        np.testing.assert_array_equal(lw[-nf:], 0.0)
        assert np.all(lw >= 0)
    # budget 1: every block, weight 1
    p1 = oracle.plan(Q, K, prob, 1.0, seed=3)
    for r in range(prob.R):
        cols, lw = p1.row(r)
        np.testing.assert_array_equal(cols, np.arange(prob.n_kb))
        np.testing.assert_array_equal(lw, 0.0)
    # same seed, same plan; another seed, another plan
    p2 = oracle.plan(Q, K, prob, 0.2, seed=3)
    np.testing.assert_array_equal(p.col_idx, p2.col_idx)
    p3 = oracle.plan(Q, K, prob, 0.2, seed=4)
    assert not np.array_equal(p.col_idx, p3.col_idx)


def test_logw_is_minus_log_pi():
    s = random_scores(1, 200, seed=2, spread=2.0)[0]
    pi = oracle.inclusion_probabilities(s, 0.15)
    cols, lw = oracle.sample_row(s, 0.15, 0, 0, 0, 99)
    want = np.where(pi[cols] == 1.0, 0.0, -np.log(pi[cols])).astype(np.float32)
    np.testing.assert_array_equal(lw, want)
    # lw is -ln(pi) rounded to fp32 (half an ulp: at most |lw| * 2^-24 off),
    # so exp(lw) * pi is 1 within that, plus float64 rounding
    lw64 = lw.astype(np.float64)
    assert np.all(np.abs(np.exp(lw64) * pi[cols] - 1.0) <= np.abs(lw64) * 2.0 ** -24 * 1.01 + 1e-15)
