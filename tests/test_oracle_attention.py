"""Pins of the oracle's attention: library SDPA, dense equality, HT unbiasedness.

The Horvitz-Thompson checks are what the pages fix about the estimator: the
expected numerator and normaliser over the draws equal the dense ones.  Exact
enumeration over every subset pins the sign and form of the logit shift.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Problem
from workloads import Workload, make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa_rows(q, k, v, shift, tau):
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    mask = torch.from_numpy(np.broadcast_to(shift, (q.shape[0], k.shape[0])).copy())[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=tau)
    lse = torch.logsumexp(tau * (qt @ kt.transpose(-1, -2)) + mask, dim=-1)
    return o[0, 0].numpy(), lse[0, 0].numpy()


def test_attend_row_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    prob = Problem(B=1, H=2, N=520, D=32)
    Q = rng.standard_normal((1, 2, 520, 32))
    K = rng.standard_normal((1, 2, 520, 32))
    V = rng.standard_normal((1, 2, 520, 32))
    for r in [0, 3, prob.R - 1]:       # row 3 is the partial last block of head 0
        cols = np.sort(rng.choice(prob.n_kb, 37, replace=False)).astype(np.int32)
        lw = rng.uniform(0, 5, 37).astype(np.float32)
        o, lse = oracle.attend_row(Q, K, V, prob, r, cols, lw)
        b, h, qb = oracle.unflatten_row(prob, r)
        tok = (cols[:, None] * 4 + np.arange(4)).reshape(-1)
        lo, hi = qb * 128, min(qb * 128 + 128, 520)
        ro, rl = _sdpa_rows(Q[b, h, lo:hi], K[b, h, tok], V[b, h, tok],
                            np.repeat(lw.astype(np.float64), 4), prob.tau)
        np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=1e-12)


def test_dense_matches_torch_sdpa():
    rng = np.random.default_rng(2)
    prob = Problem(B=1, H=2, N=300, D=16)
    Q, K, V = (rng.standard_normal((1, 2, 300, 16)) for _ in range(3))
    O, L = oracle.dense(Q, K, V, prob)
    for h in range(2):
        ro, rl = _sdpa_rows(Q[0, h], K[0, h], V[0, h], np.zeros(300), prob.tau)
        np.testing.assert_allclose(O[0, h], ro, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(L[0, h], rl, rtol=1e-12)


def test_budget_one_equals_dense():
    wl = Workload("t", B=1, H=2, D=64, grid=(2, 16, 16), dtype="f32", sigma=1.0)
    q, k, v = make_qkv(wl)
    prob = Problem(B=1, H=2, N=wl.N, D=64)
    p = oracle.plan(q, k, prob, 1.0, seed=0)
    O, L = oracle.attend(q, k, v, p, prob)
    Od, Ld = oracle.dense(q, k, v, prob)
    np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, Ld, rtol=1e-13)


def test_empty_row_and_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "sip_worked_example.json")))["attention_example"]
    prob = Problem(B=1, H=1, N=8, D=2, q_block=1, kv_block=4)
    Q = np.zeros((1, 1, 8, 2))
    K = np.random.default_rng(0).standard_normal((1, 1, 8, 2))
    V = np.zeros((1, 1, 8, 2))
    for j, val in enumerate(g["value_of_block"]):
        V[0, 0, 4 * j:4 * j + 4, :] = val
    o, lse = oracle.attend_row(Q, K, V, prob, 0, np.array(g["blocks"], np.int32),
                               np.array(g["logw"]))
    np.testing.assert_allclose(o[0], g["expected_o"], rtol=1e-15)
    np.testing.assert_allclose(lse[0], g["expected_lse"], rtol=1e-15)
    o, lse = oracle.attend_row(Q, K, V, prob, 0, np.zeros(0, np.int32), np.zeros(0, np.float32))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _row_setup(n_blocks, seed, budget):
    rng = np.random.default_rng(seed)
    D = 8
    N = 4 * n_blocks
    prob = Problem(B=1, H=1, N=N, D=D, q_block=N)
    Q = rng.standard_normal((1, 1, N, D))
    K = rng.standard_normal((1, 1, N, D))
    V = rng.standard_normal((1, 1, N, D))
    s = np.exp(rng.standard_normal(n_blocks)).astype(np.float32)
    s /= s.sum()
    pi = oracle.inclusion_probabilities(s.astype(np.float32), budget)
    Od, Ld = oracle.dense(Q, K, V, prob)
    m_ref = Ld[0, 0]                 # any fixed shift works; use the dense LSE
    n_true = Od[0, 0]                # N/D with M* = LSE gives D = 1, N = o
    return prob, Q, K, V, s, pi, m_ref, n_true


@pytest.mark.parametrize("seed,n_blocks,budget", [(0, 10, 0.3), (1, 12, 0.2), (2, 8, 0.5)])
def test_ht_unbiased_exact_enumeration(seed, n_blocks, budget):
    prob, Q, K, V, s, pi, m_ref, n_true = _row_setup(n_blocks, seed, budget)
    lw_all = np.where(pi == 1.0, 0.0, -np.log(np.where(pi > 0, pi, 1.0)))
    EN = np.zeros_like(n_true)
    ED = np.zeros(Q.shape[2])
    total = 0.0
    for bits in itertools.product([0, 1], repeat=n_blocks):
        x = np.array(bits, dtype=bool)
        pr = np.prod(np.where(x, pi, 1.0 - pi))
        if pr == 0.0:
            continue
        total += pr
        cols = np.nonzero(x)[0].astype(np.int32)
        o, lse = oracle.attend_row(Q, K, V, prob, 0, cols, lw_all[cols])
        if cols.size == 0:
            continue
        nh, dh = oracle.ht_estimates(o, lse, m_ref)
        EN += pr * nh
        ED += pr * dh
    assert abs(total - 1.0) < 1e-12
    np.testing.assert_allclose(ED, 1.0, rtol=1e-11)
    np.testing.assert_allclose(EN, n_true, rtol=1e-10, atol=1e-12)


def test_ht_wrong_sign_is_biased():
    # the plausible sign mistake (shift -log(1/pi)) is caught by the same check
    prob, Q, K, V, s, pi, m_ref, n_true = _row_setup(8, 2, 0.5)
    lw_bad = np.where(pi == 1.0, 0.0, np.log(np.where(pi > 0, pi, 1.0)))
    ED = np.zeros(Q.shape[2])
    for bits in itertools.product([0, 1], repeat=8):
        x = np.array(bits, dtype=bool)
        pr = np.prod(np.where(x, pi, 1.0 - pi))
        cols = np.nonzero(x)[0].astype(np.int32)
        if pr == 0.0 or cols.size == 0:
            continue
        o, lse = oracle.attend_row(Q, K, V, prob, 0, cols, lw_bad[cols])
        ED += pr * oracle.ht_estimates(o, lse, m_ref)[1]
    assert np.max(np.abs(ED - 1.0)) > 1e-2


def test_ht_monte_carlo_on_tiny_workload():
    wl = Workload("t", B=1, H=1, D=64, grid=(1, 16, 16), dtype="f32", sigma=1.0)
    q, k, v = make_qkv(wl)
    prob = Problem(B=1, H=1, N=wl.N, D=64)
    sc = oracle.ibcs_scores(q, k, prob, rows=[0])
    Od, Ld = oracle.dense(q, k, v, prob)
    rows = slice(0, 128)
    m_ref = Ld[0, 0, rows]
    T = 1500
    nh_sum = np.zeros((128, 64))
    nh_sq = np.zeros((128, 64))
    dh_sum = np.zeros(128)
    dh_sq = np.zeros(128)
    for seed in range(T):
        p = oracle.plan_from_scores(sc["S32"], prob, 0.1, seed, rows=[0])
        o, lse = oracle.attend_row(q, k, v, prob, 0, *p.row(0))
        nh, dh = oracle.ht_estimates(o, lse, m_ref)
        nh_sum += nh
        nh_sq += nh ** 2
        dh_sum += dh
        dh_sq += dh ** 2
    mean_d = dh_sum / T
    se_d = np.sqrt(np.maximum(dh_sq / T - mean_d ** 2, 0) / T)
    zd = (mean_d - 1.0) / se_d
    mean_n = nh_sum / T
    se_n = np.sqrt(np.maximum(nh_sq / T - mean_n ** 2, 0) / T)
    zn = (mean_n - Od[0, 0, rows]) / np.maximum(se_n, 1e-12)
    # many rows are tested at once: allow the usual tail at 4.5 sigma
    assert np.mean(np.abs(zd) < 4.5) > 0.995 and np.max(np.abs(zd)) < 6
    assert np.mean(np.abs(zn) < 4.5) > 0.995 and np.max(np.abs(zn)) < 6.5
