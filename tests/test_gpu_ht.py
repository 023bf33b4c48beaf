"""The library's sampler and attention as a Horvitz-Thompson estimator.

news.hamidun.com, "AB-Attention speeds up video generation by up to 2.23x and
skips 92% of attention", section "AB-Attention's three techniques", SIP: each
block enters with probability pi (proportional to its score, capped at 1) and
is weighted by 1/pi, which estimates both the attention numerator and the
softmax normalisation without bias (the normalised output itself is not
unbiased, and nothing here assumes it is).

Over many seeds, with the plan and the attention both run by the library on
the GPU -- the fp32 path (D = 64) and the bf16 production path (D = 128: fp16
block scores, fp16 probabilities times fp16 V, bf16 output):
  * each block's inclusion frequency matches pi = exp(-logw) of the plan (the
    scores do not depend on the seed, so every kept copy of a block carries
    the same logw) -- a z-test per block;
  * the mean number of sampled blocks per row is m = budget * n_blocks;
  * with the dense log-sum-exp as the fixed reference shift M*, the estimates
    D_hat = exp(LSE - M*) and N_hat = o * D_hat average to the exact
    normaliser (1) and numerator (the dense output) within the Monte-Carlo
    standard error.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import lib_problem, oracle_problem, say, to_dev
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")


HT_CASES = {
    "f32_d64": Workload("ht", B=1, H=1, D=64, grid=(1, 16, 16), dtype="f32", sigma=1.0),
    "bf16_d128": Workload("ht16", B=1, H=1, D=128, grid=(1, 16, 16), dtype="bf16", sigma=1.0),
}


@pytest.mark.parametrize("case", list(HT_CASES))
def test_sip_law_and_ht_unbiasedness_on_gpu(case):
    wl = HT_CASES[case]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, wl.dtype) for x in (q, k, v))
    say(f"HT law on GPU: {case}")
    Od, Ld = oracle.dense(q, k, v, op)
    budget, T = 0.1, 3000
    n, R, nq = op.n_kbs, op.R, 128
    hits = np.zeros((R, n))
    lw_seen = np.full((R, n), np.nan)
    counts = np.zeros((T, R))
    nh_sum = np.zeros((R, nq, op.D))
    nh_sq = np.zeros_like(nh_sum)
    dh_sum = np.zeros((R, nq))
    dh_sq = np.zeros_like(dh_sum)
    for seed in range(T):
        pl = ab.plan(dq, dk, budget, seed=seed, problem=prob)
        o, lse = ab.attend(dq, dk, dv, pl, problem=prob, return_lse=True)
        rp = pl.row_ptr.cpu().numpy()
        nnz = int(rp[-1])
        ci = pl.col_idx[:nnz].cpu().numpy()
        lw = pl.logw[:nnz].cpu().numpy()
        o, lse = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        for r in range(R):
            c, w = ci[rp[r]:rp[r + 1]], lw[rp[r]:rp[r + 1]]
            hits[r, c] += 1
            seen = ~np.isnan(lw_seen[r, c])
            assert np.all(lw_seen[r, c][seen] == w[seen])    # one pi per block
            lw_seen[r, c] = w
            counts[seed, r] = len(c)
            lo = r * nq
            nh, dh = oracle.ht_estimates(o[0, 0, lo:lo + nq], lse[0, 0, lo:lo + nq],
                                         Ld[0, 0, lo:lo + nq])
            nh_sum[r] += nh
            nh_sq[r] += nh ** 2
            dh_sum[r] += dh
            dh_sq[r] += dh ** 2
    # inclusion frequencies against pi = exp(-logw), on blocks expected at
    # least 20 times (the normal approximation of the binomial holds there)
    drawn = ~np.isnan(lw_seen)
    pi = np.exp(-lw_seen[drawn].astype(np.float64))
    freq = hits[drawn] / T
    ok = pi * T >= 20
    z = (freq[ok] - pi[ok]) / np.sqrt(pi[ok] * (1 - pi[ok]) / T + 1e-300)
    z = np.where(pi[ok] >= 1.0, (freq[ok] - 1.0) * 1e6, z)      # certain blocks: every time
    say(f"HT on GPU: {int(ok.sum())} blocks tested, |z| max {np.abs(z).max():.2f}, "
        f"mean count {counts.mean():.3f} (m = {budget * n:.1f})")
    assert ok.sum() >= 20
    assert np.mean(np.abs(z) < 4.0) > 0.995 and np.abs(z).max() < 5.5
    m = budget * n
    se = counts.std() / np.sqrt(counts.size)
    assert abs(counts.mean() - m) < 4.5 * max(se, 1e-9)
    # unbiased numerator and normaliser
    mean_d = dh_sum / T
    se_d = np.sqrt(np.maximum(dh_sq / T - mean_d ** 2, 0) / T)
    zd = (mean_d - 1.0) / np.maximum(se_d, 1e-12)
    mean_n = nh_sum / T
    se_n = np.sqrt(np.maximum(nh_sq / T - mean_n ** 2, 0) / T)
    ref_n = Od[0, 0].reshape(R, nq, op.D)
    zn = (mean_n - ref_n) / np.maximum(se_n, 1e-12)
    say(f"HT on GPU: |z| normaliser max {np.abs(zd).max():.2f}, numerator max {np.abs(zn).max():.2f}")
    assert np.mean(np.abs(zd) < 4.5) > 0.995 and np.max(np.abs(zd)) < 6
    assert np.mean(np.abs(zn) < 4.5) > 0.995 and np.max(np.abs(zn)) < 6.5
