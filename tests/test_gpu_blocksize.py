"""GPU parity at key/value block sizes other than 4 tokens.

The pages fix the key block at 4 tokens and compare it with 128-token blocks
(news.hamidun.com, "AB-Attention's three techniques", third technique); the
library takes any power of two from 4 to 128.  Per block size, against the
oracle (which is written for any block size): key means (fp32 sums of kb rows
against float64), the sampler fed the oracle's scores (indices bit-exact,
logw within 1 fp32 ulp), the plan end to end (>= 99% block agreement, forced
text blocks in every row), and attention on the library's plan (bf16 max-abs
1e-2 / mean-rel 1e-3, fp32 1e-4; log-sum-exp as elsewhere).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (LSE_TOL, check_output, jaccard, lib_problem, oracle_problem, plan_to_host,
                     say, to_dev, ulp_diff_f32)
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")

CASES = {
    "bf16_kb8": Workload("k8", B=1, H=2, D=128, grid=(2, 16, 32), kv_block=8),
    "bf16_kb16_text": Workload("k16", B=1, H=2, D=128, grid=(2, 16, 32), n_text=64, kv_block=16),
    "bf16_kb64": Workload("k64", B=1, H=2, D=128, grid=(4, 16, 48), kv_block=64),
    "bf16_kb128_text": Workload("k128", B=1, H=2, D=128, grid=(8, 16, 32), n_text=128,
                                kv_block=128),
    "bf16_d64_kb32": Workload("d64", B=2, H=1, D=64, grid=(2, 16, 32), kv_block=32),
    "f32_kb8": Workload("f8", B=1, H=2, D=64, grid=(2, 16, 32), dtype="f32", sigma=1.0,
                        kv_block=8),
    "f32_kb128": Workload("f128", B=1, H=1, D=64, grid=(8, 16, 32), dtype="f32", sigma=1.0,
                          kv_block=128),
}
BUDGET = 0.12


@pytest.mark.parametrize("name", list(CASES))
def test_key_means_block_sizes(name):
    wl = CASES[name]
    _, k, _ = make_qkv(wl)
    op = oracle_problem(wl)
    say(f"key means {name} kb={wl.kv_block}")
    got = ab.key_means(to_dev(k, wl.dtype), lib_problem(wl))
    torch.cuda.synchronize()
    # fp32 sum of kb values in token order: error below kb fp32 ulps of the largest |k|
    atol = wl.kv_block * 2.0 ** -24 * float(np.abs(k).max())
    np.testing.assert_allclose(got.cpu().numpy(), oracle.key_block_means(k, op), rtol=2e-6,
                               atol=atol)


@pytest.mark.parametrize("name", list(CASES))
def test_sampler_from_oracle_scores_block_sizes(name):
    wl = CASES[name]
    q, k, _ = make_qkv(wl)
    op = oracle_problem(wl)
    S32 = oracle.ibcs_scores(q, k, op)["S32"]
    ref = oracle.plan_from_scores(S32, op, BUDGET, seed=17)
    say(f"sampler {name}: n_kbs={op.n_kbs} n_kb={op.n_kb}")
    pl = ab.plan_from_scores(torch.from_numpy(np.ascontiguousarray(S32)).cuda(), BUDGET, 17,
                             lib_problem(wl))
    torch.cuda.synchronize()
    assert pl.ok()
    rp, ci, lw = plan_to_host(pl)
    np.testing.assert_array_equal(rp, ref.row_ptr)
    np.testing.assert_array_equal(ci, ref.col_idx)
    assert ulp_diff_f32(lw, ref.logw).max(initial=0) <= 1


@pytest.mark.parametrize("name", list(CASES))
def test_plan_and_attend_block_sizes(name):
    wl = CASES[name]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    ref = oracle.plan(q, k, op, BUDGET, seed=3)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, wl.dtype) for x in (q, k, v))
    pl = ab.plan(dq, dk, BUDGET, seed=3, problem=prob)
    o, lse = ab.attend(dq, dk, dv, pl, problem=prob, return_lse=True)
    torch.cuda.synchronize()
    assert pl.ok()
    rp, ci, lw = plan_to_host(pl)
    jac = jaccard(rp, ci, ref.row_ptr, ref.col_idx)
    say(f"plan {name}: kb={wl.kv_block} jaccard {jac:.5f} nnz {len(ci)}")
    assert jac >= 0.99
    nf = op.n_kb - op.n_kbs
    for r in range(op.R):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
        if nf:
            np.testing.assert_array_equal(row[-nf:], np.arange(op.n_kbs, op.n_kb))
    # attention against the oracle run on the library's own plan
    O, L = oracle.attend(q, k, v, oracle.Plan(rp.astype(np.int64), ci, lw), op)
    check_output(o, O, wl.dtype, f"attend {name}")
    lse_h = lse.cpu().numpy()
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lse_h), fin)
    assert np.abs(lse_h[fin] - L[fin]).max(initial=0.0) <= LSE_TOL[wl.dtype]


@pytest.mark.parametrize("kb,D", [(16, 128), (128, 128), (4, 64), (64, 64)])
def test_budget_one_is_dense_block_sizes(kb, D):
    # every key block of the head, the last rows included, through both gather
    # forms (one 4-key group per wave-wide load at D = 128, two at D = 64)
    wl = Workload("one", B=1, H=1, D=D, grid=(2, 16, 32), kv_block=kb)
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    Od, _ = oracle.dense(q, k, v, op)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    pl = ab.plan(dq, dk, 1.0, seed=0, problem=prob)
    o = ab.attend(dq, dk, dv, pl, problem=prob)
    torch.cuda.synchronize()
    assert pl.nnz() == op.R * op.n_kb
    check_output(o, Od, "bf16", f"budget 1, kb={kb}, D={D}")


def test_dense_ignores_block_size():
    # dense attention runs over every key: the problem's key-block size (here
    # one that does not divide N) changes nothing
    rng = np.random.default_rng(7)
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 2, 1000, 128)).astype(np.float32))
               .to(torch.bfloat16).cuda() for _ in range(3))
    ref = ab.dense(q, k, v, problem=ab.Problem(1, 2, 1000, 128))
    got = ab.dense(q, k, v, problem=ab.Problem(1, 2, 1000, 128, kv_block=128))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
