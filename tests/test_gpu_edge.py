"""GPU parity at the edges of the supported shapes.

* sequences of a single key block (N = 4) and single partial query blocks,
  bf16 (D = 128) and fp32 (D = 64), 8 and 16 clusters;
* last query blocks with fewer queries than clusters: k-means starts from
  duplicated members, so ties go to the lower index and the duplicates stay
  empty (they keep their centroid) -- weights must match exactly;
* budgets that expect less than one block per row: most rows are empty
  (output 0, log-sum-exp -inf);
* a long head, N = 2^21: offsets into the [rows, blocks] score matrix pass
  2^31 and the sampler reads its rows from global memory; plan and attention
  are checked on sampled rows.
Bars as elsewhere: tiny plans select the oracle's blocks exactly (scores
agree to ~1e-6, so a flip would need a uniform within that of pi) with
log-weights within 1e-5; the long plan
>= 99% block agreement; attention bf16 max-abs 1e-2 / mean-rel 1e-3, fp32
1e-4, against the oracle run on the same plan.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (LSE_TOL, check_output, errors, jaccard, lib_problem, oracle_problem,
                     plan_to_host, round_ref, say, to_dev)
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")

# logw = -log(pi) with pi = c * s_j: these plans use the GPU's own scores, and
# a relative score error e moves logw by about e in absolute terms, once
# through s_j and once through the water-filling constant c (a ratio of the
# row's scores).  So logw's bar is twice the scores' relative bar: 2e-3 for
# bf16 problems (fp16 operands), ~5e-6 for fp32 problems (split-bf16)
LOGW_ATOL = {"bf16": 4e-3, "f32": 1e-5}


def _plan_and_attend(wl, budget, seed=0):
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    ref = oracle.plan(q, k, op, budget, seed)
    O, L = oracle.attend(q, k, v, ref, op)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, wl.dtype) for x in (q, k, v))
    pl = ab.plan(dq, dk, budget, seed=seed, problem=prob)
    o, lse = ab.attend(dq, dk, dv, pl, problem=prob, return_lse=True)
    torch.cuda.synchronize()
    assert pl.ok()
    return (q, k, v), op, ref, (O, L), pl, (o, lse), prob, (dq, dk)


@pytest.mark.parametrize("N", [4, 8, 132, 260])
@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 8), ("bf16", 128, 16), ("f32", 64, 8)])
def test_tiny_sequences(N, dtype, D, C):
    wl = Workload("t", B=1, H=2, D=D, grid=(1, 1, N), dtype=dtype, sigma=1.0, n_clusters=C)
    say(f"tiny N={N} {dtype} D={D} C={C}")
    _, op, ref, (O, L), pl, (o, lse), _, _ = _plan_and_attend(wl, 0.5)
    rp, ci, lw = plan_to_host(pl)
    np.testing.assert_array_equal(rp, ref.row_ptr)
    np.testing.assert_array_equal(ci, ref.col_idx)
    np.testing.assert_allclose(lw, ref.logw, rtol=0, atol=LOGW_ATOL[dtype])
    check_output(o, O, dtype, f"tiny N={N} {dtype} C={C}")
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    assert np.abs(lse.cpu().numpy()[fin] - L[fin]).max(initial=0.0) <= LSE_TOL[dtype]


@pytest.mark.parametrize("C", [8, 16])
def test_kmeans_fewer_queries_than_clusters(C):
    # the last query block holds 4 queries: centroids start at members
    # floor(c*4/C), i.e. each member C/4 times
    wl = Workload("k", B=1, H=2, D=128, grid=(1, 1, 256 + 4), n_clusters=C)
    q, k, _ = make_qkv(wl)
    op = oracle_problem(wl)
    sc = oracle.ibcs_scores(q, k, op)
    S, mu, w = ab.scores(to_dev(q, "bf16"), to_dev(k, "bf16"), lib_problem(wl))
    torch.cuda.synchronize()
    w, mu, S = w.cpu().numpy(), mu.cpu().numpy(), S.cpu().numpy()
    last = [op.n_qb - 1, 2 * op.n_qb - 1]
    say(f"k-means C={C}: last-block weights {w[last[0]]}")
    # full blocks: as in the selector tests (an fp32/fp64 near tie may split a
    # block); the 4-query blocks have no near ties and must match exactly
    same = np.all(np.abs(w - sc["w"]) <= 1e-6, axis=1)
    assert all(same[r] for r in last)
    np.testing.assert_allclose(mu[same], sc["mu"][same], rtol=1e-5, atol=1e-6)
    for r in last:  # duplicated starts: only the lowest copy of each member is used
        assert np.count_nonzero(w[r]) == 4
        np.testing.assert_allclose(w[r][w[r] > 0], 0.25, rtol=0, atol=0)
    rel = np.abs(S[same] - sc["S"][same]) / sc["S"][same]
    assert rel.max() <= 2e-3 and rel.mean() <= 2e-4


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_budget_below_one_block(dtype, D):
    wl = Workload("z", B=1, H=4, D=D, grid=(2, 16, 16), dtype=dtype, sigma=1.0)
    budget = 0.004  # 128 sparse blocks per row: m = 0.512 expected blocks
    say(f"budget {budget} {dtype}")
    _, op, ref, (O, L), pl, (o, lse), _, _ = _plan_and_attend(wl, budget, seed=5)
    rp, ci, lw = plan_to_host(pl)
    np.testing.assert_array_equal(rp, ref.row_ptr)
    np.testing.assert_array_equal(ci, ref.col_idx)
    np.testing.assert_allclose(lw, ref.logw, rtol=0, atol=LOGW_ATOL[dtype])
    empty = np.diff(ref.row_ptr) == 0
    say(f"  {int(empty.sum())} of {len(empty)} rows empty")
    assert empty.any() and not empty.all()
    check_output(o, O, dtype, f"budget {budget} {dtype}")
    lse_h = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(lse_h), np.isfinite(L))
    o_h = o.float().cpu().numpy()
    for r in np.nonzero(empty)[0]:
        b, h, qb = oracle.unflatten_row(op, int(r))
        lo, hi = qb * 128, min((qb + 1) * 128, wl.N)
        assert np.all(o_h[b, h, lo:hi] == 0) and np.all(np.isneginf(lse_h[b, h, lo:hi]))


def test_long_sequence():
    wl = Workload("long", B=1, H=1, D=128, grid=(32, 256, 256))  # N = 2^21
    budget = 0.01
    say(f"long N={wl.N}: generating inputs")
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    say(f"long N={wl.N}: plan (score matrix {op.R * op.n_kbs * 4 / 2**30:.1f} GiB) + attend")
    pl = ab.plan(dq, dk, budget, seed=11, problem=prob)
    o = ab.attend(dq, dk, dv, pl, problem=prob)
    torch.cuda.synchronize()
    assert pl.ok()
    del dq, dk, dv
    rows = [0, 1, 7777, op.R - 2, op.R - 1]
    ref = oracle.plan(q, k, op, budget, 11, rows=rows)
    rp = pl.row_ptr.cpu().numpy().astype(np.int64)
    g_ci = [pl.col_idx[rp[r]:rp[r + 1]].cpu().numpy() for r in rows]
    g_lw = [pl.logw[rp[r]:rp[r + 1]].cpu().numpy() for r in rows]
    g_rp = np.cumsum([0] + [len(c) for c in g_ci])
    jac = jaccard(g_rp, np.concatenate(g_ci), ref.row_ptr, ref.col_idx)
    say(f"long: rows {rows} plan jaccard {jac:.5f}, nnz {int(rp[-1])}")
    assert jac >= 0.99
    got, want = [], []
    for r, c, lw in zip(rows, g_ci, g_lw):
        orow, _ = oracle.attend_row(q, k, v, op, r, c, lw)
        b, h, qb = oracle.unflatten_row(op, r)
        lo = qb * 128
        got.append(o[b, h, lo:lo + orow.shape[0]].float().cpu().numpy().astype(np.float64))
        want.append(orow)
    mx, mr = errors(np.concatenate(got), round_ref(np.concatenate(want), "bf16"))
    say(f"long: attend rows max-abs {mx:.3e} mean-rel {mr:.3e}")
    assert mx <= 1e-2 and mr <= 1e-3
