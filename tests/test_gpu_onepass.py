"""abatt_plan_onepass (count, scan and fill in one kernel, rows ordered by
tickets and chained by decoupled look-back) against abatt_plan (three
kernels), through the binding: the same plan bit for bit -- status, row_ptr,
col_idx and the bits of logw -- on small and ragged shapes, text tokens,
key-block sizes from 4 to 128, budget 1, long rows (18 944 to 40 000 key
blocks, with the mask words of a pass up to the LDS list's limit), many rows
(long look-back chains) and a capacity overflow (same status, same row_ptr).
One small case also checks the one-pass plan against the oracle's (block
agreement, as for abatt_plan)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import jaccard, lib_problem, oracle_problem, plan_to_host, say, to_dev
from workloads import CONFIGS, Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")

CASES = {
    "tiny_f32": (CONFIGS["tiny"], 0.1),
    "bf16_ragged": (Workload("r", B=1, H=2, D=128, grid=(3, 10, 12)), 0.12),
    "bf16_text_c16": (Workload("x", B=1, H=2, D=128, grid=(2, 8, 16), n_text=16,
                               n_clusters=16), 0.2),
    "bf16_d64_b2": (Workload("b", B=2, H=2, D=64, grid=(2, 12, 16)), 0.05),
    "bf16_kv16": (Workload("k16", B=1, H=2, D=128, grid=(4, 16, 16), kv_block=16), 0.3),
    "bf16_kv128_text": (Workload("k128", B=1, H=1, D=64, grid=(4, 16, 16), n_text=128,
                                 kv_block=128), 0.5),
    "bf16_all": (Workload("m", B=1, H=2, D=128, grid=(6, 16, 24)), 1.0),
    # long rows, read in place by both samplers: 18 944 and 18 948 key blocks
    # (two passes of the LDS list, the second one short)
    "bf16_row_18944": (Workload("L", B=1, H=1, D=64, grid=(1, 4, 18944)), 0.1),
    "bf16_row_18948": (Workload("P", B=1, H=1, D=64, grid=(1, 4, 18948)), 0.1),
    # 40 000 key blocks: 1250 mask words, three passes of the LDS list
    "bf16_row_global": (Workload("G", B=1, H=1, D=64, grid=(20, 40, 200)), 0.1),
    # many rows (12 heads x 256 query blocks): look-back over long chains
    "bf16_many_rows": (Workload("M", B=1, H=12, D=64, grid=(8, 64, 64)), 0.08),
}


def same_plan(a, b):
    assert int(a.status.item()) == int(b.status.item())
    assert torch.equal(a.row_ptr, b.row_ptr)


@pytest.mark.parametrize("name", list(CASES))
def test_onepass_equals_plan(name):
    wl, budget = CASES[name]
    prob = lib_problem(wl)
    q, k, _ = make_qkv(wl)
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    say(f"onepass {name}: R={prob.R} n_kbs={prob.n_kbs} budget {budget}")
    ref = ab.plan(dq, dk, budget, seed=5, problem=prob)
    got = ab.plan_onepass(dq, dk, budget, seed=5, problem=prob)
    again = ab.plan_onepass(dq, dk, budget, seed=5, problem=prob)
    torch.cuda.synchronize()
    assert ref.ok() and got.ok() and again.ok()
    same_plan(got, ref)
    nnz = ref.nnz()
    assert nnz > 0
    assert torch.equal(got.col_idx[:nnz], ref.col_idx[:nnz])
    assert torch.equal(got.logw[:nnz].view(torch.int32), ref.logw[:nnz].view(torch.int32))
    assert torch.equal(again.row_ptr, ref.row_ptr)
    assert torch.equal(again.col_idx[:nnz], ref.col_idx[:nnz])
    say(f"  {name}: nnz {nnz}, bit-identical")


def test_onepass_against_oracle():
    wl = CASES["bf16_ragged"][0]
    q, k, _ = make_qkv(wl)
    op = oracle_problem(wl)
    ref = oracle.plan(q, k, op, 0.12, seed=3)
    prob = lib_problem(wl)
    pl = ab.plan_onepass(to_dev(q, wl.dtype), to_dev(k, wl.dtype), 0.12, seed=3, problem=prob)
    torch.cuda.synchronize()
    assert pl.ok()
    rp, ci, _ = plan_to_host(pl)
    jac = jaccard(rp, ci, ref.row_ptr, ref.col_idx)
    say(f"onepass vs oracle: jaccard {jac:.5f}")
    assert jac >= 0.99
    nf = op.n_kb - op.n_kbs
    for r in range(op.R):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
        if nf:
            np.testing.assert_array_equal(row[-nf:], np.arange(op.n_kbs, op.n_kb))


@pytest.mark.parametrize("cap_frac", [0.0, 0.5])
def test_onepass_overflow(cap_frac):
    # capacity below the total: status 1 and row_ptr (the total needed in
    # row_ptr[R]) as abatt_plan reports them; rows that fit hold their entries
    wl = CASES["bf16_text_c16"][0]
    prob = lib_problem(wl)
    q, k, _ = make_qkv(wl)
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    full = ab.plan(dq, dk, 0.2, seed=9, problem=prob)
    torch.cuda.synchronize()
    total = full.nnz()
    nf = prob.n_kb - prob.n_kbs
    cap = max(int(total * cap_frac), prob.R * nf)
    say(f"onepass overflow: total {total} capacity {cap}")
    ref = ab.plan(dq, dk, 0.2, seed=9, problem=prob, capacity=cap)
    got = ab.plan_onepass(dq, dk, 0.2, seed=9, problem=prob, capacity=cap)
    torch.cuda.synchronize()
    assert not ref.ok() and not got.ok()
    same_plan(got, ref)
    assert got.nnz() == total
    rp = got.row_ptr.cpu().numpy()
    fit = int(np.searchsorted(rp[1:], cap, side="right"))   # rows r with rp[r+1] <= cap
    end = int(rp[fit])
    assert torch.equal(got.col_idx[:end], full.col_idx[:end])
    assert torch.equal(got.logw[:end], full.logw[:end])
