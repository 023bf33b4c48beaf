"""abatt_plan_noalloc (the plan with the library's static scratch as its
workspace) against abatt_plan with a caller workspace, through the C ABI:
the same plan bit for bit -- status, row_ptr, col_idx and logw -- on calls in
a row on one GPU, a larger problem first and a smaller one after it (the
scratch keeps the larger call's contents), then the larger one again."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import lib_problem, say, to_dev
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")

CASES = [
    # larger first: 3 heads, 5120 tokens + 64 text tokens, 16 clusters
    ("large", Workload("na_l", B=1, H=3, D=128, grid=(4, 32, 40), n_text=64, n_clusters=16), 0.10, 7),
    # smaller second: 1 head, 512 tokens, D = 64
    ("small", Workload("na_s", B=1, H=1, D=64, grid=(2, 16, 16)), 0.15, 11),
    # the larger one again after the smaller one
    ("large again", Workload("na_l", B=1, H=3, D=128, grid=(4, 32, 40), n_text=64, n_clusters=16), 0.10, 7),
]


def _garbage_plan(prob, capacity, dev):
    pl = ab.empty_plan(prob, capacity, dev)
    pl.row_ptr.fill_(-7)
    pl.col_idx.fill_(-7)
    pl.logw.fill_(-7.0)
    pl.status.fill_(5)
    return pl


def test_noalloc_equals_plan_in_a_row():
    dev = torch.device("cuda:0")
    lib = ab.load_library()
    for name, wl, budget, seed in CASES:
        prob = lib_problem(wl)
        assert ab.plan_workspace_bytes(prob) <= ab.SCRATCH_BYTES
        q, k, _ = make_qkv(wl)
        dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
        cap = ab.nnz_bound(prob, budget)
        ref = _garbage_plan(prob, cap, dev)
        got = _garbage_plan(prob, cap, dev)
        ws = ab.workspace(prob, dev)
        torch.cuda.synchronize()
        say(f"noalloc {name}: R={prob.R} n_kbs={prob.n_kbs} ws={ab.plan_workspace_bytes(prob)}")
        ab.plan(dq, dk, budget, seed=seed, problem=prob, ws=ws, out=ref)
        # straight through the C ABI with preallocated outputs: nothing allocates
        cp = got.c()
        code = lib.abatt_plan_noalloc(ctypes.byref(prob.c()), ctypes.c_void_p(dq.data_ptr()),
                                      ctypes.c_void_p(dk.data_ptr()), float(budget),
                                      ctypes.c_uint64(seed), ctypes.byref(cp),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert code == 0, code
        torch.cuda.synchronize()
        assert int(ref.status.item()) == 0 and int(got.status.item()) == 0
        assert torch.equal(got.row_ptr, ref.row_ptr)
        nnz = int(ref.row_ptr[-1].item())
        assert nnz > 0
        assert torch.equal(got.col_idx[:nnz], ref.col_idx[:nnz])
        assert torch.equal(got.logw[:nnz].view(torch.int32), ref.logw[:nnz].view(torch.int32))
        say(f"  {name}: nnz {nnz}, bit-identical")


def test_noalloc_binding_and_too_large():
    dev = torch.device("cuda:0")
    wl = Workload("na_b", B=1, H=2, D=128, grid=(2, 12, 16), n_text=16)
    prob = lib_problem(wl)
    q, k, _ = make_qkv(wl)
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    say("noalloc binding")
    a = ab.plan_noalloc(dq, dk, 0.2, seed=3, problem=prob)
    b = ab.plan(dq, dk, 0.2, seed=3, problem=prob)
    torch.cuda.synchronize()
    nnz = int(b.row_ptr[-1].item())
    assert torch.equal(a.row_ptr, b.row_ptr)
    assert torch.equal(a.col_idx[:nnz], b.col_idx[:nnz])
    assert np.array_equal(a.logw[:nnz].cpu().numpy().view(np.int32),
                          b.logw[:nnz].cpu().numpy().view(np.int32))
    # a problem whose plan workspace exceeds the scratch is refused before any launch
    big = ab.Problem(B=1, H=40, N=75600, D=128)
    assert ab.plan_workspace_bytes(big) > ab.SCRATCH_BYTES
    out = ab.empty_plan(ab.Problem(B=1, H=2, N=1024, D=128), 16, dev)
    with pytest.raises(ab.AbattError) as ei:
        cp = ab._Plan(out.row_ptr.data_ptr(), out.col_idx.data_ptr(), out.logw.data_ptr(),
                      10 ** 9, out.status.data_ptr())
        ab._check(ab.load_library().abatt_plan_noalloc(
            ctypes.byref(big.c()), ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()),
            0.1, ctypes.c_uint64(0), ctypes.byref(cp), None))
    assert ei.value.code == ab.ABATT_ESCRATCH
