"""The library under HIP graph capture and on concurrent streams.

Every entry point only enqueues kernels on the caller's stream (no memsets,
copies, allocations or synchronisations), so a plan + attend sequence (also
with the V conversion of the fp16-V form) can be captured once and replayed,
and calls on different streams with their own
workspaces and plans do not interfere.  Checked bit for bit against eager
calls: several replays with eager work and synchronisations between them, and
two streams (default priority) working at once.
"""
import pytest
import torch

from helpers import lib_problem, say, to_dev
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")


def _inputs(seed, dtype="bf16", D=128):
    wl = Workload("g", B=1, H=2, D=D, grid=(3, 16, 32), dtype=dtype, seed=seed, n_text=64)
    q, k, v = make_qkv(wl)
    return wl, [to_dev(x, dtype) for x in (q, k, v)]


def _eager(prob, q, k, v, budget, seed):
    pl = ab.plan(q, k, budget, seed=seed, problem=prob)
    o, lse = ab.attend(q, k, v, pl, problem=prob, return_lse=True)
    torch.cuda.synchronize()
    return pl, o, lse


@pytest.mark.parametrize("dtype,D,v16", [("bf16", 128, False), ("bf16", 128, True), ("f32", 64, False)])
def test_plan_attend_graph_replays(dtype, D, v16):
    wl, (q, k, v) = _inputs(1, dtype, D)
    prob = lib_problem(wl)
    budget, seed = 0.15, 9
    ref_pl, ref_o, ref_lse = _eager(prob, q, k, v, budget, seed)
    n = ref_pl.nnz()

    # buffers the graph reads and writes, allocated before capture
    qs, ks, vs = q.clone(), k.clone(), v.clone()
    ws = ab.workspace(prob, q.device)
    pl = ab.empty_plan(prob, ab.nnz_bound(prob, budget), q.device)
    o = torch.empty_like(q)
    vh = torch.empty(v.shape, dtype=torch.float16, device=v.device) if v16 else None

    def body(**kw):
        ab.plan(qs, ks, budget, seed=seed, problem=prob, ws=ws, out=pl)
        va = ab.v_to_f16(vs, prob, out=vh) if v16 else vs     # fp16-V form: same results
        return ab.attend(qs, ks, va, pl, problem=prob, out=o, **kw)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the binding's code paths off the graph
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        # the log-sum-exp tensor is allocated inside the capture (graph pool)
        _, lse_buf = body(return_lse=True)

    other_wl, (q2, k2, v2) = _inputs(2, dtype, D)
    for rep in range(4):
        # eager work between replays, on other data and on the graph's buffers
        o.zero_()
        pl.col_idx.fill_(-1)
        ab.attend(q2, k2, v2, ab.plan(q2, k2, 0.3, seed=rep, problem=prob), problem=prob)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph {dtype}{' v16' if v16 else ''} replay {rep}: nnz {pl.nnz()}")
        assert torch.equal(pl.row_ptr, ref_pl.row_ptr)
        assert torch.equal(pl.col_idx[:n], ref_pl.col_idx[:n])
        assert torch.equal(pl.logw[:n], ref_pl.logw[:n])
        assert torch.equal(o, ref_o)
        assert torch.equal(lse_buf, ref_lse)

    # new inputs copied into the captured buffers: the replay follows them
    qs.copy_(q2)
    ks.copy_(k2)
    vs.copy_(v2)
    ref2_pl, ref2_o, _ = _eager(prob, q2, k2, v2, budget, seed)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(pl.row_ptr, ref2_pl.row_ptr)
    assert torch.equal(o, ref2_o)


def test_two_streams_at_once():
    wl_a, (qa, ka, va) = _inputs(3)
    wl_b, (qb, kb, vb) = _inputs(4)
    prob = lib_problem(wl_a)
    ref_a = _eager(prob, qa, ka, va, 0.1, 1)
    ref_b = _eager(prob, qb, kb, vb, 0.2, 2)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(sa):
            pa = ab.plan(qa, ka, 0.1, seed=1, problem=prob)
            oa = ab.attend(qa, ka, va, pa, problem=prob)
        with torch.cuda.stream(sb):
            pb = ab.plan(qb, kb, 0.2, seed=2, problem=prob)
            ob = ab.attend(qb, kb, vb, pb, problem=prob)
        torch.cuda.synchronize()
        outs[rep] = (pa, oa, pb, ob)
    for rep, (pa, oa, pb, ob) in outs.items():
        for (pl, o), (rpl, ro, _) in (((pa, oa), ref_a), ((pb, ob), ref_b)):
            n = rpl.nnz()
            assert torch.equal(pl.row_ptr, rpl.row_ptr)
            assert torch.equal(pl.col_idx[:n], rpl.col_idx[:n])
            assert torch.equal(o, ro)
    say("two streams: identical to sequential calls")
