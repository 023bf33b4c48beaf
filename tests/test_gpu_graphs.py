"""The library under HIP graph capture and on concurrent streams.

Every entry point only enqueues kernels on the caller's stream (no memsets,
copies, allocations or synchronisations; outside capture the plan's key
means run on the library's side stream, forked from the caller's stream and
joined back to it), so a plan + attend sequence (also with the V conversion of the fp16-V
form) can be captured once and replayed, and calls on different streams with
their own workspaces and plans do not interfere.  Checked bit for bit against eager
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


_FRESH = r"""
import torch
import block_sparse_attention_09_amd as ab
from helpers import lib_problem, to_dev
from workloads import Workload, make_qkv

wl = Workload("g", B=1, H=2, D=128, grid=(3, 16, 32), dtype="bf16", seed=5, n_text=64)
q, k, v = (to_dev(x, "bf16") for x in make_qkv(wl))
prob = lib_problem(wl)
budget, seed = 0.15, 3
# load the plan's kernels without making the side stream (noalloc never does)
ab.plan_noalloc(q, k, budget, seed=seed, problem=prob)
torch.cuda.synchronize()
ws = ab.workspace(prob, q.device)
pl = ab.empty_plan(prob, ab.nnz_bound(prob, budget), q.device)
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # under capture the plan runs on the captured stream alone
    ab.plan(q, k, budget, seed=seed, problem=prob, ws=ws, out=pl)
g.replay()
torch.cuda.synchronize()
ref = ab.plan(q, k, budget, seed=seed, problem=prob)  # eager: makes the side stream
torch.cuda.synchronize()
n = ref.nnz()
for rep in range(2):
    assert torch.equal(pl.row_ptr, ref.row_ptr), rep
    assert torch.equal(pl.col_idx[:n], ref.col_idx[:n]), rep
    assert torch.equal(pl.logw[:n], ref.logw[:n]), rep
    pl.col_idx.fill_(-1)
    g.replay()
    torch.cuda.synchronize()
print("fresh-process capture ok", n)
"""


def test_plan_captured_before_side_stream():
    """A plan captured as the first plan call of a process, before the library
    has made its side stream (captured plans never use it): its replays
    equal eager plans made afterwards, with the side stream."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([os.path.dirname(here), here, env.get("PYTHONPATH", "")])
    say("fresh process: plan captured before the side stream exists")
    r = subprocess.run([sys.executable, "-c", _FRESH], env=env, capture_output=True, text=True,
                       timeout=110)
    say(r.stdout.strip()[-300:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "fresh-process capture ok" in r.stdout


def test_plans_from_host_threads():
    """Plan calls from several host threads at once, each on its own stream
    with its own workspace and plan (the library orders the forks onto its
    side stream with a lock): every plan equals the sequential one."""
    import threading
    wl, (q, k, v) = _inputs(6)
    prob = lib_problem(wl)
    budgets = [0.1, 0.15, 0.2, 0.3]
    refs = [ab.plan(q, k, b, seed=i, problem=prob) for i, b in enumerate(budgets)]
    torch.cuda.synchronize()
    outs, errs = {}, []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                ws = ab.workspace(prob, q.device)
                pl = ab.empty_plan(prob, ab.nnz_bound(prob, budgets[i]), q.device)
                for _ in range(3):
                    ab.plan(q, k, budgets[i], seed=i, problem=prob, ws=ws, out=pl)
            st.synchronize()
            outs[i] = pl
        except Exception as e:  # reported below, on the main thread
            errs.append(repr(e))

    ths = [threading.Thread(target=work, args=(i,)) for i in range(len(budgets))]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i, ref in enumerate(refs):
        n = ref.nnz()
        assert torch.equal(outs[i].row_ptr, ref.row_ptr), i
        assert torch.equal(outs[i].col_idx[:n], ref.col_idx[:n]), i
        assert torch.equal(outs[i].logw[:n], ref.logw[:n]), i
    say("host threads: every plan equals the sequential one")


def test_eager_plans_beside_a_capture():
    """One thread captures a plan while another runs eager plans on its own
    stream: captured plans never touch the side stream, so the eager plans
    run (and come out right) and the graph replays the captured plan."""
    import threading
    wl, (q, k, v) = _inputs(7)
    prob = lib_problem(wl)
    ref_a = ab.plan(q, k, 0.15, seed=3, problem=prob)
    ref_b = ab.plan(q, k, 0.2, seed=4, problem=prob)
    torch.cuda.synchronize()
    ws_a, ws_b = ab.workspace(prob, q.device), ab.workspace(prob, q.device)
    pl_a = ab.empty_plan(prob, ab.nnz_bound(prob, 0.15), q.device)
    pl_b = ab.empty_plan(prob, ab.nnz_bound(prob, 0.2), q.device)
    sb = torch.cuda.Stream()
    torch.cuda.synchronize()
    errs = []

    def other():
        try:
            with torch.cuda.stream(sb):
                for _ in range(3):
                    ab.plan(q, k, 0.2, seed=4, problem=prob, ws=ws_b, out=pl_b)
            sb.synchronize()
        except Exception as e:  # reported below, on the main thread
            errs.append(repr(e))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        th = threading.Thread(target=other)
        th.start()
        ab.plan(q, k, 0.15, seed=3, problem=prob, ws=ws_a, out=pl_a)
        th.join()
    assert not errs, errs
    for rep in range(2):
        pl_a.col_idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for pl, ref in ((pl_a, ref_a), (pl_b, ref_b)):
            n = ref.nnz()
            assert torch.equal(pl.row_ptr, ref.row_ptr), rep
            assert torch.equal(pl.col_idx[:n], ref.col_idx[:n]), rep
            assert torch.equal(pl.logw[:n], ref.logw[:n]), rep
    say("eager plans beside a capture: both right")
