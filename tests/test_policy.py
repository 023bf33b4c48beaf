"""Step policy (dense steps and blocks, plan every four steps, fresh seeds):
host logic on the CPU, the attention callable on the GPU.

Pins: the schedule the pages describe (news.hamidun.com, "AB-Attention speeds
up video generation by up to 2.23x and skips 92% of attention": the plan is
rebuilt every four denoising steps, section "AB-Attention's three techniques";
dense attention in block 0 at every step and in steps 0-9 of 50, section "How it was
measured and what came out"), counted by hand for a 50-step, 40-block run;
SplitMix64 against its published first outputs for state 0 (Steele et al.,
OOPSLA 2014; the sequence of Vigna's reference generator seeded with 0).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_09_amd.policy import (BUILD, DENSE, REUSE, ABAttention, StepPolicy,
                                                  splitmix64)


def test_splitmix64_known_answers():
    # consecutive outputs of the generator seeded with 0: state advances by
    # the golden-ratio increment before each output
    g = 0x9E3779B97F4A7C15
    assert splitmix64(0) == 0xE220A8397B1DCDAF
    assert splitmix64(g) == 0x6E789E6AA1B965F4
    assert splitmix64(2 * g % (1 << 64)) == 0x06C45D188009454F


def test_schedule_of_a_50_step_run():
    p = StepPolicy()
    for s in range(10):
        assert all(p.mode(s, b) == DENSE for b in range(40))
    for s in range(50):
        assert p.mode(s, 0) == DENSE
    builds = [s for s in range(50) if p.mode(s, 7) == BUILD]
    assert builds == list(range(10, 50, 4))
    assert all(p.mode(s, 7) == REUSE for s in range(10, 50) if s not in builds)
    # 10 dense steps x 40 blocks + 40 later steps of block 0; 39 blocks x 10
    # plans; the rest reuse
    assert p.counts(40) == {DENSE: 440, BUILD: 390, REUSE: 1170}


def test_seeds_fresh_per_plan_and_block():
    p = StepPolicy(base_seed=5)
    seeds = {}
    for b in range(1, 12):
        for s in range(10, 50):
            seeds.setdefault((b, p.plan_index(s)), set()).add(p.seed(s, b))
    assert all(len(v) == 1 for v in seeds.values())          # one seed per plan
    flat = [next(iter(v)) for v in seeds.values()]
    assert len(set(flat)) == len(flat)                        # all plans distinct
    assert StepPolicy(base_seed=6).seed(10, 1) != p.seed(10, 1)


def test_policy_argument_checks():
    with pytest.raises(ValueError):
        StepPolicy(plan_every=0)
    with pytest.raises(ValueError):
        StepPolicy(budget=0.0)
    with pytest.raises(ValueError):
        StepPolicy().mode(-1, 0)
    with pytest.raises(ValueError):
        ABAttention(n_text=6)


@pytest.mark.gpu
def test_attention_callable_in_a_denoising_loop():
    import block_sparse_attention_09_amd as ab
    import oracle
    from helpers import check_output, oracle_problem, say, to_dev
    from workloads import Workload, make_qkv

    wl = Workload("loop", B=1, H=2, D=128, grid=(2, 8, 16), n_text=16)
    pol = StepPolicy(total_steps=12, dense_steps=2, dense_blocks=1, plan_every=4, budget=0.2,
                     base_seed=3)
    attn = ABAttention(pol, n_text=wl.n_text)
    n_blocks = 3
    plans = {}
    for step in range(pol.total_steps):
        attn.set_step(step)
        for blk in range(n_blocks):
            q, k, v = make_qkv(wl.scaled(seed=100 * step + blk))
            dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
            o = attn(dq, dk, dv, blk)
            mode = pol.mode(step, blk)
            assert attn.log[-1] == (step, blk, mode)
            prob = attn.problem(dq)
            if mode == DENSE:
                ref = ab.dense(dq, dk, dv, problem=prob)
            else:
                pl = attn.plan_of(blk)
                if mode == BUILD:
                    # the callable's plan is the library's plan for this seed
                    own = ab.plan(dq, dk, pol.budget, seed=pol.seed(step, blk), problem=prob)
                    n = own.nnz()
                    assert pl.nnz() == n
                    assert torch.equal(pl.row_ptr, own.row_ptr)
                    assert torch.equal(pl.col_idx[:n], own.col_idx[:n])
                    assert torch.equal(pl.logw[:n], own.logw[:n])
                    plans[(blk, pol.plan_index(step))] = pl.col_idx[:n].clone()
                else:
                    # reused: the same plan object as the build step of this window
                    assert torch.equal(pl.col_idx[:pl.nnz()], plans[(blk, pol.plan_index(step))])
                ref = ab.attend(dq, dk, dv, pl, problem=prob)
                # text key blocks (the last n_text/4) are in every row
                rp = pl.row_ptr.cpu().numpy()
                ci = pl.col_idx.cpu().numpy()
                forced = set(range(prob.n_kbs, prob.n_kb))
                for r in range(prob.R):
                    assert forced <= set(ci[rp[r]:rp[r + 1]].tolist())
                if step == 7 and blk == 2:   # a reused plan, checked against the oracle
                    op = oracle_problem(wl)
                    n = int(rp[-1])
                    O, _ = oracle.attend(q, k, v, oracle.Plan(rp.astype(np.int64), ci[:n],
                                                              pl.logw.cpu().numpy()[:n]), op)
                    check_output(o, O, "bf16", "policy loop, reused plan")
            torch.cuda.synchronize()
            assert torch.equal(o, ref), (step, blk, mode)
    say(f"policy loop: modes {pol.counts(n_blocks)}")
    modes = [m for (_, _, m) in attn.log]
    assert {m: modes.count(m) for m in (DENSE, BUILD, REUSE)} == pol.counts(n_blocks)
    assert pol.counts(n_blocks) == {DENSE: 2 * 3 + 10, BUILD: 3 * 2, REUSE: 7 * 2}
    assert len(plans) == 6


@pytest.mark.gpu
def test_overflowed_plan_raises_without_a_stall_per_build():
    """A plan that outgrows its capacity still raises: at the next call once
    its status copy has landed, or at check() (which waits)."""
    import block_sparse_attention_09_amd as ab
    from helpers import say, to_dev
    from workloads import Workload, make_qkv

    wl = Workload("ovf", B=1, H=1, D=128, grid=(2, 8, 16))
    q, k, v = make_qkv(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    pol = StepPolicy(total_steps=4, dense_steps=0, dense_blocks=0, plan_every=4, budget=0.5)
    for via_check in (False, True):
        attn = ABAttention(pol)
        prob = attn.problem(dq)
        # a cached plan of this problem with room for one entry: the build at
        # step 0 writes into it and overflows
        attn._plans[0] = (-1, ab.empty_plan(prob, 1, dq.device), prob)
        attn.set_step(0)
        say(f"policy overflow (check() {via_check})")
        o = attn(dq, dk, dv, 0)                      # deferred: no raise yet
        torch.cuda.synchronize()
        assert int(attn.plan_of(0).status.item()) == 1
        assert torch.count_nonzero(o) == 0           # every row empty
        with pytest.raises(RuntimeError, match="outgrew its capacity"):
            if via_check:
                attn.check()
            else:
                attn(dq, dk, dv, 1)                  # the next call surfaces it
