"""GPU parity of the selector and sampler kernels against the CPU oracle.

* key means: to fp32 rounding;
* k-means: per query block, identical cluster counts (weights) on >= 99% of
  blocks, and centroids within 1e-4 relative where the counts agree (fp32
  distances on the GPU vs float64 in the oracle can split a near tie);
* scores: within 2e-3 relative (max) and 2e-4 (mean) on agreeing blocks;
* sampler fed the oracle's fp32 scores: plan indices bit-exact, logw within
  1 fp32 ulp (float64 log on both sides, rounded to fp32);
* abatt_plan end to end: >= 99% block agreement (Jaccard over all rows).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from helpers import (jaccard, lib_problem, oracle_problem, plan_to_host, say, to_dev,
                     ulp_diff_f32)
from workloads import CONFIGS, Workload, make_qkv, random_scores, round_like

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")

SEL = {
    "tiny_f32": CONFIGS["tiny"],
    "bf16_ragged": Workload("r", B=1, H=2, D=128, grid=(3, 10, 12)),
    "bf16_text_c16": Workload("x", B=1, H=2, D=128, grid=(2, 8, 16), n_text=16, n_clusters=16),
    "bf16_d64_b2": Workload("b", B=2, H=2, D=64, grid=(2, 12, 16)),
    "bf16_mid": Workload("m", B=1, H=2, D=128, grid=(6, 16, 24)),
}


@pytest.mark.parametrize("name", list(SEL))
def test_key_means(name):
    wl = SEL[name]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    ref = oracle.key_block_means(k, op)
    say(f"key means {name}")
    got = ab.key_means(to_dev(k, wl.dtype), lib_problem(wl))
    torch.cuda.synchronize()
    np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("name", [n for n in SEL if SEL[n].dtype == "bf16"])
def test_key_means_scoring_form(name):
    """The key means as abatt_plan's scorer reads them (bf16 problems): one fp16
    plane [B,H,n_kbs,D] at the start of the plan workspace, followed by one fp32
    scale 2^e per tile of 32 blocks of a head.  plane * scale must be the mean
    to fp16's rounding: 2^-11 relative, plus half an fp16 subnormal step (2^-25
    in plane units) for values 2^-14 below their tile's largest."""
    wl = SEL[name]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    prob = lib_problem(wl)
    ref = oracle.key_block_means(k, op)                       # [B,H,n_kbs,D] float64
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    ws = ab.workspace(prob, dq.device)
    S = torch.empty(prob.R, prob.n_kbs, dtype=torch.float32, device="cuda")
    say(f"key means scoring form {name}")
    lib = ab.load_library()
    ab._check(lib.abatt_scores(ctypes.byref(prob.c()), ab._ptr(dq), ab._ptr(dk), ab._ptr(S),
                               None, None, ab._ptr(ws), ws.numel(), ab._stream()))
    torch.cuda.synchronize()
    n_plane = prob.B * prob.H * prob.n_kbs * prob.D
    n_tiles = (prob.n_kbs + 31) // 32
    raw = ws.cpu().numpy()
    plane = raw[:2 * n_plane].view(np.float16).astype(np.float64)
    plane = plane.reshape(prob.B, prob.H, prob.n_kbs, prob.D)
    scale = raw[2 * n_plane:2 * n_plane + 4 * prob.B * prob.H * n_tiles].view(np.float32)
    scale = scale.astype(np.float64).reshape(prob.B, prob.H, n_tiles)
    # scales are powers of two that put each tile's largest |mean| in [1, 2)
    assert np.all(np.log2(scale) == np.round(np.log2(scale)))
    tile = np.repeat(scale, 32, axis=2)[:, :, :prob.n_kbs, None]
    got = plane * tile
    err = np.abs(got - ref)
    bound = 2.0 ** -11 * np.abs(ref) + 2.0 ** -25 * tile + 1e-30
    say(f"  max error / bound {np.max(err / bound):.3f}, max rel {np.max(err / np.maximum(np.abs(ref), 1e-30)):.2e}")
    assert np.all(err <= bound)
    assert np.abs(plane).max() < 2.0


@pytest.mark.parametrize("name", list(SEL))
def test_centroids_and_scores(name):
    wl = SEL[name]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    sc = oracle.ibcs_scores(q, k, op)
    say(f"scores {name} R={op.R} n_kbs={op.n_kbs}")
    S, mu, w = ab.scores(to_dev(q, wl.dtype), to_dev(k, wl.dtype), lib_problem(wl))
    torch.cuda.synchronize()
    S, mu, w = S.cpu().numpy(), mu.cpu().numpy(), w.cpu().numpy()
    same = np.all(np.abs(w - sc["w"]) <= 1e-6, axis=1)
    say(f"  k-means blocks with identical weights: {same.mean():.4f}")
    assert same.mean() >= 0.99
    np.testing.assert_allclose(mu[same], sc["mu"][same], rtol=1e-4, atol=1e-4)
    rel = np.abs(S[same] - sc["S"][same]) / sc["S"][same]
    say(f"  score rel err max {rel.max():.3e} mean {rel.mean():.3e}")
    assert rel.max() <= 2e-3 and rel.mean() <= 2e-4
    np.testing.assert_allclose(S.sum(axis=1), 1.0, rtol=1e-4)


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_ragged", "bf16_d64_b2"])
@pytest.mark.parametrize("k2", [-30, 30])
def test_scores_invariant_under_power_of_two_key_scaling(name, k2):
    # K * 2^k2 with the softmax scale * 2^-k2 gives the same logits.  The
    # scorer's operands are scaled by powers of two only (per tile of key
    # means and per work-group of centroids, or bf16 hi/lo splits), so the
    # scores must come out bit for bit the same, also with |K| near 1e9 or
    # 1e-9 (far outside fp16's range)
    wl = SEL[name]
    q, k, _ = make_qkv(wl)
    s0 = 1.0 / np.sqrt(wl.D)
    say(f"scores {name} with K * 2^{k2}")
    dq = to_dev(q, wl.dtype)
    S0, _, _ = ab.scores(dq, to_dev(k, wl.dtype), lib_problem(wl, scale=s0))
    S1, _, _ = ab.scores(dq, to_dev(np.ldexp(k, k2), wl.dtype),
                         lib_problem(wl, scale=float(np.ldexp(s0, -k2))))
    torch.cuda.synchronize()
    assert torch.equal(S0, S1)


# Inputs that send the bf16 scorer off its unit scale (where the fp16 MFMA
# yields the logits themselves and the pass offsets ride in the accumulator
# input) onto the per-logit tile-scale form: every logit below -100 (log2 units,
# so pass 1's sums underflow against the starting reference 0 and the
# work-group redoes pass 1 with a moving reference), one tile of keys 2^20
# smaller than the rest (tile scales too far apart for one fp16 factor each),
# and queries 2^14 smaller (logits near zero).
UNIT_FALLBACK = ["far_negative", "tile_spread", "tiny_logits"]


@pytest.mark.parametrize("case", UNIT_FALLBACK)
def test_scores_off_the_unit_scale(case):
    wl = SEL["bf16_mid"]
    q, k, _ = make_qkv(wl)
    if case == "far_negative":
        # q shifted by -1 and k by +16 in every dim: mu.kbar / sqrt(128) *
        # log2(e) from about -175 to -110 (q keeps its structure, so k-means
        # is as usual)
        q = round_like(q - 1.0, wl.dtype)
        k = round_like(k + 16.0, wl.dtype)
    elif case == "tile_spread":
        k = k.copy()
        k[:, :, :128] = round_like(np.ldexp(k[:, :, :128], -20), wl.dtype)  # the first tile of 32 blocks
    else:
        q = round_like(np.ldexp(q, -14), wl.dtype)
    op = oracle_problem(wl)
    sc = oracle.ibcs_scores(q, k, op)
    say(f"scores off the unit scale: {case}")
    S, mu, w = ab.scores(to_dev(q, wl.dtype), to_dev(k, wl.dtype), lib_problem(wl))
    torch.cuda.synchronize()
    S, w = S.cpu().numpy(), w.cpu().numpy()
    same = np.all(np.abs(w - sc["w"]) <= 1e-6, axis=1)
    say(f"  k-means blocks with identical weights: {same.mean():.4f}")
    assert same.mean() >= 0.99
    rel = np.abs(S[same] - sc["S"][same]) / sc["S"][same]
    say(f"  score rel err max {rel.max():.3e} mean {rel.mean():.3e}")
    assert rel.max() <= 2e-3 and rel.mean() <= 2e-4
    np.testing.assert_allclose(S.sum(axis=1), 1.0, rtol=1e-4)


SAMPLER = [
    # (problem kwargs, budget, score spread, rows checked)
    (dict(B=1, H=2, N=1024, D=64), 0.10, 3.0, None),
    (dict(B=1, H=1, N=32760, D=128), 0.10, 4.0, None),
    (dict(B=1, H=1, N=4096, D=128), 0.01, 2.0, None),
    (dict(B=1, H=1, N=4096, D=128), 0.5, 1.0, None),
    (dict(B=1, H=1, N=4096, D=128), 1.0, 2.0, None),
    (dict(B=1, H=1, N=4096 + 256, D=128, n_forced_tail=256), 0.1, 3.0, None),
    (dict(B=2, H=3, N=2048, D=128), 0.25, 6.0, None),
    # long rows (the count kernel reads every row in place; its first read
    # issues at most 10 loads of 16 bytes per thread at a time, 20 480 blocks):
    # n_kbs = 40000, two rounds of loads
    (dict(B=1, H=1, N=160000, D=128), 0.05, 3.0, [0, 1, 7, 500, 1249]),
    # n_kbs = 20224 and 20228: rows just under 20 480 blocks, the longest that
    # one round of loads covers
    (dict(B=1, H=1, N=80896, D=64), 0.1, 3.0, [0, 1, 315, 631]),
    (dict(B=1, H=1, N=80912, D=64), 0.1, 3.0, [0, 5, 632]),
]


@pytest.mark.parametrize("case", range(len(SAMPLER)))
def test_sampler_bit_exact_from_oracle_scores(case):
    kw, budget, spread, rows = SAMPLER[case]
    op = oracle.Problem(**kw)
    prob = ab.Problem(dtype="bf16", **kw)
    S = random_scores(op.R, op.n_kbs, seed=case, spread=spread)
    if case == 0:
        S[:, ::7] = 0.0          # zero scores are never drawn
    rows = list(range(op.R)) if rows is None else rows
    ref = oracle.plan_from_scores(S[rows], op, budget, seed=1234 + case, rows=rows)
    say(f"sampler case {case}: R={op.R} n_kbs={op.n_kbs} budget={budget}")
    cap = ab.nnz_bound(prob, budget)
    pl = ab.plan_from_scores(torch.from_numpy(S).cuda(), budget, 1234 + case, prob, capacity=cap)
    torch.cuda.synchronize()
    assert pl.ok()
    rp, ci, lw = plan_to_host(pl)
    for i, r in enumerate(rows):
        a, b = ref.row_ptr[i], ref.row_ptr[i + 1]
        ga, gb = rp[r], rp[r + 1]
        np.testing.assert_array_equal(ci[ga:gb], ref.col_idx[a:b], err_msg=f"row {r}")
        assert ulp_diff_f32(lw[ga:gb], ref.logw[a:b]).max(initial=0) <= 1, f"row {r}"
    if len(rows) == op.R:
        np.testing.assert_array_equal(rp, ref.row_ptr)


def test_sampler_capacity_overflow_and_determinism():
    kw = dict(B=1, H=1, N=4096, D=128)
    prob = ab.Problem(dtype="bf16", **kw)
    op = oracle.Problem(**kw)
    S = torch.from_numpy(random_scores(op.R, op.n_kbs, seed=5)).cuda()
    say("sampler overflow")
    small = ab.plan_from_scores(S, 0.3, 7, prob, capacity=10)
    a = ab.plan_from_scores(S, 0.3, 7, prob)
    b = ab.plan_from_scores(S, 0.3, 7, prob)
    torch.cuda.synchronize()
    assert not small.ok()
    assert small.nnz() == a.nnz() > 10      # row_ptr still reports the needed total
    assert torch.equal(a.row_ptr, b.row_ptr)
    n = a.nnz()
    assert torch.equal(a.col_idx[:n], b.col_idx[:n]) and torch.equal(a.logw[:n], b.logw[:n])


PLAN_PATHS = {
    "bf16_ragged": (SEL["bf16_ragged"], 0.12),
    "bf16_mid_half": (SEL["bf16_mid"], 0.5),
    "bf16_mid_all": (SEL["bf16_mid"], 1.0),
    "tiny_f32": (SEL["tiny_f32"], 0.3),
    "bf16_d64_b2": (SEL["bf16_d64_b2"], 0.05),
    # 38 000 key blocks: a row of 152 000 bytes, read from memory by the count kernel
    "bf16_long_row": (Workload("L", B=1, H=1, D=64, grid=(19, 40, 200)), 0.1),
}


@pytest.mark.parametrize("name", list(PLAN_PATHS))
def test_plan_equals_scores_then_sampler(name):
    # abatt_plan (scores in its workspace) and abatt_scores followed by
    # abatt_plan_from_scores (scores in the caller's buffer) run the same
    # kernels on the same scores: the same plan, bit for bit
    wl, budget = PLAN_PATHS[name]
    q, k, _ = make_qkv(wl)
    prob = lib_problem(wl)
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    say(f"plan paths {name} n_kbs={prob.n_kbs} budget {budget}")
    a = ab.plan(dq, dk, budget, seed=4, problem=prob)
    S, _, _ = ab.scores(dq, dk, prob)
    b = ab.plan_from_scores(S, budget, 4, prob)
    torch.cuda.synchronize()
    assert a.ok() and b.ok()
    assert torch.equal(a.row_ptr, b.row_ptr)
    n = a.nnz()
    assert torch.equal(a.col_idx[:n], b.col_idx[:n]) and torch.equal(a.logw[:n], b.logw[:n])


@pytest.mark.parametrize("name", list(SEL))
def test_plan_end_to_end_agreement(name):
    wl = SEL[name]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    budget = 0.12
    ref = oracle.plan(q, k, op, budget, seed=3)
    say(f"plan e2e {name}")
    dq, dk = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    prob = lib_problem(wl)
    pl = ab.plan(dq, dk, budget, seed=3, problem=prob)
    pl2 = ab.plan(dq, dk, budget, seed=3, problem=prob)
    torch.cuda.synchronize()
    assert pl.ok()
    rp, ci, lw = plan_to_host(pl)
    rp2, ci2, lw2 = plan_to_host(pl2)
    np.testing.assert_array_equal(rp, rp2)          # deterministic
    np.testing.assert_array_equal(ci, ci2)
    jac = jaccard(rp, ci, ref.row_ptr, ref.col_idx)
    say(f"  jaccard {jac:.5f} nnz gpu {len(ci)} oracle {len(ref.col_idx)}")
    assert jac >= 0.99
    # forced blocks present in every row
    nf = op.n_kb - op.n_kbs
    for r in range(op.R):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
        if nf:
            np.testing.assert_array_equal(row[-nf:], np.arange(op.n_kbs, op.n_kb))


def test_plan_then_attend_budget_one():
    wl = SEL["bf16_ragged"]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    say("plan budget 1 -> attend == dense")
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, wl.dtype) for x in (q, k, v))
    pl = ab.plan(dq, dk, 1.0, seed=0, problem=prob)
    o = ab.attend(dq, dk, dv, pl, problem=prob)
    torch.cuda.synchronize()
    assert pl.nnz() == op.R * op.n_kb
    assert torch.all(pl.logw[:pl.nnz()] == 0)
    from helpers import check_output
    Od, _ = oracle.dense(q, k, v, op)
    check_output(o, Od, wl.dtype, "plan@1 + attend vs dense")
