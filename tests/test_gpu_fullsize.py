"""Parity at the full layer shapes, in the launch configuration bench.py times.

The GPU runs the whole layer (every head, every plan row); the oracle checks a
sample of rows one by one:
  * plan rows against oracle.plan on the same rows (block agreement >= 99%);
  * attention rows against the oracle run on the GPU's own plan rows (bf16
    bar: max-abs 1e-2, mean-rel 1e-3 against the oracle rounded to bf16), and
    the fp16-V form (V converted once, as bench.py runs it) bit-identical to it;
  * dense rows against the oracle's dense attention of sampled queries.
Sampled rows lie in the first two heads and the last head (its first row, a
middle row and its last row, the head's partial last query block); the oracle
gets those heads' inputs, generated on the host by the same seeded recipe
(full-shape host arrays whose other heads stay zero and untouched).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import errors, jaccard, round_ref, say
from workloads import CONFIGS, Generator, make_qkv, make_qkv_sequence, round_like

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")


def checked_heads(wl):
    return sorted({0, min(1, wl.H - 1), wl.H - 1})


def gpu_inputs(wl):
    """Full [B,H,N,D] bf16 q, k, v on the GPU; host fp32 masters of q, k (reused
    plans); and host q, k, v rounded like the GPU's for the checked heads of
    batch 0, in full-shape arrays whose other heads are zero (np.zeros pages
    that are never written take no memory)."""
    shape = (wl.B, wl.H, wl.N, wl.D)
    q = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    gen = Generator(wl)
    qm = np.empty(shape, dtype=np.float32) if wl.plan_reuse > 1 else None
    km = np.empty(shape, dtype=np.float32) if wl.plan_reuse > 1 else None
    host = tuple(np.zeros(shape, dtype=np.float32) for _ in range(3))
    heads = checked_heads(wl)
    for b, h, qh, kh, vh in gen.iter_heads():
        q[b, h].copy_(torch.from_numpy(qh).to(torch.bfloat16))
        k[b, h].copy_(torch.from_numpy(kh).to(torch.bfloat16))
        v[b, h].copy_(torch.from_numpy(vh).to(torch.bfloat16))
        if qm is not None:
            qm[b, h], km[b, h] = qh, kh
        if b == 0 and h in heads:
            for arr, x in zip(host, (qh, kh, vh)):
                arr[0, h] = round_like(x, wl.dtype)
    return gen, q, k, v, qm, km, host


def problems(wl):
    prob = ab.Problem(wl.B, wl.H, wl.N, wl.D, n_clusters=wl.n_clusters,
                      kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text)
    op = oracle.Problem(wl.B, wl.H, wl.N, wl.D, n_clusters=wl.n_clusters,
                        kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text)
    return prob, op


def sample_rows(op, n=6, seed=0):
    """Rows of heads 0 and 1 (random ones and the partial last blocks) and of
    the last head: its first, a middle and its last row (R - 1)."""
    rng = np.random.default_rng(seed)
    last = op.n_qb - 1
    rows = {0, last, op.n_qb + last // 2, op.n_qb + last}      # incl. partial last blocks
    rows |= set(rng.integers(0, 2 * op.n_qb, n).tolist())
    rows = {r for r in rows if r < min(2, op.H) * op.n_qb}
    hl = (op.B * op.H - 1) * op.n_qb                            # last head of the last batch
    if op.B == 1:
        rows |= {hl, hl + last // 2, op.R - 1}
    return sorted(rows)


def check_plan_and_attend(tag, wl, budget, seed, q2, k2, v2, q, k, v, prob, op, pl, o):
    """q2/k2/v2: host fp32 (bf16-exact) inputs of the checked heads; q/k/v, pl, o: GPU."""
    rows = sample_rows(op)
    ref = oracle.plan(q2, k2, op, budget, seed, rows=rows)
    rp = pl.row_ptr.cpu().numpy().astype(np.int64)
    ci_all = pl.col_idx[: int(rp[-1])].cpu().numpy()
    lw_all = pl.logw[: int(rp[-1])].cpu().numpy()
    g_ci = [ci_all[rp[r]:rp[r + 1]] for r in rows]
    g_lw = [lw_all[rp[r]:rp[r + 1]] for r in rows]
    g_rp = np.cumsum([0] + [len(c) for c in g_ci])
    jac = jaccard(g_rp, np.concatenate(g_ci), ref.row_ptr, ref.col_idx)
    say(f"{tag}: rows {rows} plan jaccard {jac:.5f}")
    assert jac >= 0.99
    # attention on the GPU's own plan rows
    check_rows(tag, q2, k2, v2, op, rows, g_ci, g_lw, o)


def check_rows(tag, q2, k2, v2, op, rows, cols, lws, o):
    """Oracle attention of each sampled row on the given plan rows vs GPU o."""
    got, ref = [], []
    for r, c, w in zip(rows, cols, lws):
        orow, _ = oracle.attend_row(q2, k2, v2, op, r, c, w)
        b, h, qb = oracle.unflatten_row(op, r)
        lo = qb * op.q_block
        got.append(o[b, h, lo:lo + orow.shape[0]].float().cpu().numpy().astype(np.float64))
        ref.append(orow)
    got, ref = np.concatenate(got), np.concatenate(ref)
    mx, mr = errors(got, round_ref(ref, "bf16"))
    say(f"{tag}: attend rows max-abs {mx:.3e} mean-rel {mr:.3e}")
    assert mx <= 1e-2 and mr <= 1e-3


@pytest.mark.parametrize("name", ["wan1p3b_480p", "wan14b_720p", "hunyuan_720p"])
def test_fullsize_plan_attend(name):
    wl = CONFIGS[name]
    say(f"{name}: generating inputs")
    gen, q, k, v, _, _, (q2, k2, v2) = gpu_inputs(wl)
    prob, op = problems(wl)
    # every sparse budget the layer is quoted at (8%, 10%, 12% for the 14B layer)
    for budget in [b for b in wl.budgets if b < 1.0]:
        pl = ab.plan(q, k, budget, seed=wl.plan_seed, problem=prob)
        o = ab.attend(q, k, v, pl, problem=prob)
        torch.cuda.synchronize()
        assert pl.ok()
        nnz = pl.nnz()
        m = budget * op.n_kbs
        expect = op.R * (m + (op.n_kb - op.n_kbs))
        say(f"{name} budget {budget}: nnz {nnz} expected {expect:.0f}")
        assert abs(nnz - expect) < 6 * np.sqrt(op.R * m)
        check_plan_and_attend(f"{name} budget {budget}", wl, budget, wl.plan_seed, q2, k2, v2,
                              q, k, v, prob, op, pl, o)
        # the one-pass sampler: the same plan, bit for bit
        p1 = ab.plan_onepass(q, k, budget, seed=wl.plan_seed, problem=prob)
        torch.cuda.synchronize()
        assert p1.ok() and torch.equal(p1.row_ptr, pl.row_ptr)
        assert torch.equal(p1.col_idx[:nnz], pl.col_idx[:nnz])
        assert torch.equal(p1.logw[:nnz].view(torch.int32), pl.logw[:nnz].view(torch.int32))
        del p1
        # the fp16-V form bench.py times: bit-identical to the attention just checked
        o16 = ab.attend(q, k, ab.v_to_f16(v, prob), pl, problem=prob)
        torch.cuda.synchronize()
        assert torch.equal(o16, o)
        del pl, o, o16
    if name == "wan14b_720p":
        od = ab.dense(q, k, v, problem=prob)
        torch.cuda.synchronize()
        rng = np.random.default_rng(1)
        qi = np.unique(np.concatenate([[0, wl.N - 1], rng.integers(0, wl.N, 30)]))
        for h in checked_heads(wl):
            Od, _ = oracle.dense_rows(q2, k2, v2, op, 0, h, qi)
            got = od[0, h, qi].float().cpu().numpy().astype(np.float64)
            mx, mr = errors(got, round_ref(Od, "bf16"))
            say(f"{name}: dense head {h} rows max-abs {mx:.3e} mean-rel {mr:.3e}")
            assert mx <= 1e-2 and mr <= 1e-3


def test_fullsize_stress_plan_reuse():
    """1% budget, 16 clusters; one plan serves four calls with drifting q/k."""
    wl = CONFIGS["stress_1pct"]
    budget = wl.budgets[0]
    say("stress_1pct: generating inputs")
    gen, q, k, v, qm, km, (q2, k2, v2) = gpu_inputs(wl)
    prob, op = problems(wl)
    pl = ab.plan(q, k, budget, seed=wl.plan_seed, problem=prob)
    torch.cuda.synchronize()
    assert pl.ok()
    seq = make_qkv_sequence(wl, wl.plan_reuse, heads=2)
    np.testing.assert_array_equal(q2[0, :2], seq[0][0][0])
    o = ab.attend(q, k, v, pl, problem=prob)
    torch.cuda.synchronize()
    check_plan_and_attend("stress call 0", wl, budget, wl.plan_seed, q2, k2, v2, q, k, v,
                          prob, op, pl, o)
    # calls 1..3: drift q/k of every head (same draw order as make_qkv_sequence),
    # keep the plan, attend again and check the last call's rows
    for c in range(1, wl.plan_reuse):
        for b in range(wl.B):
            for h in range(wl.H):
                qm[b, h] = gen.drift(qm[b, h])
                km[b, h] = gen.drift(km[b, h])
                q[b, h].copy_(torch.from_numpy(qm[b, h]).to(torch.bfloat16))
                k[b, h].copy_(torch.from_numpy(km[b, h]).to(torch.bfloat16))
        o = ab.attend(q, k, v, pl, problem=prob)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q[0, :2].float().cpu().numpy(), seq[-1][0][0])
    # host inputs of the last call for the checked heads (the drifted masters)
    q3, k3 = np.zeros_like(q2), np.zeros_like(k2)
    for h in checked_heads(wl):
        q3[0, h] = round_like(qm[0, h], wl.dtype)
        k3[0, h] = round_like(km[0, h], wl.dtype)
    np.testing.assert_array_equal(q3[0, :2], seq[-1][0][0])
    v3 = v2
    rows = sample_rows(op)
    rp = pl.row_ptr.cpu().numpy().astype(np.int64)
    ci = pl.col_idx[: int(rp[-1])].cpu().numpy()
    lw = pl.logw[: int(rp[-1])].cpu().numpy()
    check_rows("stress call 3", q3, k3, v3, op, rows,
               [ci[rp[r]:rp[r + 1]] for r in rows], [lw[rp[r]:rp[r + 1]] for r in rows], o)


@pytest.mark.parametrize("pe_amp", [2.0, 3.0])
def test_sharp_inputs_plan_attend(pe_amp):
    """Sharper attention (position code amplitude 2 and 3): the logits spread
    wider, so the scorer's fp16 products err more in relative terms; the plan
    still has to agree with the oracle's (>= 99%) and attention to hold its bar."""
    wl = CONFIGS["wan1p3b_480p"].scaled(H=2, pe_amp=pe_amp)
    say(f"wan1p3b_480p H=2 pe_amp={pe_amp}: generating inputs")
    gen, q, k, v, _, _, (q2, k2, v2) = gpu_inputs(wl)
    prob, op = problems(wl)
    budget = 0.10
    pl = ab.plan(q, k, budget, seed=wl.plan_seed, problem=prob)
    o = ab.attend(q, k, v, pl, problem=prob)
    torch.cuda.synchronize()
    assert pl.ok()
    check_plan_and_attend(f"pe_amp {pe_amp}", wl, budget, wl.plan_seed, q2, k2, v2,
                          q, k, v, prob, op, pl, o)
