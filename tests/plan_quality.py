"""Plan-quality harness: attention mass kept and output error of block
selections, against dense attention, at equal block counts.

What is compared (news.hamidun.com, "AB-Attention speeds up video generation
by up to 2.23x and skips 92% of attention"):
  * section "Where earlier sparse schemes break down": ideal top-k selection
    keeps only part of the attention mass (about 69% at 10.8% of the keys);
  * section "AB-Attention's three techniques": against ideal top-k, IBCS
    leaves half the recall shortfall of mean-pooled block scoring; with equally
    many blocks, SIP's output error is 41% smaller than ideal top-k's; under
    ideal selection 4-token blocks retain 69% of the mass against 59% for
    128-token blocks.
Those figures come from real model activations; on the synthetic inputs here
they are context, not targets (parity unpinned).

Definitions (readings; the pages give none):
  * attention mass of key block j for plan row r: the mean over the row's
    queries of the dense softmax probability summed over the block's keys
    (each row's masses sum to 1);
  * recall of a selection: the mass of its blocks;
  * a top-k method keeps the k highest-scoring blocks of a row, k being the
    number of blocks SIP drew for that row (equal counts row by row), and
    attends with a plain softmax over the kept keys; SIP attends with the
    log(1/pi) shift (the oracle's attention);
  * error: ||O - O_dense||_F / ||O_dense||_F over all queries of the rows;
  * block averaging scores a block by the softmax over blocks of
    scale * mean(q of the row) . mean(k of the block).
Test infrastructure: computes everything with the oracle (NumPy, fp64), the
plan either from the oracle or from the library.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, List, Optional

import numpy as np

if __name__ == "__main__":   # run as a script: oracle/ and workloads/ sit at the repo root
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402


@dataclasses.dataclass
class RowQuality:
    mass: np.ndarray          # [n_kbs] attention mass per sparse key block
    dense: np.ndarray         # [n_q, D] dense output


def row_reference(Q, K, V, prob: "oracle.Problem", r: int) -> RowQuality:
    """Dense attention of row r's queries over all keys, and its block masses."""
    b, h, qb = oracle.unflatten_row(prob, r)
    lo, hi = qb * prob.q_block, min((qb + 1) * prob.q_block, prob.N)
    q = np.asarray(Q[b, h, lo:hi], dtype=np.float64)
    k = np.asarray(K[b, h], dtype=np.float64)
    v = np.asarray(V[b, h], dtype=np.float64)
    z = prob.tau * (q @ k.T)
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    nk = prob.n_kbs * prob.kv_block
    mass = p[:, :nk].reshape(p.shape[0], prob.n_kbs, prob.kv_block).sum(axis=2).mean(axis=0)
    return RowQuality(mass=mass, dense=p @ v)


def topk_output(Q, K, V, prob, r: int, cols: np.ndarray) -> np.ndarray:
    """Plain softmax attention of row r over the keys of the given blocks."""
    out, _ = oracle.attend_row(Q, K, V, prob, r, np.sort(cols).astype(np.int32),
                               np.zeros(len(cols), dtype=np.float32))
    return out


def block_average_scores(Q, K, prob, r: int) -> np.ndarray:
    """Softmax over blocks of scale * mean query . mean key (block averaging)."""
    b, h, qb = oracle.unflatten_row(prob, r)
    lo, hi = qb * prob.q_block, min((qb + 1) * prob.q_block, prob.N)
    qm = np.asarray(Q[b, h, lo:hi], dtype=np.float64).mean(axis=0)
    km = oracle.key_block_means(K[b:b + 1, h:h + 1], prob)[0, 0]
    z = prob.tau * (km @ qm)
    e = np.exp(z - z.max())
    return e / e.sum()


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (ties to the lower index)."""
    order = np.lexsort((np.arange(len(scores)), -scores))
    return np.sort(order[:k])


def evaluate(Q, K, V, prob, plan: "oracle.Plan", rows: Iterable[int],
             ibcs_scores: Optional[np.ndarray] = None) -> Dict[str, float]:
    """Recall and relative error of ideal top-k, block-average top-k, IBCS top-k
    and the SIP plan on the given rows (plan rows indexed like ``rows``' order
    in ``plan`` when plan holds only those rows, else by row id)."""
    rows = list(rows)
    if ibcs_scores is None:
        ibcs_scores = oracle.ibcs_scores(Q, K, prob, rows=rows)["S"]
    rec = {m: [] for m in ("ideal", "average", "ibcs", "sip")}
    err_num = {m: 0.0 for m in ("ideal", "average", "ibcs", "sip")}
    den = 0.0
    kept = 0
    for i, r in enumerate(rows):
        pr = i if plan.row_ptr.shape[0] == len(rows) + 1 else r
        cols, lw = plan.row(pr)
        ref = row_reference(Q, K, V, prob, r)
        k = len(cols)
        kept += k
        sel = {"ideal": topk(ref.mass, k),
               "average": topk(block_average_scores(Q, K, prob, r), k),
               "ibcs": topk(np.asarray(ibcs_scores[i], dtype=np.float64), k)}
        sparse_cols = cols[cols < prob.n_kbs]
        for m, c in sel.items():
            rec[m].append(ref.mass[c].sum())
            err_num[m] += float(((topk_output(Q, K, V, prob, r, c) - ref.dense) ** 2).sum())
        rec["sip"].append(ref.mass[sparse_cols].sum())
        o_sip, _ = oracle.attend_row(Q, K, V, prob, r, cols, lw)
        err_num["sip"] += float(((o_sip - ref.dense) ** 2).sum())
        den += float((ref.dense ** 2).sum())
    out = {f"recall_{m}": float(np.mean(v)) for m, v in rec.items()}
    out.update({f"err_{m}": float(np.sqrt(err_num[m] / den)) for m in err_num})
    out["blocks_per_row"] = kept / len(rows)
    out["key_fraction"] = out["blocks_per_row"] / prob.n_kbs
    gap_avg = out["recall_ideal"] - out["recall_average"]
    out["recall_gap_ratio"] = (out["recall_ideal"] - out["recall_ibcs"]) / gap_avg \
        if gap_avg > 0 else float("nan")
    out["err_ratio_sip_vs_ideal"] = out["err_sip"] / out["err_ideal"] \
        if out["err_ideal"] > 0 else float("nan")
    return out


def ideal_recall_by_block_size(Q, K, prob, rows: Iterable[int], key_fraction: float,
                               sizes=(4, 128)) -> Dict[int, float]:
    """Mass kept by ideal top-k at a fixed share of keys for several block sizes
    (blocks of ``size`` consecutive keys; the last partial block counts whole)."""
    out = {}
    for size in sizes:
        vals = []
        for r in rows:
            b, h, qb = oracle.unflatten_row(prob, r)
            lo, hi = qb * prob.q_block, min((qb + 1) * prob.q_block, prob.N)
            q = np.asarray(Q[b, h, lo:hi], dtype=np.float64)
            k = np.asarray(K[b, h], dtype=np.float64)
            z = prob.tau * (q @ k.T)
            z -= z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            nb = -(-prob.N // size)
            pad = nb * size - prob.N
            pm = np.pad(p, ((0, 0), (0, pad))).reshape(p.shape[0], nb, size).sum(axis=2).mean(0)
            kb = max(1, int(round(key_fraction * prob.N / size)))
            vals.append(np.sort(pm)[::-1][:kb].sum())
        out[size] = float(np.mean(vals))
    return out


def report(name: str, res: Dict[str, float], by_size: Dict[int, float]) -> List[str]:
    """Markdown lines for one evaluated configuration."""
    return [
        f"| {name} | {res['key_fraction']:.3f} | {res['recall_ideal']:.3f} | "
        f"{res['recall_average']:.3f} | {res['recall_ibcs']:.3f} | {res['recall_sip']:.3f} | "
        f"{res['recall_gap_ratio']:.2f} | {res['err_ideal']:.4f} | {res['err_sip']:.4f} | "
        f"{res['err_ratio_sip_vs_ideal']:.2f} | {by_size.get(4, float('nan')):.3f} | "
        f"{by_size.get(128, float('nan')):.3f} |"]


REPORT_HEADER = [
    "| workload | keys kept | recall ideal | recall block-avg | recall IBCS | recall SIP | "
    "IBCS gap / avg gap | err ideal top-k | err SIP | SIP / ideal | ideal recall K_b=4 | "
    "ideal recall K_b=128 |",
    "|---|---|---|---|---|---|---|---|---|---|---|---|"]


def sweep(amps, budgets, nrows: int = 24, workload: str = "wan1p3b_480p",
          v_pe: float = 0.0) -> List[str]:
    """Markdown table of the harness over position-code amplitudes and budgets
    on one head of a workload, with the oracle's own plans (plans from the
    library agree with them on >= 99.9% of blocks); v_pe gives the values a
    positional structure of that amplitude (workloads' v_pe_amp)."""
    from workloads import CONFIGS, make_qkv
    lines = list(REPORT_HEADER) + ["|" + " --- |" * 12]
    for a in amps:
        wl = CONFIGS[workload].scaled(H=1, pe_amp=a, v_pe_amp=v_pe)
        q, k, v = make_qkv(wl)
        prob = oracle.Problem(B=1, H=1, N=wl.N, D=wl.D, n_clusters=wl.n_clusters,
                              kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text)
        rows = list(np.linspace(0, prob.R - 1, nrows).astype(int))
        sc = oracle.ibcs_scores(q, k, prob, rows=rows)
        for budget in budgets:
            pl = oracle.plan_from_scores(sc["S32"], prob, budget, wl.plan_seed, rows)
            res = evaluate(q, k, v, prob, pl, rows, ibcs_scores=sc["S"])
            by = ideal_recall_by_block_size(q, k, prob, rows, res["key_fraction"])
            tag = f"{workload} H=1 pe_amp={a}" + (f" v_pe={v_pe}" if v_pe else "")
            lines += report(f"{tag}, budget {budget}, {nrows} rows", res, by)
            print(lines[-1], flush=True)
    return lines


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="plan-quality sweep (oracle plans, CPU)")
    ap.add_argument("--amps", default="4,5,6")
    ap.add_argument("--budgets", default="0.05,0.1,0.2")
    ap.add_argument("--rows", type=int, default=24)
    ap.add_argument("--workload", default="wan1p3b_480p")
    ap.add_argument("--v-pe", type=float, default=0.0,
                    help="amplitude of the positional structure in v (0: v is pure noise)")
    args = ap.parse_args()
    out = sweep([float(x) for x in args.amps.split(",")],
                [float(x) for x in args.budgets.split(",")], args.rows, args.workload,
                args.v_pe)
    print("\n".join(out))
