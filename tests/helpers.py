"""Shared helpers for the GPU parity tests (comparison metrics, conversions)."""
import os
import sys

import numpy as np
import torch

import oracle
from workloads import Workload, bf16_bits_to_f32, make_qkv, to_bf16_bits


def say(msg: str) -> None:
    """Progress line, flushed (names the case before each GPU step)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to("cuda").contiguous()


def oracle_problem(wl: Workload, **kw) -> "oracle.Problem":
    return oracle.Problem(B=wl.B, H=wl.H, N=wl.N, D=wl.D, q_block=wl.q_block,
                          kv_block=wl.kv_block, n_clusters=wl.n_clusters,
                          kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text, **kw)


def lib_problem(wl: Workload, **kw):
    import block_sparse_attention_09_amd as ab
    return ab.Problem(B=wl.B, H=wl.H, N=wl.N, D=wl.D, q_block=wl.q_block,
                      kv_block=wl.kv_block, n_clusters=wl.n_clusters,
                      kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text,
                      dtype=wl.dtype, **kw)


def round_ref(ref: np.ndarray, dtype: str) -> np.ndarray:
    """The oracle's float64 output as the GPU stores it (bf16 RNE or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    return ref.astype(np.float32).astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs, mean-rel = sum|d| / sum|ref|) over finite reference entries."""
    m = np.isfinite(ref)
    d = np.abs(got[m].astype(np.float64) - ref[m])
    return float(d.max(initial=0.0)), float(d.sum() / max(np.abs(ref[m]).sum(), 1e-300))


# output tolerances (max-abs, mean-rel) by dtype
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-4, 1e-4)}
LSE_TOL = {"bf16": 2e-3, "f32": 1e-4}


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_output(o_gpu: torch.Tensor, o_ref: np.ndarray, dtype: str, what: str):
    """Output bar: max-abs and mean-rel against the oracle rounded like the
    output.  Two values rounded to bf16 can sit one bf16 step apart when the
    exact result lies near a rounding boundary, and above |x| = 2 that step
    (2^-6) exceeds the 1e-2 absolute bar, so for bf16 each element may also
    differ by one step of its reference."""
    got = o_gpu.float().cpu().numpy().astype(np.float64)
    ref = round_ref(o_ref, dtype)
    mx, mr = errors(got, ref)
    say(f"{what}: max-abs {mx:.3e} mean-rel {mr:.3e}")
    tol = TOL[dtype]
    assert mr <= tol[1], (what, mx, mr)
    if mx > tol[0]:
        fin = np.isfinite(ref)
        allowed = np.maximum(tol[0], bf16_ulp(ref[fin])) if dtype == "bf16" else tol[0]
        over = np.abs(got[fin] - ref[fin]) > allowed
        assert not over.any(), (what, mx, mr, int(over.sum()))
    return mx, mr


def plan_to_host(pl):
    rp = pl.row_ptr.cpu().numpy().astype(np.int64)
    nnz = int(rp[-1])
    return rp, pl.col_idx[:nnz].cpu().numpy(), pl.logw[:nnz].cpu().numpy()


def jaccard(rp_a, ci_a, rp_b, ci_b) -> float:
    inter = union = 0
    for r in range(len(rp_a) - 1):
        a = set(ci_a[rp_a[r]:rp_a[r + 1]].tolist())
        b = set(ci_b[rp_b[r]:rp_b[r + 1]].tolist())
        inter += len(a & b)
        union += len(a | b)
    return inter / max(union, 1)


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)
