"""Python binding of libabatt: AB-Attention block-sparse video attention (gfx950).

Argument marshalling only.  Every step of the path -- key-block means,
k-means, block scores, sampling, gathered attention, dense attention -- runs
in the library's HIP kernels; torch supplies device memory and the current
stream.  There is no CPU fallback: if the library is missing, importing the
calls raises.

    prob = Problem.like(q, n_clusters=8)
    pl = plan(q, k, budget=0.10, seed=0, problem=prob)   # CSR plan on the GPU
    o = attend(q, k, v, pl, problem=prob)                # gathered attention
    o_dense = dense(q, k, v, problem=prob)
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libabatt.so")

ABATT_F32, ABATT_BF16 = 0, 1
ABATT_ESCRATCH = -6
SCRATCH_BYTES = 256 * 1024 * 1024   # ABATT_SCRATCH_BYTES in abatt.h

SYMBOLS = (
    "abatt_plan_rows", "abatt_plan_max_nnz", "abatt_plan_nnz_bound",
    "abatt_plan_workspace_bytes", "abatt_sampler_workspace_bytes", "abatt_plan",
    "abatt_plan_onepass", "abatt_plan_noalloc", "abatt_attend", "abatt_v_to_f16", "abatt_attend_v16", "abatt_dense",
    "abatt_dense_v16",
    "abatt_key_means", "abatt_scores", "abatt_plan_from_scores", "abatt_status_str",
    "abatt_version",
)


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
                ("n_clusters", ctypes.c_int32), ("kmeans_iters", ctypes.c_int32),
                ("n_forced_tail", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int)]


class _Plan(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("logw", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("status", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libabatt.so (built in-tree); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    vp, i64, sz, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "abatt_plan_rows": (i64, [P]),
        "abatt_plan_max_nnz": (i64, [P]),
        "abatt_plan_nnz_bound": (i64, [P, ctypes.c_double]),
        "abatt_plan_workspace_bytes": (sz, [P]),
        "abatt_sampler_workspace_bytes": (sz, [P]),
        "abatt_plan": (st, [P, vp, vp, ctypes.c_double, ctypes.c_uint64, vp, sz,
                            ctypes.POINTER(_Plan), vp]),
        "abatt_plan_onepass": (st, [P, vp, vp, ctypes.c_double, ctypes.c_uint64, vp, sz,
                                    ctypes.POINTER(_Plan), vp]),
        "abatt_plan_noalloc": (st, [P, vp, vp, ctypes.c_double, ctypes.c_uint64,
                                    ctypes.POINTER(_Plan), vp]),
        "abatt_attend": (st, [P, vp, vp, vp, ctypes.POINTER(_Plan), vp, vp, vp]),
        "abatt_v_to_f16": (st, [P, vp, vp, vp]),
        "abatt_attend_v16": (st, [P, vp, vp, vp, ctypes.POINTER(_Plan), vp, vp, vp]),
        "abatt_dense": (st, [P, vp, vp, vp, vp, vp, vp]),
        "abatt_dense_v16": (st, [P, vp, vp, vp, vp, vp, vp]),
        "abatt_key_means": (st, [P, vp, vp, vp]),
        "abatt_scores": (st, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
        "abatt_plan_from_scores": (st, [P, vp, ctypes.c_double, ctypes.c_uint64, vp, sz,
                                        ctypes.POINTER(_Plan), vp]),
        "abatt_status_str": (ctypes.c_char_p, [st]),
        "abatt_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class AbattError(RuntimeError):
    def __init__(self, code: int):
        msg = load_library().abatt_status_str(code).decode()
        super().__init__(f"abatt status {code}: {msg}")
        self.code = code


def _check(code: int) -> None:
    if code != 0:
        raise AbattError(code)


@dataclasses.dataclass(frozen=True)
class Problem:
    """Sizes and hyper-parameters of one layer; mirrors abatt_problem_t."""

    B: int
    H: int
    N: int
    D: int
    q_block: int = 128
    kv_block: int = 4
    n_clusters: int = 8
    kmeans_iters: int = 10
    n_forced_tail: int = 0
    scale: Optional[float] = None
    dtype: str = "bf16"

    @staticmethod
    def like(q: torch.Tensor, **kw) -> "Problem":
        B, H, N, D = q.shape
        dt = {torch.bfloat16: "bf16", torch.float32: "f32"}[q.dtype]
        return Problem(B, H, N, D, dtype=dt, **kw)

    def c(self) -> _Problem:
        scale = 1.0 / math.sqrt(self.D) if self.scale is None else float(self.scale)
        return _Problem(self.B, self.H, self.N, self.D, self.q_block, self.kv_block,
                        self.n_clusters, self.kmeans_iters, self.n_forced_tail, scale,
                        ABATT_BF16 if self.dtype == "bf16" else ABATT_F32)

    @property
    def n_qb(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def n_kbs(self) -> int:
        return (self.N - self.n_forced_tail) // self.kv_block

    @property
    def n_kb(self) -> int:
        return self.n_kbs + self.n_forced_tail // self.kv_block

    @property
    def R(self) -> int:
        return self.B * self.H * self.n_qb

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


@dataclasses.dataclass
class Plan:
    """Device CSR plan: row_ptr [R+1], col_idx/logw [capacity], status [1]."""

    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    logw: torch.Tensor
    status: Optional[torch.Tensor] = None

    def c(self) -> _Plan:
        return _Plan(self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.logw.data_ptr(),
                     self.col_idx.numel(),
                     None if self.status is None else self.status.data_ptr())

    def nnz(self) -> int:
        """Kept blocks in the plan (reads row_ptr[R]; synchronises)."""
        return int(self.row_ptr[-1].item())

    def ok(self) -> bool:
        """False if the plan outgrew its capacity (synchronises)."""
        return self.status is None or int(self.status.item()) == 0


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _qkv_check(prob: Problem, *ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")
        if t.dtype != prob.torch_dtype or tuple(t.shape) != (prob.B, prob.H, prob.N, prob.D):
            raise ValueError(f"expected {prob.dtype} [{prob.B},{prob.H},{prob.N},{prob.D}], "
                             f"got {t.dtype} {tuple(t.shape)}")


def _plan_check(prob: Problem, pl: Plan, device=None, need_status: bool = False) -> None:
    """Checks a plan's arrays against the problem before the library sees them:
    the C ABI gets pointers and a capacity only, so a short or mistyped array
    would be written or read out of bounds by the kernels."""
    if pl.row_ptr.numel() != prob.R + 1 or pl.row_ptr.dtype != torch.int32:
        raise ValueError(f"row_ptr must be int32 [{prob.R + 1}]")
    if pl.col_idx.dtype != torch.int32 or pl.logw.dtype != torch.float32 \
            or pl.logw.numel() < pl.col_idx.numel():
        raise ValueError("col_idx must be int32 and logw float32 of the same capacity")
    arrays = [pl.row_ptr, pl.col_idx, pl.logw]
    if need_status:
        if pl.status is None:
            raise ValueError("a plan written by plan() needs a status tensor")
        if pl.status.dtype != torch.int32 or pl.status.numel() < 1:
            raise ValueError("status must be an int32 tensor of at least one element")
    if pl.status is not None:
        arrays.append(pl.status)
    for t in arrays:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("plan arrays must be contiguous CUDA tensors")
        if device is not None and t.device != device:
            raise ValueError(f"plan arrays must be on {device}, found one on {t.device}")


def _out_check(prob: Problem, out: torch.Tensor, like: torch.Tensor) -> None:
    """A caller-supplied output must hold exactly [B,H,N,D] of the problem's
    dtype, contiguous, on the inputs' device (the kernels write all of it)."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous CUDA tensor")
    if out.device != like.device:
        raise ValueError(f"out must be on {like.device}, found {out.device}")
    if out.dtype != prob.torch_dtype or tuple(out.shape) != (prob.B, prob.H, prob.N, prob.D):
        raise ValueError(f"out must be {prob.dtype} [{prob.B},{prob.H},{prob.N},{prob.D}], "
                         f"got {out.dtype} {tuple(out.shape)}")


def plan_rows(prob: Problem) -> int:
    return int(load_library().abatt_plan_rows(ctypes.byref(prob.c())))


def max_nnz(prob: Problem) -> int:
    return int(load_library().abatt_plan_max_nnz(ctypes.byref(prob.c())))


def nnz_bound(prob: Problem, budget: float) -> int:
    return int(load_library().abatt_plan_nnz_bound(ctypes.byref(prob.c()), float(budget)))


def plan_workspace_bytes(prob: Problem) -> int:
    return int(load_library().abatt_plan_workspace_bytes(ctypes.byref(prob.c())))


def sampler_workspace_bytes(prob: Problem) -> int:
    return int(load_library().abatt_sampler_workspace_bytes(ctypes.byref(prob.c())))


def empty_plan(prob: Problem, capacity: int, device) -> Plan:
    return Plan(torch.empty(prob.R + 1, dtype=torch.int32, device=device),
                torch.empty(max(capacity, 1), dtype=torch.int32, device=device),
                torch.empty(max(capacity, 1), dtype=torch.float32, device=device),
                torch.zeros(1, dtype=torch.int32, device=device))


def workspace(prob: Problem, device) -> torch.Tensor:
    return torch.empty(max(plan_workspace_bytes(prob), 1), dtype=torch.uint8, device=device)


def plan(q: torch.Tensor, k: torch.Tensor, budget: float, seed: int = 0,
         problem: Optional[Problem] = None, capacity: Optional[int] = None,
         ws: Optional[torch.Tensor] = None, out: Optional[Plan] = None) -> Plan:
    """IBCS + SIP on the GPU: returns a device CSR plan (abatt_plan)."""
    return _plan_call("abatt_plan", q, k, budget, seed, problem, capacity, ws, out)


def plan_onepass(q: torch.Tensor, k: torch.Tensor, budget: float, seed: int = 0,
                 problem: Optional[Problem] = None, capacity: Optional[int] = None,
                 ws: Optional[torch.Tensor] = None, out: Optional[Plan] = None) -> Plan:
    """abatt_plan_onepass: the plan of plan(), bit for bit, with the sampler's
    count, scan and fill done by one kernel (decoupled look-back)."""
    return _plan_call("abatt_plan_onepass", q, k, budget, seed, problem, capacity, ws, out)


def _plan_call(entry: str, q, k, budget, seed, problem, capacity, ws, out) -> Plan:
    prob = problem or Problem.like(q)
    _qkv_check(prob, q, k)
    lib = load_library()
    if out is None:
        cap = nnz_bound(prob, budget) if capacity is None else capacity
        out = empty_plan(prob, cap, q.device)
    else:
        _plan_check(prob, out, q.device, need_status=True)
    if ws is None:
        ws = workspace(prob, q.device)
    elif not ws.is_cuda or not ws.is_contiguous() or ws.device != q.device \
            or ws.dtype != torch.uint8:
        raise ValueError(f"ws must be a contiguous uint8 tensor on {q.device}")
    cp = out.c()
    _check(getattr(lib, entry)(ctypes.byref(prob.c()), _ptr(q), _ptr(k), float(budget),
                               ctypes.c_uint64(seed), _ptr(ws), ws.numel(), ctypes.byref(cp),
                               _stream()))
    return out


def plan_noalloc(q: torch.Tensor, k: torch.Tensor, budget: float, seed: int = 0,
                 problem: Optional[Problem] = None, out: Optional[Plan] = None,
                 capacity: Optional[int] = None) -> Plan:
    """abatt_plan_noalloc: the same plan as plan(), with the library's static
    scratch as workspace.  Pass `out` (from empty_plan) to allocate nothing."""
    prob = problem or Problem.like(q)
    _qkv_check(prob, q, k)
    if out is None:
        cap = nnz_bound(prob, budget) if capacity is None else capacity
        out = empty_plan(prob, cap, q.device)
    else:
        _plan_check(prob, out, q.device, need_status=True)
    cp = out.c()
    _check(load_library().abatt_plan_noalloc(ctypes.byref(prob.c()), _ptr(q), _ptr(k),
                                             float(budget), ctypes.c_uint64(seed),
                                             ctypes.byref(cp), _stream()))
    return out


def _v16_check(prob: Problem, v16: torch.Tensor) -> None:
    if prob.dtype != "bf16":
        raise ValueError("fp16 V is for bf16 problems")
    if not v16.is_cuda or not v16.is_contiguous() or v16.dtype != torch.float16 \
            or tuple(v16.shape) != (prob.B, prob.H, prob.N, prob.D):
        raise ValueError(f"expected contiguous float16 [{prob.B},{prob.H},{prob.N},{prob.D}]")


def v_to_f16(v: torch.Tensor, problem: Optional[Problem] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 V -> fp16 (round toward zero) for attend's fp16-V form (abatt_v_to_f16)."""
    prob = problem or Problem.like(v)
    _qkv_check(prob, v)
    v16 = torch.empty(v.shape, dtype=torch.float16, device=v.device) if out is None else out
    _v16_check(prob, v16)
    if v16.device != v.device:
        raise ValueError(f"out must be on {v.device}, found {v16.device}")
    _check(load_library().abatt_v_to_f16(ctypes.byref(prob.c()), _ptr(v), _ptr(v16), _stream()))
    return v16


def attend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pl: Plan,
           problem: Optional[Problem] = None, return_lse: bool = False,
           out: Optional[torch.Tensor] = None):
    """Gathered attention with the log(1/pi) shift (abatt_attend).

    A float16 `v` (from v_to_f16) selects abatt_attend_v16, with bit-identical results.
    """
    prob = problem or Problem.like(q)
    v16 = v.dtype == torch.float16
    _qkv_check(prob, q, k)
    if v16:
        _v16_check(prob, v)
    else:
        _qkv_check(prob, v)
    _plan_check(prob, pl, q.device)
    for t in (k, v):
        if t.device != q.device:
            raise ValueError(f"q, k and v must be on one device ({q.device}, {t.device})")
    if out is None:
        o = torch.empty_like(q)
    else:
        _out_check(prob, out, q)
        o = out
    lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=q.device) \
        if return_lse else None
    cp = pl.c()
    fn = load_library().abatt_attend_v16 if v16 else load_library().abatt_attend
    _check(fn(ctypes.byref(prob.c()), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cp), _ptr(o),
              _ptr(lse), _stream()))
    return (o, lse) if return_lse else o


def dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, problem: Optional[Problem] = None,
          return_lse: bool = False, out: Optional[torch.Tensor] = None):
    """Dense softmax attention over every key (abatt_dense).

    A float16 `v` (from v_to_f16) selects abatt_dense_v16, with bit-identical results.
    """
    prob = problem or Problem.like(q)
    v16 = v.dtype == torch.float16
    _qkv_check(prob, q, k)
    if v16:
        _v16_check(prob, v)
    else:
        _qkv_check(prob, v)
    for t in (k, v):
        if t.device != q.device:
            raise ValueError(f"q, k and v must be on one device ({q.device}, {t.device})")
    if out is None:
        o = torch.empty_like(q)
    else:
        _out_check(prob, out, q)
        o = out
    lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=q.device) \
        if return_lse else None
    fn = load_library().abatt_dense_v16 if v16 else load_library().abatt_dense
    _check(fn(ctypes.byref(prob.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream()))
    return (o, lse) if return_lse else o


def key_means(k: torch.Tensor, problem: Optional[Problem] = None) -> torch.Tensor:
    """[B,H,n_kbs,D] fp32 mean of every sparse 4-token key block."""
    prob = problem or Problem.like(k)
    _qkv_check(prob, k)
    out = torch.empty(prob.B, prob.H, prob.n_kbs, prob.D, dtype=torch.float32, device=k.device)
    _check(load_library().abatt_key_means(ctypes.byref(prob.c()), _ptr(k), _ptr(out), _stream()))
    return out


def scores(q: torch.Tensor, k: torch.Tensor, problem: Optional[Problem] = None
           ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(S [R,n_kbs], centroids [R,C,D], weights [R,C]) fp32 from the selector kernels."""
    prob = problem or Problem.like(q)
    _qkv_check(prob, q, k)
    dev = q.device
    S = torch.empty(prob.R, prob.n_kbs, dtype=torch.float32, device=dev)
    mu = torch.empty(prob.R, prob.n_clusters, prob.D, dtype=torch.float32, device=dev)
    w = torch.empty(prob.R, prob.n_clusters, dtype=torch.float32, device=dev)
    ws = workspace(prob, dev)
    _check(load_library().abatt_scores(ctypes.byref(prob.c()), _ptr(q), _ptr(k), _ptr(S),
                                       _ptr(mu), _ptr(w), _ptr(ws), ws.numel(), _stream()))
    return S, mu, w


def plan_from_scores(S: torch.Tensor, budget: float, seed: int, problem: Problem,
                     capacity: Optional[int] = None) -> Plan:
    """SIP sampling of caller scores [R, n_kbs] fp32 (abatt_plan_from_scores)."""
    prob = problem
    if S.dtype != torch.float32 or tuple(S.shape) != (prob.R, prob.n_kbs) or not S.is_cuda \
            or not S.is_contiguous():
        raise ValueError("S must be a contiguous fp32 CUDA tensor [R, n_kbs]")
    cap = nnz_bound(prob, budget) if capacity is None else capacity
    out = empty_plan(prob, cap, S.device)
    nws = max(sampler_workspace_bytes(prob), 1)
    ws = torch.empty(nws, dtype=torch.uint8, device=S.device)
    cp = out.c()
    _check(load_library().abatt_plan_from_scores(ctypes.byref(prob.c()), _ptr(S), float(budget),
                                                 ctypes.c_uint64(seed), _ptr(ws), nws,
                                                 ctypes.byref(cp), _stream()))
    return out


def make_plan(row_ptr, col_idx, logw, device) -> Plan:
    """Wraps a caller-built CSR plan (host arrays) as a device Plan without status."""
    rp = torch.as_tensor(row_ptr).to(dtype=torch.int32, device=device).contiguous()
    ci = torch.as_tensor(col_idx).to(dtype=torch.int32, device=device).contiguous()
    lw = torch.as_tensor(logw).to(dtype=torch.float32, device=device).contiguous()
    if ci.numel() == 0:
        ci = torch.zeros(1, dtype=torch.int32, device=device)
        lw = torch.zeros(1, dtype=torch.float32, device=device)
    return Plan(rp, ci, lw, None)
