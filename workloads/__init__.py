"""Seeded synthetic inputs for the AB-Attention hot path.

This module only makes inputs: token grids, shapes and seeded random tensors.
It holds none of the method's arithmetic (no block means, clustering, scores,
sampling or attention), so both the CPU oracle's tests and the GPU path's
tests and benchmark can draw their inputs from it.

The pages measure on Wan2.1 and HunyuanVideo activations from a prompt suite
that is not available here; the tensors below stand in for them.  They keep
the latent token shapes of those runs (720p with 81 frames is a 21x45x80
latent grid, 129 frames is 33x45x80) and give the logits a local-plus-tail
structure: q and k share a 3D sinusoidal position code, so a query's largest
logits sit at nearby positions in space and time, over a noise floor.

Recipe (per config):
  * ``rng = numpy.random.default_rng(seed)``; for b, then h, draw ``z_q``,
    ``z_k`` and ``z_v`` of shape [N, d] as float32 standard normals, in that
    order.
  * Position code PE(t, y, x) in R^d, amplitude 1: the dimensions split as
    d_y = d_x = 2*floor(d/6) and d_t = d - d_y - d_x; an axis with d_a
    dimensions holds [sin(p*w_i) for i < d_a/2] then [cos(p*w_i) ...], with
    w_i = 10000 ** (-2 i / d_a).  Tokens are in raster order
    i = (t*H_g + y)*W_g + x.
  * q = sigma*z_q + PE, k = sigma*z_k + PE, v = z_v.  Text tokens (appended at
    the tail, HunyuanVideo shape only) get q, k = sigma*z with no PE.
  * Optional (plan-quality sweeps only; 0 everywhere else): v also gets
    v_pe_amp * PE with its dimensions rotated by D/2, a smooth positional
    structure in the values that is not a copy of q's and k's.
  * bf16 configs round the float32 values to bfloat16 (round to nearest even);
    both sides of any comparison see the same bits.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and sampling settings of one synthetic attention layer."""

    name: str
    B: int
    H: int
    D: int
    grid: Tuple[int, int, int]          # (T, H_g, W_g) latent video grid
    n_text: int = 0                     # text tokens appended at the tail
    dtype: str = "bf16"                 # "bf16" or "f32"
    sigma: float = 0.5                  # noise std of q and k
    q_block: int = 128
    kv_block: int = 4
    n_clusters: int = 8
    kmeans_iters: int = 10
    budgets: Tuple[float, ...] = (0.10,)
    seed: int = 0                       # input seed (numpy PCG64)
    plan_seed: int = 0                  # sampler seed
    plan_reuse: int = 1                 # calls that share one plan
    drift: float = 0.0                  # per-call q/k drift std when reused
    pe_amp: float = 1.0                 # amplitude of the position code (1 everywhere
                                        # except the plan-quality sweep)
    v_pe_amp: float = 0.0               # positional structure in v (plan-quality sweep)

    @property
    def N(self) -> int:
        t, hg, wg = self.grid
        return t * hg * wg + self.n_text

    @property
    def n_video(self) -> int:
        t, hg, wg = self.grid
        return t * hg * wg

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes the measurements are quoted on.
CONFIGS: Dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, H=2, D=64, grid=(4, 16, 16), dtype="f32",
                     sigma=1.0, budgets=(0.10,)),
    "wan1p3b_480p": Workload("wan1p3b_480p", B=1, H=12, D=128,
                             grid=(21, 30, 52), budgets=(0.10,)),
    "wan14b_720p": Workload("wan14b_720p", B=1, H=40, D=128,
                            grid=(21, 45, 80), budgets=(0.08, 0.10, 0.12, 1.0)),
    "hunyuan_720p": Workload("hunyuan_720p", B=1, H=24, D=128,
                             grid=(33, 45, 80), n_text=256, budgets=(0.10,)),
    "stress_1pct": Workload("stress_1pct", B=1, H=40, D=128, grid=(21, 45, 80),
                            n_clusters=16, budgets=(0.01,), plan_reuse=4,
                            drift=0.05),
}


def position_code(grid: Tuple[int, int, int], d: int) -> np.ndarray:
    """3D sinusoidal position code, float64 [T*H_g*W_g, d], raster order."""
    t_n, y_n, x_n = grid
    d_y = d_x = 2 * (d // 6)
    d_t = d - d_y - d_x

    def axis(n: int, d_a: int) -> np.ndarray:
        half = d_a // 2
        p = np.arange(n, dtype=np.float64)[:, None]
        w = 10000.0 ** (-2.0 * np.arange(half, dtype=np.float64) / d_a)
        out = np.zeros((n, d_a), dtype=np.float64)
        out[:, :half] = np.sin(p * w)
        out[:, half:2 * half] = np.cos(p * w)
        return out

    pt, py, px = axis(t_n, d_t), axis(y_n, d_y), axis(x_n, d_x)
    pe = np.empty((t_n, y_n, x_n, d), dtype=np.float64)
    pe[..., :d_t] = pt[:, None, None, :]
    pe[..., d_t:d_t + d_y] = py[None, :, None, :]
    pe[..., d_t + d_y:] = px[None, None, :, :]
    return pe.reshape(t_n * y_n * x_n, d)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_like(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 copy of x after rounding to the workload's storage dtype."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(to_bf16_bits(x))
    if dtype == "f32":
        return x.copy()
    raise ValueError(dtype)


class Generator:
    """Seeded q/k/v producer for one workload (float32 master copies)."""

    def __init__(self, wl: Workload, heads: Optional[List[Tuple[int, int]]] = None):
        self.wl = wl
        self.rng = np.random.default_rng(wl.seed)
        self.pe = (wl.pe_amp * position_code(wl.grid, wl.D)).astype(np.float32)

    def _one(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        wl = self.wl
        n, d, nv = wl.N, wl.D, wl.n_video
        zq = self.rng.standard_normal((n, d), dtype=np.float32)
        zk = self.rng.standard_normal((n, d), dtype=np.float32)
        zv = self.rng.standard_normal((n, d), dtype=np.float32)
        s = np.float32(wl.sigma)
        q = s * zq
        k = s * zk
        q[:nv] += self.pe
        k[:nv] += self.pe
        if wl.v_pe_amp:
            zv[:nv] += np.float32(wl.v_pe_amp / wl.pe_amp if wl.pe_amp else 0.0) * \
                np.roll(self.pe, d // 2, axis=1)
        return q, k, zv

    def iter_heads(self) -> Iterator[Tuple[int, int, np.ndarray, np.ndarray, np.ndarray]]:
        """Yields (b, h, q, k, v) float32 masters in generation order."""
        for b in range(self.wl.B):
            for h in range(self.wl.H):
                q, k, v = self._one()
                yield b, h, q, k, v

    def drift(self, x: np.ndarray) -> np.ndarray:
        """One drift step x + drift*z for a reused plan (fresh draws)."""
        z = self.rng.standard_normal(x.shape, dtype=np.float32)
        return x + np.float32(self.wl.drift) * z


def make_qkv(wl: Workload, heads: Optional[int] = None
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full [B, H', N, D] float32 q, k, v, already rounded to the storage dtype.

    ``heads`` limits generation to the first H' heads of batch 0 (the draw
    order is the same as for the full tensor, so head h is identical either
    way).
    """
    H = wl.H if heads is None else heads
    B = wl.B if heads is None else 1
    q = np.empty((B, H, wl.N, wl.D), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    gen = Generator(wl)
    for b, h, qh, kh, vh in gen.iter_heads():
        if b >= B or h >= H:
            break                       # heads come in order: the subset is done
        q[b, h] = round_like(qh, wl.dtype)
        k[b, h] = round_like(kh, wl.dtype)
        v[b, h] = round_like(vh, wl.dtype)
    return q, k, v


def make_qkv_sequence(wl: Workload, calls: int, heads: Optional[int] = None
                      ) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """q/k/v for ``calls`` consecutive calls that share one plan.

    Call 0 is ``make_qkv``; each later call adds drift*z to the float32 master
    q and k (fresh draws from the same generator, q before k, head by head)
    and re-rounds; v is unchanged.
    """
    H = wl.H if heads is None else heads
    B = wl.B if heads is None else 1
    gen = Generator(wl)
    qm = np.empty((B, H, wl.N, wl.D), dtype=np.float32)
    km = np.empty_like(qm)
    vm = np.empty_like(qm)
    for b, h, qh, kh, vh in gen.iter_heads():
        if b < B and h < H:
            qm[b, h], km[b, h], vm[b, h] = qh, kh, vh
    out = []
    v = round_like(vm, wl.dtype)
    shape = (wl.N, wl.D)
    for c in range(calls):
        if c > 0:
            # draws for every head in order (so a subset matches the full layer)
            for b in range(wl.B):
                for h in range(wl.H):
                    if b < B and h < H:
                        qm[b, h] = gen.drift(qm[b, h])
                        km[b, h] = gen.drift(km[b, h])
                    else:
                        gen.drift(np.zeros(shape, dtype=np.float32))
                        gen.drift(np.zeros(shape, dtype=np.float32))
        out.append((round_like(qm, wl.dtype), round_like(km, wl.dtype), v))
    return out


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the arrays (input-stability pin)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def random_scores(rows: int, n: int, seed: int, spread: float = 3.0) -> np.ndarray:
    """Positive float32 score rows that sum to ~1, log-normal spread.

    Stand-in for selector output when testing the sampler on its own.
    """
    rng = np.random.default_rng(seed)
    x = np.exp(spread * rng.standard_normal((rows, n)))
    x /= x.sum(axis=1, keepdims=True)
    return x.astype(np.float32)
