"""Step policy for a denoising loop: when to run dense attention, when to
build a new sampling plan and when to reuse the last one.

Source: news.hamidun.com, "AB-Attention speeds up video generation by up to
2.23x and skips 92% of attention":
  * section "AB-Attention's three techniques": the sampling plan is rebuilt
    once every four denoising steps while the attention itself runs at every
    step;
  * section "How it was measured and what came out": in the evaluation the
    opening transformer block (all steps) and steps 0-9 of the 50 run dense
    (for every method compared).
Readings where the pages are silent:
  * a plan belongs to one transformer block (each block has its own q/k);
    the first sparse step of a block builds it, the next ``plan_every - 1``
    steps of that block reuse it;
  * each rebuilt plan draws with a fresh seed, derived from the base seed, the
    block and the plan's ordinal by SplitMix64 (Steele et al., OOPSLA 2014),
    so runs are reproducible and plans of different blocks/steps independent;
  * text tokens sit at the tail of the sequence; their key blocks are always
    kept (forced tail), as for the HunyuanVideo shape.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import torch

from . import Plan, Problem, attend, dense, plan, v_to_f16

DENSE, BUILD, REUSE = "dense", "build", "reuse"

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One SplitMix64 output for state x (Steele, Lea, Flood, OOPSLA 2014)."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


@dataclasses.dataclass(frozen=True)
class StepPolicy:
    """Which attention a (step, block) call gets; steps and blocks count from 0."""

    total_steps: int = 50
    dense_steps: int = 10      # the first steps run dense in every block
    dense_blocks: int = 1      # the first blocks run dense at every step
    plan_every: int = 4        # a plan serves this many consecutive sparse steps
    budget: float = 0.10
    base_seed: int = 0

    def __post_init__(self):
        if self.plan_every < 1 or self.dense_steps < 0 or self.dense_blocks < 0:
            raise ValueError("plan_every >= 1, dense_steps >= 0, dense_blocks >= 0")
        if not 0.0 < self.budget <= 1.0:
            raise ValueError("budget must be in (0, 1]")

    def mode(self, step: int, block: int) -> str:
        """DENSE, BUILD (a new plan at this step) or REUSE (the block's last plan)."""
        if step < 0 or block < 0:
            raise ValueError("step and block count from 0")
        if step < self.dense_steps or block < self.dense_blocks:
            return DENSE
        return BUILD if (step - self.dense_steps) % self.plan_every == 0 else REUSE

    def plan_index(self, step: int) -> int:
        """Ordinal of the plan serving a sparse step (0 for the first plan)."""
        return (step - self.dense_steps) // self.plan_every

    def seed(self, step: int, block: int) -> int:
        """Sampler seed of the plan serving (step, block): fresh per plan and block."""
        k = self.plan_index(step)
        return splitmix64(splitmix64(splitmix64(self.base_seed & _M64) ^ block) ^ k)

    def counts(self, n_blocks: int) -> Dict[str, int]:
        """How many calls of a full run (total_steps x n_blocks) get each mode."""
        out = {DENSE: 0, BUILD: 0, REUSE: 0}
        for s in range(self.total_steps):
            for b in range(n_blocks):
                out[self.mode(s, b)] += 1
        return out


class ABAttention:
    """Attention callable for a DiT loop: ``o = attn(q, k, v, block)``.

    q, k, v: contiguous [B, H, N, D] device tensors (bf16 or fp32), the last
    ``n_text`` tokens being text.  Call ``set_step(s)`` before the blocks of
    denoising step s.  Each call runs the library's dense kernel, builds a new
    plan (abatt_plan) and attends with it, or attends with the block's cached
    plan (abatt_attend), as the policy says.  Plans stay on the device between
    steps.  A plan that outgrew its capacity raises, without stalling the
    host at every build: its status is copied to pinned host memory behind an
    event, and checked at the next call once that event has completed (and at
    the block's next build, or by ``check()``, which waits).  An overflowed
    plan makes attention return zeros for the calls made before the error
    surfaces.  For bf16 inputs every call converts V to fp16 once and uses
    the attention's fp16-V forms (abatt_v_to_f16 + abatt_attend_v16 or
    abatt_dense_v16: the same results, faster kernels) unless ``fp16_v`` is
    False.
    """

    def __init__(self, policy: StepPolicy = StepPolicy(), n_text: int = 0,
                 n_clusters: int = 8, kmeans_iters: int = 10, fp16_v: bool = True):
        if n_text % 4:
            raise ValueError("text tokens must fill whole 4-token key blocks")
        self.policy = policy
        self.n_text = n_text
        self.n_clusters = n_clusters
        self.kmeans_iters = kmeans_iters
        self.fp16_v = fp16_v
        self.step = 0
        self._plans: Dict[int, Tuple[int, Plan, Problem]] = {}
        self._v16: Optional[torch.Tensor] = None   # reused fp16 copy of V
        # plan status checks in flight: block -> (event, pinned int32 [1], step)
        self._pending: Dict[int, Tuple[torch.cuda.Event, torch.Tensor, int]] = {}
        self._status_host: Dict[int, torch.Tensor] = {}
        self.log: list = []    # (step, block, mode) of every call

    def set_step(self, step: int) -> None:
        self.step = step

    def _check_block(self, block: int, wait: bool) -> None:
        entry = self._pending.get(block)
        if entry is None:
            return
        ev, host, step = entry
        if not wait and not ev.query():
            return
        ev.synchronize()
        del self._pending[block]
        if int(host[0]) != 0:
            raise RuntimeError(f"the plan of block {block} built at step {step} outgrew its "
                               "capacity (its attention calls returned zeros)")

    def check(self) -> None:
        """Waits for every plan-status check in flight; raises on an overflow."""
        for block in list(self._pending):
            self._check_block(block, wait=True)

    def problem(self, q: torch.Tensor) -> Problem:
        return Problem.like(q, n_forced_tail=self.n_text, n_clusters=self.n_clusters,
                            kmeans_iters=self.kmeans_iters)

    def plan_of(self, block: int) -> Optional[Plan]:
        entry = self._plans.get(block)
        return None if entry is None else entry[1]

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int,
                 return_lse: bool = False):
        for b in list(self._pending):       # completed checks only: no host stall
            self._check_block(b, wait=False)
        mode = self.policy.mode(self.step, block)
        prob = self.problem(q)
        if mode == REUSE:
            entry = self._plans.get(block)
            if entry is None or entry[2] != prob:
                mode = BUILD   # no usable plan (first call after a skipped build, or new shape)
        self.log.append((self.step, block, mode))
        if self.fp16_v and v.dtype == torch.bfloat16:
            if self._v16 is None or self._v16.shape != v.shape or self._v16.device != v.device:
                self._v16 = torch.empty(v.shape, dtype=torch.float16, device=v.device)
            v = v_to_f16(v, prob, out=self._v16)
        if mode == DENSE:
            return dense(q, k, v, problem=prob, return_lse=return_lse)
        if mode == BUILD:
            old = self._plans.get(block)
            reuse_buf = old[1] if old is not None and old[2] == prob else None
            self._check_block(block, wait=True)   # the last build's copy (long finished)
            pl = plan(q, k, self.policy.budget, seed=self.policy.seed(self.step, block),
                      problem=prob, out=reuse_buf)
            host = self._status_host.get(block)
            if host is None:
                host = torch.empty(1, dtype=torch.int32, pin_memory=True)
                self._status_host[block] = host
            host.copy_(pl.status, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self._pending[block] = (ev, host, self.step)
            self._plans[block] = (self.step, pl, prob)
        return attend(q, k, v, self._plans[block][1], problem=prob, return_lse=return_lse)
