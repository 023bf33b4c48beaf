"""CPU oracle for the AB-Attention hot path: TEST INFRASTRUCTURE ONLY.

Plain NumPy, float64 arithmetic.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and this module imports nothing from it.

Pages cited (the method's only description available here):
  [hamidun]  news.hamidun.com, "AB-Attention speeds up video generation by up
             to 2.23x and skips 92% of attention"
  [zerohour] zerohour.day, "AB-Attention approximates dense video attention at
             high sparsity"

AB-Attention is an approximation reached by a heuristic selector plus random
sampling, so this oracle is the algorithm written out step by step, in the
pages' order: key-block means -> per-query-block k-means -> cluster-weighted
block scores (IBCS) -> inclusion probabilities proportional to score, capped
at 1 -> Philox draws -> CSR plan with log-weights (SIP) -> softmax attention
with a logit shift over the gathered 4-token blocks.

Readings of what the pages leave open (each also listed with its reason in
the design notes):
  * tokens stay in raster order; query block qb = tokens [128qb, 128qb+128),
    the last one partial; key block j = tokens [4j, 4j+4);
  * k-means: squared Euclidean distance on the raw query rows, init at the
    evenly spaced members X[floor(c*n/C)], ties to the smaller cluster index,
    an empty cluster keeps its centroid, weights from the last assignment;
  * score of key block j: sum_c w_c softmax_j(scale * mu_c . mean_key_j),
    normalised per centroid over the sparse key blocks, then rounded to fp32;
  * budget b means m = b * n_sparse_blocks expected blocks per row; b = 1
    takes every block; independent (Poisson) draws, so the row count varies;
  * randomness: Philox4x32-10, counter (j//4, qb, h, b), key (seed low,
    seed high); word j%4 is block j's 32-bit uniform integer w, and the
    block is kept iff w < pi * 2^32 (exact in float64), so it enters with
    probability ceil(pi * 2^32) / 2^32, within 2^-32 of pi;
  * trailing text tokens (if any) form forced key blocks with pi = 1 that are
    not scored and not counted in the budget.

Parity unpinned: how well a plan keeps attention mass on real model
activations (the pages' recall and error percentages) -- those need trained
weights that are not available; nothing here claims to reproduce them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

@dataclasses.dataclass(frozen=True)
class Problem:
    """Sizes and hyper-parameters of one attention layer ([B, H, N, D])."""

    B: int
    H: int
    N: int
    D: int
    q_block: int = 128        # [hamidun] three techniques, IBCS: 128-token query blocks
    kv_block: int = 4         # [hamidun] three techniques, third technique: 4-token K/V blocks
    n_clusters: int = 8       # [hamidun] three techniques, IBCS: 8 clusters per query block
    kmeans_iters: int = 10
    n_forced_tail: int = 0    # trailing tokens whose key blocks are always kept
    scale: Optional[float] = None

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale is None else float(self.scale)

    @property
    def n_qb(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def n_kbs(self) -> int:
        """Sparse (scored, sampled) key blocks."""
        return (self.N - self.n_forced_tail) // self.kv_block

    @property
    def n_kb(self) -> int:
        """All key blocks, forced ones included (they come last)."""
        return self.n_kbs + self.n_forced_tail // self.kv_block

    @property
    def R(self) -> int:
        return self.B * self.H * self.n_qb

    def check(self) -> None:
        assert self.N > 0 and self.D > 0 and self.B > 0 and self.H > 0
        assert self.n_forced_tail % self.kv_block == 0
        assert (self.N - self.n_forced_tail) % self.kv_block == 0
        assert self.n_kbs > 0 and self.kmeans_iters >= 1 and self.n_clusters >= 1


@dataclasses.dataclass
class Plan:
    """CSR sampling plan: row r = (b*H + h)*n_qb + qb."""

    row_ptr: np.ndarray   # int64 [R+1]
    col_idx: np.ndarray   # int32 [nnz], ascending within a row
    logw: np.ndarray      # float32 [nnz], log(1/pi) of the block

    def row(self, r: int) -> Tuple[np.ndarray, np.ndarray]:
        a, b = int(self.row_ptr[r]), int(self.row_ptr[r + 1])
        return self.col_idx[a:b], self.logw[a:b]


# --------------------------------------------------------------------------
# IBCS: key-block means, per-query-block k-means, block scores
# [hamidun] "AB-Attention's three techniques", IBCS paragraph
# --------------------------------------------------------------------------

def key_block_means(K: np.ndarray, prob: Problem) -> np.ndarray:
    """Mean key of every sparse 4-token key block: [B, H, n_kbs, D] float64.

    [hamidun] three techniques: a key block is scored through its averaged
    keys; the blocks are 4 consecutive tokens (third technique).
    """
    kb, n = prob.kv_block, prob.n_kbs
    Ks = np.asarray(K, dtype=np.float64)[:, :, : n * kb, :]
    return Ks.reshape(K.shape[0], K.shape[1], n, kb, K.shape[3]).mean(axis=3)


def kmeans(X: np.ndarray, C: int, iters: int) -> Tuple[np.ndarray, np.ndarray]:
    """Lloyd k-means on the rows of X (n x D).  Returns (centroids, counts).

    [hamidun] three techniques, IBCS: the queries of a block are grouped into
    clusters; each cluster keeps a centroid and the share of queries in it.
    Init: centroid c starts at X[floor(c*n/C)].  Each iteration assigns every
    row to its nearest centroid (squared Euclidean, computed from the
    differences; ties go to the lower index) and moves each centroid to the
    mean of its members; a centroid with no members stays where it is.  The
    counts are those of the last assignment, the one averaged into the
    returned centroids.
    """
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    mu = X[[(c * n) // C for c in range(C)]].copy()
    assign = np.zeros(n, dtype=np.int64)
    for _ in range(iters):
        diff = X[:, None, :] - mu[None, :, :]
        dist = (diff * diff).sum(axis=2)            # [n, C]
        assign = np.argmin(dist, axis=1)            # first minimum on ties
        for c in range(C):
            members = X[assign == c]
            if members.shape[0] > 0:
                mu[c] = members.mean(axis=0)
    counts = np.bincount(assign, minlength=C)
    return mu, counts


def query_clusters(Q: np.ndarray, prob: Problem, rows: Optional[List[int]] = None
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """k-means of every query block (or of the listed plan rows).

    Returns centroids [R', C, D] float64, weights [R', C] float64 (share of the
    block's queries) and counts [R', C] int64.
    """
    rows = range(prob.R) if rows is None else rows
    mus, ws, cnts = [], [], []
    for r in rows:
        b, h, qb = unflatten_row(prob, r)
        X = Q[b, h, qb * prob.q_block: min((qb + 1) * prob.q_block, prob.N)]
        mu, counts = kmeans(X, prob.n_clusters, prob.kmeans_iters)
        mus.append(mu)
        cnts.append(counts)
        ws.append(counts / float(X.shape[0]))
    return np.array(mus), np.array(ws), np.array(cnts)


def block_scores(mu: np.ndarray, w: np.ndarray, kbar: np.ndarray, tau: float) -> np.ndarray:
    """s_j = sum_c w_c softmax_j(tau * mu_c . kbar_j) over the sparse key blocks j.

    [hamidun] three techniques, IBCS.  Every centroid mu_c of the query
    block spreads one softmax over the means kbar_j of all sparse key blocks;
    the block scores are those probabilities summed with the cluster shares
    w_c as weights (so they sum to 1).  Returns float64 [n_kbs].
    """
    logits = tau * (mu @ kbar.T)                        # [C, n_kbs]
    shifted = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(shifted)
    p = e / e.sum(axis=1, keepdims=True)
    return w @ p


def ibcs_scores(Q: np.ndarray, K: np.ndarray, prob: Problem,
                rows: Optional[List[int]] = None) -> dict:
    """Scores of every plan row (or the listed rows), as float64 and fp32.

    The fp32 copy (round to nearest even) is the value both samplers consume.
    """
    prob.check()
    rows = list(range(prob.R)) if rows is None else list(rows)
    kbar = {}                       # key means of the heads the rows need
    for r in rows:
        b, h, _ = unflatten_row(prob, r)
        if (b, h) not in kbar:
            kbar[(b, h)] = key_block_means(K[b:b + 1, h:h + 1], prob)[0, 0]
    mu, w, counts = query_clusters(Q, prob, rows)
    S = np.empty((len(rows), prob.n_kbs), dtype=np.float64)
    for i, r in enumerate(rows):
        b, h, _ = unflatten_row(prob, r)
        S[i] = block_scores(mu[i], w[i], kbar[(b, h)], prob.tau)
    return {"rows": rows, "kbar": kbar, "mu": mu, "w": w, "counts": counts,
            "S": S, "S32": S.astype(np.float32)}


# --------------------------------------------------------------------------
# SIP: inclusion probabilities, Philox draws, CSR plan with log-weights
# [hamidun] "AB-Attention's three techniques", SIP paragraph
# --------------------------------------------------------------------------

def inclusion_probabilities(s32: np.ndarray, budget: float) -> np.ndarray:
    """pi_j proportional to the score, capped at 1, summing to the budget.

    [hamidun] three techniques, SIP: pi scales with the block's score, is
    capped at 1 for the top-scored blocks (always drawn), and stays above zero
    for every other block with a positive score.  With m = budget * n
    expected blocks, start with no certain blocks and repeat: c = (m - #certain)
    / (sum of the scores of the uncertain positive blocks); every uncertain
    block with c*s >= 1 becomes certain; stop when none does.  Then pi = 1 on
    the certain set, c*s elsewhere (0 where s = 0).  budget >= 1 keeps every
    block; m >= #positive keeps every positive block.  float64 throughout.
    """
    s = np.asarray(s32, dtype=np.float32).astype(np.float64)
    n = s.shape[0]
    m = float(budget) * float(n)
    if m >= n:
        return np.ones(n, dtype=np.float64)
    pos = s > 0
    if m >= int(pos.sum()):
        return pos.astype(np.float64)
    certain = np.zeros(n, dtype=bool)
    c = 0.0
    while True:
        rest = pos & ~certain
        if not rest.any():
            break
        c = (m - float(certain.sum())) / math.fsum(s[rest].tolist())
        new = rest & (c * s >= 1.0)
        if not new.any():
            break
        certain |= new
    return np.where(certain, 1.0, np.where(pos & ~certain, c * s, 0.0))


# Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy
# as 1, 2, 3", SC'11): per round two 32x32->64 multiplies of counter words 0
# and 2 by fixed multipliers, the high halves XORed into the other words with
# the key, a Weyl key schedule between rounds, ten rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
M32 = 0xFFFFFFFF


def philox4x32_10(ctr: Tuple[np.ndarray, ...], key: Tuple[int, int]) -> Tuple[np.ndarray, ...]:
    """Philox4x32 with 10 rounds on arrays of counters (32-bit words held in
    uint64); returns the 4 output words (uint64 arrays, values < 2^32)."""
    m32 = np.uint64(M32)
    s32 = np.uint64(32)
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & m32 for x in ctr)
    k0, k1 = key[0] & M32, key[1] & M32
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & M32
            k1 = (k1 + PHILOX_W1) & M32
        p0 = c0 * np.uint64(PHILOX_M0)      # < 2^64: exact in uint64
        p1 = c2 * np.uint64(PHILOX_M1)
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ np.uint64(k0), p1 & m32,
                          (p0 >> s32) ^ c3 ^ np.uint64(k1), p0 & m32)
    return c0, c1, c2, c3


def block_words(b: int, h: int, qb: int, n: int, seed: int) -> np.ndarray:
    """32-bit uniform integers (uint64 holding values < 2^32) for sparse key
    blocks 0..n-1 of a row: block j is word j%4 of Philox4x32-10 with counter
    (j//4, qb, h, b) and key (low, high 32 bits of the seed)."""
    quads = -(-n // 4)
    g = np.arange(quads, dtype=np.uint64)
    z = np.zeros(quads, dtype=np.uint64)
    w = philox4x32_10((g, z + np.uint64(qb), z + np.uint64(h), z + np.uint64(b)),
                      (seed & M32, (seed >> 32) & M32))
    return np.stack(w, axis=1).reshape(-1)[:n]


def sample_row(s32: np.ndarray, budget: float, b: int, h: int, qb: int, seed: int,
               n_forced_blocks: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """One plan row: ascending key-block ids and fp32 log-weights.

    [hamidun] three techniques, SIP: each block enters independently with
    probability pi; a kept block is weighted by 1/pi (Horvitz-Thompson),
    applied as the logit shift log(1/pi).  Block j is kept iff its 32-bit
    uniform integer w satisfies w < pi * 2^32 (exact in float64).  Forced
    blocks (ids n..n+n_forced_blocks-1) are always kept with weight 1.
    """
    n = s32.shape[0]
    pi = inclusion_probabilities(s32, budget)
    w = block_words(b, h, qb, n, seed).astype(np.float64)
    keep = w < pi * float(1 << 32)
    idx = np.nonzero(keep)[0]
    pik = pi[idx]
    lw = np.where(pik == 1.0, 0.0, -np.log(np.where(pik == 1.0, 1.0, pik)))
    cols = np.concatenate([idx, n + np.arange(n_forced_blocks)]).astype(np.int32)
    logw = np.concatenate([lw, np.zeros(n_forced_blocks)]).astype(np.float32)
    return cols, logw


def plan_from_scores(S32: np.ndarray, prob: Problem, budget: float, seed: int,
                     rows: Optional[List[int]] = None) -> Plan:
    """CSR plan from fp32 scores [R', n_kbs] (all rows, or the listed ones)."""
    rows = list(range(prob.R)) if rows is None else list(rows)
    n_forced = prob.n_kb - prob.n_kbs
    ptr = [0]
    cols, lws = [], []
    for i, r in enumerate(rows):
        b, h, qb = unflatten_row(prob, r)
        c, lw = sample_row(S32[i], budget, b, h, qb, seed, n_forced)
        cols.append(c)
        lws.append(lw)
        ptr.append(ptr[-1] + c.shape[0])
    return Plan(np.array(ptr, dtype=np.int64),
                np.concatenate(cols) if cols else np.zeros(0, np.int32),
                np.concatenate(lws) if lws else np.zeros(0, np.float32))


def plan(Q: np.ndarray, K: np.ndarray, prob: Problem, budget: float, seed: int,
         rows: Optional[List[int]] = None) -> Plan:
    """IBCS scores followed by SIP sampling: the full selector."""
    sc = ibcs_scores(Q, K, prob, rows)
    return plan_from_scores(sc["S32"], prob, budget, seed, sc["rows"])


# --------------------------------------------------------------------------
# Attention over the plan, and dense attention
# [hamidun] three techniques, SIP (logit shift) and third technique (gather);
# [zerohour] key facts (sub-tile K/V blocks packed into full tiles)
# --------------------------------------------------------------------------

def unflatten_row(prob: Problem, r: int) -> Tuple[int, int, int]:
    bh, qb = divmod(r, prob.n_qb)
    b, h = divmod(bh, prob.H)
    return b, h, qb


def attend_row(Q: np.ndarray, K: np.ndarray, V: np.ndarray, prob: Problem, r: int,
               cols: np.ndarray, logw: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query block over its selected key blocks.

    For query i and selected key token t in block j(t):
        z_t = tau * q_i.k_t + logw_j(t)
        o_i = sum_t exp(z_t - M) v_t / sum_t exp(z_t - M),  LSE_i = M + log l.
    An empty selection gives o = 0 and LSE = -inf.
    """
    b, h, qb = unflatten_row(prob, r)
    lo, hi = qb * prob.q_block, min((qb + 1) * prob.q_block, prob.N)
    q = np.asarray(Q[b, h, lo:hi], dtype=np.float64)
    if cols.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    kb = prob.kv_block
    tok = (cols.astype(np.int64)[:, None] * kb + np.arange(kb)[None, :]).reshape(-1)
    k = np.asarray(K[b, h, tok], dtype=np.float64)
    v = np.asarray(V[b, h, tok], dtype=np.float64)
    shift = np.repeat(np.asarray(logw, dtype=np.float64), kb)
    z = prob.tau * (q @ k.T) + shift[None, :]
    M = z.max(axis=1, keepdims=True)
    e = np.exp(z - M)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (M + np.log(l))[:, 0]


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, plan: Plan, prob: Problem,
           rows: Optional[List[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O [B,H,N,D] float64 and LSE [B,H,N] for the plan's rows.

    With ``rows`` given, only those rows are computed (plan row i belongs to
    rows[i] when the plan was built for the same list); other outputs are NaN.
    """
    B, H, N, D = prob.B, prob.H, prob.N, prob.D
    O = np.full((B, H, N, D), np.nan)
    L = np.full((B, H, N), np.nan)
    rows = list(range(prob.R)) if rows is None else list(rows)
    for i, r in enumerate(rows):
        cols, lw = plan.row(i)
        o, lse = attend_row(Q, K, V, prob, r, cols, lw)
        b, h, qb = unflatten_row(prob, r)
        lo = qb * prob.q_block
        O[b, h, lo:lo + o.shape[0]] = o
        L[b, h, lo:lo + o.shape[0]] = lse
    return O, L


def dense_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, prob: Problem,
               b: int, h: int, qi: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Full softmax attention of the listed queries of head (b, h) over every key.

    o_i = sum_t exp(tau q_i.k_t - M) v_t / sum_t exp(tau q_i.k_t - M).
    """
    q = np.asarray(Q[b, h, qi], dtype=np.float64)
    k = np.asarray(K[b, h], dtype=np.float64)
    v = np.asarray(V[b, h], dtype=np.float64)
    z = prob.tau * (q @ k.T)
    M = z.max(axis=1, keepdims=True)
    e = np.exp(z - M)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (M + np.log(l))[:, 0]


def dense(Q: np.ndarray, K: np.ndarray, V: np.ndarray, prob: Problem
          ) -> Tuple[np.ndarray, np.ndarray]:
    """Dense attention over all tokens: the 100%-density path."""
    B, H, N, D = prob.B, prob.H, prob.N, prob.D
    O = np.empty((B, H, N, D))
    L = np.empty((B, H, N))
    step = 1024
    for b in range(B):
        for h in range(H):
            for lo in range(0, N, step):
                qi = np.arange(lo, min(lo + step, N))
                O[b, h, qi], L[b, h, qi] = dense_rows(Q, K, V, prob, b, h, qi)
    return O, L


# --------------------------------------------------------------------------
# Horvitz-Thompson probes (test-only quantities)
# --------------------------------------------------------------------------

def ht_estimates(o: np.ndarray, lse: np.ndarray, m_ref: np.ndarray
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Numerator and normaliser estimates with a fixed reference shift.

    D_hat = exp(LSE - M*), N_hat = o * D_hat.  Their expectations over the
    draws equal the dense sums exp(tau q.k - M*) v and exp(tau q.k - M*):
    [hamidun] three techniques, SIP: both the numerator and the softmax
    normalisation are estimated without bias.  The ratio o is not.
    """
    d_hat = np.exp(lse - m_ref)
    return o * d_hat[..., None], d_hat
