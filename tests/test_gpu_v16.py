"""The fp16-V forms of the attention: abatt_v_to_f16, then abatt_attend_v16
(gathered rows) or abatt_dense_v16 (every key).

* the conversion against an independent reference: bf16 -> fp16 rounded
  toward zero (NumPy's round-to-nearest, stepped one fp16 ulp toward zero
  where it rounded away), over normal, subnormal and overflowing magnitudes,
  signed zeros, infinities and NaN;
* attention on the converted V is bit-identical to abatt_attend on the bf16 V
  (output and log-sum-exp), for D = 128 and 64, several key-block sizes, text
  tokens, and values beyond fp16's range;
* and against the oracle, at the bf16 bar (max-abs 1e-2, mean-rel 1e-3);
* dense attention on the converted V is bit-identical to abatt_dense (output
  and log-sum-exp), for D = 128 and 64 and token counts that are not a
  multiple of the 64-key chunk or of 4.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import LSE_TOL, check_output, lib_problem, oracle_problem, plan_to_host, say, to_dev
from workloads import Workload, make_qkv, round_like

pytestmark = pytest.mark.gpu

ab = pytest.importorskip("block_sparse_attention_09_amd")


def rtz_f16(x: np.ndarray) -> np.ndarray:
    """float64 values -> float16, rounded toward zero."""
    with np.errstate(over="ignore"):
        y = x.astype(np.float16)
    away = np.isfinite(x) & (np.abs(y.astype(np.float64)) > np.abs(x))
    return np.where(away, np.nextafter(y, np.float16(0)), y).astype(np.float16)


def test_v_to_f16_rounds_toward_zero():
    rng = np.random.default_rng(11)
    n = 64 * 128 * 16
    # magnitudes 2^-40 .. 2^40 (fp16 subnormals, normals, overflow), both signs
    mag = np.exp2(rng.uniform(-40.0, 40.0, n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.0, 65520.0, 1e38,
                        2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3.0 * 2.0 ** -26, -6.0e-8],
                       dtype=np.float32)
    x[:special.size] = special
    x = round_like(x, "bf16")
    prob = ab.Problem(1, 16, 64, 128)
    v = torch.from_numpy(x.reshape(1, 16, 64, 128)).to(torch.bfloat16).cuda()
    got = ab.v_to_f16(v, prob)
    torch.cuda.synchronize()
    got = got.cpu().numpy().reshape(-1)
    ref = rtz_f16(x.astype(np.float64))
    nan = np.isnan(x)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.nonzero(got[~nan].view(np.uint16) != ref[~nan].view(np.uint16))[0]
    say(f"v_to_f16: {n} values, {bad.size} differ from round-toward-zero")
    assert bad.size == 0, (x[~nan][bad[:5]], got[~nan][bad[:5]], ref[~nan][bad[:5]])


CASES = {
    "bf16_d128": Workload("v1", B=1, H=2, D=128, grid=(3, 16, 32)),
    "bf16_d128_text": Workload("v2", B=1, H=2, D=128, grid=(2, 16, 32), n_text=64),
    "bf16_d128_kb16": Workload("v3", B=1, H=2, D=128, grid=(2, 16, 32), kv_block=16),
    "bf16_d128_kb128": Workload("v4", B=1, H=1, D=128, grid=(8, 16, 32), kv_block=128),
    "bf16_d64": Workload("v5", B=2, H=1, D=64, grid=(2, 16, 32)),
    "bf16_d64_kb32": Workload("v6", B=1, H=2, D=64, grid=(2, 16, 32), kv_block=32),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("budget", [0.1, 1.0])
def test_attend_v16_is_bit_identical(name, budget):
    wl = CASES[name]
    q, k, v = make_qkv(wl)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    pl = ab.plan(dq, dk, budget, seed=5, problem=prob)
    o, lse = ab.attend(dq, dk, dv, pl, problem=prob, return_lse=True)
    v16 = ab.v_to_f16(dv, prob)
    o16, lse16 = ab.attend(dq, dk, v16, pl, problem=prob, return_lse=True)
    torch.cuda.synchronize()
    say(f"v16 {name} budget {budget}: nnz {pl.nnz()}")
    assert torch.equal(o16, o)
    assert torch.equal(lse16, lse)


def test_attend_v16_large_values_bit_identical():
    # |v| up to 1e6: beyond fp16's range both forms saturate the same way
    wl = CASES["bf16_d128"]
    q, k, _ = make_qkv(wl)
    rng = np.random.default_rng(3)
    v = round_like((rng.standard_normal(q.shape) * np.exp2(rng.uniform(-4, 20, q.shape)))
                   .astype(np.float32), "bf16")
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    pl = ab.plan(dq, dk, 0.2, seed=1, problem=prob)
    o = ab.attend(dq, dk, dv, pl, problem=prob)
    o16 = ab.attend(dq, dk, ab.v_to_f16(dv, prob), pl, problem=prob)
    torch.cuda.synchronize()
    assert torch.equal(o16, o)


def test_attend_v16_against_oracle():
    wl = CASES["bf16_d128_text"]
    q, k, v = make_qkv(wl)
    op = oracle_problem(wl)
    prob = lib_problem(wl)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    pl = ab.plan(dq, dk, 0.15, seed=2, problem=prob)
    o, lse = ab.attend(dq, dk, ab.v_to_f16(dv, prob), pl, problem=prob, return_lse=True)
    torch.cuda.synchronize()
    rp, ci, lw = plan_to_host(pl)
    O, L = oracle.attend(q, k, v, oracle.Plan(rp.astype(np.int64), ci, lw), op)
    check_output(o, O, "bf16", "attend v16")
    lse_h = lse.cpu().numpy()
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lse_h), fin)
    assert np.abs(lse_h[fin] - L[fin]).max(initial=0.0) <= LSE_TOL["bf16"]


def test_v16_rejects_fp32_and_wrong_shapes():
    p32 = ab.Problem(1, 1, 256, 64, dtype="f32")
    v = torch.zeros(1, 1, 256, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        ab.v_to_f16(v, p32)
    pb = ab.Problem(1, 1, 256, 64)
    with pytest.raises(ValueError):
        ab.v_to_f16(torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16, device="cuda"), pb,
                    out=torch.empty(1, 1, 256, 32, dtype=torch.float16, device="cuda"))


@pytest.mark.parametrize("D,N", [(128, 2048), (128, 1150), (64, 1027), (64, 300)])
def test_dense_v16_is_bit_identical(D, N):
    rng = np.random.default_rng(D + N)
    q, k, v = (round_like(rng.standard_normal((1, 2, N, D)).astype(np.float32), "bf16")
               for _ in range(3))
    prob = ab.Problem(1, 2, N, D)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    say(f"dense fp16-V D={D} N={N}")
    o, lse = ab.dense(dq, dk, dv, problem=prob, return_lse=True)
    o16, lse16 = ab.dense(dq, dk, ab.v_to_f16(dv, prob), problem=prob, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o16, o)
    assert torch.equal(lse16, lse)
