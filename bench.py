"""Benchmark of the AB-Attention hot path on one MI355X.

One step = abatt_plan (IBCS selector + SIP sampler), then, for bf16 layers,
abatt_v_to_f16 (V to fp16 once per call) and abatt_attend_v16 (gathered
sparse attention, bit-identical to abatt_attend), over one synthetic layer,
inputs already resident in HBM.  Default workload: the Wan2.1-14B 720p layer shape (B=1, 40 heads,
75600 tokens = 21x45x80 latent grid, D=128, bf16) at a 10% block budget.

Printed: one JSON line with the step throughput as dense-equivalent TFLOP/s
(4*B*H*N^2*D per step / step time), the per-call times of attend, the V
conversion, plan, attend + conversion + plan/4 (one plan every four denoising
steps) and the library's own dense kernel, the roofline of the attention
kernel (HIP events around each attention launch on the stream it runs on), and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload wan14b_720p] [--budget 0.10]
    python bench.py --probe copy     # plain device copy, for counter calibration
    python bench.py --record-traffic DIR   # write the attention kernel's HBM traffic record
                                           # from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, Generator, Workload  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
# one (query block, key block) pair of kb keys: QK^T + PV over 128 queries
PAIR_FLOP = lambda D, kb=4: 4 * 128 * kb * D
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(wl: Workload, torch, heads=None):
    """q, k, v bf16 [B,H,N,D] on the GPU, generated head by head on the host."""
    H = wl.H if heads is None else heads
    shape = (wl.B, H, wl.N, wl.D)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = torch.empty(shape, dtype=dt, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    gen = Generator(wl)
    for b, h, qh, kh, vh in gen.iter_heads():
        if h >= H:
            break
        q[b, h].copy_(torch.from_numpy(qh).to(dt))
        k[b, h].copy_(torch.from_numpy(kh).to(dt))
        v[b, h].copy_(torch.from_numpy(vh).to(dt))
    return q, k, v


def src_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def cpu_baseline(wl: Workload, budget: float, dense_flop_per_head: float):
    """The oracle (NumPy fp64) on one head of the workload: plan + attend."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    host_cores = len(os.sched_getaffinity(0))
    from workloads import make_qkv
    q, k, v = make_qkv(wl, heads=1)
    op = oracle.Problem(B=1, H=1, N=wl.N, D=wl.D, kv_block=wl.kv_block, n_clusters=wl.n_clusters,
                        kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text)
    rows = list(range(op.R))
    t0 = time.perf_counter()
    pl = oracle.plan(q, k, op, budget, wl.plan_seed, rows=rows)
    t1 = time.perf_counter()
    oracle.attend(q, k, v, pl, op, rows=rows)
    t2 = time.perf_counter()
    sec = t2 - t0
    # the oracle's matrix products run on the BLAS threads; the rest of it is
    # single-threaded NumPy, so the BLAS thread count is what it used
    return {
        "value": dense_flop_per_head / sec / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(threads),
        "blas_threads": int(threads),
        "host_cores": int(host_cores),
        "kind": "oracle",
        "sample": f"1 of {wl.H * wl.B} heads ({op.R} plan rows) of {wl.name}: oracle.plan + "
                  f"oracle.attend at budget {budget}; plan {t1 - t0:.1f} s, attend "
                  f"{t2 - t1:.1f} s; value is that head's rate, extrapolated to the layer "
                  f"(heads are independent units of the same work)",
        "extrapolated": True,
        "ms_per_call_extrapolated": sec * wl.H * wl.B * 1e3,
    }


def probe_copy(torch, steps: int):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": ms,
                      "GB/s": 2 * n / ms / 1e6}))


ATTEND_KERNEL = "abatt::k_attend_bf16<128, true, true>"
TRAFFIC_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch -- "
    "python3 -u bench.py --steps 2 --warmup 1 --no-cpu --no-dense",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write -- "
    "python3 -u bench.py --steps 2 --warmup 1 --no-cpu --no-dense",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copyf -o copyf -- "
    "python3 -u bench.py --probe copy --steps 3",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copyw -o copyw -- "
    "python3 -u bench.py --probe copy --steps 3",
]


def counter_dispatches(path: str, counter: str) -> dict:
    """Kernel name -> per-dispatch totals of the counter (summed over its
    instances), from the rocprofv3 counter_collection CSVs under `path`."""
    import csv
    import glob
    from collections import defaultdict
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    per = defaultdict(lambda: defaultdict(float))
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                name = r["Kernel_Name"]
                name = name[5:] if name.startswith("void ") else name
                per[name.split("(")[0]][(f, r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def counter_means(path: str, counter: str) -> dict:
    """Kernel name -> (mean over dispatches, dispatch count)."""
    return {k: (sum(v) / len(v), len(v)) for k, v in counter_dispatches(path, counter).items()}


def record_traffic(d: str, workload: str = "wan14b_720p", budget: float = 0.10) -> dict:
    """HBM bytes per launch of the gathered attention kernel: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the 1 GiB device copy of `--probe copy`; written to TRAFFIC_FILE with
    the attention source's hash, so that bench.py reports it only while that
    source is unchanged."""
    n = 1 << 30
    # the 1 GiB copy is the largest copy dispatch of each run
    cf = [x for k, v in counter_dispatches(os.path.join(d, "copyf"), "FETCH_SIZE").items()
          if "copyBuffer" in k for x in v]
    cw = [x for k, v in counter_dispatches(os.path.join(d, "copyw"), "WRITE_SIZE").items()
          if "copyBuffer" in k for x in v]
    if not cf or not cw:
        raise SystemExit("the copy runs hold no copyBuffer dispatch")
    fetch_copy, write_copy = max(cf), max(cw)
    fs, ws_ = n / (fetch_copy * 1024), n / (write_copy * 1024)
    fe = counter_means(os.path.join(d, "fetch"), "FETCH_SIZE")
    wr = counter_means(os.path.join(d, "write"), "WRITE_SIZE")
    if ATTEND_KERNEL not in fe or ATTEND_KERNEL not in wr:
        raise SystemExit(f"no {ATTEND_KERNEL} dispatch in the counter runs")
    rec = {
        "kernel": ATTEND_KERNEL,
        "workload": workload,
        "budget": budget,
        "attend_src_sha": src_sha(os.path.join(ROOT, "block_sparse_attention_09_amd", "csrc",
                                               "attend.hip")),
        "fetch_kib_per_launch": fe[ATTEND_KERNEL][0],
        "write_kib_per_launch": wr[ATTEND_KERNEL][0],
        "copy_calibration": {"bytes_copied": n, "fetch_kib": fetch_copy, "write_kib": write_copy,
                             "fetch_scale": fs, "write_scale": ws_},
        "bytes_per_launch": (fe[ATTEND_KERNEL][0] * fs + wr[ATTEND_KERNEL][0] * ws_) * 1024,
        "commands": [c.replace("DIR", d) for c in TRAFFIC_COMMANDS],
        "other_kernels_kib_per_launch": {
            k: {"fetch": fe[k][0], "write": wr.get(k, (0.0, 0))[0]} for k in fe
            if k != ATTEND_KERNEL},
    }
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p", choices=sorted(CONFIGS))
    ap.add_argument("--budget", type=float, default=None)
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="attend reps, each after a 512 MB overwrite that evicts K/V from the "
                         "Infinity Cache; reported as a median (0 skips)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--kv-block", type=int, default=4,
                    help="key/value block size (a power of two from 4 to 128)")
    ap.add_argument("--grid", default=None,
                    help="T,H,W latent grid in place of the workload's (block-size sweep)")
    ap.add_argument("--probe", choices=["copy"], default=None)
    ap.add_argument("--record-traffic", default=None, metavar="DIR",
                    help="write the attention traffic record from the counter runs under DIR "
                         "(fetch/, write/, copyf/, copyw/) and exit; needs no GPU")
    args = ap.parse_args()

    if args.record_traffic:
        rec = record_traffic(args.record_traffic)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"{TRAFFIC_FILE}: {rec['bytes_per_launch'] / 1e9:.2f} GB per launch")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the method shards by (batch, head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_09_amd as ab

    if args.probe == "copy":
        probe_copy(torch, args.steps)
        return

    wl = CONFIGS[args.workload]
    if args.grid:
        wl = wl.scaled(grid=tuple(int(x) for x in args.grid.split(",")))
    if args.kv_block != wl.kv_block:
        wl = wl.scaled(kv_block=args.kv_block)
    stock = wl == CONFIGS[args.workload]
    budget = args.budget if args.budget is not None else \
        (0.10 if 0.10 in wl.budgets else wl.budgets[0])
    if budget >= 1.0:
        raise SystemExit("use a budget below 1 for the sparse path")
    log(f"workload {wl.name}: B={wl.B} H={wl.H} N={wl.N} D={wl.D} budget={budget}")
    t0 = time.time()
    q, k, v = make_inputs(wl, torch)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    prob = ab.Problem(wl.B, wl.H, wl.N, wl.D, kv_block=wl.kv_block, n_clusters=wl.n_clusters,
                      kmeans_iters=wl.kmeans_iters, n_forced_tail=wl.n_text, dtype=wl.dtype)
    ws = ab.workspace(prob, q.device)
    pl = ab.empty_plan(prob, ab.nnz_bound(prob, budget), q.device)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    # bf16 problems: V converted to fp16 once per call (abatt_v_to_f16), then the
    # attention's fp16-V form (abatt_attend_v16, bit-identical to abatt_attend)
    v16 = torch.empty(v.shape, dtype=torch.float16, device=v.device) \
        if wl.dtype == "bf16" else None
    va = v if v16 is None else v16

    def step(i, ev=None):
        ab.plan(q, k, budget, seed=wl.plan_seed + i, problem=prob, ws=ws, out=pl)
        if v16 is not None:
            ab.v_to_f16(v, prob, out=v16)
        if ev is not None:
            ev[0].record(stream)
        ab.attend(q, k, va, pl, problem=prob, out=o)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert pl.ok(), "plan exceeded its capacity"
    log("warm-up done")

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nnz_list = []
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / args.steps
    attend_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nnz = pl.nnz()      # plan of the last timed step (every step's nnz is within ~0.1% of it)
    log(f"timed {args.steps} steps: {step_ms:.3f} ms/step, attend {attend_ms:.3f} ms")

    # plan alone (same workspace), for the per-call split
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record(stream)
    for i in range(args.steps):
        ab.plan(q, k, budget, seed=wl.plan_seed + i, problem=prob, ws=ws, out=pl)
    e2.record(stream)
    torch.cuda.synchronize()
    plan_ms = s2.elapsed_time(e2) / args.steps

    # the opt-in one-pass plan entry point (the same plan), for comparison
    s3, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s3.record(stream)
    for i in range(args.steps):
        ab.plan_onepass(q, k, budget, seed=wl.plan_seed + i, problem=prob, ws=ws, out=pl)
    e3.record(stream)
    torch.cuda.synchronize()
    plan_onepass_ms = s3.elapsed_time(e3) / args.steps
    assert pl.ok(), "one-pass plan exceeded its capacity"
    log(f"plan {plan_ms:.3f} ms, one-pass plan {plan_onepass_ms:.3f} ms")

    # the V conversion alone
    convert_ms = 0.0
    if v16 is not None:
        s4, e4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s4.record(stream)
        for _ in range(args.steps):
            ab.v_to_f16(v, prob, out=v16)
        e4.record(stream)
        torch.cuda.synchronize()
        convert_ms = s4.elapsed_time(e4) / args.steps
    call_ms = attend_ms + convert_ms       # the attention path per call

    # attend from a cold Infinity Cache: a 512 MB overwrite before each rep,
    # outside the event pair; median over the reps
    attend_cold_ms = None
    if args.cold_reps > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
        cold = []
        for i in range(args.cold_reps):
            scratch.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ab.attend(q, k, va, pl, problem=prob, out=o)
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        attend_cold_ms = float(np.median(cold))
        del scratch
        log(f"attend from a cold cache: median {attend_cold_ms:.3f} ms over {args.cold_reps} reps")

    # per-row counts of the timed plan: executed tiles include the padding of
    # each row's last key chunk (32 keys in both the bf16 and the fp32 kernel);
    # useful work excludes the padded query rows of a head's last query block
    kb = wl.kv_block
    rp = pl.row_ptr.cpu().numpy().astype(np.int64)
    row_nnz = np.diff(rp)
    valid_q = np.minimum(128, wl.N - 128 * (np.arange(prob.R) % prob.n_qb))
    chunk = 32
    executed_keys = int((np.ceil(row_nnz * kb / chunk) * chunk).sum())
    useful_flop = float((row_nnz * valid_q).sum()) * 4 * kb * wl.D

    # the library's dense attention, the speed-up denominator: for bf16 layers
    # its fastest form (V to fp16, then abatt_dense_v16; the conversion is
    # counted), and the one-call form beside it
    dense_ms = dense_onecall_ms = None
    if not args.no_dense:
        od = torch.empty_like(q)

        def time_dense(fn):
            fn()
            torch.cuda.synchronize()
            s3, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s3.record(stream)
            for _ in range(args.dense_reps):
                fn()
            e3.record(stream)
            torch.cuda.synchronize()
            return s3.elapsed_time(e3) / args.dense_reps

        dense_onecall_ms = time_dense(lambda: ab.dense(q, k, v, problem=prob, out=od))
        dense_ms = dense_onecall_ms
        if v16 is not None:
            dense_ms = time_dense(lambda: ab.dense(q, k, ab.v_to_f16(v, prob, out=v16),
                                                   problem=prob, out=od))
        del od
        log(f"dense {dense_ms:.3f} ms (one-call form {dense_onecall_ms:.3f} ms)")

    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    dense_flop = 4.0 * B * H * N * N * D
    attend_flop = PAIR_FLOP(D, kb) * nnz
    achieved = attend_flop / (attend_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("attend_src_sha") == src_sha(os.path.join(
                ROOT, "block_sparse_attention_09_amd", "csrc", "attend.hip")) \
                and stock and t.get("workload") == wl.name \
                and abs(t.get("budget", -1) - budget) < 1e-9:
            traffic = t.get("bytes_per_launch")

    out = {
        "metric": "sparse attn ms/call + dense-equiv TFLOP/s, Wan2.1-14B shape, ~10% density",
        "value": dense_flop / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent, plan + attend per step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded video-grid q/k/v; no model weights)",
        "config": {
            "workload": f"{wl.name}: B={B} H={H} N={N} ({'x'.join(map(str, wl.grid))}"
                        f"{' + %d text' % wl.n_text if wl.n_text else ''}) D={D} {wl.dtype}, "
                        f"budget {budget}, {wl.n_clusters} clusters, q block 128, "
                        f"kv block {wl.kv_block}",
            "budget": budget,
            "plan_rows": prob.R,
            "nnz": nnz,
            "density": nnz / (prob.R * prob.n_kb),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "k_attend_bf16<128,gather,fp16 V>" if wl.dtype == "bf16" else "k_attend_f32",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
        "detail": {
            "attend_ms": attend_ms,
            "v_to_f16_ms": convert_ms,
            "plan_ms": plan_ms,
            "plan_onepass_ms": plan_onepass_ms,
            "attend_plus_plan_over_4_ms": call_ms + plan_ms / 4,
            "dense_ms": dense_ms,
            "dense_onecall_ms": dense_onecall_ms,
            "attend_dense_equiv_tflops": dense_flop / (call_ms * 1e-3) / 1e12,
            "speedup_attend_vs_dense": (dense_ms / call_ms) if dense_ms else None,
            "speedup_step_vs_dense": (dense_ms / step_ms) if dense_ms else None,
            "speedup_amortized_vs_dense": (dense_ms / (call_ms + plan_ms / 4)) if dense_ms else None,
            "dense_mfma_frac": (dense_flop / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS) if dense_ms else None,
            "attend_flop_per_launch": attend_flop,
            "attend_ms_cold_median": attend_cold_ms,
            "attend_mfma_frac_executed_tiles": PAIR_FLOP(D, 1) * executed_keys / (attend_ms * 1e-3)
                                              / 1e12 / PEAK_BF16_TFLOPS,
            "attend_mfma_frac_useful": useful_flop / (attend_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            # algorithmic selector traffic: Q and K read, S written once and read
            # twice (4 + 8 bytes per pair), the plan written
            "plan_hbm_gbps": (2 * B * H * N * D * 2 + 12 * prob.R * prob.n_kbs + 8 * nnz
                              + 4 * (prob.R + 1)) / (plan_ms * 1e-3) / 1e9,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        log("timing the CPU oracle on a one-head sample ...")
        out["cpu_baseline"] = cpu_baseline(wl, budget, 4.0 * N * N * D)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
