"""The C ABI on the CPU: the library loads without a GPU, exports what the
header declares, sizes its buffers, and rejects bad arguments before any HIP
call (so nothing here touches a device)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_09_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return ab.load_library()


def header_symbols():
    text = open(os.path.join(ROOT, "include", "abatt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(abatt_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    syms = header_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(ab.SYMBOLS) == syms
    assert b"gfx950" in lib.abatt_version()


def prob(**kw):
    base = dict(B=1, H=2, N=1024, D=128, n_clusters=8, dtype="bf16")
    base.update(kw)
    return ab.Problem(**base)


def test_sizes(lib):
    p = prob()
    assert ab.plan_rows(p) == 16
    assert ab.max_nnz(p) == 16 * 256
    b = ab.nnz_bound(p, 0.1)
    assert 16 * 25.6 < b <= ab.max_nnz(p)
    assert ab.nnz_bound(p, 1.0) == ab.max_nnz(p)
    ws = ab.plan_workspace_bytes(p)
    # means + centroids + weights + scores + the scorer's partial normalisers
    # (2 groups of 256 centroid rows, each group's 8 key tiles in 2 splits, 8
    # bytes per row and split) + sampler scratch (row counts, kept-block
    # bitmasks of 256/32 words per row, 16-byte row solves)
    sampler = 16 * 4 + 16 * 8 * 4 + 16 * 16
    partial = 2 * 2 * 256 * 8
    need = 2 * 256 * 128 * 4 + 16 * 8 * 128 * 4 + 16 * 8 * 4 + 16 * 256 * 4 + partial + sampler
    assert need <= ws <= need + 8 * 256
    assert sampler <= ab.sampler_workspace_bytes(p) <= sampler + 4 * 256
    pf = prob(N=1024 + 256, n_forced_tail=256)
    assert ab.max_nnz(pf) == pf.R * (256 + 64)
    assert ab.nnz_bound(pf, 0.1) - ab.nnz_bound(prob(N=1280, n_forced_tail=256), 0.1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -2), (dict(n_clusters=4), -2), (dict(q_block=64), -2),
    (dict(kv_block=256), -2), (dict(kv_block=2), -2), (dict(kv_block=12, N=1020), -2),
    (dict(kv_block=16, N=1032), -1), (dict(N=0), -1), (dict(H=0), -1), (dict(N=1022), -1),
    (dict(n_forced_tail=6), -1), (dict(scale=-1.0), -1), (dict(kmeans_iters=0), -1),
])
def test_bad_problems(lib, kw, code):
    p = prob(**kw)
    assert lib.abatt_plan_rows(ctypes.byref(p.c())) == -1
    assert lib.abatt_plan_workspace_bytes(ctypes.byref(p.c())) == 0
    fake = ctypes.c_void_p(0x1000)
    pl = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, 0x1000)
    r = lib.abatt_plan(ctypes.byref(p.c()), fake, fake, 0.1, 0, fake, 1 << 40,
                       ctypes.byref(pl), None)
    assert r == code


@pytest.mark.parametrize("entry", ["abatt_plan", "abatt_plan_onepass"])
def test_plan_entries_check_alike(lib, entry):
    # both planning entry points take the same arguments and reject the same
    # ones with the same codes, before any HIP call
    f = getattr(lib, entry)
    P = ctypes.byref
    fake = ctypes.c_void_p(0x1000)
    good = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, 0x1000)
    for kw, code in ((dict(D=96), -2), (dict(kv_block=256), -2), (dict(N=0), -1),
                     (dict(n_forced_tail=6), -1), (dict(kmeans_iters=0), -1)):
        assert f(P(prob(**kw).c()), fake, fake, 0.1, 0, fake, 1 << 40, P(good), None) == code
    p = prob()
    c = p.c()
    ws = ab.plan_workspace_bytes(p)
    assert f(P(c), None, fake, 0.1, 0, fake, ws, P(good), None) == -1
    for b in (0.0, -0.1, 1.5, float("nan")):
        assert f(P(c), fake, fake, b, 0, fake, ws, P(good), None) == -1
    assert f(P(c), fake, fake, 0.1, 0, fake, ws - 1, P(good), None) == -3
    assert f(P(c), fake, fake, 0.1, 0, None, ws, P(good), None) == -1
    nostat = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, None)
    assert f(P(c), fake, fake, 0.1, 0, fake, ws, P(nostat), None) == -1
    pf = prob(N=1280, n_forced_tail=256).c()
    small = ab._Plan(0x1000, 0x1000, 0x1000, 10, 0x1000)
    assert f(P(pf), fake, fake, 0.1, 0, fake, lib.abatt_plan_workspace_bytes(P(pf)),
             P(small), None) == -4
    odd = ctypes.c_void_p(0x1008)
    assert f(P(c), fake, odd, 0.1, 0, fake, ws, P(good), None) == -1
    assert f(P(c), fake, fake, 0.1, 0, odd, ws, P(good), None) == -1


@pytest.mark.parametrize("kb", [4, 8, 16, 32, 64, 128])
def test_key_block_sizes(lib, kb):
    # powers of two from 4 to 128 tokens; blocks and forced blocks scale with kb
    p = prob(N=2048 + 2 * kb, kv_block=kb, n_forced_tail=2 * kb)
    assert lib.abatt_plan_rows(ctypes.byref(p.c())) == p.R
    assert p.n_kbs == 2048 // kb and p.n_kb == p.n_kbs + 2
    assert ab.max_nnz(p) == p.R * p.n_kb


def test_argument_checks_before_any_hip_call(lib):
    p = prob()
    c = p.c()
    fake = ctypes.c_void_p(0x1000)
    ws = ab.plan_workspace_bytes(p)
    good = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, 0x1000)
    P = ctypes.byref
    # null tensors
    assert lib.abatt_plan(P(c), None, fake, 0.1, 0, fake, ws, P(good), None) == -1
    assert lib.abatt_attend(P(c), fake, None, fake, P(good), fake, None, None) == -1
    assert lib.abatt_dense(P(c), fake, fake, fake, None, None, None) == -1
    assert lib.abatt_key_means(P(c), None, fake, None) == -1
    assert lib.abatt_scores(P(c), fake, fake, None, None, None, fake, ws, None) == -1
    # budget outside (0, 1]
    for b in (0.0, -0.1, 1.5, float("nan")):
        assert lib.abatt_plan(P(c), fake, fake, b, 0, fake, ws, P(good), None) == -1
        assert lib.abatt_plan_from_scores(P(c), fake, b, 0, fake, 1 << 20, P(good), None) == -1
    # workspace too small
    assert lib.abatt_plan(P(c), fake, fake, 0.1, 0, fake, ws - 1, P(good), None) == -3
    assert lib.abatt_scores(P(c), fake, fake, fake, None, None, fake, ws - 1, None) == -3
    assert lib.abatt_plan_from_scores(P(c), fake, 0.1, 0, fake, 3, P(good), None) == -3
    # plan without status, or without arrays
    nostat = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, None)
    assert lib.abatt_plan(P(c), fake, fake, 0.1, 0, fake, ws, P(nostat), None) == -1
    noarr = ab._Plan(None, 0x1000, 0x1000, 10 ** 6, 0x1000)
    assert lib.abatt_attend(P(c), fake, fake, fake, P(noarr), fake, None, None) == -1
    assert lib.abatt_attend(P(c), fake, fake, fake, None, fake, None, None) == -1
    # capacity below the forced blocks
    pf = prob(N=1280, n_forced_tail=256).c()
    small = ab._Plan(0x1000, 0x1000, 0x1000, 10, 0x1000)
    wsf = lib.abatt_plan_workspace_bytes(P(pf))
    assert lib.abatt_plan(P(pf), fake, fake, 0.1, 0, fake, wsf, P(small), None) == -4
    # misaligned tensors or workspace (the kernels move 16 bytes at a time)
    odd = ctypes.c_void_p(0x1008)
    assert lib.abatt_plan(P(c), fake, odd, 0.1, 0, fake, ws, P(good), None) == -1
    assert lib.abatt_plan(P(c), fake, fake, 0.1, 0, odd, ws, P(good), None) == -1
    assert lib.abatt_attend(P(c), fake, fake, odd, P(good), fake, None, None) == -1
    assert lib.abatt_attend(P(c), fake, fake, fake, P(good), odd, None, None) == -1
    assert lib.abatt_dense(P(c), odd, fake, fake, fake, None, None) == -1
    assert lib.abatt_v_to_f16(P(c), fake, odd, None) == -1
    assert lib.abatt_attend_v16(P(c), fake, fake, odd, P(good), fake, None, None) == -1
    assert lib.abatt_key_means(P(c), odd, fake, None) == -1
    # fp16 V: nulls, V16 aliasing V, fp32 problems
    assert lib.abatt_v_to_f16(P(c), None, fake, None) == -1
    assert lib.abatt_v_to_f16(P(c), fake, fake, None) == -1
    assert lib.abatt_attend_v16(P(c), fake, fake, None, P(good), fake, None, None) == -1
    assert lib.abatt_attend_v16(P(c), fake, fake, fake, P(noarr), fake, None, None) == -1
    assert lib.abatt_dense_v16(P(c), fake, fake, None, fake, None, None) == -1
    assert lib.abatt_dense_v16(P(c), fake, fake, odd, fake, None, None) == -1
    c32 = prob(dtype="f32", D=64).c()
    assert lib.abatt_dense_v16(P(c32), fake, fake, fake, fake, None, None) == -2
    assert lib.abatt_v_to_f16(P(c32), fake, ctypes.c_void_p(0x2000), None) == -2
    assert lib.abatt_attend_v16(P(c32), fake, fake, fake, P(good), fake, None, None) == -2
    # dense accepts N not a multiple of 4 (keys past N are masked) but still checks D
    assert lib.abatt_dense(P(prob(N=1023, D=96).c()), fake, fake, fake, fake, None, None) == -2


def test_noalloc_checks_before_any_hip_call(lib):
    """abatt_plan_noalloc refuses a problem whose plan workspace exceeds the
    static scratch (ABATT_ESCRATCH), and bad arguments, with nothing enqueued."""
    P = ctypes.byref
    fake = ctypes.c_void_p(0x1000)
    good = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 9, 0x1000)
    big = ab.Problem(B=1, H=40, N=75600, D=128)          # 14B 720p layer: ~2.3 GB
    assert ab.plan_workspace_bytes(big) > ab.SCRATCH_BYTES
    assert lib.abatt_plan_noalloc(P(big.c()), fake, fake, 0.1, 0, P(good), None) == -6
    fits = ab.Problem(B=1, H=12, N=32760, D=128)          # 1.3B 480p layer fits
    assert ab.plan_workspace_bytes(fits) <= ab.SCRATCH_BYTES
    c = prob().c()
    assert lib.abatt_plan_noalloc(P(c), None, fake, 0.1, 0, P(good), None) == -1
    assert lib.abatt_plan_noalloc(P(c), fake, ctypes.c_void_p(0x1008), 0.1, 0, P(good), None) == -1
    assert lib.abatt_plan_noalloc(P(c), fake, fake, 0.0, 0, P(good), None) == -1
    nostat = ab._Plan(0x1000, 0x1000, 0x1000, 10 ** 6, None)
    assert lib.abatt_plan_noalloc(P(c), fake, fake, 0.1, 0, P(nostat), None) == -1
    pf = prob(N=1280, n_forced_tail=256).c()
    small = ab._Plan(0x1000, 0x1000, 0x1000, 10, 0x1000)
    assert lib.abatt_plan_noalloc(P(pf), fake, fake, 0.1, 0, P(small), None) == -4
    assert lib.abatt_plan_noalloc(P(prob(D=96).c()), fake, fake, 0.1, 0, P(good), None) == -2


def test_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "abatt.h")).read()
    m = re.search(r"#define ABATT_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m is not None
    assert int(m.group(1)) * 1024 * 1024 == ab.SCRATCH_BYTES


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert len(lib.abatt_status_str(code)) > 0
    with pytest.raises(ab.AbattError):
        ab._check(-1)
