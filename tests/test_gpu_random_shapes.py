"""Seeded random configurations against the fp64 oracle, whole problem, to the same bars
as the fixed cases: lengths drawn around the tile edges (1, 31-33, 63-65, 127-129,
255-257, ... and arbitrary), GQA ratios 1-8, both head dims, all dtypes, causal or not,
softmax scales from a quarter to four times 1/sqrt(d), query magnitudes up to 4 (large
score ranges exercise the moves of the running reference max) and key outliers.  The
split-KV forward gets its own draws of query and key counts and chunkings, the
interval-masked forward and backward draws of mask kinds and query/key counts, and the
fp8 forward draws of shapes, head dims and scales (against its derived bound).  The case
lists are fixed by the seeds, so a failure names a reproducible case."""

import numpy as np
import pytest

import synthetic as S
from gpu_parity import check_full, need_gpu

pytestmark = pytest.mark.gpu

EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 513]


def _draw_cases(n, seed):
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(r.choice(EDGES)) if r.random() < 0.6 else int(r.integers(1, 700))
        Hkv = int(r.choice([1, 1, 2, 3]))
        n_rep = int(r.choice([1, 2, 3, 4, 8]))
        cases.append(dict(
            idx=i, dtype=str(r.choice(["fp32", "fp16", "bf16", "bf16"])), B=int(r.integers(1, 3)),
            H=Hkv * n_rep, Hkv=Hkv, N=N, d=int(r.choice([64, 128])), causal=bool(r.random() < 0.5),
            scale_mult=float(2.0 ** r.uniform(-2, 2)), q_mult=float(r.choice([1.0, 1.0, 2.0, 4.0])),
            outliers=float(r.choice([0.0, 0.0, 0.01, 0.05]))))
    return cases


CASES = _draw_cases(36, 20261202)


def _cid(c):
    return (f"{c['idx']}-{c['dtype']}-B{c['B']}H{c['H']}Hkv{c['Hkv']}N{c['N']}d{c['d']}"
            f"{'-c' if c['causal'] else ''}-s{c['scale_mult']:.2f}-q{c['q_mult']:g}-o{c['outliers']:g}")


@pytest.mark.parametrize("c", CASES, ids=_cid)
def test_random_shape(c):
    need_gpu()
    kw = {"k_outlier_frac": c["outliers"], "k_outlier_seed": 1000 + c["idx"]} if c["outliers"] else {}
    w = S.custom(c["dtype"], c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["causal"],
                 seed_base=60000 + 100 * c["idx"], **kw)
    inp = S.make_inputs(w)
    if c["q_mult"] != 1.0:
        inp["q"] = (inp["q"].float() * c["q_mult"]).to(inp["q"].dtype)
    check_full(inp, c["dtype"], c["causal"], w.scale * c["scale_mult"], backward=True, label=_cid(c))


def _draw_split(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(r.choice([1, 2, 4]))
        n_rep = int(r.choice([1, 2, 4, 8]))
        Nq = int(r.choice([1, 1, 2, 3, 7, 16, 33]))
        Nk = int(r.integers(max(1, Nq), 3000))
        out.append(dict(idx=i, dtype=str(r.choice(["fp16", "bf16"])), B=int(r.integers(1, 3)),
                        H=Hkv * n_rep, Hkv=Hkv, Nq=Nq, Nk=Nk, d=int(r.choice([64, 128])),
                        causal=bool(r.random() < 0.5),
                        n_splits=int(r.choice([0, 0, 1, 3, 17, 1000]))))
    return out


SPLIT_CASES = _draw_split(16, 20261203)


@pytest.mark.parametrize("c", SPLIT_CASES, ids=lambda c: (
    f"{c['idx']}-{c['dtype']}-B{c['B']}H{c['H']}Hkv{c['Hkv']}Nq{c['Nq']}Nk{c['Nk']}d{c['d']}"
    f"{'-c' if c['causal'] else ''}-s{c['n_splits']}"))
def test_random_splitkv(c):
    need_gpu()
    from test_gpu_splitkv import check_split
    w = S.custom(c["dtype"], c["B"], c["H"], c["Hkv"], c["Nq"], c["d"], c["causal"],
                 seed_base=70000 + 100 * c["idx"], Nk=c["Nk"])
    check_split(w, n_splits=c["n_splits"])


def _draw_masked(n, seed):
    r = np.random.default_rng(seed)
    kinds = [("random", lambda: {"empty_frac": float(r.choice([0.0, 0.1, 0.3]))}),
             ("sliding", lambda: {"left": int(r.integers(0, 300)), "right": int(r.integers(0, 50)),
                                  "causal": bool(r.random() < 0.5)}),
             ("prefix", lambda: {"prefix": int(r.integers(1, 400))}),
             ("causal", lambda: {})]
    out = []
    for i in range(n):
        Hkv = int(r.choice([1, 2]))
        n_rep = int(r.choice([1, 2, 4]))
        Nk = int(r.choice(EDGES)) if r.random() < 0.5 else int(r.integers(1, 600))
        Nq = Nk if r.random() < 0.5 else int(r.integers(1, Nk + 1))
        kind, mk = kinds[int(r.integers(0, len(kinds)))]
        out.append(dict(idx=i, dtype=str(r.choice(["fp32", "fp16", "bf16"])), B=int(r.integers(1, 3)),
                        H=Hkv * n_rep, Hkv=Hkv, Nq=Nq, Nk=Nk, d=int(r.choice([64, 128])), kind=kind,
                        mk=mk()))
    return out


MASKED_CASES = _draw_masked(16, 20261204)


@pytest.mark.parametrize("c", MASKED_CASES, ids=lambda c: (
    f"{c['idx']}-{c['dtype']}-{c['kind']}-B{c['B']}H{c['H']}Hkv{c['Hkv']}Nq{c['Nq']}Nk{c['Nk']}d{c['d']}"))
def test_random_masked_fwd_bwd(c):
    need_gpu()
    from test_gpu_masked import check_masked_bwd
    check_masked_bwd(c["dtype"], c["B"], c["H"], c["Hkv"], c["Nq"], c["Nk"], c["d"], c["kind"],
                     80000 + 100 * c["idx"], **c["mk"])


def _draw_fp8(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(r.choice([1, 2]))
        out.append(dict(idx=i, B=int(r.integers(1, 3)), H=Hkv * int(r.choice([1, 2, 4])), Hkv=Hkv,
                        N=int(r.choice(EDGES)) if r.random() < 0.6 else int(r.integers(1, 700)),
                        d=int(r.choice([64, 128])), causal=bool(r.random() < 0.5),
                        scale_mult=float(2.0 ** r.uniform(-1, 1))))
    return out


FP8_CASES = _draw_fp8(12, 20261205)


@pytest.mark.parametrize("c", FP8_CASES, ids=lambda c: (
    f"{c['idx']}-B{c['B']}H{c['H']}Hkv{c['Hkv']}N{c['N']}d{c['d']}{'-c' if c['causal'] else ''}"
    f"-s{c['scale_mult']:.2f}"))
def test_random_fp8(c):
    need_gpu()
    from test_gpu_fp8 import bound_check, run_fp8
    w = S.custom("bf16", c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["causal"],
                 seed_base=90000 + 100 * c["idx"])
    inp = S.make_fp8_inputs(w)
    scale = w.scale * c["scale_mult"]
    o, lse = run_fp8(inp, c["causal"], scale)
    bound_check(inp, c["causal"], scale, o, lse, f"random fp8 {c['idx']}")
