"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding and
compare with the fp64 oracle on the same seeded inputs.

Tolerances (stated for this path): output O and LSE absolute, gradients relative
to each gradient's largest oracle magnitude.
    fp32: 1e-5      fp16: 2e-3      bf16: 1e-2 (O, LSE), 2e-2 (gradients)

Two readings of those bars, needed at the edges:
  * bf16 only: O is compared as |O - O_ref| / max(1, |O_ref|) per element, absolute
    for |O| <= 1 and relative above.  Rounding the output to bf16 alone costs half
    an ulp, which exceeds 1e-2 once |O| >= 4 (possible in the first rows of a causal
    head, where O mixes few value rows); no bf16-returning kernel could meet an
    absolute 1e-2 there.  fp32 and fp16 outputs are held to the absolute bar (half
    an ulp is 2.4e-7 for fp32 and at most 2e-3 for fp16 below |O| = 8).
  * The relative gradient error divides by max(max |g_ref|, 1e-2), so a gradient
    that is nearly zero is held to 1e-2 * tolerance in absolute terms.  At N = 1,
    dQ and dK are exactly zero in real arithmetic (the single weight is 1 and
    dS = dP - D cancels); there they are checked in absolute terms against the
    tolerance itself, since what remains is cancellation residue of |dP| ~ 10.
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle.attention as A

TOL_O = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 1e-2}
TOL_G = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 2e-2}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    import online_softmax_attn_amd as osa
    osa.library()  # raises if the HIP library is missing: no fallback exists


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return x.to("cuda", non_blocking=False).contiguous()


def run_fwd(inp, causal, scale):
    import online_softmax_attn_amd as osa
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = osa.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def run_bwd(inp, causal, scale, o=None, lse=None):
    import online_softmax_attn_amd as osa
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    if o is None:
        o, lse = osa.attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = osa.attn_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def f64(t):
    return t.detach().cpu().double().numpy()


def max_abs(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def out_err(got, ref, dtype):
    """The O metric: max |got - ref| / max(1, |ref|) for bf16, max |got - ref| for
    fp32 and fp16."""
    if not ref.size:
        return 0.0
    if dtype != "bf16":
        return max_abs(got, ref)
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))


GRAD_FLOOR = 1e-2


def rel_err(got, ref, floor=GRAD_FLOOR):
    denom = max(float(np.max(np.abs(ref))) if ref.size else 0.0, floor)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / denom


def check_full(inp, dtype, causal, scale, backward=True, label=""):
    """Whole-problem comparison (small shapes)."""
    say(f"[parity] {label} dtype={dtype} causal={causal} shape={tuple(inp['q'].shape)} kv={tuple(inp['k'].shape)}")
    if backward:
        o, lse, dq, dk, dv = run_bwd(inp, causal, scale)
        ref = A.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    else:
        o, lse = run_fwd(inp, causal, scale)
        r_o, r_lse = A.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
        ref = {"o": r_o, "lse": r_lse}
    errs = {"o": out_err(f64(o), ref["o"], dtype), "o_abs": max_abs(f64(o), ref["o"]),
            "lse": max_abs(f64(lse), ref["lse"])}
    assert np.all(np.isfinite(f64(o))) and np.all(np.isfinite(f64(lse)))
    if backward:
        n_keys = inp["q"].shape[2]
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            g = f64(t)
            assert np.all(np.isfinite(g)), name
            zero_grad = n_keys == 1 and name in ("dq", "dk")
            errs[name] = rel_err(g, ref[name], floor=1.0 if zero_grad else GRAD_FLOOR)
    say(f"[parity]   errors {', '.join(f'{k}={v:.2e}' for k, v in errs.items())}")
    assert errs["o"] <= TOL_O[dtype], errs
    assert errs["lse"] <= TOL_O[dtype], errs
    for name in ("dq", "dk", "dv"):
        if name in errs:
            assert errs[name] <= TOL_G[dtype], errs
    return errs


def pick_rows(B, H, N, per_head, seed):
    r = np.random.default_rng(seed)
    picks = []
    for b in range(B):
        for h in range(H):
            rows = {0, N - 1}
            rows.update(int(x) for x in r.integers(0, N, size=max(0, per_head - 2)))
            picks += [(b, h, i) for i in sorted(rows)]
    return picks


def check_sampled_fwd(inp, o, lse, dtype, causal, scale, per_head=3, seed=0, label=""):
    """Rows picked across every head, each computed by the oracle on its own."""
    B, H, N, _ = inp["q"].shape
    picks = pick_rows(B, H, N, per_head, seed)
    r_o, r_lse = A.attention_forward_rows(inp["q"], inp["k"], inp["v"], scale, causal, picks)
    idx = tuple(np.array(x) for x in zip(*picks))
    g_o = o.detach()[idx[0], idx[1], idx[2]].cpu().double().numpy()
    g_lse = lse.detach()[idx[0], idx[1], idx[2]].cpu().double().numpy()
    e_o, e_l = out_err(g_o, r_o, dtype), max_abs(g_lse, r_lse)
    say(f"[parity] {label} sampled fwd rows={len(picks)} o={e_o:.2e} lse={e_l:.2e}")
    assert e_o <= TOL_O[dtype] and e_l <= TOL_O[dtype], (e_o, e_l)
    return e_o, e_l


def check_group_bwd(inp, outs, dtype, causal, scale, groups, label=""):
    """Full-oracle backward for the query heads of the given (b, kv head) groups."""
    o, lse, dq, dk, dv = outs
    H, Hkv = inp["q"].shape[1], inp["k"].shape[1]
    n_rep = H // Hkv
    ref = A.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, heads=groups)
    errs = {}
    for b, g in groups:
        hs = slice(g * n_rep, (g + 1) * n_rep)
        errs_g = {
            "o": out_err(f64(o[b, hs]), ref["o"][b, hs], dtype),
            "lse": max_abs(f64(lse[b, hs]), ref["lse"][b, hs]),
            "dq": rel_err(f64(dq[b, hs]), ref["dq"][b, hs]),
            "dk": rel_err(f64(dk[b, g]), ref["dk"][b, g]),
            "dv": rel_err(f64(dv[b, g]), ref["dv"][b, g]),
        }
        for k_, v_ in errs_g.items():
            errs[k_] = max(errs.get(k_, 0.0), v_)
    say(f"[parity] {label} group bwd {groups}: {', '.join(f'{k}={v:.2e}' for k, v in errs.items())}")
    assert errs["o"] <= TOL_O[dtype] and errs["lse"] <= TOL_O[dtype], errs
    for name in ("dq", "dk", "dv"):
        assert errs[name] <= TOL_G[dtype], errs
    return errs


def oracle_workers() -> int:
    """Threads for whole-problem oracle checks: the host cores this process may use,
    at most 16 (the host CPU share that comes with one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def check_all_heads(inp, outs, dtype, causal, scale, label=""):
    """Whole-problem comparison at full workload sizes: O, LSE and dQ of every query
    head and dK, dV of every key/value head against the oracle.

    Query heads are independent, so each runs alone (oracle.attention.attention_head
    on its own query head and its key/value head) on a thread pool: NumPy releases
    the GIL inside its products and ufuncs, and BLAS is held to one thread per
    worker.  A key/value head's dK, dV are the sum of its query heads'
    contributions, added in head order once all of them are back.  Progress is
    printed per group.
    """
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    o, lse, dq, dk, dv = (t.detach().cpu() for t in outs)
    B, H, N, d = inp["q"].shape
    Hkv, Nk = inp["k"].shape[1], inp["k"].shape[2]
    n_rep = H // Hkv
    say(f"[parity] {label} all heads: B={B} H={H} Hkv={Hkv} N={N} d={d} dtype={dtype} "
        f"causal={causal}, {oracle_workers()} oracle threads")

    def head(b, h):
        g = A.kv_head_of(h, H, Hkv)
        ro, rl, rdq, rdk, rdv, _ = A.attention_head(
            A._f64(inp["q"][b, h]), A._f64(inp["k"][b, g]), A._f64(inp["v"][b, g]), scale,
            causal, A._f64(inp["do"][b, h]))
        go, gdq = f64(o[b, h]), f64(dq[b, h])
        e = {"o": out_err(go, ro, dtype), "lse": max_abs(f64(lse[b, h]), rl),
             "dq": rel_err(gdq, rdq)}
        finite = bool(np.all(np.isfinite(go)) and np.all(np.isfinite(gdq)))
        return e, finite, rdk, rdv

    errs = {k_: 0.0 for k_ in ("o", "lse", "dq", "dk", "dv")}

    def collect(futs):
        for b in range(B):
            for g in range(Hkv):
                dk_ref = np.zeros((Nk, d))
                dv_ref = np.zeros((Nk, d))
                for h in range(g * n_rep, (g + 1) * n_rep):
                    e, finite, rdk, rdv = futs.pop((b, h)).result()
                    assert finite, (label, b, h)
                    for k_, v_ in e.items():
                        errs[k_] = max(errs[k_], v_)
                    dk_ref += rdk
                    dv_ref += rdv
                errs["dk"] = max(errs["dk"], rel_err(f64(dk[b, g]), dk_ref))
                errs["dv"] = max(errs["dv"], rel_err(f64(dv[b, g]), dv_ref))
                say(f"[parity]   group ({b},{g}) done; running max "
                    f"{', '.join(f'{k_}={v_:.2e}' for k_, v_ in errs.items())}")

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(oracle_workers()) as ex:
            futs = {(b, h): ex.submit(head, b, h) for b in range(B) for h in range(H)}
            try:
                collect(futs)
            except BaseException:
                for f in futs.values():
                    f.cancel()
                raise
    say(f"[parity] {label} all heads: {', '.join(f'{k_}={v_:.2e}' for k_, v_ in errs.items())}")
    assert errs["o"] <= TOL_O[dtype] and errs["lse"] <= TOL_O[dtype], errs
    for name in ("dq", "dk", "dv"):
        assert errs[name] <= TOL_G[dtype], errs
    return errs
