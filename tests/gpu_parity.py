"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding and
compare with the fp64 oracle on the same seeded inputs.

Tolerances (stated for this path): output O and LSE absolute, gradients relative
to each gradient's largest oracle magnitude.
    fp32: 1e-5      fp16: 2e-3      bf16: 1e-2 (O, LSE), 2e-2 (gradients)

Two readings of those bars, needed at the edges:
  * O is compared as |O - O_ref| / max(1, |O_ref|) per element: absolute for
    |O| <= 1, relative above.  Rounding the output to bf16 alone costs half an
    ulp, which exceeds 1e-2 once |O| >= 4 (possible in the first rows of a causal
    head, where O mixes few value rows); no bf16-returning kernel could meet an
    absolute 1e-2 there.
  * The relative gradient error divides by max(max |g_ref|, 1e-2), so a gradient
    that is nearly zero is held to 1e-2 * tolerance in absolute terms.  At N = 1,
    dQ and dK are exactly zero in real arithmetic (the single weight is 1 and
    dS = dP - D cancels); there they are checked in absolute terms against the
    tolerance itself, since what remains is cancellation residue of |dP| ~ 10.
"""

from __future__ import annotations

import math
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


def out_err(got, ref):
    """max |got - ref| / max(1, |ref|): the O / LSE metric."""
    if not ref.size:
        return 0.0
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
    errs = {"o": out_err(f64(o), ref["o"]), "o_abs": max_abs(f64(o), ref["o"]),
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
    e_o, e_l = out_err(g_o, r_o), max_abs(g_lse, r_lse)
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
            "o": out_err(f64(o[b, hs]), ref["o"][b, hs]),
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
