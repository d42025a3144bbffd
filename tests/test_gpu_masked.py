"""GPU parity of the interval-masked forward (general masks; queries may be fewer
than keys) against the fp64 oracle, element by element on small and ragged shapes and
on sampled rows at full size."""

import numpy as np
import pytest
import torch

import oracle.attention as A
import synthetic as S
from gpu_parity import TOL_O, f64, max_abs, need_gpu, out_err, say, to_dev

pytestmark = pytest.mark.gpu


def run_masked_bwd(inp, lo, hi, scale):
    import online_softmax_attn_amd as osa
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    lo_d, hi_d = to_dev(lo), to_dev(hi)
    o, lse = osa.attn_fwd_masked(q, k, v, lo_d, hi_d, scale=scale)
    dq, dk, dv = osa.attn_bwd_masked(q, k, v, o, lse, do, lo_d, hi_d, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def run_masked(inp, lo, hi, scale):
    import online_softmax_attn_amd as osa
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = osa.attn_fwd_masked(q, k, v, to_dev(lo), to_dev(hi), scale=scale)
    torch.cuda.synchronize()
    return o, lse


def compare(o, lse, r_o, r_lse, dtype, label):
    g_o, g_l = f64(o), f64(lse)
    assert np.all(np.isfinite(g_o))
    # Rows that see no key: LSE = -inf on both sides, O = 0.
    assert np.array_equal(np.isneginf(g_l), np.isneginf(r_lse)), label
    fin = np.isfinite(r_lse)
    e_o, e_l = out_err(g_o, r_o, dtype), max_abs(g_l[fin], r_lse[fin])
    say(f"[masked] {label} o={e_o:.2e} lse={e_l:.2e}")
    assert e_o <= TOL_O[dtype] and e_l <= TOL_O[dtype], (e_o, e_l)


def check_masked(dtype, B, H, Hkv, Nq, Nk, d, kind, seed, **mk):
    w = S.custom(dtype, B, H, Hkv, Nq, d, False, seed_base=seed, Nk=Nk if Nk != Nq else 0)
    inp = S.make_inputs(w, with_grad=False)
    lo, hi = S.mask_intervals(kind, B, Nq, Nk, seed=seed, **mk)
    o, lse = run_masked(inp, lo, hi, w.scale)
    r_o, r_lse = A.attention_forward_intervals(inp["q"], inp["k"], inp["v"], w.scale,
                                               lo.numpy(), hi.numpy())
    compare(o, lse, r_o, r_lse, dtype, f"{kind} {dtype} B{B}H{H}Hkv{Hkv}Nq{Nq}Nk{Nk}d{d} {mk}")


MASKS = [
    ("causal", {}),
    ("sliding", {"left": 40, "causal": True}),
    ("sliding", {"left": 17, "right": 30, "causal": False}),
    ("prefix", {"prefix": 50}),
    ("random", {"empty_frac": 0.1}),
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m[0] + "_" + "_".join(f"{k}{v}" for k, v in m[1].items()))
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 1), (2, 4, 2, 200, 200), (1, 3, 1, 333, 333),
                                   (1, 4, 2, 77, 300)],
                         ids=lambda s: "B{}H{}Hkv{}Nq{}Nk{}".format(*s))
def test_masked_small(dtype, d, mask, shape):
    need_gpu()
    kind, mk = mask
    B, H, Hkv, Nq, Nk = shape
    check_masked(dtype, B, H, Hkv, Nq, Nk, d, kind, 9600 + Nq, **mk)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_documents(dtype, causal):
    """Packed variable-length sequences: each row sees only its own document."""
    need_gpu()
    lens = [[100, 3, 250, 1, 46], [400]]
    check_masked(dtype, 2, 4, 2, 400, 400, 128, "document", 9700, doc_lens=lens, causal=causal)


def test_masked_causal_matches_attn_fwd():
    """The causal mask as intervals agrees with the causal forward."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w = S.custom("bf16", 1, 4, 2, 700, 128, True, seed_base=9750)
    inp = S.make_inputs(w, with_grad=False)
    lo, hi = S.mask_intervals("causal", 1, 700, 700)
    o1, l1 = run_masked(inp, lo, hi, w.scale)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o2, l2 = osa.attn_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert max_abs(f64(o1), f64(o2)) <= 2 * TOL_O["bf16"]
    assert max_abs(f64(l1), f64(l2)) <= TOL_O["bf16"]


def test_masked_all_rows_empty():
    """Every interval empty: O = 0 and LSE = -inf everywhere, no NaN."""
    need_gpu()
    w = S.custom("fp16", 1, 2, 1, 64, 64, False, seed_base=9760)
    inp = S.make_inputs(w, with_grad=False)
    lo = torch.full((1, 64), 10, dtype=torch.int32)
    hi = torch.full((1, 64), 3, dtype=torch.int32)
    o, lse = run_masked(inp, lo, hi, w.scale)
    assert torch.count_nonzero(o).item() == 0
    assert torch.all(torch.isneginf(lse)).item()


FULL = [  # (name, dtype, B, H, Hkv, N, d, kind, params)
    ("sliding4096_bf16_gqa", "bf16", 1, 32, 8, 16384, 128, "sliding", {"left": 4095, "causal": True}),
    ("documents_bf16", "bf16", 4, 16, 16, 8192, 128, "document",
     {"doc_lens": [[3000, 2000, 3192], [8192], [1, 4095, 4096], [100] * 81 + [92]], "causal": True}),
]


@pytest.mark.slow
@pytest.mark.parametrize("case", FULL, ids=lambda c: c[0])
def test_masked_full_size_sampled(case):
    """Full-size masked workloads, rows sampled in every head against the oracle."""
    need_gpu()
    name, dtype, B, H, Hkv, N, d, kind, mk = case
    w = S.custom(dtype, B, H, Hkv, N, d, False, seed_base=9800)
    inp = S.make_inputs(w, with_grad=False)
    lo, hi = S.mask_intervals(kind, B, N, N, **mk)
    o, lse = run_masked(inp, lo, hi, w.scale)
    r = np.random.default_rng(5)
    err_o = err_l = 0.0
    for b in range(B):
        for h in range(H):
            rows = np.unique(np.concatenate([[0, N - 1], r.integers(0, N, 2)]))
            g = A.kv_head_of(h, H, Hkv)
            ro, rl = A.attention_head_intervals(A._f64(inp["q"][b, h])[rows], A._f64(inp["k"][b, g]),
                                                A._f64(inp["v"][b, g]), w.scale,
                                                lo[b].numpy()[rows], hi[b].numpy()[rows])
            err_o = max(err_o, out_err(f64(o[b, h])[rows], ro, dtype))
            err_l = max(err_l, max_abs(f64(lse[b, h])[rows], rl))
    say(f"[masked] {name} sampled o={err_o:.2e} lse={err_l:.2e}")
    assert err_o <= TOL_O[dtype] and err_l <= TOL_O[dtype]


def check_masked_bwd(dtype, B, H, Hkv, Nq, Nk, d, kind, seed, **mk):
    from gpu_parity import TOL_G, rel_err
    w = S.custom(dtype, B, H, Hkv, Nq, d, False, seed_base=seed, Nk=Nk if Nk != Nq else 0)
    inp = S.make_inputs(w, with_grad=True)
    lo, hi = S.mask_intervals(kind, B, Nq, Nk, seed=seed, **mk)
    o, lse, dq, dk, dv = run_masked_bwd(inp, lo, hi, w.scale)
    ref = A.attention_backward_intervals(inp["q"], inp["k"], inp["v"], inp["do"], w.scale,
                                         lo.numpy(), hi.numpy())
    label = f"bwd {kind} {dtype} B{B}H{H}Hkv{Hkv}Nq{Nq}Nk{Nk}d{d} {mk}"
    compare(o, lse, ref["o"], ref["lse"], dtype, label)
    errs = {}
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = f64(t)
        assert np.all(np.isfinite(g)), name
        # A gradient that is exactly zero in real arithmetic (every row sees one key)
        # is checked in absolute terms, as the unmasked parity tests do at N = 1.
        zero = not np.any(ref[name])
        errs[name] = rel_err(g, ref[name], floor=1.0 if zero else 1e-2)
    say(f"[masked]   grads {', '.join(f'{k}={v:.2e}' for k, v in errs.items())}")
    for name, e in errs.items():
        assert e <= TOL_G[dtype], errs


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m[0] + "_" + "_".join(f"{k}{v}" for k, v in m[1].items()))
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 1), (2, 4, 2, 200, 200), (1, 3, 1, 333, 333),
                                   (1, 4, 2, 77, 300)],
                         ids=lambda s: "B{}H{}Hkv{}Nq{}Nk{}".format(*s))
def test_masked_bwd_small(dtype, d, mask, shape):
    need_gpu()
    kind, mk = mask
    B, H, Hkv, Nq, Nk = shape
    check_masked_bwd(dtype, B, H, Hkv, Nq, Nk, d, kind, 9900 + Nq, **mk)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_bwd_documents(dtype, causal):
    need_gpu()
    lens = [[100, 3, 250, 1, 46], [400]]
    check_masked_bwd(dtype, 2, 4, 2, 400, 400, 128, "document", 9950, doc_lens=lens, causal=causal)


def test_masked_bwd_causal_matches_attn_bwd():
    """The causal mask as intervals gives the causal backward's gradients."""
    need_gpu()
    import online_softmax_attn_amd as osa
    from gpu_parity import TOL_G, rel_err
    w = S.custom("bf16", 1, 4, 2, 700, 128, True, seed_base=9960)
    inp = S.make_inputs(w, with_grad=True)
    lo, hi = S.mask_intervals("causal", 1, 700, 700)
    _, _, dq1, dk1, dv1 = run_masked_bwd(inp, lo, hi, w.scale)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = osa.attn_fwd(q, k, v, causal=True, scale=w.scale)
    dq2, dk2, dv2 = osa.attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert rel_err(f64(a), f64(b)) <= TOL_G["bf16"]


@pytest.mark.slow
@pytest.mark.parametrize("case", FULL, ids=lambda c: c[0])
def test_masked_bwd_full_size_groups(case):
    """Full-size masked backward: two (batch, kv-head) groups against the oracle."""
    need_gpu()
    from gpu_parity import TOL_G, rel_err
    name, dtype, B, H, Hkv, N, d, kind, mk = case
    w = S.custom(dtype, B, H, Hkv, N, d, False, seed_base=9800)
    inp = S.make_inputs(w, with_grad=True)
    lo, hi = S.mask_intervals(kind, B, N, N, **mk)
    o, lse, dq, dk, dv = run_masked_bwd(inp, lo, hi, w.scale)
    groups = [(0, 0), (B - 1, Hkv - 1)]
    ref = A.attention_backward_intervals(inp["q"], inp["k"], inp["v"], inp["do"], w.scale,
                                         lo.numpy(), hi.numpy(), heads=groups)
    n_rep = H // Hkv
    for b, g in groups:
        hs = slice(g * n_rep, (g + 1) * n_rep)
        e = {"dq": rel_err(f64(dq[b, hs]), ref["dq"][b, hs]),
             "dk": rel_err(f64(dk[b, g]), ref["dk"][b, g]),
             "dv": rel_err(f64(dv[b, g]), ref["dv"][b, g]),
             "o": out_err(f64(o[b, hs]), ref["o"][b, hs], dtype)}
        say(f"[masked] {name} group ({b},{g}) {', '.join(f'{k}={v:.2e}' for k, v in e.items())}")
        assert e["o"] <= TOL_O[dtype]
        assert max(e["dq"], e["dk"], e["dv"]) <= TOL_G[dtype], e
