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
    e_o, e_l = out_err(g_o, r_o), max_abs(g_l[fin], r_lse[fin])
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
            err_o = max(err_o, out_err(f64(o[b, h])[rows], ro))
            err_l = max(err_l, max_abs(f64(lse[b, h])[rows], rl))
    say(f"[masked] {name} sampled o={err_o:.2e} lse={err_l:.2e}")
    assert err_o <= TOL_O[dtype] and err_l <= TOL_O[dtype]
