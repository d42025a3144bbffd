"""GPU parity of the fp8 (e4m3) forward against the fp64 oracle on the decoded inputs
(oracle.fp8: O_ref and LSE_ref of every checked row come from it).

Bar (derived from the arithmetic, element by element).  The scores are exact fp8
products summed in fp32; the probabilities P (formed against a running reference that
never exceeds the row max, P * 256 <= 446) are rounded to e4m3 after scaling by 256,
and O = sum P8 v / sum P8 with the same P8.  With p_j = exp(s_j - max s) (so p <= 1,
L = sum p = exp(LSE - max s) >= 1), each rounded weight is p_j (1 + delta_j) + eps_j with |delta_j| <= 2^-4 (three mantissa
bits) and |eps_j| <= 2^-18 (half the subnormal spacing 2^-9 of e4m3, over the factor
256; earlier tiles are rescaled by factors <= 1, which only shrinks their errors).
Then for every output element
    |O - O_ref| <= (2^-4 * L * W + 2^-18 * A) / (L (1 - 2^-4) - n 2^-18)
                   + 2^-8 |O_ref| (bf16 output rounding) + 1e-5 max|v| (fp32)
with W = sum_j P_j |v_j - O_ref| (P the exact normalised weights), A = sum_j
|v_j - O_ref| and n the number of visible keys; and
    |LSE - LSE_ref| <= -ln(1 - 2^-4 - n 2^-18 / L) + 1e-5 (1 + |LSE_ref|).
Sharp cases on top: rows of V all equal give O = v (the weights cancel), and Q = 0
gives exact uniform weights (256 is exact in e4m3): O = the mean of the visible rows
of V and LSE = ln n.
"""

import numpy as np
import pytest
import torch

import oracle.attention as A
import oracle.fp8 as F8
import synthetic as S
from gpu_parity import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DLT, EPS = 2.0 ** -4, 2.0 ** -18


def run_fp8(inp, causal, scale):
    import online_softmax_attn_amd as osa
    o, lse = osa.attn_fwd_fp8(to_dev(inp["q8"]), to_dev(inp["k8"]), to_dev(inp["v8"]), inp["dq"],
                              inp["dk"], inp["dv"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_reference(inp, causal, scale, heads, rows):
    """O_ref, LSE_ref [B][len(heads)][len(rows)] from the pinned fp8 oracle (the plain
    attention of the decoded inputs): whole problems through attention_forward_fp8,
    row subsets through its row variant."""
    B, H, N, _ = inp["q8"].shape
    args = (inp["q8"], inp["k8"], inp["v8"], inp["dq"], inp["dk"], inp["dv"])
    if len(heads) == H and len(rows) == N:
        return F8.attention_forward_fp8(*args, scale, causal)
    picks = [(b, h, int(i)) for b in range(B) for h in heads for i in rows]
    o, lse = F8.attention_forward_fp8_rows(*args, scale, causal, picks)
    return (o.reshape(B, len(heads), len(rows), -1), lse.reshape(B, len(heads), len(rows)))


def bound_check(inp, causal, scale, o, lse, label, heads=None, rows=None, block=16):
    """|O - O_ref| and |LSE - LSE_ref| against the oracle, within the derived bound.
    O_ref and LSE_ref come from oracle.fp8; the terms of the bound (the exact weights
    P, their sum L, W, A and the visible key count n) are formed here from the decoded
    inputs, and the O_ref they imply is checked to agree with the oracle's."""
    q = F8.dequantize(inp["q8"], inp["dq"])
    k = F8.dequantize(inp["k8"], inp["dk"])
    v = F8.dequantize(inp["v8"], inp["dv"])
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    ref_o, ref_l = oracle_reference(inp, causal, scale, heads, rows)
    if ref_o.shape[1] == H and ref_o.shape[2] == N:  # whole problem: pick the same sub-arrays
        ref_o, ref_l = ref_o[:, heads][:, :, rows], ref_l[:, heads][:, :, rows]
    worst_o = worst_l = -1.0
    err = agree = 0.0
    for b in range(B):
        for hi_, h in enumerate(heads):
            g = A.kv_head_of(h, H, Hkv)
            vg = v[b, g]
            vmax = np.abs(vg).max()
            for r0 in range(0, len(rows), block):
                ri = rows[r0:r0 + block]
                o_ref = ref_o[b, hi_, r0:r0 + block]
                lse_ref = ref_l[b, hi_, r0:r0 + block]
                s = scale * (q[b, h][ri] @ k[b, g].T)
                if causal:
                    s = np.where(np.arange(N)[None, :] <= ri[:, None], s, -np.inf)
                mx = s.max(-1, keepdims=True)
                p = np.exp(s - mx)
                L = p.sum(-1, keepdims=True)
                P = p / L
                agree = max(agree, float(np.abs(P @ vg - o_ref).max()))
                n = np.isfinite(s).sum(-1, keepdims=True).astype(float)
                dev = np.abs(vg[None, :, :] - o_ref[:, None, :])  # [rows, Nk, d]
                W = np.einsum("ij,ijc->ic", P, dev)
                Asum = dev.sum(1)
                bound = (DLT * L * W + EPS * Asum) / (L * (1 - DLT) - n * EPS) \
                    + 2.0 ** -8 * np.abs(o_ref) + 1e-5 * vmax
                got = o[b, h][ri]
                worst_o = max(worst_o, float((np.abs(got - o_ref) - bound).max()))
                lb = -np.log(1 - DLT - n[:, 0] * EPS / L[:, 0]) + 1e-5 * (1 + np.abs(lse_ref))
                worst_l = max(worst_l, float((np.abs(lse[b, h][ri] - lse_ref) - lb).max()))
                err = max(err, float(np.abs(got - o_ref).max()))
    say(f"[fp8] {label}: max |dO| {err:.2e}, worst excess O {worst_o:.2e} LSE {worst_l:.2e}; "
        f"bound terms vs oracle {agree:.1e}")
    assert agree <= 1e-12 * max(1.0, float(np.abs(v).max())), (label, agree)
    assert worst_o <= 0 and worst_l <= 0, (label, worst_o, worst_l)


def case(B, H, Hkv, N, causal, seed, d=128):
    w = S.custom("bf16", B, H, Hkv, N, d, causal, seed_base=seed)
    return w, S.make_fp8_inputs(w)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 1), (1, 2, 2, 77), (2, 4, 2, 300), (1, 4, 1, 1000),
                                   (1, 2, 1, 256)],
                         ids=lambda s: "B{}H{}Hkv{}N{}".format(*s))
def test_fp8_forward(shape, causal, d):
    need_gpu()
    B, H, Hkv, N = shape
    w, inp = case(B, H, Hkv, N, causal, 31000 + N + d, d)
    o, lse = run_fp8(inp, causal, w.scale)
    bound_check(inp, causal, w.scale, o, lse, f"B{B}H{H}Hkv{Hkv}N{N}d{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_equal_value_rows(causal, d):
    """Every row of V the same vector: O is that vector whatever the weights."""
    need_gpu()
    w, inp = case(1, 2, 1, 333, causal, 32000 + d, d)
    v8 = inp["v8"].clone()
    v8[:] = v8[:, :, :1, :]
    inp["v8"] = v8.contiguous()
    o, _ = run_fp8(inp, causal, w.scale)
    v = F8.dequantize(inp["v8"], inp["dv"])[0, 0, 0]
    err = np.abs(o - v[None, None, None, :]) - (2.0 ** -8 * np.abs(v) + 1e-6)
    say(f"[fp8] equal V rows d={d} causal={causal}: worst excess {err.max():.2e}")
    assert err.max() <= 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_zero_query(causal, d):
    """Q = 0: every visible key has weight exactly 1 (256 in e4m3 is exact), so O is
    the mean (the prefix mean when causal) of V and LSE = ln(number of keys)."""
    need_gpu()
    w, inp = case(1, 2, 1, 200, causal, 33000 + d, d)
    inp["q8"] = torch.zeros_like(inp["q8"])
    o, lse = run_fp8(inp, causal, w.scale)
    v = F8.dequantize(inp["v8"], inp["dv"])[0, 0]
    n = np.arange(1, 201, dtype=float) if causal else np.full(200, 200.0)
    mean = (np.cumsum(v, 0) / n[:, None]) if causal else np.broadcast_to(v.mean(0), v.shape)
    err_o = np.abs(o[0] - mean[None]) - (2.0 ** -8 * np.abs(mean[None]) + 1e-5 * np.abs(v).max())
    err_l = np.abs(lse[0] - np.log(n)[None]) - 1e-5 * (1 + np.log(n)[None])
    say(f"[fp8] Q=0 d={d} causal={causal}: worst excess O {err_o.max():.2e} LSE {err_l.max():.2e}")
    assert err_o.max() <= 0 and err_l.max() <= 0


@pytest.mark.slow
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_headline_shape_sampled_heads(causal):
    """B4 H16 N8192 d128 at full size (the shape bench.py times); the bound checked on
    32 sampled rows of two heads of batch 0 (the kernel runs the whole problem)."""
    need_gpu()
    w, inp = case(4, 16, 16, 8192, causal, 34000)
    o, lse = run_fp8(inp, causal, w.scale)
    sub = {n: (t[:1] if hasattr(t, "shape") else t) for n, t in inp.items()}
    rows = np.unique(np.r_[0, 1, 255, 256, 4095, 8191, np.random.default_rng(5).choice(8192, 26, replace=False)])
    bound_check(sub, causal, w.scale, o[:1], lse[:1], f"B4H16N8192 causal={causal}", heads=[0, 9],
                rows=rows, block=4)
