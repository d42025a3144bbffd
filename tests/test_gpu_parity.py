"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and ragged shapes are compared element by element over the whole problem.
The named workloads run at their full sizes: the fp32 head, the bf16 forward, the
fp16 causal and the bf16 GQA causal workloads, and the sweep point that bench.py
times, are compared element by element over the whole problem (forward and
backward); the other sweep points on rows sampled across every head and one whole
key/value group.
"""

import math

import numpy as np
import pytest
import torch

import synthetic as S
from gpu_parity import (TOL_G, TOL_O, check_all_heads, check_full, check_group_bwd,
                         check_sampled_fwd, f64,
                        max_abs, need_gpu, rel_err, run_bwd, run_fwd, say)

pytestmark = pytest.mark.gpu

SMALL_SHAPES = [  # (B, H, Hkv, N)
    (1, 1, 1, 1),
    (1, 2, 1, 17),
    (2, 2, 2, 64),
    (1, 4, 2, 200),
    (1, 3, 1, 333),
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "B{}H{}Hkv{}N{}".format(*s))
def test_small_full(dtype, d, causal, shape):
    need_gpu()
    B, H, Hkv, N = shape
    w = S.custom(dtype, B, H, Hkv, N, d, causal, seed_base=7000 + N + d + 3 * H)
    inp = S.make_inputs(w)
    check_full(inp, dtype, causal, w.scale, backward=True, label=w.name)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_outlier_keys_small(dtype):
    """Key rows scaled x8 make the running max move late in the loop."""
    need_gpu()
    w = S.custom(dtype, 1, 4, 2, 700, 128, True, seed_base=7700, k_outlier_frac=0.02,
                 k_outlier_seed=7701)
    check_full(S.make_inputs(w), dtype, True, w.scale, label=w.name)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows(dtype, causal):
    """All value rows equal w: every output row is w (up to the output rounding)
    and dQ, dK vanish (pin of the definition; here checked on the GPU)."""
    need_gpu()
    w_ = S.custom(dtype, 1, 2, 1, 300, 64, causal, seed_base=7800)
    inp = S.make_inputs(w_)
    row = torch.linspace(-2, 2, 64).to(S.DTYPES[dtype])
    inp["v"] = row.expand_as(inp["v"]).contiguous()
    o, lse, dq, dk, dv = run_bwd(inp, causal, w_.scale)
    assert max_abs(f64(o), row.double().numpy()) <= TOL_O[dtype]
    gmax = max(float(f64(dv).__abs__().max()), 1e-30)
    assert float(np.abs(f64(dq)).max()) <= TOL_G[dtype] * gmax
    assert float(np.abs(f64(dk)).max()) <= TOL_G[dtype] * gmax


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_query_uniform(dtype):
    """Q = 0: O is the mean (causal: prefix mean) of V and LSE = ln(visible keys)."""
    need_gpu()
    w_ = S.custom(dtype, 1, 1, 1, 257, 128, True, seed_base=7900)
    inp = S.make_inputs(w_)
    inp["q"] = torch.zeros_like(inp["q"])
    o, lse = run_fwd(inp, True, w_.scale)
    v = inp["v"][0, 0].double().numpy()
    n = np.arange(1, 258)
    assert max_abs(f64(o)[0, 0], np.cumsum(v, axis=0) / n[:, None]) <= TOL_O[dtype]
    assert max_abs(f64(lse)[0, 0], np.log(n)) <= TOL_O[dtype]


def test_backward_deterministic():
    """Every output element has a single writer: repeated runs are bitwise equal."""
    need_gpu()
    w = S.custom("bf16", 1, 4, 2, 1000, 128, True, seed_base=8000)
    inp = S.make_inputs(w)
    a = run_bwd(inp, True, w.scale)
    b = run_bwd(inp, True, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype,causal,order", [("bf16", False, "dkdv_first"),
                                                 ("fp16", True, "dq_first"),
                                                 ("fp32", True, "dkdv_first")])
def test_backward_stages_match_attn_bwd(dtype, causal, order):
    """The three stage entry points, run one by one on a shared workspace, write
    exactly what attn_bwd writes (same kernels, single writer per element)."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w = S.custom(dtype, 1, 4, 2, 300, 64 if dtype == "fp16" else 128, causal, seed_base=8050)
    inp = S.make_inputs(w)
    o, lse, dq, dk, dv = run_bwd(inp, causal, w.scale)
    q, k, v, do = (t.to("cuda") for t in (inp["q"], inp["k"], inp["v"], inp["do"]))
    ws = osa.new_bwd_workspace(q, k)
    ws.fill_(0xFF)  # stale contents must not matter
    osa.attn_bwd_preprocess(q, k, o, lse, do, ws)
    kw = dict(causal=causal, scale=w.scale)
    if order == "dq_first":
        dq2 = osa.attn_bwd_dq(q, k, v, o, lse, do, ws, **kw)
        dk2, dv2 = osa.attn_bwd_dkdv(q, k, v, o, lse, do, ws, **kw)
    else:
        dk2, dv2 = osa.attn_bwd_dkdv(q, k, v, o, lse, do, ws, **kw)
        dq2 = osa.attn_bwd_dq(q, k, v, o, lse, do, ws, **kw)
    torch.cuda.synchronize()
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(x, y)


def test_side_stream_matches_default_stream():
    need_gpu()
    w = S.custom("fp16", 1, 2, 2, 513, 64, False, seed_base=8100)
    inp = S.make_inputs(w)
    a = run_bwd(inp, False, w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_bwd(inp, False, w.scale)
    s.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_medium_ragged_two_block_tiles():
    """Enough rows to select the 256-row forward tiles, with a ragged last tile."""
    need_gpu()
    w = S.custom("bf16", 1, 32, 8, 4500, 128, False, seed_base=8200)
    inp = S.make_inputs(w)
    outs = run_bwd(inp, False, w.scale)
    check_sampled_fwd(inp, outs[0], outs[1], "bf16", False, w.scale, per_head=4, label=w.name)
    check_group_bwd(inp, outs, "bf16", False, w.scale, [(0, 3)], label=w.name)


def test_medium_ragged_wide_rows_d64():
    """d = 64 non-causal with a grid of at least one 512-row workgroup per CU (so the
    two-block-per-wave forward runs) and a ragged last tile."""
    need_gpu()
    w = S.custom("bf16", 4, 16, 16, 2500, 64, False, seed_base=8400)
    inp = S.make_inputs(w)
    outs = run_bwd(inp, False, w.scale)
    check_sampled_fwd(inp, outs[0], outs[1], "bf16", False, w.scale, per_head=8, label=w.name)
    check_group_bwd(inp, outs, "bf16", False, w.scale, [(2, 9)], label=w.name)


def test_medium_ragged_causal_fp16():
    need_gpu()
    w = S.custom("fp16", 2, 16, 16, 4477, 64, True, seed_base=8300)
    inp = S.make_inputs(w)
    outs = run_bwd(inp, True, w.scale)
    check_sampled_fwd(inp, outs[0], outs[1], "fp16", True, w.scale, per_head=4, label=w.name)
    check_group_bwd(inp, outs, "fp16", True, w.scale, [(1, 15)], label=w.name)


# ---- the five named workloads at full size ------------------------------------------

def test_workload_fp32_single_head():
    need_gpu()
    w = S.WORKLOADS["fp32_single_head"]
    check_full(S.make_inputs(w), "fp32", False, w.scale, backward=True, label=w.name)


def test_workload_bf16_fwd_full():
    need_gpu()
    w = S.WORKLOADS["bf16_fwd"]
    check_full(S.make_inputs(w), "bf16", False, w.scale, backward=False, label=w.name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_workload_fp16_causal():
    """fp16 causal B2 H32 N8192 d64, every output element of the forward and the
    backward against the oracle."""
    need_gpu()
    w = S.WORKLOADS["fp16_causal"]
    inp = S.make_inputs(w)
    outs = run_bwd(inp, True, w.scale)
    check_all_heads(inp, outs, "fp16", True, w.scale, label=w.name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_workload_bf16_gqa_causal():
    """bf16 GQA causal B1 H32 Hkv8 N16384 d128 with 1% of key rows x8, every output
    element of the forward and the backward against the oracle."""
    need_gpu()
    w = S.WORKLOADS["bf16_gqa_causal"]
    inp = S.make_inputs(w)
    outs = run_bwd(inp, True, w.scale)
    check_all_heads(inp, outs, "bf16", True, w.scale, label=w.name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_workload_headline_full():
    """The sweep point bench.py times (bf16 B4 H16 N8192 d128, non-causal), every
    output element of the forward and the backward against the oracle."""
    need_gpu()
    w = S.HEADLINE
    inp = S.make_inputs(w)
    outs = run_bwd(inp, False, w.scale)
    check_all_heads(inp, outs, "bf16", False, w.scale, label=w.name)


@pytest.mark.slow
@pytest.mark.parametrize("point", range(len(S.sweep_points())))
def test_workload_sweep(point):
    need_gpu()
    w = S.sweep_points()[point]
    inp = S.make_inputs(w)
    outs = run_bwd(inp, False, w.scale)
    check_sampled_fwd(inp, outs[0], outs[1], "bf16", False, w.scale, per_head=2,
                      seed=point, label=w.name)
    check_group_bwd(inp, outs, "bf16", False, w.scale, [(point % 4, (5 * point) % 16)],
                    label=w.name)
