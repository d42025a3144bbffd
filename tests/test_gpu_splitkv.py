"""GPU parity of the split-KV forward (few queries against many keys) against the
fp64 oracle: O and LSE element by element, for GQA groups, ragged key counts,
every chunking from one chunk to one chunk per 32-key tile, causal masks aligned
bottom-right, and the decoding workloads at full size."""

import numpy as np
import pytest
import torch

import oracle.attention as A
import synthetic as S
from gpu_parity import TOL_O, f64, max_abs, need_gpu, out_err, say, to_dev

pytestmark = pytest.mark.gpu


def run_split(inp, causal, scale, n_splits=0):
    import online_softmax_attn_amd as osa
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = osa.attn_fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=n_splits)
    torch.cuda.synchronize()
    return o, lse


def check_split(w, n_splits=0, label=""):
    inp = S.make_inputs(w, with_grad=False)
    say(f"[splitkv] {label or w.name} q={tuple(inp['q'].shape)} kv={tuple(inp['k'].shape)} "
        f"causal={w.causal} n_splits={n_splits}")
    o, lse = run_split(inp, w.causal, w.scale, n_splits)
    r_o, r_lse = A.attention_forward(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    g_o, g_l = f64(o), f64(lse)
    assert np.all(np.isfinite(g_o)) and np.all(np.isfinite(g_l))
    e_o, e_l = out_err(g_o, r_o, w.dtype), max_abs(g_l, r_lse)
    say(f"[splitkv]   errors o={e_o:.2e} lse={e_l:.2e}")
    assert e_o <= TOL_O[w.dtype] and e_l <= TOL_O[w.dtype], (e_o, e_l)
    return o, lse


SHAPES = [  # (B, H, Hkv, Nq, Nk)
    (1, 1, 1, 1, 1),
    (1, 2, 1, 1, 31),
    (2, 4, 2, 3, 100),
    (1, 8, 2, 5, 333),
    (1, 4, 4, 16, 1000),
    (1, 2, 1, 33, 257),     # 66 rows per group: three 32-row blocks, the last partial
    (1, 32, 8, 1, 2048),    # n_rep = 4 packed rows of one group
    (1, 8, 1, 20, 500),     # 160 rows per group: four-wave workgroups, one wave all padding
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}Hkv{}Nq{}Nk{}".format(*s))
def test_splitkv_small(dtype, d, causal, shape):
    need_gpu()
    B, H, Hkv, Nq, Nk = shape
    w = S.custom(dtype, B, H, Hkv, Nq, d, causal, seed_base=9000 + Nk, Nk=Nk)
    check_split(w)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 1000])
def test_splitkv_chunkings(n_splits):
    """From one chunk to one per tile (1000 is capped), with uneven last chunks and,
    under the causal mask, chunks some rows see nothing of."""
    need_gpu()
    w = S.custom("bf16", 1, 4, 2, 40, 128, True, seed_base=9100, Nk=300)
    check_split(w, n_splits, label=f"chunks={n_splits}")


def test_splitkv_all_chunkings_agree_closely():
    """Different chunkings agree to the dtype's rounding: each chunk rounds P to fp16
    against its own running max (and sums the rounded values), so chunkings differ
    by up to about 2^-11 relative in l and O, well inside the fp16 bar."""
    need_gpu()
    w = S.custom("fp16", 1, 4, 1, 2, 64, False, seed_base=9200, Nk=1500)
    inp = S.make_inputs(w, with_grad=False)
    outs = [run_split(inp, False, w.scale, n) for n in (1, 4, 47)]
    for o, lse in outs[1:]:
        assert max_abs(f64(o), f64(outs[0][0])) <= TOL_O["fp16"]
        assert max_abs(f64(lse), f64(outs[0][1])) <= TOL_O["fp16"]


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_equals_attn_fwd_for_square(causal):
    """Nq == Nk: the split-KV path and the main forward solve the same problem (they
    round P against different running maxima, so they agree to the bf16 bar)."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w = S.custom("bf16", 1, 4, 2, 300, 128, causal, seed_base=9300)
    inp = S.make_inputs(w, with_grad=False)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o1, l1 = osa.attn_fwd(q, k, v, causal=causal, scale=w.scale)
    o2, l2 = osa.attn_fwd_splitkv(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert max_abs(f64(o1), f64(o2)) <= 2 * TOL_O["bf16"]
    assert max_abs(f64(l1), f64(l2)) <= TOL_O["bf16"]
    check_split(w)


def test_splitkv_outlier_keys():
    """A few keys scaled by 8 put the max late in some chunks: the merge must rescale."""
    need_gpu()
    w = S.custom("bf16", 1, 8, 2, 4, 128, True, seed_base=9400, Nk=4096, k_outlier_frac=0.01,
                 k_outlier_seed=9401)
    check_split(w)


def test_splitkv_workspace_reuse_and_side_stream():
    """A dirty, reused workspace and a non-default stream give identical results."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w = S.custom("fp16", 2, 8, 2, 3, 128, True, seed_base=9500, Nk=777)
    inp = S.make_inputs(w, with_grad=False)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    a = run_split(inp, True, w.scale)
    need = osa.attn_fwd_splitkv_workspace_bytes(2, 8, 2, 3, 777, 128, True, q.dtype)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = osa.attn_fwd_splitkv(q, k, v, causal=True, scale=w.scale, workspace=ws)
        c = osa.attn_fwd_splitkv(q, k, v, causal=True, scale=w.scale, workspace=ws)
    s.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


@pytest.mark.parametrize("name", sorted(S.DECODE))
def test_splitkv_decode_workloads(name):
    """The decoding workloads at full size, every row against the oracle."""
    need_gpu()
    check_split(S.DECODE[name])
