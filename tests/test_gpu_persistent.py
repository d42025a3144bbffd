"""Persistent grids (the forward without an interval mask, the causal dK/dV kernel).

Their workgroups walk a fixed schedule of tiles (one block of tiles per XCD, taken in
snake-ordered rounds) instead of one tile each.  These tests check that many launches
in a row, and launches on two streams at once, give results bit for bit equal to the
first launch, which the oracle checks, on shapes whose tile counts do not divide
evenly among the workgroups.
"""

import pytest
import torch

import synthetic as S
from gpu_parity import check_full, check_sampled_fwd, need_gpu, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu

N_LAUNCHES = 20


def _run(inp, scale, stream=None, causal=True):
    import online_softmax_attn_amd as osa
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    if stream is None:
        stream = torch.cuda.current_stream()
    else:
        stream.wait_stream(torch.cuda.current_stream())  # the inputs' copies
    with torch.cuda.stream(stream):
        o, lse = osa.attn_fwd(q, k, v, causal=causal, scale=scale)
        dq, dk, dv = osa.attn_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    return o, lse, dq, dk, dv


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_many_launches_bitwise(d, causal):
    need_gpu()
    w = S.custom("bf16", 2, 4, 2, 1100, d, causal, seed_base=9100 + d + 7 * causal)
    inp = S.make_inputs(w)
    check_full(inp, "bf16", causal, w.scale, label=w.name)
    first = _run(inp, w.scale, causal=causal)
    torch.cuda.synchronize()
    for i in range(N_LAUNCHES):
        again = _run(inp, w.scale, causal=causal)
        torch.cuda.synchronize()
        assert _same(first, again), f"launch {i} differs"
    say(f"[persistent] {w.name}: {N_LAUNCHES} launches bit-identical")


@pytest.mark.parametrize("d,B,H,Hkv,N", [(128, 2, 48, 8, 1700), (64, 2, 96, 8, 1700),
                                           (128, 1, 35, 7, 2100), (64, 1, 35, 5, 2100)])
def test_many_tiles_per_workgroup(d, B, H, Hkv, N):
    """Non-causal forwards with several query tiles per workgroup and a ragged last tile
    per head: 672 and 768 tiles, and 315 (256-row tiles at both head dims; 315 is not a
    multiple of the 8 XCD blocks).  Sampled rows of every head against the oracle."""
    need_gpu()
    w = S.custom("fp16", B, H, Hkv, N, d, False, seed_base=9400 + d + N)
    inp = S.make_inputs(w)
    o, lse = run_fwd(inp, False, w.scale)
    check_sampled_fwd(inp, o, lse, "fp16", False, w.scale, per_head=4, label=w.name)


@pytest.mark.parametrize("causal", [True, False])
def test_two_streams_at_once(causal):
    need_gpu()
    w1 = S.custom("bf16", 1, 8, 8, 2048, 128, causal, seed_base=9200 + 7 * causal)
    w2 = S.custom("fp16", 2, 4, 1, 1500, 64, causal, seed_base=9300 + 7 * causal)
    in1, in2 = S.make_inputs(w1), S.make_inputs(w2)
    ref1, ref2 = _run(in1, w1.scale, causal=causal), _run(in2, w2.scale, causal=causal)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(8):
        got1 = _run(in1, w1.scale, s1, causal=causal)
        got2 = _run(in2, w2.scale, s2, causal=causal)
        torch.cuda.synchronize()
        assert _same(ref1, got1) and _same(ref2, got2), f"round {i} differs"
    check_full(in1, "bf16", causal, w1.scale, label=w1.name)
    check_full(in2, "fp16", causal, w2.scale, label=w2.name)
