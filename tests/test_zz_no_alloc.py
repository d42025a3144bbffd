"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd, through the C ABI.

Both launch the same three kernels; only where their workspace lives differs (a
fixed device array in the library instead of caller memory), so every gradient
must be bit-identical to attn_bwd's, which the parity tests hold to the oracle.
Two calls in a row, the second on a smaller problem, show that what a previous
call left in the shared array does not matter.
"""

import pytest
import torch

import synthetic as S
from gpu_parity import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(dtype, B, H, Hkv, N, d, causal, seed):
    import online_softmax_attn_amd as osa
    w = S.custom(dtype, B, H, Hkv, N, d, causal, seed_base=seed)
    inp = S.make_inputs(w)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = osa.attn_fwd(q, k, v, causal=causal, scale=w.scale)
    return w, (q, k, v, o, lse, do)


def test_noalloc_matches_attn_bwd_twice():
    need_gpu()
    import online_softmax_attn_amd as osa
    cases = [("bf16", 2, 8, 2, 3001, 128, True, 9500),   # larger first
             ("fp16", 1, 4, 1, 700, 64, False, 9510)]    # then smaller
    for dtype, B, H, Hkv, N, d, causal, seed in cases:
        say(f"[noalloc] {dtype} B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
        w, (q, k, v, o, lse, do) = _inputs(dtype, B, H, Hkv, N, d, causal, seed)
        ref = osa.attn_bwd(q, k, v, o, lse, do, causal=causal, scale=w.scale)
        out = [torch.full_like(t, float("nan")) for t in ref]
        got = osa.attn_bwd_noalloc(q, k, v, o, lse, do, causal=causal, scale=w.scale,
                                   dq=out[0], dk=out[1], dv=out[2])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), (name, float((a.float() - b.float()).abs().max()))
        say("[noalloc]   bit-identical to attn_bwd")


def test_noalloc_fp32_and_refusal():
    """The fp32 kernels take the same workspace; a problem over the fixed size is
    refused with its own status (the binding raises) and nothing is written."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w, (q, k, v, o, lse, do) = _inputs("fp32", 1, 2, 1, 257, 64, True, 9520)
    ref = osa.attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    got = osa.attn_bwd_noalloc(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    lib = osa.library()
    dq = torch.zeros(4, device="cuda")
    st = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dq.data_ptr(),
                              dq.data_ptr(), 1, 1, 1, 4194305, 64, 0.125, 0, 0,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == osa.STATUS["ATTN_ERR_SCRATCH"]
    assert torch.count_nonzero(dq) == 0
