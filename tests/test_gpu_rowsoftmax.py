"""GPU parity of row softmax, log-softmax and cross-entropy with logits (forward and
backward) against the fp64 oracle in oracle/rowsoftmax.py, element by element.

Bar, per element (derived from the arithmetic; the kernels keep fp32 statistics):
    |got - ref| <= rtol[dtype] * |ref| + 3e-5 * scale + atol[dtype]
  * rtol is the output's rounding to its dtype, half an ulp relative: 2^-8 (bf16),
    2^-11 (fp16), and 0 for fp32, plus 1e-6 of slack;
  * 3e-5 * scale bounds the fp32 arithmetic: the exponent argument carries a relative
    rounding error of a few 2^-24, i.e. an absolute one of |argument| * 2^-23 or so
    (|argument| stays below about 150 here), and the row sums are fp32 sums.  `scale`
    is the size of the terms the result is made of, with a row sum counted by the sum
    of its terms' magnitudes (the sum may cancel, its rounding error does not): |ref|
    for the softmax output, |x| + |lse| for the log-softmax output,
    y * (|dy| + sum_j |y_j dy_j|) for the softmax backward, |dy| + exp(y) * sum_j |dy_j|
    for the log-softmax backward, dloss * (p + [j == target]) for the cross-entropy
    backward;
  * atol covers fp16's subnormals (spacing 2^-24): 6e-8; 1e-30 for fp32 and bf16.
The loss and the row logsumexp are fp32 outputs: |got - ref| <= 3e-5 * max(1, |lse|).

Inputs of the backward passes (y, lse) are the oracle's forward outputs rounded to
the kernel's input types, so both sides see the same values.
"""

import numpy as np
import pytest
import torch

import oracle.rowsoftmax as R
import synthetic as S
from gpu_parity import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

RTOL = {"fp32": 1e-6, "fp16": 2.0 ** -11 + 1e-6, "bf16": 2.0 ** -8 + 1e-6}
ATOL = {"fp32": 1e-30, "fp16": 6e-8, "bf16": 1e-30}
ARITH = 3e-5


def f64(t):
    return t.detach().cpu().double().numpy()


def check(got, ref, scale, dtype, label):
    got = f64(got) if isinstance(got, torch.Tensor) else got
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, label
    same_inf = (np.isinf(ref) & (got == ref))
    assert np.all(np.isfinite(got) | same_inf), label
    fin = np.isfinite(ref)
    excess = np.abs(got[fin] - ref[fin]) - (RTOL[dtype] * np.abs(ref[fin]) + ARITH * scale[fin]
                                            + ATOL[dtype])
    worst = float(excess.max()) if excess.size else -1.0
    say(f"[rows] {label}: worst excess {worst:.2e}")
    assert worst <= 0, (label, worst)


def case(op, dtype, rows, cols, seed, std=1.0, ignore_frac=0.0):
    w = S.RowWorkload(f"case_{op}_{dtype}_{rows}x{cols}", op, dtype, rows, cols, seed, std,
                      ignore_frac)
    return w, S.row_inputs(w)


def check_softmax(dtype, rows, cols, log, seed, std=1.0, neg_inf_frac=0.0, offset=0.0):
    import online_softmax_attn_amd as osa
    op = "log_softmax" if log else "softmax"
    w, inp = case(op, dtype, rows, cols, seed, std)
    x = inp["x"]
    if offset:
        x = (x.float() + offset).to(x.dtype)
    if neg_inf_frac > 0:  # masked classes; every row keeps its first entry
        g = torch.Generator().manual_seed(seed + 7)
        m = torch.rand(x.shape, generator=g) < neg_inf_frac
        m[:, 0] = False
        x = x.masked_fill(m, float("-inf"))
    label = f"{op} {dtype} {rows}x{cols}" + (f" -inf{neg_inf_frac}" if neg_inf_frac else "")
    xd = to_dev(x)
    y = osa.rowsoftmax_fwd(xd, log_softmax=log)
    torch.cuda.synchronize()
    x64 = f64(x)
    if log:
        ref = R.log_softmax(x64)
        lse = R.logsumexp(x64)[:, None]
        scale = np.abs(np.where(np.isfinite(x64), x64, 0.0)) + np.abs(lse)
    else:
        ref = R.softmax(x64)
        scale = np.abs(ref)
    check(y, ref, scale, dtype, label + " fwd")

    # Backward from the oracle's forward output, rounded to the dtype.
    y_in = torch.from_numpy(ref).to(S.DTYPES[dtype]).contiguous()
    dy = inp["dy"]
    dx = osa.rowsoftmax_bwd(to_dev(y_in), to_dev(dy), log_softmax=log)
    torch.cuda.synchronize()
    y64, dy64 = f64(y_in), f64(dy)
    if log:
        ref_b = R.log_softmax_backward(y64, dy64)
        scale_b = np.abs(dy64) + np.exp(y64) * np.abs(dy64).sum(-1, keepdims=True)
    else:
        ref_b = R.softmax_backward(y64, dy64)
        scale_b = y64 * (np.abs(dy64) + np.abs(y64 * dy64).sum(-1, keepdims=True))
    check(dx, ref_b, scale_b, dtype, label + " bwd")


# Column counts that reach every register-kernel shape in each dtype (64 .. 1024
# threads per row, several rows per workgroup below 256 threads, 1 .. 16 chunks of 16
# bytes per thread; the forward and the backward pick different shapes for one row
# length) and the streaming kernels (rows too long to hold, and rows whose length is
# not a whole number of 16-byte chunks).
COLS = [1, 3, 8, 64, 100, 512, 1000, 1001, 2048, 4096, 8192, 12345, 16000, 32768, 65536,
        131072, 200000]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("log", [False, True], ids=["softmax", "log_softmax"])
def test_rowsoftmax(dtype, cols, log):
    need_gpu()
    rows = max(1, min(37, 2_000_000 // cols))  # ragged: not a multiple of 4 rows per block
    check_softmax(dtype, rows, cols, log, seed=20000 + cols)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("cols", [64, 4096, 32768, 131072, 1001])
@pytest.mark.parametrize("log", [False, True], ids=["softmax", "log_softmax"])
def test_rowsoftmax_masked_classes(dtype, cols, log):
    """Entries of -inf (masked classes) get probability 0 and log-probability -inf."""
    need_gpu()
    check_softmax(dtype, 6, cols, log, seed=21000 + cols, neg_inf_frac=0.3)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rowsoftmax_large_logits(dtype):
    """Logits of std 20 around +50: exponent arguments up to ~150 and a dominant entry."""
    need_gpu()
    check_softmax(dtype, 9, 4096, False, seed=22000, std=20.0, offset=50.0)
    check_softmax(dtype, 9, 12345, True, seed=22001, std=20.0, offset=50.0)


def test_rowsoftmax_many_rows():
    """More rows than a single launch covers (2^20 workgroups of 4 one-wave rows):
    the rows go out in several launches."""
    need_gpu()
    import online_softmax_attn_amd as osa
    rows, cols = (1 << 22) + 5, 8
    g = torch.Generator().manual_seed(23000)
    x = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    y = osa.rowsoftmax_fwd(to_dev(x))
    torch.cuda.synchronize()
    idx = np.r_[0:3, (1 << 22) - 2:(1 << 22) + 5]
    ref = R.softmax(f64(x[idx]))
    check(y[idx], ref, np.abs(ref), "bf16", f"softmax bf16 {rows}x{cols} sampled")


def check_xent(dtype, rows, cols, seed, std=2.0, ignore_frac=0.1, extra_ignored=(),
               neg_inf_frac=0.0, offset=0.0):
    import online_softmax_attn_amd as osa
    w, inp = case("xent", dtype, rows, cols, seed, std, ignore_frac)
    x, t = inp["x"], inp["targets"].clone()
    if offset:
        x = (x.float() + offset).to(x.dtype)
    for r, val in extra_ignored:  # targets outside 0 .. cols-1 of other kinds
        if r < rows:
            t[r] = val
    if neg_inf_frac > 0:
        g = torch.Generator().manual_seed(seed + 7)
        m = torch.rand(x.shape, generator=g) < neg_inf_frac
        m[torch.arange(rows), t.clamp(0, cols - 1).long()] = False
        x = x.masked_fill(m, float("-inf"))
    label = f"xent {dtype} {rows}x{cols}" + (f" -inf{neg_inf_frac}" if neg_inf_frac else "")
    g = torch.Generator().manual_seed(seed + 5)
    dloss = torch.rand((rows,), generator=g, dtype=torch.float32) + 0.5
    xd, td = to_dev(x), to_dev(t)
    loss, lse = osa.rowxent_fwd(xd, td)
    torch.cuda.synchronize()
    x64, t64 = f64(x), t.numpy().astype(np.int64)
    t_or = t64
    r_loss, r_lse = R.cross_entropy(x64, t_or)
    s = np.maximum(1.0, np.abs(r_lse))
    check(lse, r_lse, s, "fp32", label + " lse")
    check(loss, r_loss, s, "fp32", label + " loss")

    lse_in = torch.from_numpy(r_lse).to(torch.float32)
    dx = osa.rowxent_bwd(xd, td, to_dev(lse_in), to_dev(dloss))
    torch.cuda.synchronize()
    d64 = f64(dloss)
    ref = R.cross_entropy_backward(x64, t_or, d64)
    p = R.softmax(x64)
    onehot = np.zeros_like(p)
    live = (t_or >= 0) & (t_or < cols)
    onehot[np.nonzero(live)[0], t_or[live]] = 1.0
    scale = (np.abs(d64) * live)[:, None] * (p + onehot)
    check(dx, ref, scale, dtype, label + " bwd")
    assert np.all(f64(dx)[~live] == 0.0), "ignored rows must get a zero gradient"


XENT_COLS = [1, 3, 8, 1000, 1001, 8192, 8193, 32000, 50257, 128256]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("cols", XENT_COLS)
def test_rowxent(dtype, cols):
    need_gpu()
    rows = max(2, min(41, 4_000_000 // cols))
    check_xent(dtype, rows, cols, seed=24000 + cols,
               extra_ignored=((1, -1), (2, cols), (3, 2**31 - 1), (4, -2**31)))


@pytest.mark.parametrize("cols", [1000, 1001, 32000])
def test_rowxent_masked_classes(cols):
    need_gpu()
    check_xent("bf16", 9, cols, seed=25000 + cols, neg_inf_frac=0.5)


def test_rowxent_large_logits():
    need_gpu()
    check_xent("fp32", 7, 50257, seed=26000, std=20.0, offset=50.0)
    check_xent("bf16", 7, 8193, seed=26001, std=20.0, offset=-50.0)


def test_rowxent_all_ignored():
    need_gpu()
    check_xent("bf16", 5, 1000, seed=27000, ignore_frac=1.0)


# ---- the bench workloads at full size, on sampled rows ------------------------------
def sample_rows(rows, n=24, seed=0):
    g = np.random.default_rng(seed)
    return np.unique(np.r_[0, rows - 1, g.choice(rows, size=n, replace=False)])


@pytest.mark.slow
@pytest.mark.parametrize("name", list(S.ROWS))
def test_row_workload_full_size(name):
    """The workload bench.py times, at its full size and in its launch configuration,
    checked on sampled rows.  The backward's row inputs (y, lse) are the GPU forward's
    outputs with the sampled rows overwritten by the oracle's values, so every row
    that is compared was computed from oracle inputs."""
    need_gpu()
    import online_softmax_attn_amd as osa
    w = S.ROWS[name]
    inp = S.row_inputs(w)
    idx = sample_rows(w.rows, seed=w.seed)
    idx_d = torch.from_numpy(idx).cuda()
    x = inp["x"]
    xd = to_dev(x)
    x64 = f64(x[idx])
    if w.op == "xent":
        td = to_dev(inp["targets"])
        loss, lse = osa.rowxent_fwd(xd, td)
        torch.cuda.synchronize()
        t_or = inp["targets"].numpy().astype(np.int64)[idx]
        r_loss, r_lse = R.cross_entropy(x64, t_or)
        s = np.maximum(1.0, np.abs(r_lse))
        check(lse[idx_d], r_lse, s, "fp32", name + " lse")
        check(loss[idx_d], r_loss, s, "fp32", name + " loss")
        lse_in = lse.clone()
        lse_in[idx_d] = to_dev(torch.from_numpy(r_lse).to(torch.float32))
        dx = osa.rowxent_bwd(xd, td, lse_in, to_dev(inp["dloss"]))
        torch.cuda.synchronize()
        d64 = f64(inp["dloss"][idx])
        ref = R.cross_entropy_backward(x64, t_or, d64)
        p = R.softmax(x64)
        onehot = np.zeros_like(p)
        live = (t_or >= 0) & (t_or < w.cols)
        onehot[np.nonzero(live)[0], t_or[live]] = 1.0
        check(dx[idx_d], ref, (np.abs(d64) * live)[:, None] * (p + onehot), w.dtype,
              name + " bwd")
        return
    log = w.op == "log_softmax"
    y = osa.rowsoftmax_fwd(xd, log_softmax=log)
    torch.cuda.synchronize()
    if log:
        ref = R.log_softmax(x64)
        scale = np.abs(x64) + np.abs(R.logsumexp(x64))[:, None]
    else:
        ref = R.softmax(x64)
        scale = np.abs(ref)
    check(y[idx_d], ref, scale, w.dtype, name + " fwd")
    y_rows = torch.from_numpy(ref).to(S.DTYPES[w.dtype])
    y[idx_d] = to_dev(y_rows)
    dx = osa.rowsoftmax_bwd(y, to_dev(inp["dy"]), log_softmax=log)
    torch.cuda.synchronize()
    y64, dy64 = f64(y_rows), f64(inp["dy"][idx])
    if log:
        ref_b = R.log_softmax_backward(y64, dy64)
        scale_b = np.abs(dy64) + np.exp(y64) * np.abs(dy64).sum(-1, keepdims=True)
    else:
        ref_b = R.softmax_backward(y64, dy64)
        scale_b = y64 * (np.abs(dy64) + np.abs(y64 * dy64).sum(-1, keepdims=True))
    check(dx[idx_d], ref_b, scale_b, w.dtype, name + " bwd")
