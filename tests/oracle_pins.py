"""Pins for the fp64 oracle: each returns an error figure, tests compare it to a bound.

Kept as plain functions so that ``test_oracle_mutations.py`` can re-run them on an
oracle with a planted mistake and show that at least one pin catches it.  None of
these retypes the oracle's formulas: each checks the oracle against something
else the pages or the mathematics fix (printed values, closed forms, invariants,
finite differences, brute-force loops, a library routine).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.attention as A
import oracle.brute as BR
import oracle.fp8 as F8
import oracle.online_walk as W
import oracle.rowsoftmax as RS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fa2_worked_example.json")


def rng_case(seed, B=1, H=2, Hkv=1, N=7, d=4, scale=None):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    do = r.standard_normal((B, H, N, d))
    return q, k, v, do, (1.0 / math.sqrt(d) if scale is None else scale)


def closed_form(terms):
    return sum(c * math.exp(e) for c, e in terms)


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def worked_example_arrays(g):
    q = np.array(g["Q"], dtype=np.float64)
    k = np.array(g["K_T"], dtype=np.float64).T.copy()
    v = np.array(g["V"], dtype=np.float64)
    return q, k, v


# --- p1: the worked example -------------------------------------------------------

def pin_worked_example_walk():
    """Max error of the tiled walk's (m, l, Ot) after each step vs the page's closed forms."""
    g = load_golden()
    q, k, v = worked_example_arrays(g)
    _, _, steps = W.tiled_forward(q, k, v, g["block_rows"], g["block_cols"], g["scale"],
                                  trace=True)
    err = 0.0
    for st in g["steps"]:
        got = steps[st["j"] - 1]          # query tile 1 is i = 0, key tile j is index j-1
        assert got["i"] == 0
        err = max(err, np.max(np.abs(got["m"] - np.array(st["m"], dtype=float))))
        err = max(err, max(abs(got["l"][r] - closed_form(st["l"][r])) for r in range(2)))
        for r in range(2):
            for c in range(2):
                err = max(err, abs(got["Ot"][r, c] - closed_form(st["Ot"][r][c])))
    return err


def pin_worked_example_scores():
    """S_1j = Q_1 K_j^T from the oracle's score function vs the page's printed tiles."""
    g = load_golden()
    q, k, v = worked_example_arrays(g)
    s = A.scores(q[:2], k, g["scale"], False)
    err = 0.0
    for st in g["steps"]:
        j = st["j"] - 1
        err = max(err, np.max(np.abs(s[:, 2 * j:2 * j + 2] - np.array(st["S"], dtype=float))))
    return err


def pin_worked_example_naive():
    """The plain-definition oracle's O, LSE of rows 1-2 vs Ot/l and m + ln l of the last step."""
    g = load_golden()
    q, k, v = worked_example_arrays(g)
    o, lse = A.attention_forward(q[None, None], k[None, None], v[None, None], g["scale"])
    last = g["steps"][-1]
    err = 0.0
    for r in range(2):
        l = closed_form(last["l"][r])
        err = max(err, abs(lse[0, 0, r] - (last["m"][r] + math.log(l))))
        for c in range(2):
            err = max(err, abs(o[0, 0, r, c] - closed_form(last["Ot"][r][c]) / l))
    return err


def pin_tiled_equals_naive(seed=0, N=13, d=5, br=4, bc=3, causal=False):
    q, k, v, _, scale = rng_case(seed, 1, 1, 1, N, d)
    o_t, lse_t = W.tiled_forward(q[0, 0], k[0, 0], v[0, 0], br, bc, scale, causal)
    o_n, lse_n = A.attention_forward(q, k, v, scale, causal)
    return max(np.max(np.abs(o_t - o_n[0, 0])), np.max(np.abs(lse_t - lse_n[0, 0])))


# --- p2..p9: invariants and closed forms ------------------------------------------

def pin_rows_sum_to_one(seed=1, causal=True):
    q, k, _, _, scale = rng_case(seed, 1, 1, 1, 9, 3)
    p = A.softmax_rows(A.scores(q[0, 0], k[0, 0], scale, causal))
    return np.max(np.abs(p.sum(axis=1) - 1.0))


def pin_shift_invariance(seed=2, causal=False):
    """Adding u to every key row shifts each score row by scale*q_i.u: O and all
    gradients are unchanged and LSE_i moves by exactly scale*q_i.u."""
    q, k, v, do, scale = rng_case(seed, 1, 2, 1, 8, 4)
    u = np.random.default_rng(seed + 100).standard_normal(4) * 3.0
    a = A.attention_backward(q, k, v, do, scale, causal)
    b = A.attention_backward(q, k + u, v, do, scale, causal)
    err = 0.0
    for name in ("o", "dq", "dk", "dv"):
        err = max(err, np.max(np.abs(a[name] - b[name])))
    shift = scale * np.einsum("bhnd,d->bhn", q, u)
    err = max(err, np.max(np.abs(b["lse"] - a["lse"] - shift)))
    return err


def pin_softmax_jvp(seed=3, n=6):
    """s*(g - <s,g>) equals the full Jacobian product with J = diag(s) - s s^T; J is
    symmetric; each result row sums to zero."""
    r = np.random.default_rng(seed)
    z = r.standard_normal((4, n)) * 2
    gr = r.standard_normal((4, n))
    s = A.softmax_rows(z)
    got = A.softmax_backward_rows(s, gr)
    err = 0.0
    for i in range(4):
        jac = np.diag(s[i]) - np.outer(s[i], s[i])
        err = max(err, np.max(np.abs(jac - jac.T)))
        err = max(err, np.max(np.abs(jac @ gr[i] - got[i])))
    err = max(err, np.max(np.abs(got.sum(axis=1))))
    return err


def pin_softmax_jvp_fd(seed=4, n=7, h=1e-6):
    """The softmax JVP against central differences of <g, softmax(z)> in z."""
    r = np.random.default_rng(seed)
    z = r.standard_normal(n)
    gr = r.standard_normal(n)
    got = A.softmax_backward_rows(A.softmax_rows(z[None])[0], gr)
    fd = np.empty(n)
    for j in range(n):
        zp, zm = z.copy(), z.copy()
        zp[j] += h
        zm[j] -= h
        fd[j] = (gr @ A.softmax_rows(zp[None])[0] - gr @ A.softmax_rows(zm[None])[0]) / (2 * h)
    return np.max(np.abs(fd - got))


def pin_d_identity(seed=5, causal=True):
    """rowsum(dO * O) equals rowsum(P * dP), the row dot of the softmax JVP."""
    q, k, v, do, scale = rng_case(seed, 2, 2, 2, 10, 4)
    out = A.attention_backward(q, k, v, do, scale, causal)
    return np.max(np.abs(np.sum(do * out["o"], axis=-1) - out["D"]))


def pin_equal_value_rows(seed=6, causal=False):
    """All value rows equal to one vector w: O is w for every row and dQ = dK = 0."""
    q, k, _, do, scale = rng_case(seed, 1, 2, 1, 9, 4)
    w = np.array([0.5, -1.25, 2.0, 3.0])
    v = np.broadcast_to(w, k.shape).copy()
    out = A.attention_backward(q, k, v, do, scale, causal)
    return max(np.max(np.abs(out["o"] - w)), np.max(np.abs(out["dq"])),
               np.max(np.abs(out["dk"])))


def pin_zero_query(seed=7, causal=False):
    """Q = 0: every score is 0, P is uniform over the visible keys, O is the mean
    (causal: prefix mean) of V and LSE is ln(number of visible keys)."""
    _, k, v, _, scale = rng_case(seed, 1, 1, 1, 8, 3)
    q = np.zeros((1, 1, 8, 3))
    o, lse = A.attention_forward(q, k, v, scale, causal)
    n = np.arange(1, 9) if causal else np.full(8, 8)
    if causal:
        mean = np.cumsum(v[0, 0], axis=0) / n[:, None]
    else:
        mean = np.broadcast_to(v[0, 0].mean(axis=0), (8, 3))
    return max(np.max(np.abs(o[0, 0] - mean)), np.max(np.abs(lse[0, 0] - np.log(n))))


def pin_causal_row0_and_single_key(seed=8):
    """Causal row 0 sees only key 0: O_0 = v_0, LSE_0 = scale q_0.k_0.  N = 1 likewise."""
    q, k, v, _, scale = rng_case(seed, 1, 1, 1, 6, 4)
    o, lse = A.attention_forward(q, k, v, scale, True)
    err = max(np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])),
              abs(lse[0, 0, 0] - scale * q[0, 0, 0] @ k[0, 0, 0]))
    o1, lse1 = A.attention_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale, False)
    err = max(err, np.max(np.abs(o1[0, 0, 0] - v[0, 0, 0])),
              abs(lse1[0, 0, 0] - scale * q[0, 0, 0] @ k[0, 0, 0]))
    return err


def pin_gqa_is_repeated_mha(seed=9, causal=True):
    """GQA equals MHA on K, V repeated n_rep times per head; dK, dV are the group sums."""
    q, k, v, do, scale = rng_case(seed, 2, 6, 2, 7, 3)
    n_rep = 3
    kr = np.repeat(k, n_rep, axis=1)
    vr = np.repeat(v, n_rep, axis=1)
    g = A.attention_backward(q, k, v, do, scale, causal)
    m = A.attention_backward(q, kr, vr, do, scale, causal)
    err = max(np.max(np.abs(g[n] - m[n])) for n in ("o", "lse", "dq"))
    for name in ("dk", "dv"):
        summed = m[name].reshape(2, 2, n_rep, 7, 3).sum(axis=2)
        err = max(err, np.max(np.abs(g[name] - summed)))
    return err


# --- p7, p10, p11: independent computations --------------------------------------

def pin_finite_differences(seed=10, N=12, d=5, causal=False, gqa=False, h=1e-6):
    """dQ, dK, dV vs central differences of L = sum(dO * O) (relative to max |grad|)."""
    H, Hkv = (4, 2) if gqa else (2, 2)
    q, k, v, do, scale = rng_case(seed, 1, H, Hkv, N, d)
    out = A.attention_backward(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        o, _ = A.attention_forward(qq, kk, vv, scale, causal)
        return float(np.sum(do * o))

    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        worst = max(worst, np.max(np.abs(fd - out[name])) / np.max(np.abs(fd)))
    return worst


def pin_brute_force(seed=11, N=6, d=3, causal=False):
    q, k, v, do, scale = rng_case(seed, 1, 1, 1, N, d)
    out = A.attention_backward(q, k, v, do, scale, causal)
    ql, kl, vl, dol = (x[0, 0].tolist() for x in (q, k, v, do))
    o_b, lse_b = BR.forward(ql, kl, vl, scale, causal)
    dq_b, dk_b, dv_b = BR.backward(ql, kl, vl, dol, scale, causal)
    err = max(np.max(np.abs(out["o"][0, 0] - np.array(o_b))),
              np.max(np.abs(out["lse"][0, 0] - np.array(lse_b))))
    for name, ref in (("dq", dq_b), ("dk", dk_b), ("dv", dv_b)):
        err = max(err, np.max(np.abs(out[name][0, 0] - np.array(ref))))
    return err


def pin_torch_library(seed=12, causal=False, gqa=False):
    """Second opinion: torch CPU scaled_dot_product_attention in float64 plus autograd."""
    import torch
    H, Hkv = (4, 2) if gqa else (2, 2)
    q, k, v, do, scale = rng_case(seed, 2, H, Hkv, 11, 6)
    out = A.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    rep = H // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1),
        is_causal=causal, scale=scale)
    o.backward(torch.tensor(do))
    err = np.max(np.abs(o.detach().numpy() - out["o"]))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        err = max(err, np.max(np.abs(t.grad.numpy() - out[name])))
    return err


def pin_row_sampling(seed=13, causal=True):
    """Row-by-row evaluation equals the full forward (the large-shape parity path)."""
    q, k, v, _, scale = rng_case(seed, 2, 4, 2, 9, 3)
    o, lse = A.attention_forward(q, k, v, scale, causal, row_block=4)
    picks = [(1, 3, 0), (0, 1, 8), (1, 0, 4), (0, 2, 5)]
    o_r, lse_r = A.attention_forward_rows(q, k, v, scale, causal, picks)
    err = 0.0
    for n, (b, h, i) in enumerate(picks):
        err = max(err, np.max(np.abs(o_r[n] - o[b, h, i])), abs(lse_r[n] - lse[b, h, i]))
    return err


def pin_row_blocking(seed=14, causal=True):
    """Row blocks of complete rows (size 3) equal a single block."""
    q, k, v, do, scale = rng_case(seed, 1, 2, 1, 10, 4)
    a = A.attention_backward(q, k, v, do, scale, causal, row_block=3)
    b = A.attention_backward(q, k, v, do, scale, causal, row_block=1024)
    return max(np.max(np.abs(a[n] - b[n])) for n in ("o", "lse", "dq", "dk", "dv", "D"))


# --- queries fewer than keys (decoding) and the split-KV merge ------------------------

def rect_case(seed, B=1, H=2, Hkv=1, Nq=3, Nk=9, d=4):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, Nq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    return q, k, v, 1.0 / math.sqrt(d)


def pin_rect_causal_is_tail_of_square(seed=20, Nq=3, Nk=9):
    """Bottom-right alignment: Nq queries against Nk keys give the last Nq rows of the
    square causal problem whose final query rows are those queries."""
    q, k, v, scale = rect_case(seed, 1, 2, 1, Nq, Nk)
    r = np.random.default_rng(seed + 1)
    q_full = np.concatenate([r.standard_normal((1, 2, Nk - Nq, q.shape[-1])), q], axis=2)
    o_sq, lse_sq = A.attention_forward(q_full, k, v, scale, causal=True)
    o, lse = A.attention_forward(q, k, v, scale, causal=True)
    return max(np.max(np.abs(o - o_sq[:, :, Nk - Nq:])), np.max(np.abs(lse - lse_sq[:, :, Nk - Nq:])))


def pin_decode_row_sees_all_keys(seed=21, Nk=10):
    """A single causal query is the last position: it sees every key (equals non-causal),
    and with Nk = 1 its output is v_0."""
    q, k, v, scale = rect_case(seed, 1, 2, 2, 1, Nk)
    o_c, lse_c = A.attention_forward(q, k, v, scale, causal=True)
    o_n, lse_n = A.attention_forward(q, k, v, scale, causal=False)
    o1, _ = A.attention_forward(q, k[:, :, :1], v[:, :, :1], scale, causal=True)
    return max(np.max(np.abs(o_c - o_n)), np.max(np.abs(lse_c - lse_n)),
               np.max(np.abs(o1 - v[:, :, :1])))


def pin_brute_force_rect(seed=22, Nq=3, Nk=7, d=3, causal=True):
    """The pure-Python loops (their own mask test) against the oracle for Nq < Nk."""
    q, k, v, scale = rect_case(seed, 1, 1, 1, Nq, Nk, d)
    o, lse = A.attention_forward(q, k, v, scale, causal)
    o_b, lse_b = BR.forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, causal)
    return max(np.max(np.abs(o[0, 0] - np.array(o_b))), np.max(np.abs(lse[0, 0] - np.array(lse_b))))


def _chunk_results(q, k, v, scale, causal, bounds):
    """Per-chunk (O_s, LSE_s) of one head computed on the chunk's keys alone, with
    the causal mask at the keys' absolute positions; rows that see none of the
    chunk's keys get O_s = 0 and LSE_s = -inf."""
    nq, nk = q.shape[0], k.shape[0]
    off = nk - nq
    o_parts, lse_parts = [], []
    for a, b in bounds:
        s = A.scores(q, k[a:b], scale, causal, np.arange(nq), off - a)
        vis = np.isfinite(s).any(axis=1)
        o_s = np.zeros((nq, v.shape[1]))
        l_s = np.full(nq, -np.inf)
        if vis.any():
            o_s[vis] = A.softmax_rows(s[vis]) @ v[a:b]
            l_s[vis] = A.logsumexp_rows(s[vis])
        o_parts.append(o_s)
        lse_parts.append(l_s)
    return np.array(o_parts), np.array(lse_parts)


def pin_merge_exact(seed=23, Nq=4, Nk=23, causal=False, order=None):
    """Splitting the keys into chunks and merging the chunk results gives the whole-row
    attention, for uneven chunks, in any order, and (causal) with chunks that some
    rows cannot see at all."""
    q, k, v, scale = rect_case(seed, 1, 1, 1, Nq, Nk, 5)
    bounds = [(0, 5), (5, 6), (6, 14), (14, 20), (20, 23)]
    if order is not None:
        bounds = [bounds[i] for i in order]
    o_p, l_p = _chunk_results(q[0, 0], k[0, 0], v[0, 0], scale, causal, bounds)
    o_m, lse_m = A.merge_partials(o_p, l_p)
    o, lse = A.attention_forward(q, k, v, scale, causal)
    return max(np.max(np.abs(o_m - o[0, 0])), np.max(np.abs(lse_m - lse[0, 0])))


def pin_merge_single_chunk(seed=24):
    """One chunk holding every key: the merge returns it unchanged."""
    q, k, v, scale = rect_case(seed, 1, 1, 1, 3, 8, 4)
    o, lse = A.attention_forward(q, k, v, scale, False)
    o_m, lse_m = A.merge_partials(o[0, 0][None], lse[0, 0][None])
    return max(np.max(np.abs(o_m - o[0, 0])), np.max(np.abs(lse_m - lse[0, 0])))


# --- interval (general) masks ------------------------------------------------------

def _np(t):
    return t.numpy().astype(np.int64)


def pin_intervals_causal(seed=30, Nq=6, Nk=6):
    """The causal mask written as intervals gives the causal oracle's forward and
    backward (square and with queries at the end of a longer key sequence)."""
    import synthetic as S
    q, k, v, do, scale = rng_case(seed, 2, 4, 2, Nq, 5)
    if Nk != Nq:
        r = np.random.default_rng(seed + 1)
        k, v = r.standard_normal((2, 2, Nk, 5)), r.standard_normal((2, 2, Nk, 5))
    lo, hi = S.mask_intervals("causal", 2, Nq, Nk)
    a = A.attention_backward_intervals(q, k, v, do, scale, _np(lo), _np(hi))
    if Nk == Nq:
        b = A.attention_backward(q, k, v, do, scale, True)
        names = ("o", "lse", "dq", "dk", "dv", "D")
    else:
        o, l = A.attention_forward(q, k, v, scale, True)
        b, names = {"o": o, "lse": l}, ("o", "lse")
    return max(np.max(np.abs(a[n] - b[n])) for n in names)


def pin_intervals_documents(seed=31, causal=True):
    """A document mask equals attention run on each document on its own."""
    import synthetic as S
    lens = [[3, 5, 1, 4], [13]]
    q, k, v, do, scale = rng_case(seed, 2, 2, 1, 13, 4)
    lo, hi = S.mask_intervals("document", 2, 13, 13, doc_lens=lens, causal=causal)
    a = A.attention_backward_intervals(q, k, v, do, scale, _np(lo), _np(hi))
    err = 0.0
    for b in range(2):
        s0 = 0
        for n in lens[b]:
            sl = slice(s0, s0 + n)
            part = A.attention_backward(q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl],
                                        do[b:b + 1, :, sl], scale, causal)
            for name in ("o", "lse", "dq", "dk", "dv"):
                err = max(err, np.max(np.abs(a[name][b, :, sl] - part[name][0])))
            s0 += n
    return err


def pin_intervals_brute(seed=32, Nq=7, Nk=9, d=3):
    """Random intervals, some empty: the vectorised oracle against the scalar loops
    (forward and all three gradients; empty rows give O = 0, LSE = -inf, dQ = 0)."""
    import synthetic as S
    r = np.random.default_rng(seed)
    q, k, v, do = (r.standard_normal(s) for s in ((1, 1, Nq, d), (1, 1, Nk, d), (1, 1, Nk, d),
                                                  (1, 1, Nq, d)))
    scale = 0.7
    lo, hi = S.mask_intervals("random", 1, Nq, Nk, seed=seed, empty_frac=0.3)
    lo, hi = _np(lo)[0], _np(hi)[0]
    assert np.any(lo > hi) and np.any(lo <= hi)
    out = A.attention_backward_intervals(q, k, v, do, scale, lo[None], hi[None])
    vis = lambda i, j: lo[i] <= j <= hi[i]
    ql, kl, vl, dol = (x[0, 0].tolist() for x in (q, k, v, do))
    o_b, lse_b = BR.forward(ql, kl, vl, scale, visible=vis)
    dq_b, dk_b, dv_b = BR.backward(ql, kl, vl, dol, scale, visible=vis)
    lse_o = out["lse"][0, 0]
    lse_ref = np.array(lse_b)
    if not np.array_equal(np.isinf(lse_o), np.isinf(lse_ref)):
        return np.inf
    fin = np.isfinite(lse_ref)
    err = max(np.max(np.abs(out["o"][0, 0] - np.array(o_b))),
              np.max(np.abs(lse_o[fin] - lse_ref[fin])))
    for name, ref in (("dq", dq_b), ("dk", dk_b), ("dv", dv_b)):
        err = max(err, np.max(np.abs(out[name][0, 0] - np.array(ref))))
    return err


def pin_intervals_wide_window(seed=33):
    """A sliding window wider than the sequence is the plain (causal or full) mask."""
    import synthetic as S
    q, k, v, _, scale = rng_case(seed, 1, 2, 2, 9, 4)
    err = 0.0
    for causal in (True, False):
        lo, hi = S.mask_intervals("sliding", 1, 9, 9, left=50, right=50, causal=causal)
        o, l = A.attention_forward_intervals(q, k, v, scale, _np(lo), _np(hi))
        o2, l2 = A.attention_forward(q, k, v, scale, causal)
        err = max(err, np.max(np.abs(o - o2)), np.max(np.abs(l - l2)))
    return err


def pin_intervals_finite_differences(seed=34, h=1e-6):
    """Gradients under a sliding-window mask against central differences of
    L = sum(dO * O) (relative to max |grad|)."""
    import synthetic as S
    q, k, v, do, scale = rng_case(seed, 1, 2, 1, 8, 3)
    lo, hi = S.mask_intervals("sliding", 1, 8, 8, left=2, causal=True)
    lo, hi = _np(lo), _np(hi)
    out = A.attention_backward_intervals(q, k, v, do, scale, lo, hi)

    def loss(qq, kk, vv):
        o, _ = A.attention_forward_intervals(qq, kk, vv, scale, lo, hi)
        return float(np.sum(do * o))

    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        worst = max(worst, np.max(np.abs(fd - out[name])) / np.max(np.abs(fd)))
    return worst


# --- row softmax, log-softmax, cross-entropy ---------------------------------------

def _fd_rows(f, x, h=1e-6):
    """Central differences of the scalar f(x) with respect to every entry of x."""
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


def pin_row_softmax_fd(seed=40):
    """Softmax and log-softmax backward against central differences of <g, f(x)>."""
    r = np.random.default_rng(seed)
    x, g = r.standard_normal((3, 7)) * 2, r.standard_normal((3, 7))
    e1 = np.max(np.abs(RS.softmax_backward(RS.softmax(x), g)
                       - _fd_rows(lambda z: float(np.sum(g * RS.softmax(z))), x)))
    e2 = np.max(np.abs(RS.log_softmax_backward(RS.log_softmax(x), g)
                       - _fd_rows(lambda z: float(np.sum(g * RS.log_softmax(z))), x)))
    return max(e1, e2)


def pin_row_xent_fd(seed=41):
    """Cross-entropy loss gradient against central differences of sum(dloss * loss)."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((4, 9)) * 3
    t = np.array([2, 0, 8, 5])
    dl = r.standard_normal(4)
    g = RS.cross_entropy_backward(x, t, dl)
    fd = _fd_rows(lambda z: float(np.sum(dl * RS.cross_entropy(z, t)[0])), x)
    return float(np.max(np.abs(g - fd)))


def pin_row_xent_three_routes(seed=42):
    """The page's three routes to the logits gradient agree: p - y directly, the
    softmax JVP with dL/dS = -y/p, and the log-softmax backward with dL/dY = -y."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((5, 6))
    t = r.integers(0, 6, 5)
    y = np.zeros_like(x)
    y[np.arange(5), t] = 1.0
    p = RS.softmax(x)
    a = RS.cross_entropy_backward(x, t, np.ones(5))
    b = RS.softmax_backward(p, -y / p)
    c = RS.log_softmax_backward(RS.log_softmax(x), -y)
    return max(np.max(np.abs(a - b)), np.max(np.abs(a - c)))


def pin_row_invariants(seed=43):
    """Rows of P sum to 1, softmax-backward rows sum to 0, exp(log-softmax) = softmax,
    adding a constant to a row changes nothing, and the loss of a row equals
    -log p_t; an ignored row (target outside 0 .. cols-1) has loss 0 and zero gradient."""
    r = np.random.default_rng(seed)
    x, g = r.standard_normal((4, 11)) * 4, r.standard_normal((4, 11))
    p = RS.softmax(x)
    t = np.array([3, -1, 10, 0])
    loss, lse = RS.cross_entropy(x, t)
    gx = RS.cross_entropy_backward(x, t, np.ones(4))
    t_big = np.array([3, 11, -100, 0])  # 11 = cols: outside the classes, ignored too
    loss_b, _ = RS.cross_entropy(x, t_big)
    gx_b = RS.cross_entropy_backward(x, t_big, np.ones(4))
    errs = [np.max(np.abs(p.sum(-1) - 1)),
            np.max(np.abs(RS.softmax_backward(p, g).sum(-1))),
            np.max(np.abs(np.exp(RS.log_softmax(x)) - p)),
            np.max(np.abs(RS.softmax(x + 7.5) - p)),
            np.max(np.abs(RS.log_softmax(x - 3.0) - RS.log_softmax(x))),
            abs(loss[1]), np.max(np.abs(gx[1])),
            np.max(np.abs(loss_b[1:3])), np.max(np.abs(gx_b[1:3])),
            np.max(np.abs(loss_b[[0, 3]] - loss[[0, 3]])), np.max(np.abs(gx_b[[0, 3]] - gx[[0, 3]])),
            np.max(np.abs(loss[[0, 2, 3]] + np.log(p[[0, 2, 3], t[[0, 2, 3]]])))]
    return float(max(errs))


def pin_row_torch_library(seed=44):
    """Second opinion: torch CPU softmax, log_softmax and cross_entropy in float64 with
    autograd (reduction 'none', ignore_index -1)."""
    import torch
    r = np.random.default_rng(seed)
    x = r.standard_normal((6, 13)) * 2
    g = r.standard_normal((6, 13))
    t = np.array([1, 12, -1, 0, 7, 7])
    dl = r.standard_normal(6)
    err = 0.0
    for fn, ofn, bfn in ((torch.softmax, RS.softmax, RS.softmax_backward),
                         (torch.log_softmax, RS.log_softmax, RS.log_softmax_backward)):
        tx = torch.tensor(x, requires_grad=True)
        out = fn(tx, dim=-1)
        out.backward(torch.tensor(g))
        err = max(err, np.max(np.abs(out.detach().numpy() - ofn(x))),
                  np.max(np.abs(tx.grad.numpy() - bfn(ofn(x), g))))
    tx = torch.tensor(x, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(tx, torch.tensor(t), reduction="none", ignore_index=-1)
    loss.backward(torch.tensor(dl))
    l_o, _ = RS.cross_entropy(x, t)
    err = max(err, np.max(np.abs(loss.detach().numpy() - l_o)),
              np.max(np.abs(tx.grad.numpy() - RS.cross_entropy_backward(x, t, dl))))
    return float(err)


def pin_row_large_logits(seed=45):
    """Logits near 1e4 (exp overflows without the max): the stable forms stay finite
    and equal those of the shifted row."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((2, 8))
    big = x + 1e4
    errs = [np.max(np.abs(RS.softmax(big) - RS.softmax(x))),
            np.max(np.abs(RS.logsumexp(big) - 1e4 - RS.logsumexp(x)))]
    return float(max(errs)) if np.all(np.isfinite(RS.softmax(big))) else np.inf


def pin_fp8_decode_library(seed=50):
    """All 256 e4m3 codes against torch's float8_e4m3fn decoding (NaN codes compared
    as NaN), and a round trip: encoding the decoded finite values with torch gives
    back the codes (up to the sign of zero)."""
    import torch
    codes = np.arange(256)
    mine = F8.decode_e4m3(codes)
    lib = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(np.isnan(mine), np.isnan(lib)):
        return np.inf
    fin = ~np.isnan(lib)
    err = float(np.max(np.abs(mine[fin] - lib[fin])))
    back = torch.tensor(mine[fin]).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(int)
    same = (back == codes[fin]) | ((back & 0x7F) == 0) & ((codes[fin] & 0x7F) == 0)
    return err if np.all(same) else np.inf


def pin_fp8_decode_closed_forms():
    """Values the format fixes: 1.0 = 0x38, 448 = 0x7E (largest), 2^-6 = 0x08 (smallest
    normal), 2^-9 = 0x01 (smallest subnormal), 1.125 = 0x39, -2 = 0xC0, -0 = 0x80,
    0x7F and 0xFF are NaN."""
    want = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x39: 1.125, 0xC0: -2.0,
            0x80: 0.0, 0x07: 7 * 2.0 ** -9, 0x77: 240.0}
    got = F8.decode_e4m3(list(want))
    err = float(np.max(np.abs(got - np.array(list(want.values())))))
    nan_ok = np.isnan(F8.decode_e4m3([0x7F, 0xFF])).all() and np.isfinite(F8.decode_e4m3([0x7E, 0xFE])).all()
    return err if nan_ok and F8.E4M3_MAX == 448.0 else np.inf


def pin_fp8_attention_is_attention_of_decoded(seed=51):
    """The fp8 forward (and its row variant, on picked rows) equals the plain forward
    of the decoded, dequantised tensors computed by hand here (codes drawn at random,
    scales chosen as powers of two so the products are exact), against the
    pure-Python loops."""
    r = np.random.default_rng(seed)
    q8 = r.integers(0, 0x7F, (1, 2, 5, 4)) | (r.integers(0, 2, (1, 2, 5, 4)) << 7)
    k8 = r.integers(0, 0x7F, (1, 1, 5, 4)) | (r.integers(0, 2, (1, 1, 5, 4)) << 7)
    v8 = r.integers(0, 0x7F, (1, 1, 5, 4)) | (r.integers(0, 2, (1, 1, 5, 4)) << 7)
    # keep the exponents small so that exp(scores) stays moderate
    q8, k8, v8 = (np.where((x >> 3) & 0xF > 9, x & 0x87, x) for x in (q8, k8, v8))
    dq, dk, dv, scale = 0.25, 0.5, 2.0, 0.125
    o, lse = F8.attention_forward_fp8(q8, k8, v8, dq, dk, dv, scale, causal=True)
    q = F8.decode_e4m3(q8) * dq
    k = F8.decode_e4m3(k8) * dk
    v = F8.decode_e4m3(v8) * dv
    picks = [(0, 1, 4), (0, 0, 0), (0, 1, 2)]
    o_r, lse_r = F8.attention_forward_fp8_rows(q8, k8, v8, dq, dk, dv, scale, True, picks)
    err = 0.0
    for h in range(2):  # GQA: both query heads read the one key/value head
        ob, lb = BR.forward(q[0, h].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, True)
        err = max(err, float(np.max(np.abs(o[0, h] - np.array(ob)))),
                  float(np.max(np.abs(lse[0, h] - np.array(lb)))))
        for n, (_, hp, i) in enumerate(picks):  # the row variant, row by row
            if hp == h:
                err = max(err, float(np.max(np.abs(o_r[n] - np.array(ob[i])))),
                          abs(float(lse_r[n]) - lb[i]))
    return err


ALL_PINS = {
    "worked_example_walk": (pin_worked_example_walk, 1e-12),
    "worked_example_scores": (pin_worked_example_scores, 0.0),
    "worked_example_naive": (pin_worked_example_naive, 1e-12),
    "tiled_equals_naive": (pin_tiled_equals_naive, 1e-13),
    "tiled_equals_naive_causal": (lambda: pin_tiled_equals_naive(causal=True, br=3, bc=4), 1e-13),
    "rows_sum_to_one": (pin_rows_sum_to_one, 1e-14),
    "shift_invariance": (pin_shift_invariance, 1e-12),
    "shift_invariance_causal": (lambda: pin_shift_invariance(causal=True), 1e-12),
    "softmax_jvp": (pin_softmax_jvp, 1e-14),
    "softmax_jvp_fd": (pin_softmax_jvp_fd, 1e-8),
    "d_identity": (pin_d_identity, 1e-13),
    "equal_value_rows": (pin_equal_value_rows, 1e-13),
    "equal_value_rows_causal": (lambda: pin_equal_value_rows(causal=True), 1e-13),
    "zero_query": (pin_zero_query, 1e-14),
    "zero_query_causal": (lambda: pin_zero_query(causal=True), 1e-14),
    "causal_row0_single_key": (pin_causal_row0_and_single_key, 1e-14),
    "gqa_is_repeated_mha": (pin_gqa_is_repeated_mha, 1e-13),
    "finite_differences": (pin_finite_differences, 1e-7),
    "finite_differences_causal_gqa": (lambda: pin_finite_differences(causal=True, gqa=True, N=9), 1e-7),
    "brute_force": (pin_brute_force, 1e-13),
    "brute_force_causal": (lambda: pin_brute_force(causal=True, N=7), 1e-13),
    "torch_library": (pin_torch_library, 1e-12),
    "torch_library_causal_gqa": (lambda: pin_torch_library(causal=True, gqa=True), 1e-12),
    "row_sampling": (pin_row_sampling, 1e-13),
    "row_blocking": (pin_row_blocking, 1e-13),
    "rect_causal_is_tail_of_square": (pin_rect_causal_is_tail_of_square, 1e-13),
    "rect_causal_one_query": (lambda: pin_rect_causal_is_tail_of_square(Nq=1, Nk=6), 1e-13),
    "decode_row_sees_all_keys": (pin_decode_row_sees_all_keys, 1e-13),
    "brute_force_rect_causal": (pin_brute_force_rect, 1e-13),
    "brute_force_rect": (lambda: pin_brute_force_rect(causal=False, Nq=2, Nk=5), 1e-13),
    "merge_exact": (pin_merge_exact, 1e-13),
    "merge_exact_causal": (lambda: pin_merge_exact(causal=True, Nq=9), 1e-13),
    "merge_exact_reordered": (lambda: pin_merge_exact(causal=True, Nq=9, order=[3, 0, 4, 2, 1]), 1e-13),
    "merge_single_chunk": (pin_merge_single_chunk, 1e-14),
    "intervals_causal": (pin_intervals_causal, 1e-13),
    "intervals_causal_rect": (lambda: pin_intervals_causal(Nq=4, Nk=9), 1e-13),
    "intervals_documents_causal": (pin_intervals_documents, 1e-13),
    "intervals_documents": (lambda: pin_intervals_documents(causal=False), 1e-13),
    "intervals_brute": (pin_intervals_brute, 1e-13),
    "intervals_wide_window": (pin_intervals_wide_window, 1e-13),
    "intervals_finite_differences": (pin_intervals_finite_differences, 1e-7),
    "row_softmax_fd": (pin_row_softmax_fd, 1e-8),
    "row_xent_fd": (pin_row_xent_fd, 1e-7),
    "row_xent_three_routes": (pin_row_xent_three_routes, 1e-14),
    "row_invariants": (pin_row_invariants, 1e-13),
    "row_torch_library": (pin_row_torch_library, 1e-12),
    "row_large_logits": (pin_row_large_logits, 1e-9),
    "fp8_decode_library": (pin_fp8_decode_library, 0.0),
    "fp8_decode_closed_forms": (pin_fp8_decode_closed_forms, 0.0),
    "fp8_attention_is_attention_of_decoded": (pin_fp8_attention_is_attention_of_decoded, 1e-12),
}
