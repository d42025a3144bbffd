"""Plain fp64 CPU oracle for scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, header, table or helper with the
HIP library, and it never imports that library.

What it computes is the plain definition of attention, with the N x N score and
probability matrices materialised (FlashAttention-2 page, "Standard Attention"):

    S = scale * Q K^T                      (scores, one per query/key pair)
    S_ij = -inf where j > i   if causal    ("Causal masking": mask M, N=4 example)
    P = rowwise softmax(S), max-subtracted (each row of P sums to 1)
    O = P V
    LSE_i = m_i + ln sum_j exp(S_ij - m_i) (logsumexp, stabilised by the row max:
                                            softmax-backward page, "LogSoftmax Backward")

The tiled algorithm on the FlashAttention-2 page reaches exactly this result, up to
the order of floating-point rounding ("FLOPs are unchanged", and the worked-example
"Sanity check"), so the oracle is the definition, not the tiling.

Backward (softmax-backward page, "Backpropagating Through Softmax": the Jacobian-
vector product S * (g - <S, g>); matmul chain rule for the two products):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij                 (the row "dot" of the softmax JVP)
    dS = P * (dP - D)
    dQ = scale * dS K
    dK = scale * dS^T Q

Grouped-query attention: query head h reads key/value head floor(h / n_rep), with
n_rep = H / Hkv (contiguous groups, as in the SnapKV ``view(b, n_kv_head, n_rep, ...)``
grouping on the KV-cache page); dK and dV of a key/value head are the sums over the
n_rep query heads of its group.

Layouts: q, o, do, dq are [B, H, Nq, d]; k, v, dk, dv are [B, Hkv, Nk, d]; lse is
[B, H, Nq].  Inputs are upcast to float64 exactly as given (the GPU receives the
dtype-rounded tensors; the oracle receives those same values).

Queries and keys may differ in number (decoding: a few new queries against a long
key/value history).  The pages only draw the square causal mask, so the reading
taken for Nq != Nk is the bottom-right alignment: the Nq queries are the last Nq
positions of the sequence, query i sits at position i + (Nk - Nq) and sees keys
0 .. i + Nk - Nq.  For Nq == Nk this is the square mask above.

Split-KV merge (ml-notes page, the split-K sparse-attention notes: each key chunk
keeps its max m, denominator l and unnormalised output o, and rescaling by
exp(m_s - m) onto a common max makes the merge exact and order-free; the
attnres-kernel-lab page merges two softmax partitions the same way): with the
chunk results written as a normalised output O_s = o_s / l_s and a logsumexp
LSE_s = m_s + ln l_s, the whole-row result is

    LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,

where a chunk with no visible key has LSE_s = -inf and weight 0.

General masks: each query row i of batch b sees the keys lo[b, i] <= j <= hi[b, i]
(an interval, clamped to 0 .. Nk-1; the same for every head).  Causal, bottom-right
causal, sliding-window, prefix-LM and document (packed variable-length) masks are all
such intervals (the FlashAttention-2 page's mask-then-softmax of "Option A" with the
predicate replaced).  A row whose interval holds no key has no softmax; the reading
taken is O = 0, LSE = -inf, dQ = 0, and no contribution to dK, dV or D = 0.

Large shapes are processed in blocks of complete rows: each row's full set of N
scores is formed before its softmax, so no online rescaling happens here.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head_of",
    "scores",
    "softmax_rows",
    "logsumexp_rows",
    "softmax_backward_rows",
    "attention_forward",
    "attention_backward",
    "attention_forward_rows",
    "attention_head",
    "causal_key_offset",
    "merge_partials",
    "interval_scores",
    "attention_head_intervals",
    "attention_forward_intervals",
    "attention_backward_intervals",
]


def _f64(x) -> np.ndarray:
    """Upcast to a C-contiguous float64 array (torch tensors go through numpy)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """Key/value head read by query head h: floor(h / (H / Hkv)) (contiguous groups)."""
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return h // (H // Hkv)


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float, causal: bool,
           row_ids: np.ndarray | None = None, key_offset: int = 0) -> np.ndarray:
    """S = scale * Q K^T for the given query rows against all Nk keys.

    q_rows is [R, d], k is [Nk, d]; row_ids are the query indices of the R rows.
    The causal mask keeps key index <= query index + key_offset, where key_offset =
    Nk - Nq places the queries at the end of the key sequence (0 when Nq == Nk).
    """
    s = scale * (q_rows @ k.T)
    if causal:
        if row_ids is None:
            row_ids = np.arange(q_rows.shape[0])
        key_ids = np.arange(k.shape[0])
        s = np.where(key_ids[None, :] > row_ids[:, None] + key_offset, -np.inf, s)
    return s


def causal_key_offset(nq: int, nk: int, causal: bool) -> int:
    """Nk - Nq: position of query 0 in the key sequence (bottom-right alignment).
    A causal problem needs Nk >= Nq so that every query sees at least key 0."""
    if causal and nk < nq:
        raise ValueError("causal attention needs at least as many keys as queries")
    return nk - nq


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax with the row max subtracted before exponentiating."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def logsumexp_rows(s: np.ndarray) -> np.ndarray:
    """ln sum_j exp(s_j) per row, computed as m + ln sum exp(s - m)."""
    m = np.max(s, axis=-1)
    return m + np.log(np.sum(np.exp(s - m[..., None]), axis=-1))


def softmax_backward_rows(p: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Softmax Jacobian-vector product per row: p * (g - <p, g>).

    p is the softmax output, g the upstream gradient with respect to it; the
    result is the gradient with respect to the logits.
    """
    dot = np.sum(p * g, axis=-1, keepdims=True)
    return p * (g - dot)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, do: np.ndarray | None = None,
                   row_block: int = 1024):
    """One query head against its key/value head, all rows.

    Returns (O, LSE) when do is None, else (O, LSE, dQ, dK, dV, D) where dK and dV
    are this query head's contributions (a GQA group sums them).
    """
    n = q.shape[0]
    off = causal_key_offset(n, k.shape[0], causal)
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    want_grad = do is not None
    if want_grad:
        dq = np.empty_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        dvec = np.empty(n)
    for r0 in range(0, n, row_block):
        rows = np.arange(r0, min(n, r0 + row_block))
        s = scores(q[rows], k, scale, causal, rows, off)
        p = softmax_rows(s)
        o[rows] = p @ v
        lse[rows] = logsumexp_rows(s)
        if want_grad:
            dp = do[rows] @ v.T
            ds = softmax_backward_rows(p, dp)
            dvec[rows] = np.sum(p * dp, axis=-1)
            dq[rows] = scale * (ds @ k)
            dk += scale * (ds.T @ q[rows])
            dv += p.T @ do[rows]
    if want_grad:
        return o, lse, dq, dk, dv, dvec
    return o, lse


def attention_forward(q, k, v, scale: float, causal: bool = False,
                      row_block: int = 1024):
    """O [B,H,Nq,d] and LSE [B,H,Nq] in float64 for the whole batch (k, v may
    hold a different number of rows Nk; see causal_key_offset)."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            o[b, h], lse[b, h] = attention_head(_f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g]),
                                                scale, causal, row_block=row_block)
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool = False,
                       row_block: int = 1024, heads=None):
    """Full forward + backward in float64.

    Returns a dict with o, lse, dq, dk, dv, D.  With ``heads`` = a list of
    (b, kv_head) pairs, only the query heads of those groups are computed (the
    other entries are NaN); this keeps parity checks at large shapes bounded.
    Each head is upcast to float64 only when it is used.
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    n_rep = H // Hkv
    out = {name: np.full((B, H, N, d), np.nan) for name in ("o", "dq")}
    out["lse"] = np.full((B, H, N), np.nan)
    out["D"] = np.full((B, H, N), np.nan)
    out["dk"] = np.full((B, Hkv, N, d), np.nan)
    out["dv"] = np.full((B, Hkv, N, d), np.nan)
    groups = heads if heads is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in groups:
        kg, vg = _f64(k[b, g]), _f64(v[b, g])
        dk_sum = np.zeros((N, d))
        dv_sum = np.zeros((N, d))
        for h in range(g * n_rep, (g + 1) * n_rep):
            o, lse, dq, dk, dv, dvec = attention_head(_f64(q[b, h]), kg, vg, scale,
                                                      causal, _f64(do[b, h]), row_block)
            out["o"][b, h], out["lse"][b, h], out["dq"][b, h], out["D"][b, h] = o, lse, dq, dvec
            dk_sum += dk
            dv_sum += dv
        out["dk"][b, g] = dk_sum
        out["dv"][b, g] = dv_sum
    return out


def attention_forward_rows(q, k, v, scale: float, causal: bool, picks):
    """O and LSE for individually picked rows: picks is a list of (b, h, i).

    Each row needs only its own query vector and the whole key/value head, so
    rows of a large problem can be checked one by one.
    """
    H, Hkv = q.shape[1], k.shape[1]
    o_rows = np.empty((len(picks), q.shape[-1]))
    lse_rows = np.empty(len(picks))
    by_head = {}
    for n, (b, h, i) in enumerate(picks):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        g = kv_head_of(h, H, Hkv)
        kg, vg = _f64(k[b, g]), _f64(v[b, g])
        idx = np.array([i for _, i in items])
        qi = _f64(q[b, h])[idx] if isinstance(q, np.ndarray) else _f64(q[b, h, idx])
        s = scores(qi, kg, scale, causal, idx, causal_key_offset(q.shape[2], kg.shape[0], causal))
        p = softmax_rows(s)
        for (n, _), o_row, l_row in zip(items, p @ vg, logsumexp_rows(s)):
            o_rows[n] = o_row
            lse_rows[n] = l_row
    return o_rows, lse_rows


def merge_partials(o_parts, lse_parts):
    """Exact merge of per-chunk results: o_parts [S, ..., d], lse_parts [S, ...].

    Chunk s contributes exp(LSE_s - LSE) of its normalised output, LSE being the
    logsumexp of the chunk LSEs (taken about their max); chunks with LSE_s = -inf
    (no visible key) get weight zero.  Returns (O, LSE).
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m[None])            # 0 for -inf chunks
    z = np.sum(w, axis=0)
    o = np.sum(w[..., None] * o_parts, axis=0) / z[..., None]
    return o, m + np.log(z)


def interval_scores(q_rows: np.ndarray, k: np.ndarray, scale: float, lo: np.ndarray,
                    hi: np.ndarray) -> np.ndarray:
    """S = scale * Q K^T with S_ij = -inf unless lo_i <= j <= hi_i."""
    s = scale * (q_rows @ k.T)
    key_ids = np.arange(k.shape[0])[None, :]
    keep = (key_ids >= np.asarray(lo)[:, None]) & (key_ids <= np.asarray(hi)[:, None])
    return np.where(keep, s, -np.inf)


def attention_head_intervals(q, k, v, scale, lo, hi, do=None):
    """One query head under an interval mask; rows with an empty interval give O = 0,
    LSE = -inf, dQ = 0, D = 0 and add nothing to dK, dV.  Same returns as
    attention_head."""
    n = q.shape[0]
    lo = np.clip(np.asarray(lo, dtype=np.int64), 0, k.shape[0])
    hi = np.clip(np.asarray(hi, dtype=np.int64), -1, k.shape[0] - 1)
    live = lo <= hi
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    want_grad = do is not None
    if want_grad:
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        dvec = np.zeros(n)
    rows = np.nonzero(live)[0]
    if rows.size:
        s = interval_scores(q[rows], k, scale, lo[rows], hi[rows])
        p = softmax_rows(s)
        o[rows] = p @ v
        lse[rows] = logsumexp_rows(s)
        if want_grad:
            dp = do[rows] @ v.T
            ds = softmax_backward_rows(p, dp)
            dvec[rows] = np.sum(p * dp, axis=-1)
            dq[rows] = scale * (ds @ k)
            dk += scale * (ds.T @ q[rows])
            dv += p.T @ do[rows]
    if want_grad:
        return o, lse, dq, dk, dv, dvec
    return o, lse


def attention_forward_intervals(q, k, v, scale: float, kv_lo, kv_hi):
    """O [B,H,Nq,d] and LSE [B,H,Nq] under per-row key intervals kv_lo, kv_hi [B,Nq]."""
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    kv_lo, kv_hi = np.asarray(kv_lo), np.asarray(kv_hi)
    o = np.empty((B, H, Nq, d))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            o[b, h], lse[b, h] = attention_head_intervals(_f64(q[b, h]), _f64(k[b, g]),
                                                          _f64(v[b, g]), scale, kv_lo[b], kv_hi[b])
    return o, lse


def attention_backward_intervals(q, k, v, do, scale: float, kv_lo, kv_hi, heads=None):
    """Forward + backward under per-row key intervals; same dict as attention_backward
    (dk, dv have the keys' length Nk)."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    n_rep = H // Hkv
    kv_lo, kv_hi = np.asarray(kv_lo), np.asarray(kv_hi)
    out = {name: np.full((B, H, Nq, d), np.nan) for name in ("o", "dq")}
    out["lse"] = np.full((B, H, Nq), np.nan)
    out["D"] = np.full((B, H, Nq), np.nan)
    out["dk"] = np.full((B, Hkv, Nk, d), np.nan)
    out["dv"] = np.full((B, Hkv, Nk, d), np.nan)
    groups = heads if heads is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in groups:
        kg, vg = _f64(k[b, g]), _f64(v[b, g])
        dk_sum = np.zeros((Nk, d))
        dv_sum = np.zeros((Nk, d))
        for h in range(g * n_rep, (g + 1) * n_rep):
            o, lse, dq, dk, dv, dvec = attention_head_intervals(
                _f64(q[b, h]), kg, vg, scale, kv_lo[b], kv_hi[b], _f64(do[b, h]))
            out["o"][b, h], out["lse"][b, h], out["dq"][b, h], out["D"][b, h] = o, lse, dq, dvec
            dk_sum += dk
            dv_sum += dv
        out["dk"][b, g] = dk_sum
        out["dv"][b, g] = dv_sum
    return out
