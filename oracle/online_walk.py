"""Online softmax over key blocks, in float64, written as a fold of block summaries.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): it exists to pin
the plain-definition oracle against the worked example printed on the
FlashAttention-2 page ("Worked Example") and to show that going block by block
changes nothing but the order of rounding.  The HIP library never uses it.

The recurrence.  For one query row, a set of keys with scores s_j and value rows
v_j is summarised by three numbers (one vector):

    m = max_j s_j,    l = sum_j exp(s_j - m),    u = sum_j exp(s_j - m) v_j .

The summaries of two disjoint key sets give the summary of their union exactly,
by moving both onto the larger of the two maxima M = max(m1, m2):

    l = exp(m1 - M) l1 + exp(m2 - M) l2,    u = exp(m1 - M) u1 + exp(m2 - M) u2 .

This combination is associative and commutative, and the empty key set
(m = -inf, l = 0, u = 0) is its identity (exp(-inf - M) is 0).  A row's
attention output is u / l and its logsumexp is m + ln l.  Summarising each key
block on its own and folding the summaries from the first block to the last is
the online softmax of the pages: the state after each block is the running max,
running denominator and unnormalised output that the FlashAttention-2 page tracks
through its example.  The page's example uses scale = 1 (no 1/sqrt(d)).

A key block in which every score of a row is masked summarises to the identity
for that row.
"""

from __future__ import annotations

from itertools import accumulate

import numpy as np

__all__ = ["block_summary", "combine", "finish", "tiled_forward", "EMPTY"]


def _weight(m: np.ndarray, m_to: np.ndarray) -> np.ndarray:
    """exp(m - m_to), taken as 0 where m = -inf (an empty summary weighs nothing)."""
    out = np.zeros_like(m)
    live = np.isfinite(m)
    out[live] = np.exp(m[live] - m_to[live])
    return out


def block_summary(s: np.ndarray, v: np.ndarray):
    """(m, l, u) of the score rows s [R, C] over one key block with values v [C, d]."""
    m = np.max(s, axis=1)
    e = np.zeros_like(s)
    live = np.isfinite(m)
    e[live] = np.exp(s[live] - m[live, None])
    return m, e.sum(axis=1), e @ v


def combine(a, b):
    """The summary of the union of two disjoint key sets (exact, order-free)."""
    (m1, l1, u1), (m2, l2, u2) = a, b
    mm = np.maximum(m1, m2)
    w1, w2 = _weight(m1, mm), _weight(m2, mm)
    return mm, w1 * l1 + w2 * l2, w1[:, None] * u1 + w2[:, None] * u2


def finish(state):
    """(O rows, logsumexp) of a whole-row summary."""
    m, l, u = state
    return u / l[:, None], m + np.log(l)


def EMPTY(rows: int, d: int):
    """The identity summary for `rows` rows of width d."""
    return np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d))


def tiled_forward(q, k, v, block_rows: int, block_cols: int, scale: float = 1.0,
                  causal: bool = False, trace: bool = False):
    """Block-by-block forward for one head: q [N, d], k [Nk, d], v [Nk, d].

    Returns (O, LSE) and, with trace=True, also a list with one entry per
    (query block i, key block j): dict(i, j, m, l, Ot) holding the folded state
    of query block i after key block j (Ot is the unnormalised output u).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    nk = k.shape[0]
    o, lse, states = np.empty_like(q), np.empty(n), []
    for i, r0 in enumerate(range(0, n, block_rows)):
        rows = np.arange(r0, min(n, r0 + block_rows))

        def summaries():
            for c0 in range(0, nk, block_cols):
                cols = np.arange(c0, min(nk, c0 + block_cols))
                s = scale * (q[rows] @ k[cols].T)
                if causal:
                    s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
                yield block_summary(s, v[cols])

        folded = list(accumulate(summaries(), combine, initial=EMPTY(len(rows), d)))[1:]
        if trace:
            states += [{"i": i, "j": j, "m": m.copy(), "l": l.copy(), "Ot": u.copy()}
                       for j, (m, l, u) in enumerate(folded)]
        o[rows], lse[rows] = finish(folded[-1])
    if trace:
        return o, lse, states
    return o, lse
