"""The tiled online-softmax forward, in float64, in the order the pages give it.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): it exists to pin
the plain-definition oracle against the worked example printed on the
FlashAttention-2 page and to show that tiling changes nothing but the order of
rounding.  The HIP library never uses it.

Per query tile Q_i (B_r rows) the inner loop over key/value tiles (K_j, V_j) of
B_c rows takes the five steps of the FlashAttention-2 page's inner loop:

  1. S_ij = scale * Q_i K_j^T
  2. m_ij = rowmax(S_ij);  Pt_ij = exp(S_ij - m_ij)
  3. l_ij = rowsum(Pt_ij)
  4. m_new = max(m_old, m_ij);
     l_new = exp(m_old - m_new) * l_old + exp(m_ij - m_new) * l_ij
  5. Ot_new = exp(m_old - m_new) * Ot_old + exp(m_ij - m_new) * (Pt_ij V_j)

starting from m = -inf, l = 0, Ot = 0 ("Initialization"), and after the last
tile O_i = Ot_i / l_i ("final safe normalization").  The logsumexp of a row is
m + ln l.  The page's worked example uses scale = 1 (no 1/sqrt(d)).

exp(-inf - finite) = 0 makes the first step's correction vanish, as on the page.
A row whose scores in a tile are all masked has m_ij = -inf; its tile terms are
then taken as zero (exp(-inf - m_new) with m_new finite), which is the limit the
formula has.
"""

from __future__ import annotations

import numpy as np

__all__ = ["tiled_forward"]


def _exp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """exp(a - b) with exp(-inf - x) = 0 for finite or -inf x."""
    out = np.zeros_like(a)
    ok = np.isfinite(a)
    out[ok] = np.exp(a[ok] - b[ok])
    return out


def tiled_forward(q, k, v, block_rows: int, block_cols: int, scale: float = 1.0,
                  causal: bool = False, trace: bool = False):
    """Tiled forward for one head: q [N, d], k [N, d], v [N, d] (float64).

    Returns (O, LSE) and, with trace=True, also a list with one entry per
    (i, j) inner step: dict(i, j, m, l, Ot) holding the running statistics of
    query tile i after key tile j.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    t_r = -(-n // block_rows)
    t_c = -(-k.shape[0] // block_cols)
    o = np.empty_like(q)
    lse = np.empty(n)
    steps = []
    for i in range(t_r):
        rows = np.arange(i * block_rows, min(n, (i + 1) * block_rows))
        q_i = q[rows]
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        ot = np.zeros((len(rows), d))
        for j in range(t_c):
            cols = np.arange(j * block_cols, min(k.shape[0], (j + 1) * block_cols))
            # step 1
            s_ij = scale * (q_i @ k[cols].T)
            if causal:
                s_ij = np.where(cols[None, :] > rows[:, None], -np.inf, s_ij)
            # step 2
            m_ij = np.max(s_ij, axis=1)
            pt = np.zeros_like(s_ij)
            live = np.isfinite(m_ij)
            pt[live] = np.exp(s_ij[live] - m_ij[live, None])
            # step 3
            l_ij = np.sum(pt, axis=1)
            # step 4
            m_new = np.maximum(m, m_ij)
            alpha = _exp_diff(m, m_new)
            beta = _exp_diff(m_ij, m_new)
            l = alpha * l + beta * l_ij
            # step 5
            ot = alpha[:, None] * ot + beta[:, None] * (pt @ v[cols])
            m = m_new
            if trace:
                steps.append({"i": i, "j": j, "m": m.copy(), "l": l.copy(), "Ot": ot.copy()})
        o[rows] = ot / l[:, None]
        lse[rows] = m + np.log(l)
    if trace:
        return o, lse, steps
    return o, lse
