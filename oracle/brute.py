"""Pure-Python loops for tiny attention problems (N <= 8): an independent pin.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``).  No NumPy, no
vector ops: every score, probability and gradient entry is a scalar sum written
out, so an index or transpose slip in the vectorised oracle shows up as a
mismatch.  Single head; q, k, v, do are lists of rows (lists of floats).
"""

from __future__ import annotations

import math

__all__ = ["forward", "backward"]


def _probs(q, k, scale, causal, visible=None):
    """visible(i, j) -> bool overrides the causal rule when given; a row that sees no
    key gets all-zero probabilities and LSE = -inf."""
    n, nk = len(q), len(k)
    p = []
    lse = []
    for i in range(n):
        row = []
        for j in range(nk):
            # Query i is position i + nk - n of the sequence (bottom-right alignment).
            hidden = (not visible(i, j)) if visible is not None else (causal and j > i + nk - n)
            if hidden:
                row.append(None)
            else:
                row.append(scale * sum(q[i][c] * k[j][c] for c in range(len(q[i]))))
        seen = [x for x in row if x is not None]
        if not seen:
            p.append([0.0] * nk)
            lse.append(-math.inf)
            continue
        m = max(seen)
        z = sum(math.exp(x - m) for x in seen)
        p.append([0.0 if x is None else math.exp(x - m) / z for x in row])
        lse.append(m + math.log(z))
    return p, lse


def forward(q, k, v, scale, causal=False, visible=None):
    """Returns (O, LSE) as nested lists."""
    p, lse = _probs(q, k, scale, causal, visible)
    d = len(v[0])
    o = [[sum(p[i][j] * v[j][c] for j in range(len(k))) for c in range(d)]
         for i in range(len(q))]
    return o, lse


def backward(q, k, v, do, scale, causal=False, visible=None):
    """Returns (dQ, dK, dV) as nested lists, each entry a scalar sum."""
    n, nk, d = len(q), len(k), len(q[0])
    p, _ = _probs(q, k, scale, causal, visible)
    dv = [[sum(p[i][j] * do[i][c] for i in range(n)) for c in range(d)] for j in range(nk)]
    dp = [[sum(do[i][c] * v[j][c] for c in range(d)) for j in range(nk)] for i in range(n)]
    ds = []
    for i in range(n):
        dot = sum(p[i][t] * dp[i][t] for t in range(nk))
        ds.append([p[i][j] * (dp[i][j] - dot) for j in range(nk)])
    dq = [[scale * sum(ds[i][j] * k[j][c] for j in range(nk)) for c in range(d)]
          for i in range(n)]
    dk = [[scale * sum(ds[i][j] * q[i][c] for i in range(n)) for c in range(d)]
          for j in range(nk)]
    return dq, dk, dv
