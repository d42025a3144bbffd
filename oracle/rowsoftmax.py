"""Plain fp64 CPU oracle for row softmax, log-softmax and cross-entropy with logits,
forward and backward.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it; it
shares nothing with the HIP library.

What it computes (softmax-backward page on shreyansh26.github.io):
  * softmax of each row, max-subtracted ("Setup", "The Softmax Derivative");
  * softmax backward: the row Jacobian-vector product S * (g - <S, g>)
    ("Backpropagating Through Softmax");
  * log-softmax z - logsumexp(z) and its backward g - softmax(z) * rowsum(g)
    ("LogSoftmax Backward");
  * cross-entropy with logits against a class index t: logsumexp(z) - z_t per row,
    and its gradient (softmax(z) - onehot(t)) times the row's upstream gradient
    ("Cross-Entropy With Logits").  A target outside 0 .. cols-1 (negative, such as
    -100, or too large) marks an ignored row: loss 0, zero gradient (a reading; the
    page's plain version has no ignored labels).
Rows are independent; x is [rows, cols].
"""

from __future__ import annotations

import numpy as np

__all__ = ["softmax", "softmax_backward", "log_softmax", "log_softmax_backward",
           "cross_entropy", "cross_entropy_backward", "logsumexp"]


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def logsumexp(x):
    """ln sum_j exp(x_j) per row, about the row max."""
    x = _f64(x)
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def softmax(x):
    x = _f64(x)
    e = np.exp(x - np.max(x, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def softmax_backward(y, dy):
    """dx = y * (dy - rowsum(dy * y)), y the softmax output."""
    y, dy = _f64(y), _f64(dy)
    return y * (dy - np.sum(dy * y, axis=-1, keepdims=True))


def log_softmax(x):
    x = _f64(x)
    return x - logsumexp(x)[..., None]


def log_softmax_backward(y, dy):
    """dx = dy - exp(y) * rowsum(dy), y the log-softmax output (exp(y) is the softmax)."""
    y, dy = _f64(y), _f64(dy)
    return dy - np.exp(y) * np.sum(dy, axis=-1, keepdims=True)


def _live(t, cols):
    return (t >= 0) & (t < cols)


def cross_entropy(x, t):
    """Per-row loss logsumexp(x) - x_t, and the row logsumexp; ignored rows give 0."""
    x = _f64(x)
    t = np.asarray(t, dtype=np.int64)
    lse = logsumexp(x)
    live = _live(t, x.shape[-1])
    zt = np.where(live, x[np.arange(x.shape[0]), np.where(live, t, 0)], 0.0)
    return np.where(live, lse - zt, 0.0), lse


def cross_entropy_backward(x, t, dloss):
    """dlogits = dloss_row * (softmax(x) - onehot(t)); zero for ignored rows."""
    x = _f64(x)
    t = np.asarray(t, dtype=np.int64)
    live = _live(t, x.shape[-1])
    g = softmax(x)
    rows = np.nonzero(live)[0]
    g[rows, t[rows]] -= 1.0
    g *= _f64(dloss)[:, None]
    g[~live] = 0.0
    return g
