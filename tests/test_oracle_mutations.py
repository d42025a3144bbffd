"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

This is the evidence that the pins in ``oracle_pins.py`` constrain every step of
the oracle: a dropped term, a wrong sign, a missing scale, a transposed operand or
a wrong head map each make at least one pin fail.
"""

import numpy as np
import pytest

import oracle.attention as A
import oracle.fp8 as F8
import oracle.online_walk as W
import oracle.rowsoftmax as RS
import oracle_pins as P


def _mutant_head(variant):
    orig = A.attention_head

    def head(q, k, v, scale, causal, do=None, row_block=1024):
        if do is None or variant is None:
            return orig(q, k, v, scale, causal, do, row_block)
        n = q.shape[0]
        s = A.scores(q, k, scale, causal, np.arange(n))
        p = A.softmax_rows(s)
        o = p @ v
        lse = A.logsumexp_rows(s)
        dp = do @ v.T
        ds = A.softmax_backward_rows(p, dp)
        dvec = np.sum(p * dp, axis=-1)
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        dv = p.T @ do
        if variant == "dk_no_scale":
            dk = ds.T @ q
        elif variant == "dk_transposed":
            dk = scale * (ds @ q)
        elif variant == "dv_transposed":
            dv = p @ do
        elif variant == "dq_uses_v":
            dq = scale * (ds @ v)
        elif variant == "dp_transposed":
            ds = A.softmax_backward_rows(p, (do @ v.T).T)
            dq = scale * (ds @ k)
            dk = scale * (ds.T @ q)
        return o, lse, dq, dk, dv, dvec

    return head


MUTANTS = {
    "jvp_drops_dot": ("softmax_backward_rows", lambda p, g: p * g),
    "jvp_sign_flip": ("softmax_backward_rows",
                      lambda p, g: p * (np.sum(p * g, axis=-1, keepdims=True) - g)),
    "scores_no_scale": ("scores", lambda q, k, scale, causal, row_ids=None, key_offset=0:
                        P_orig_scores(q, k, 1.0, causal, row_ids, key_offset)),
    "causal_off_by_one": ("scores", lambda q, k, scale, causal, row_ids=None, key_offset=0:
                          _shifted_mask(q, k, scale, causal, row_ids, key_offset + 1)),
    "causal_top_left_for_rect": ("scores", lambda q, k, scale, causal, row_ids=None, key_offset=0:
                                 P_orig_scores(q, k, scale, causal, row_ids, 0)),
    "causal_offset_sign": ("scores", lambda q, k, scale, causal, row_ids=None, key_offset=0:
                           P_orig_scores(q, k, scale, causal, row_ids, -key_offset)),
    "interval_hi_exclusive": ("interval_scores", lambda q, k, scale, lo, hi:
                              P_orig_interval(q, k, scale, lo, np.asarray(hi) - 1)),
    "interval_lo_ignored": ("interval_scores", lambda q, k, scale, lo, hi:
                            P_orig_interval(q, k, scale, np.zeros_like(np.asarray(lo)), hi)),
    "interval_transposed_keep": ("interval_scores", lambda q, k, scale, lo, hi:
                                 _interval_rows_as_keys(q, k, scale, lo, hi)),
    "merge_unnormalised": ("merge_partials", lambda o, l: _bad_merge(o, l, "unnormalised")),
    "merge_plain_mean": ("merge_partials", lambda o, l: _bad_merge(o, l, "mean")),
    "merge_lse_is_max": ("merge_partials", lambda o, l: _bad_merge(o, l, "lse_max")),
    "lse_drops_max": ("logsumexp_rows",
                      lambda s: np.log(np.sum(np.exp(s - np.max(s, axis=-1, keepdims=True)), axis=-1))),
    "gqa_modulo_map": ("kv_head_of", lambda h, H, Hkv: h % Hkv),
    "dk_no_scale": ("attention_head", "dk_no_scale"),
    "dk_transposed": ("attention_head", "dk_transposed"),
    "dv_transposed": ("attention_head", "dv_transposed"),
    "dq_uses_v": ("attention_head", "dq_uses_v"),
    "dp_transposed": ("attention_head", "dp_transposed"),
}

P_orig_scores = A.scores
P_orig_interval = A.interval_scores


def _interval_rows_as_keys(q, k, scale, lo, hi):
    """Masks by query index instead of key index (a transposed keep test)."""
    s = scale * (q @ k.T)
    rows = np.arange(q.shape[0])[:, None]
    keep = (rows >= np.asarray(lo)[:, None]) & (rows <= np.asarray(hi)[:, None])
    return np.where(np.broadcast_to(keep, s.shape), s, -np.inf)


def _shifted_mask(q, k, scale, causal, row_ids, key_offset):
    s = scale * (q @ k.T)
    if causal:
        if row_ids is None:
            row_ids = np.arange(q.shape[0])
        s = np.where(np.arange(k.shape[0])[None, :] > row_ids[:, None] + key_offset, -np.inf, s)
    return s


def _bad_merge(o_parts, lse_parts, how):
    o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m[None])
    z = np.sum(w, axis=0)
    if how == "unnormalised":
        return np.sum(w[..., None] * o_parts, axis=0), m + np.log(z)
    if how == "mean":
        return np.mean(o_parts, axis=0), m + np.log(z)
    return np.sum(w[..., None] * o_parts, axis=0) / z[..., None], m


ROW_MUTANTS = {
    "row_softmax_bwd_no_dot": ("softmax_backward", lambda y, dy: np.asarray(y) * np.asarray(dy)),
    "row_logsoftmax_bwd_sign": ("log_softmax_backward",
                                lambda y, dy: np.asarray(dy) + np.exp(y) * np.sum(dy, -1, keepdims=True)),
    "row_xent_grad_no_onehot": ("cross_entropy_backward",
                                lambda x, t, dl: RS.softmax(x) * np.asarray(dl)[:, None]),
    "row_xent_loss_no_lse": ("cross_entropy", lambda x, t: _xent_no_lse(x, t)),
    "row_softmax_no_max": ("softmax", lambda x: _softmax_no_max(x)),
}


def _xent_no_lse(x, t):
    x = np.asarray(x, float)
    t = np.asarray(t)
    live = t >= 0
    zt = np.where(live, x[np.arange(x.shape[0]), np.where(live, t, 0)], 0.0)
    return np.where(live, -zt, 0.0), np.zeros(x.shape[0])


def _softmax_no_max(x):
    e = np.exp(np.asarray(x, float))
    return e / np.sum(e, axis=-1, keepdims=True)


@pytest.mark.parametrize("mutant", sorted(ROW_MUTANTS))
def test_row_mutant_is_caught(mutant, monkeypatch):
    target, repl = ROW_MUTANTS[mutant]
    monkeypatch.setattr(RS, target, repl)
    assert _failing_pins(), f"no pin caught mutant {mutant}"


FP8_MUTANTS = {
    # exponent bias 8 instead of 7
    "fp8_bias_off_by_one": lambda c: _decode_bias(c, 8),
    # subnormals read as if they had the implicit leading one
    "fp8_subnormal_as_normal": lambda c: _decode_no_subnormal(c),
    # the sign bit ignored
    "fp8_no_sign": lambda c: np.abs(_ORIG_DECODE(c)),
}
_ORIG_DECODE = F8.decode_e4m3


def _decode_bias(codes, bias):
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    out = np.where(e == 0, sign * np.ldexp(m / 8.0, 1 - bias), sign * np.ldexp(1.0 + m / 8.0, (e - bias).astype(np.int64)))
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _decode_no_subnormal(codes):
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    out = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


@pytest.mark.parametrize("mutant", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(F8, "decode_e4m3", FP8_MUTANTS[mutant])
    assert _failing_pins(), f"no pin caught mutant {mutant}"


def _failing_pins():
    failed = []
    for name, (fn, bound) in P.ALL_PINS.items():
        try:
            with np.errstate(all="ignore"):
                err = fn()
            if not np.isfinite(err) or err > bound:
                failed.append(name)
        except Exception:  # a shape error or NaN assertion also counts as caught
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    target, repl = MUTANTS[mutant]
    if target == "attention_head":
        monkeypatch.setattr(A, "attention_head", _mutant_head(repl))
    else:
        monkeypatch.setattr(A, target, repl)
    failed = _failing_pins()
    assert failed, f"no pin caught mutant {mutant}"


# Mistakes in the block fold (the exact combination of two summaries, and the final
# output / logsumexp): each mutant replaces one of them with a copy that has one
# thing changed.
def _combine_mutant(kind):
    def combine(a, b):
        (m1, l1, u1), (m2, l2, u2) = a, b
        mm = np.maximum(m1, m2)
        w1, w2 = W._weight(m1, mm), W._weight(m2, mm)
        if kind == "running_not_rescaled":       # the earlier blocks keep their old max
            return mm, l1 + w2 * l2, u1 + w2[:, None] * u2
        if kind == "block_not_rescaled":         # the new block keeps its own max
            return mm, w1 * l1 + l2, w1[:, None] * u1 + u2
        if kind == "correction_inverted":        # exp(M - m) instead of exp(m - M)
            inv = np.where(np.isfinite(m1), np.exp(mm - np.where(np.isfinite(m1), m1, 0)), 0.0)
            return mm, inv * l1 + w2 * l2, inv[:, None] * u1 + w2[:, None] * u2
        if kind == "u_not_rescaled":             # only the denominator is moved
            return mm, w1 * l1 + w2 * l2, u1 + u2
        return mm, w1 * l1 + w2 * l2, w1[:, None] * u1 + w2[:, None] * u2
    return combine


def _finish_drops_max(state):
    m, l, u = state
    return u / l[:, None], np.log(l)


WALK_MUTANTS = ["running_not_rescaled", "block_not_rescaled", "correction_inverted",
                "u_not_rescaled", "lse_drops_max"]


def test_walk_mutant_harness_is_the_fold(monkeypatch):
    """With nothing changed, the test's copy of the combination passes every pin."""
    monkeypatch.setattr(W, "combine", _combine_mutant(None))
    assert _failing_pins() == []


@pytest.mark.parametrize("mutant", WALK_MUTANTS)
def test_walk_mutant_is_caught(mutant, monkeypatch):
    if mutant == "lse_drops_max":
        monkeypatch.setattr(W, "finish", _finish_drops_max)
    else:
        monkeypatch.setattr(W, "combine", _combine_mutant(mutant))
    assert _failing_pins(), f"no pin caught mutant {mutant}"
