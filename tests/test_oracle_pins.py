"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""

import math

import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(name):
    fn, bound = P.ALL_PINS[name]
    err = fn()
    assert err <= bound, f"{name}: error {err:.3e} above {bound:.1e}"


def test_worked_example_printed_decimals():
    """The decimals the page prints for l and Ot after the last step agree with the
    closed forms to the printed precision, except the one printed slip (Ot[0][0]),
    which the page's own closed form contradicts by 4.5e-3."""
    g = P.load_golden()
    last = g["steps"][-1]
    pr = last["printed"]
    for r in range(2):
        assert round(P.closed_form(last["l"][r]), pr["l_decimals"]) == pytest.approx(pr["l"][r], abs=1e-12)
        for c in range(2):
            if pr["Ot"][r][c] is None:
                continue
            val = P.closed_form(last["Ot"][r][c])
            assert abs(val - pr["Ot"][r][c]) <= 0.5 * 10 ** -pr["Ot_decimals"] + 1e-12
    slip = last["printed_slip"]["Ot_0_0"]
    assert abs(P.closed_form(last["Ot"][0][0]) - slip) == pytest.approx(0.0045, abs=3e-4)


def test_worked_example_tiled_vs_naive_machine_precision():
    """Tiled and naive agree on the worked example to a few ulps (page: about 2.2e-16)."""
    g = P.load_golden()
    q, k, v = P.worked_example_arrays(g)
    import oracle.attention as A
    import oracle.online_walk as W
    o_t, _ = W.tiled_forward(q, k, v, 2, 2, 1.0)
    o_n, _ = A.attention_forward(q[None, None], k[None, None], v[None, None], 1.0)
    assert np.max(np.abs(o_t - o_n[0, 0])) <= 4 * 2.2e-16 * 4


def test_oracle_handles_large_row_block_shapes():
    """A ragged row-blocked problem with N not a multiple of the block."""
    import oracle.attention as A
    q, k, v, do, scale = P.rng_case(20, 1, 2, 1, 37, 8)
    a = A.attention_backward(q, k, v, do, scale, True, row_block=16)
    assert np.all(np.isfinite(a["dq"])) and np.all(np.isfinite(a["dk"]))
    assert a["lse"].shape == (1, 2, 37)
    # causal: the last row sees every key, the first sees one
    assert math.isclose(a["lse"][0, 0, 0], scale * float(q[0, 0, 0] @ k[0, 0, 0]), abs_tol=1e-14)
