"""Pins of the oracle's joint token + neuron sparsity (paper §6.1): it must
reduce to Eq. 4 on every row when all rows are selected, to the anchor output
when none are, treat rows independently, and give the anchor output back on a
selected row whose input equals the anchor's."""
import numpy as np

import oracle as O
from cgs_inputs import act_tokens, ffn_weights, rng


def _setup():
    w = ffn_weights(90, 0, 128, 192, down_layout="fd", down_lognormal_sigma=1.5)
    t = act_tokens(90, 0, 12, 128, noise_sigma=0.33)
    ya, ha = O.act_ffn_masked(w, t["x_pert"], np.arange(192))
    idx = np.sort(rng(90, 0, "perm").permutation(192)[:60])
    return w, t["x"], t["x_pert"], ya.astype(np.float32), ha.astype(np.float32), idx


def test_all_rows_is_eq4():
    w, x, _, ya, ha, idx = _setup()
    y = O.act_ffn_joint(w, x, np.arange(12), idx, ya, ha)
    y4, _ = O.act_ffn_masked(w, x, idx, ya, ha)
    assert np.array_equal(y, y4)


def test_no_rows_is_the_anchor():
    w, x, _, ya, ha, idx = _setup()
    assert np.array_equal(O.act_ffn_joint(w, x, [], idx, ya, ha), ya.astype(np.float64))


def test_rows_are_independent():
    w, x, _, ya, ha, idx = _setup()
    tok = np.array([1, 4, 5, 9])
    y = O.act_ffn_joint(w, x, tok, idx, ya, ha)
    for p in tok:
        yp = O.act_ffn_joint(w, x, [p], idx, ya, ha)
        assert np.allclose(y[p], yp[p], rtol=0, atol=1e-12)
    rest = np.setdiff1d(np.arange(12), tok)
    assert np.array_equal(y[rest], ya[rest].astype(np.float64))


def test_selected_row_at_the_anchor_input_returns_the_anchor():
    w, x, xa, ya, ha, idx = _setup()
    xs = np.array(x)
    xs[3] = xa[3]   # row 3 sees the anchor step's input again
    y = O.act_ffn_joint(w, xs, [3, 7], idx, ya, ha)
    assert np.allclose(y[3], ya[3], rtol=0, atol=1e-6 * np.abs(ya).max())
