"""The parity tolerance for bf16 outputs (gpu_helpers.assert_close), pinned on
the CPU.

The bound is max |y - y_oracle| <= 1e-2 x RMS(y_oracle).  A bf16 output is a
computed value stored with round-to-nearest-even, and that rounding alone moves
an element by up to 2^-9 |y|.  So a literal, unrounded comparison would reject
even the oracle's own correctly rounded output wherever |y| exceeds about 2.6
RMS: the first test shows this on an FFN output.  The check used instead is that
the stored bf16 is the rounding of some value within the bound.  It accepts that
output and rejects a result off by the bound or by two ulps of a large element."""
import numpy as np
import pytest

import oracle as O
from cgs_inputs import ffn_weights, random_bf16
from gpu_helpers import assert_close, bf16_bracket


def _ffn_output():
    w = ffn_weights(60, 0, 256, 1024)
    x = random_bf16(60, 0, "x", (64, 256))
    return O.ffn_geglu(O.decode(x, "bf16"), w)


def test_literal_bound_rejects_a_correctly_rounded_output():
    y = _ffn_output()
    rms = float(np.sqrt(np.mean(y ** 2)))
    stored = O.decode(O.round_to_bf16_bits(y), "bf16")
    over = np.abs(stored - y) > 1e-2 * rms
    assert over.any(), "the storage rounding alone should exceed the literal bound somewhere"
    assert np.all(np.abs(y[over]) > 2.5 * rms)          # only at large elements
    assert_close(stored, y, "correctly rounded output", out="bf16")


def test_bracket_rejects_errors_at_the_bound_and_two_ulps():
    y = _ffn_output()
    rms = float(np.sqrt(np.mean(y ** 2)))
    stored = O.decode(O.round_to_bf16_bits(y), "bf16")
    j = int(np.argmax(np.abs(y)))                       # the largest element
    bad = stored.copy()
    bad.flat[j] = O.decode(O.round_to_bf16_bits(y.flat[j] + 2.5e-2 * rms), "bf16")
    with pytest.raises(AssertionError):
        assert_close(bad, y, "off by 2.5 x the bound", out="bf16")
    bits = O.round_to_bf16_bits(y)
    two_ulp = bits.copy()
    two_ulp.flat[j] = np.uint16(int(two_ulp.flat[j]) + 2)  # two bf16 steps away from |y| max
    with pytest.raises(AssertionError):
        assert_close(O.decode(two_ulp, "bf16"), y, "two ulps off at the largest element", out="bf16")
    # one ulp off at a small element is within the bound
    s = int(np.argmin(np.abs(y) + (np.abs(y) < 1e-3 * rms)))
    one_ulp = bits.copy()
    one_ulp.flat[s] = np.uint16(int(one_ulp.flat[s]) + 1)
    assert_close(O.decode(one_ulp, "bf16"), y, "one ulp off at a small element", out="bf16")


def test_bracket_is_the_rounding_of_the_interval():
    """Every bf16 value inside [RNE(y - a), RNE(y + a)] is RNE of a point of
    [y - a, y + a] and none outside is: checked by enumerating bf16 neighbours."""
    g = np.random.default_rng(3)
    y = g.standard_normal(200) * 4.0
    a = 0.05
    lo, hi = bf16_bracket(y, a)
    for v, l_, h_ in zip(y, lo, hi):
        base = int(O.round_to_bf16_bits(np.array([v]))[0])
        for step in range(-6, 7):
            b = np.uint16(base + step)
            val = float(O.decode(np.array([b]), "bf16")[0])
            # is val the RNE of some point in [v - a, v + a]? sample the interval densely
            pts = np.linspace(v - a, v + a, 4001)
            hit = np.any(O.decode(O.round_to_bf16_bits(pts), "bf16") == val)
            assert hit == (l_ <= val <= h_), (v, val, l_, h_)


def test_f32_outputs_use_the_literal_bound():
    y = _ffn_output()
    rms = float(np.sqrt(np.mean(y ** 2)))
    ok = y + 0.9e-2 * rms
    assert_close(ok, y, "inside", out="f32")
    with pytest.raises(AssertionError):
        assert_close(y + 1.1e-2 * rms, y, "outside", out="f32")
