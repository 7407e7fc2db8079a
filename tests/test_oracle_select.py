"""Pins of the oracle's token selection (rMuscle §4.1, Eq. 2 and the top ceil(rho_p P) set).

Each test checks the oracle against something other than itself: the pages'
constants and a hand-worked example (tests/golden), exact rational arithmetic,
closed forms, and an exhaustive brute force on tiny inputs.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from cgs_inputs import ctx_layer_inputs, f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_ratio_to_count_page_values():
    g = _load("page_constants.json")
    P = g["token_counts"]["P"]
    for rho, k in g["token_counts"]["cases"]:
        assert O.ratio_to_count(rho, P) == k
    m = g["mask_topk"]
    assert O.ratio_to_count(m["rho_n"], m["H"]) == m["K"]
    # guarded ceil: 0.07 * 100 evaluates to 7.000000000000001 in binary
    assert 0.07 * 100 > 7 and O.ratio_to_count(0.07, 100) == 7
    assert O.ratio_to_count(1.5, 10) == 10 and O.ratio_to_count(-0.1, 10) == 0


def test_eq2_worked_example():
    g = _load("eq2_worked_example.json")
    x = np.array(g["x"], dtype=np.float32)
    xr = np.array(g["x_ref"], dtype=np.float32)
    keys = O.ctx_score_keys(x, xr, "f32")
    assert keys.tolist() == g["keys_fixed_point"]
    # Same ranking as the real-valued Eq. 2 (d^2 values computed by hand).
    eq2 = np.array(g["d_squared_eq2"])
    for k in range(len(x) + 1):
        expect = g["topk"][str(k)]
        assert O.topk_ascending(keys, k).tolist() == expect
        assert O.topk_ascending(eq2, k).tolist() == expect
    # bf16 encoding of the same values gives the same keys (all values exact in bf16)
    kb = O.ctx_score_keys(f32_to_bf16_bits(x), f32_to_bf16_bits(xr), "bf16")
    assert kb.tolist() == g["keys_fixed_point"]


def _is_valid_topk(keys, k, sel):
    """Independent check of a top-k set: correct size, ascending, and every chosen
    index beats every unchosen one under (key desc, index asc)."""
    sel = list(sel)
    if len(sel) != k or sel != sorted(set(sel)):
        return False
    rest = [q for q in range(len(keys)) if q not in set(sel)]
    return all(keys[p] > keys[q] or (keys[p] == keys[q] and p < q) for p in sel for q in rest)


def test_topk_exhaustive_ties():
    for P in range(0, 7):
        for pattern in itertools.product([0.0, 1.0, 2.0], repeat=P):
            keys = np.array(pattern)
            for k in range(P + 1):
                assert _is_valid_topk(keys, k, O.topk_ascending(keys, k))


def test_topk_random_vs_lexsort():
    rng = np.random.default_rng(3)
    for _ in range(50):
        P = int(rng.integers(1, 300))
        keys = rng.integers(0, 20, P).astype(np.float64)  # many ties
        k = int(rng.integers(0, P + 1))
        ref = np.sort(np.lexsort((np.arange(P), -keys))[:k])
        assert np.array_equal(O.topk_ascending(keys, k), ref)


def _bf16_values(rng, shape, lo_exp=-4):
    """bf16 numbers with |v| >= 2^lo_exp, so 2^24 v^2 is an integer (exact terms)."""
    m = rng.integers(128, 256, size=shape)              # 8 significant bits
    e = rng.integers(lo_exp - 7, 2 - 7, size=shape)
    s = rng.choice([-1.0, 1.0], size=shape)
    v = (s * np.ldexp(m.astype(np.float64), e)).astype(np.float32)
    return f32_to_bf16_bits(v), v


def test_score_closed_forms():
    rng = np.random.default_rng(1)
    xb, xv = _bf16_values(rng, (6, 64))
    z = np.zeros_like(xb)
    # identical reference -> 0; zero reference -> exactly 1; negated -> exactly 4
    assert np.all(O.ctx_score_keys(xb, xb) == 0.0)
    assert np.all(O.ctx_score_keys(xb, z) == 1.0)
    assert np.all(O.ctx_score_keys(xb, f32_to_bf16_bits(-xv)) == 4.0)
    # xbar = x / 2: diff = x / 2 exactly, so d^2 = 1/4 exactly
    xr = f32_to_bf16_bits(xv * np.float32(0.5))
    assert np.all(O.ctx_score_keys(xb, xr) == 0.25)
    # identical x_ref and k tokens -> the first k indices
    assert O.ctx_select(xb, xb, 4)[0].tolist() == [0, 1, 2, 3]
    # cosine kind: identical -> 0, negated -> 2, disjoint support -> 1
    assert np.all(O.ctx_score_keys(xb, xb, kind="cosine") == 0.0)
    assert np.all(O.ctx_score_keys(xb, f32_to_bf16_bits(-xv), kind="cosine") == 2.0)
    a = xv.copy(); a[:, 32:] = 0
    b = xv.copy(); b[:, :32] = 0
    kc = O.ctx_score_keys(f32_to_bf16_bits(a), f32_to_bf16_bits(b), kind="cosine")
    assert np.all(kc == 1.0)


def test_score_matches_exact_eq2():
    """Keys equal the exact rational d_p^2 of Eq. 2 within the fixed-point bound."""
    d = 48
    x = ctx_layer_inputs(5, 0, 24, d, 6, 1.0, 0.05)
    keys = O.ctx_score_keys(x["x"], x["x_ref"])
    xd = O.decode(x["x"], "bf16")
    rd = O.decode(x["x_ref"], "bf16")
    for p in range(len(keys)):
        sd = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(xd[p], rd[p]))
        sx = sum(Fraction(float(a)) ** 2 for a in xd[p])
        exact = sd / max(sx, d * Fraction(1, 10 ** 12))
        # |rint error| <= 1/2 per term at 2^-24 resolution, in numerator and denominator
        q = Fraction(d, 2 * 2 ** 24)
        bound = Fraction(101, 100) * (q / sx) * (exact + 1) + Fraction(1, 2 ** 50) * exact
        assert abs(Fraction(float(keys[p])) - exact) <= bound


def test_cosine_equals_rel_rms_for_equal_norms():
    """With ||xbar|| = ||x|| the squared relative RMS is 2 (1 - cos): both kinds rank alike."""
    rng = np.random.default_rng(7)
    P, d = 40, 64
    x = rng.standard_normal((P, d)).astype(np.float32)
    # reference = the same row with some elements permuted: same norm, more change
    # for more permuted elements
    xr = x.copy()
    for p in range(P):
        m = 2 + 2 * p % 50
        m = min(m, d)
        sub = rng.permutation(m)
        xr[p, :m] = x[p, sub]
    xb, rb = f32_to_bf16_bits(x), f32_to_bf16_bits(xr)
    k1 = O.ctx_score_keys(xb, rb, kind="rel_rms")
    k2 = O.ctx_score_keys(xb, rb, kind="cosine")
    for k in (5, 10, 20):
        s1 = O.topk_ascending(k1, k)
        s2 = O.topk_ascending(k2, k)
        # compare only where the cut is not a near tie
        o1 = np.sort(k1)[::-1]
        if o1[k - 1] - o1[k] > 1e-6 * o1[k - 1]:
            assert np.array_equal(s1, s2)
    # the cosine key is 1 - cos|cos|; recover cos and check rel-RMS^2 = 2 (1 - cos)
    c = np.sign(1 - k2) * np.sqrt(np.abs(1 - k2))
    np.testing.assert_allclose(k1, 2 * (1 - c), rtol=1e-5, atol=1e-7)


def test_planted_recovery_tiny_fp32():
    """Tiny check, fp32: 16 of 64 tokens drift with std 1.0, the rest 0.02 (25% ratio)."""
    P, d = 64, 256
    inp = ctx_layer_inputs(0, 0, P, d, 16, 1.0, 0.02, dtype="f32")
    k = O.ratio_to_count(0.25, P)
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], k, "f32")
    assert k == 16 and np.array_equal(idx, inp["changed"])
    assert O.ctx_select(inp["x"], inp["x_ref"], 0, "f32")[0].size == 0
    assert np.array_equal(O.ctx_select(inp["x"], inp["x_ref"], P, "f32")[0], np.arange(P))


@pytest.mark.parametrize("kind", ["rel_rms", "cosine"])
def test_planted_recovery_full_layer(kind):
    """One VLM layer: 231 of 768 tokens at cosine ~0.6, the rest ~0.985; rho_p = 0.3."""
    P, d = 768, 2048
    inp = ctx_layer_inputs(1, 0, P, d, 231, 1.3333, 0.1752)
    k = O.ratio_to_count(0.3, P)
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], k, kind=kind)
    assert k == 231 and np.array_equal(idx, inp["changed"])
