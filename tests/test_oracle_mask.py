"""Pins of the oracle's contribution score (rMuscle §3.4 Eq. 1) and group masks (§5,
and the coverage share of §3.4).

Independent references: the plain real-valued Eq. 1 (torch norms and sums),
a stable argsort, exact rational coverage sums, planted heavy neurons and the
coverage extremes.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from cgs_inputs import ffn_weights, synthetic_h_ref


def _setup(seed=0, T=3, ff=96, S=6, d=32, sigma=1.0):
    w = ffn_weights(seed, 0, d, ff, down_layout="fd", down_lognormal_sigma=sigma)
    h = synthetic_h_ref(seed, 0, T, ff, S, neuron_sigma=sigma)
    return w, h


def test_contribution_matches_eq1():
    """c_{t,n} = (sum_r |h_{t,r,n}|) ||W_n||_2, scaled by the fixed point's 2^44."""
    w, h = _setup()
    c, s = O.contribution_scores(h, w)
    ht = torch.from_numpy(h.astype(np.float64))
    wd = torch.from_numpy(O.decode(w["w_down"], "bf16"))
    norm = torch.linalg.vector_norm(wd, dim=1)
    eq1 = ht.abs().sum(dim=2) * norm[None, :]                    # [T][ff]
    np.testing.assert_allclose(c / 2.0 ** 44, eq1.numpy(), rtol=1e-6)
    np.testing.assert_allclose(s / 2.0 ** 44, eq1.sum(0).numpy(), rtol=1e-6)


def test_contribution_uses_down_rows_of_the_neuron():
    """Scaling neuron n's down weights by 4 scales its score by 4 (to the fixed
    point's resolution) and leaves every other neuron's score unchanged."""
    w, h = _setup(T=1)
    c, _ = O.contribution_scores(h, w)
    w2 = dict(w)
    a = O.decode(w["w_down"], "bf16")
    a[7] *= 4.0
    from cgs_inputs import f32_to_bf16_bits
    w2["w_down"] = f32_to_bf16_bits(a.astype(np.float32))
    c2, _ = O.contribution_scores(h, w2)
    assert abs(c2[0, 7] - 4.0 * c[0, 7]) <= 1e-9 * c2[0, 7]
    assert np.array_equal(np.delete(c2, 7, axis=1), np.delete(c, 7, axis=1))


def test_topk_single_step_is_plain_topk():
    w, h = _setup(T=1)
    c, s = O.contribution_scores(h, w)
    for K in (0, 1, 10, 50, 96):
        ref = np.sort(np.lexsort((np.arange(len(s)), -c[0]))[:K])
        assert np.array_equal(O.mask_topk(c, s, K), ref)


def test_topk_union_properties():
    """§5: result = top K, by summed score, of the union of the per-step top-K sets."""
    w, h = _setup(T=3, sigma=0.3)
    c, s = O.contribution_scores(h, w)
    ff = len(s)
    for K in (5, 20, 48):
        m = O.mask_topk(c, s, K)
        steps = [set(np.lexsort((np.arange(ff), -c[t]))[:K].tolist()) for t in range(3)]
        union = set().union(*steps)
        assert len(m) == K and set(m) <= union
        rest = union - set(m)
        for a in m:
            for b in rest:
                assert s[a] > s[b] or (s[a] == s[b] and a < b)
        # a neuron outside every step's top K is never chosen, even with a large sum
        assert not (set(m) - union)


def test_topk_planted_heavy_neurons():
    w, h = _setup(T=2, sigma=0.2)
    h = h.copy()
    heavy = [3, 40, 77]
    h[:, heavy, :] *= 100.0
    c, s = O.contribution_scores(h, w)
    m = O.mask_topk(c, s, 8)
    assert set(heavy) <= set(m.tolist())


def test_coverage_extremes_and_monotone():
    w, h = _setup(T=2)
    _, s = O.contribution_scores(h, w)
    assert O.mask_coverage(s, 0.0).size == 0
    full = O.mask_coverage(s, 1.0)
    assert np.array_equal(full, np.nonzero(s > 0)[0])
    prev = set()
    for tau in np.linspace(0, 1, 21):
        m = set(O.mask_coverage(s, float(tau)).tolist())
        assert prev <= m
        prev = m
    assert O.mask_coverage(np.zeros(10), 0.5).size == 0


def test_coverage_is_shortest_prefix_exact():
    """Exact rational check: the mask's share of the total reaches tau and dropping its
    lowest-ranked member falls short, up to the fixed point's 2^-Q resolution."""
    w, h = _setup(T=2, ff=200)
    _, s = O.contribution_scores(h, w)
    total = sum(Fraction(float(v)) for v in s)
    Q = O.coverage_exponent_bits(len(s))
    tol = Fraction(len(s), 2 ** Q)
    order = np.lexsort((np.arange(len(s)), -s))
    for tau in (0.1, 0.5, 0.844, 0.95):
        m = O.mask_coverage(s, tau)
        assert np.array_equal(np.sort(order[:len(m)]), m)     # a prefix of the ranking
        share = sum(Fraction(float(s[n])) for n in m) / total
        assert share >= Fraction(tau) - tol
        last = order[len(m) - 1]
        assert (share - Fraction(float(s[last])) / total) < Fraction(tau) + tol


def test_coverage_brute_force_tiny():
    rng = np.random.default_rng(5)
    for _ in range(200):
        ff = int(rng.integers(1, 9))
        s = rng.integers(0, 5, ff).astype(np.float64) * 2.0 ** 40   # ties, zeros
        # dyadic tau: tau * total is exact in float64, so the exact rational
        # definition and the float64 threshold coincide
        tau = float(rng.choice([0.0, 0.25, 0.5, 0.75, 0.875, 1.0]))
        m = O.mask_coverage(s, tau)
        total = Fraction(int(s.sum()))
        order = sorted(range(ff), key=lambda n: (-s[n], n))
        best = None
        for mm in range(ff + 1):
            if sum(Fraction(int(s[n])) for n in order[:mm]) >= Fraction(tau) * total:
                best = mm
                break
        assert np.array_equal(m, np.array(sorted(order[:best]), dtype=np.int32))


def test_coverage_planted_dominant_neuron():
    s = np.full(50, 1.0)
    s[17] = 9 * 49.0          # 90% of the total
    assert O.mask_coverage(s, 0.5).tolist() == [17]
    assert O.mask_coverage(s, 0.9).tolist() == [17]
    assert len(O.mask_coverage(s, 0.95)) == 1 + 25


def test_mask_bits_layout():
    words = O.mask_bits([0, 63, 64, 130], 131)
    assert words.tolist() == [1 | (1 << 63), 1, 4]
    with pytest.raises(ValueError):
        O.mask_coverage(np.ones(3), 1.5)


def test_mask_indices_reads_the_stored_words():
    """Bit (n mod 64) of word n // 64 is neuron n: a hand-written example, the
    little-endian byte view through numpy's unpackbits on random words, the
    empty and full masks, and bits past ff (ignored)."""
    words = np.array([0b1011, 1 << 63, 0], dtype=np.uint64)
    assert O.mask_indices(words, 192).tolist() == [0, 1, 3, 127]
    assert O.mask_indices(words.view(np.int64), 192).tolist() == [0, 1, 3, 127]   # as stored, signed
    assert O.mask_indices(words, 100).tolist() == [0, 1, 3]                        # 127 is past ff
    g = np.random.default_rng(5)
    for ff in (1, 63, 64, 65, 200, 4096):
        nw = (ff + 63) // 64
        w = g.integers(0, 2 ** 63, size=nw, dtype=np.int64).view(np.uint64) ^ \
            (g.integers(0, 2, size=nw, dtype=np.uint64) << np.uint64(63))
        bits = np.unpackbits(w.astype("<u8").view(np.uint8), bitorder="little")[:ff]
        assert np.array_equal(O.mask_indices(w, ff), np.flatnonzero(bits).astype(np.int32)), ff
        full = np.full(nw, np.uint64(2 ** 64 - 1))
        assert O.mask_indices(full, ff).tolist() == list(range(ff))
        assert len(O.mask_indices(np.zeros(nw, np.uint64), ff)) == 0
    idx = np.sort(g.choice(4096, 1251, replace=False))
    assert np.array_equal(O.mask_indices(O.mask_bits(idx, 4096), 4096), idx)


def test_down_weight_norms_against_the_plain_norm_and_closed_forms():
    """||W_n||_2 of Eq. 1 scaled by the fixed point's 2^20: the plain
    Euclidean norm (torch) to rounding; a row of d copies of 2^-5 gives
    B = d 2^30 exactly, so nrm = 2^15 sqrt(d) (= 2^20 at d = 1024); a zero row
    gives 0; and a pure-Python brute force of the fixed-point sum on a few
    rows is matched exactly."""
    w, _ = _setup(d=64)
    nrm = O.down_weight_norms(w)
    wd = torch.from_numpy(O.decode(w["w_down"], "bf16"))
    np.testing.assert_allclose(nrm / 2.0 ** 20, torch.linalg.vector_norm(wd, dim=1).numpy(), rtol=1e-6)
    from cgs_inputs import f32_to_bf16_bits
    d = 1024
    rows = np.zeros((3, d), dtype=np.float32)
    rows[0] = 2.0 ** -5
    rows[2, ::7] = -0.75
    wc = {"d": d, "ff": 3, "dtype": "bf16", "down_layout": "fd",
          "w_gate": f32_to_bf16_bits(np.zeros((3, d), np.float32)),
          "w_up": f32_to_bf16_bits(np.zeros((3, d), np.float32)),
          "w_down": f32_to_bf16_bits(rows)}
    got = O.down_weight_norms(wc)
    assert got[0] == 2.0 ** 20 and got[1] == 0.0
    b2 = sum(round(float(v) * float(v) * 2.0 ** 40) for v in rows[2])
    assert got[2] == float(np.sqrt(np.float64(b2)))
    # the contribution scores use exactly these norms
    h = synthetic_h_ref(3, 0, 2, 3, 4)
    c, _ = O.contribution_scores(h, wc)
    assert c[0, 1] == 0.0
