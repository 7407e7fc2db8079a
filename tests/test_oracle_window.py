"""Pins of the working-set model (oracle/cgs_window.py) against what the
paper states (rMuscle §4.2, Figure 12, Eq. 5, Table 2 and §5's capacity
example), and of the native planner in libcgs against the model."""
import math
import random

import pytest

import cache_guided_sparse_amd as cgs
import numpy as np

import oracle as O
from oracle.cgs_window import WindowModel, denoise_schedule, prep_budget, window_entries


def test_window_size_of_the_representative_configuration():
    # T = 4 episodes, the matched position plus L = 4 more: T (L + 1) = 20 entries
    win = window_entries([3, 7, 11, 20], [5, 0, 9, 2], [40, 40, 40, 40], 4)
    assert len(win) == 20


def test_sliding_by_one_keeps_shared_entries_and_rebuilds_only_new_ones():
    m = WindowModel(32)
    eps, lens = [0, 1, 2, 3], [40] * 4
    entered, left, n = m.advance(eps, [0] * 4, lens, 4)
    assert len(entered) == 20 and left == [] and n == 20
    slots_before = dict(m.where)
    entered, left, n = m.advance(eps, [1] * 4, lens, 4)
    # each episode loses position 0 and gains position 5; 16 entries are shared
    assert sorted((e, p) for e, p, _ in entered) == [(e, 5) for e in eps]
    assert len(left) == 4
    shared = {k: v for k, v in slots_before.items() if k[1] >= 1}
    assert len(shared) == 16 and all(m.where[k] == v for k, v in shared.items())


def test_window_stops_at_the_end_of_an_episode():
    win = window_entries([0], [38], [40], 4)
    assert sorted(win) == [(0, 38), (0, 39)]


def test_budget_of_the_paper_example():
    # §5: ~25 ms per entry and a ~500 ms execution window allow about 20
    # entries; transfers of ~1.7 MB per entry add little; memory holds > 100
    mem = 24e9 - 10e9
    entry = 107e6
    assert math.floor(mem / entry) > 100
    t_trans = 20 * 1.7e6 / 25e9 * 1e3  # 20 compact inputs over a ~25 GB/s link, ms
    assert prep_budget(40, mem, entry, 500.0, t_trans, 25.0) == 19  # just under 20 with transfers
    assert prep_budget(40, mem, entry, 500.0, 0.0, 25.0) == 20
    assert prep_budget(12, mem, entry, 500.0, 0.0, 25.0) == 12   # bounded by the candidates
    assert prep_budget(40, 5 * entry, entry, 500.0, 0.0, 25.0) == 5  # bounded by memory
    assert prep_budget(40, mem, entry, 10.0, 20.0, 25.0) == 0    # no time left


def test_deferred_candidates_are_nearest_first_and_return_later():
    m = WindowModel(64)
    eps, lens = [5, 9], [40, 40]
    budget = (1e12, 1.0, 75.0, 0.0, 25.0)  # three entries per advance
    entered, _, n = m.advance(eps, [0, 0], lens, 4, budget)
    assert n == 10
    assert [(e, p) for e, p, _ in entered] == [(5, 0), (9, 0), (5, 1)]
    entered, _, n = m.advance(eps, [0, 0], lens, 4, budget)
    assert n == 7 and [(e, p) for e, p, _ in entered] == [(9, 1), (5, 2), (9, 2)]


def test_slots_bound_the_admissions():
    m = WindowModel(6)
    entered, _, n = m.advance([0, 1], [0, 0], [40, 40], 4)
    assert n == 10 and len(entered) == 6 and sorted(s for *_, s in entered) == list(range(6))


def _random_walk(seed, slots, steps):
    rng = random.Random(seed)
    n_ep = rng.randint(1, 6)
    pool = rng.sample(range(50), 12)
    lens = {e: rng.randint(1, 45) for e in pool}
    eps = rng.sample(pool, n_ep)
    pos = {e: 0 for e in pool}
    for _ in range(steps):
        if rng.random() < 0.2:
            eps = rng.sample(pool, rng.randint(0, 6))
        for e in eps:
            pos[e] = max(0, pos[e] + rng.choice([-1, 0, 1, 1, 2]))
        L = rng.randint(0, 5)
        budget = None if rng.random() < 0.5 else (rng.uniform(0, 2e9), 1.07e8, rng.uniform(0, 300),
                                                  rng.uniform(0, 20), rng.uniform(5, 40))
        yield eps, [pos[e] for e in eps], [lens[e] for e in eps], L, budget


@pytest.mark.parametrize("seed", range(6))
def test_native_planner_matches_the_model(seed):
    slots = [4, 16, 20, 64, 7, 1][seed]
    model, native = WindowModel(slots), cgs.Window(slots)
    for eps, pos, lens, L, budget in _random_walk(seed, slots, 200):
        want = model.advance(eps, pos, lens, L, budget)
        got = native.advance(eps, pos, lens, L, budget)
        assert got == want
        assert native.resident() == len(model.where)
        for (e, p), s in model.where.items():
            assert native.slot(e, p) == s


def test_native_budget_matches_the_model():
    rng = random.Random(7)
    for _ in range(2000):
        args = (rng.randint(0, 60), rng.uniform(0, 5e9), rng.uniform(1e6, 2e8), rng.uniform(-50, 600),
                rng.uniform(0, 100), rng.uniform(0.5, 60))
        assert cgs.prep_budget(*args) == prep_budget(*args)


def test_native_planner_rejects_bad_arguments_without_changing_state():
    w = cgs.Window(8)
    w.advance([1, 2], [0, 0], [10, 10], 1)
    before = w.resident()
    for bad in (([1, 1], [0, 0], [10, 10], 1, None),       # an episode twice
                ([1], [-1], [10], 1, None),                  # negative position
                ([1], [0], [10], -1, None),                  # negative L
                ([1], [0], [10], 1, (1e9, 0.0, 1.0, 0.0, 1.0))):  # M_entry = 0
        with pytest.raises(cgs.CgsError):
            w.advance(*bad)
        assert w.resident() == before
    with pytest.raises(cgs.CgsError):
        cgs.Window(0)
    with pytest.raises(cgs.CgsError):
        cgs.prep_budget(3, 1.0, 1.0, 1.0, 0.0, 0.0)


def _words(lists, ff):
    return np.array([[O.mask_bits(m, ff) for m in row] for row in lists], dtype=np.uint64)


def test_denoise_schedule_of_stored_masks():
    """The schedule of an entry's masks: the one-group [all, G, G, G] and
    two-group [all, G1, all, G2] layouts by hand, then the native planner
    against the plain model on random layouts; refusals: an update before any
    anchor, and counts that disagree with the bits."""
    ff, L = 200, 3
    full = list(range(ff))
    g = np.random.default_rng(7)
    G = [sorted(g.choice(ff, 50, replace=False)) for _ in range(L)]
    H = [sorted(g.choice(ff, 70, replace=False)) for _ in range(L)]
    one = [[full, G[l], G[l], G[l]] for l in range(L)]
    two = [[full, G[l], full, H[l]] for l in range(L)]
    assert denoise_schedule(_words(one, ff), ff) == ([0, 1, 1, 1], [0, 0, 0, 0], [-1, 1, 1, 1])
    assert denoise_schedule(_words(two, ff), ff) == ([0, 1, 0, 1], [0, 0, 1, 1], [-1, 1, -1, 3])
    # a layer with every neuron does not make an anchor step on its own
    part = [[full, full if l == 0 else G[l], G[l], G[l]] for l in range(L)]
    assert denoise_schedule(_words(part, ff), ff) == ([0, 1, 1, 1], [0, 0, 0, 0], [-1, 1, 2, 2])
    for trial in range(30):
        T = int(g.integers(1, 7))
        pool = [[sorted(g.choice(ff, int(g.integers(0, ff)), replace=False)) for _ in range(L)] for _ in range(3)]
        steps = [None if (t == 0 or g.random() < 0.3) else pool[int(g.integers(0, 3))] for t in range(T)]
        lists = [[full if steps[t] is None else steps[t][l] for t in range(T)] for l in range(L)]
        words = _words(lists, ff)
        counts = np.array([[len(m) for m in row] for row in lists], dtype=np.int32)
        assert cgs.denoise_schedule(counts, words, ff) == denoise_schedule(words, ff), trial
    with pytest.raises(ValueError):
        denoise_schedule(_words([[G[l], full] for l in range(L)], ff), ff)
    bad = _words([[G[l], full] for l in range(L)], ff)
    cnt = np.array([[50, ff]] * L, dtype=np.int32)
    with pytest.raises(cgs.CgsError, match="size or count"):
        cgs.denoise_schedule(cnt, bad, ff)
    ok = _words(one, ff)
    cnt = np.array([[ff, 50, 50, 50]] * L, dtype=np.int32)
    cnt[1, 2] = 51
    with pytest.raises(cgs.CgsError, match="invalid argument"):
        cgs.denoise_schedule(cnt, ok, ff)
    # bits past ff are ignored by both
    wpad = ok.copy()
    wpad[:, :, -1] |= np.uint64(1) << np.uint64(63)
    cnt = np.array([[ff, 50, 50, 50]] * L, dtype=np.int32)
    assert cgs.denoise_schedule(cnt, wpad, ff) == denoise_schedule(wpad, ff) == ([0, 1, 1, 1], [0] * 4, [-1, 1, 1, 1])
