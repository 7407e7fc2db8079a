"""Pins of the retrieval model (oracle/cgs_retrieval.py): closed forms of the
cosine and of the RMS distance, brute-force ranking, and the fallback rule
(rMuscle §4.2, §5)."""
import math

import numpy as np

from cgs_inputs import rng
from oracle import round_to_bf16_bits
from oracle.cgs_retrieval import feature_cosines, history_distance, ret_select


def _bf16(x):
    return round_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_cosine_closed_forms():
    g = rng(60, 0, "misc")
    q = _bf16(g.standard_normal(4096))
    neg = _bf16(-np.asarray(q.view(np.uint16).astype(np.uint32) << 16, dtype=np.uint32).view(np.float32))
    refs = np.stack([q, neg])
    keys = feature_cosines(q, refs)
    assert keys[0] == 1.0 and keys[1] == -1.0           # identical / negated features
    orth = np.zeros(4096, dtype=np.uint16)
    orth[:] = _bf16(np.where(np.arange(4096) % 2 == 0, 1.0, 0.0))
    q2 = _bf16(np.where(np.arange(4096) % 2 == 1, 1.0, 0.0))
    assert feature_cosines(q2, orth[None])[0] == 0.0    # disjoint supports
    assert feature_cosines(q2, np.zeros((1, 4096), dtype=np.uint16))[0] == 0.0  # zero norm


def test_cosine_matches_the_float_definition():
    g = rng(61, 0, "misc")
    q = _bf16(g.standard_normal(100_000))
    refs = _bf16(g.standard_normal((5, 100_000)) + 0.5 * (q.astype(np.uint32) << 16).view(np.float32))
    keys = feature_cosines(q, refs)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rf = (refs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = rf @ qf / (np.linalg.norm(rf, axis=1) * np.linalg.norm(qf))
    assert np.max(np.abs(keys - want)) < 1e-7


def test_history_distance_closed_forms():
    L, J = 4, 14
    q = np.zeros((L, J))
    c = np.zeros((L, J))
    c[:, :7] = 0.25       # arm 0 off by 0.25 everywhere
    c[:, 7:] = -0.5       # arm 1 off by 0.5
    assert history_distance(q, c, 0) == 0.25
    assert history_distance(q, c, 1) == 0.5
    assert history_distance(q, c, -1) == 0.5              # dual arm: the larger
    c2 = np.zeros((L, J))
    c2[0, 0] = 1.0                                        # one joint of one step
    assert math.isclose(history_distance(q, c2, 0), math.sqrt(1.0 / 28))


def test_ranking_rerank_and_fallback_brute_force():
    g = rng(62, 0, "misc")
    F, N = 2048, 9
    base = g.standard_normal(F)
    q = _bf16(base)
    mix = np.array([0.99, 0.2, 0.95, 0.95, -0.3, 0.97, 0.0, 0.9, 0.96])
    refs = np.stack([_bf16(m * base + math.sqrt(1 - m * m) * g.standard_normal(F)) for m in mix])
    hist = g.standard_normal((N, 4, 14))
    qh = hist[2] + 0.0                                   # entry 2 has the same history
    keys, top, dist, choice = ret_select(q, refs, 4, qh, hist)
    order = sorted(range(N), key=lambda n: (-keys[n], n))
    assert list(top) == order[:4]
    assert 2 in top and choice == 2 and dist[list(top).index(2)] == 0.0
    # T = 1: the best visual match wins regardless of history
    assert ret_select(q, refs, 1, qh, hist)[3] == order[0]
    # nothing above the threshold: fallback
    assert ret_select(q, refs, 4, qh, hist, min_cos=0.999)[3] == -1
    # equal keys rank by index: two identical entries
    refs2 = np.stack([refs[1], refs[0], refs[0]])
    assert list(ret_select(q, refs2, 3, qh, hist[:3])[1]) == [1, 2, 0]
