"""GPU parity of ret_select (rMuscle §4.2 visual match over the prepared
entries, §5 joint-history rerank and fallback): cosines, ranks, distances and
the choice equal the oracle's bit for bit (exact integer sums, the same
float64 operations in the same order)."""
import math

import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
from cgs_inputs import rng
from gpu_helpers import dev, say, to_dev
from oracle import round_to_bf16_bits
from oracle.cgs_retrieval import ret_select as oracle_select

pytestmark = pytest.mark.gpu


def _case(seed, N, F, dtype="bf16", planted=None, L=4, J=14):
    g = rng(seed, N, "misc")
    base = g.standard_normal(F)
    mix = g.uniform(-0.2, 0.99, N)
    if planted is not None:
        mix[planted] = 0.97
    refs = np.stack([m * base + math.sqrt(1 - m * m) * g.standard_normal(F) for m in mix])
    q = base + 0.05 * g.standard_normal(F)
    if dtype == "bf16":
        refs, q = round_to_bf16_bits(refs), round_to_bf16_bits(q)
    else:
        refs, q = refs.astype(np.float32), q.astype(np.float32)
    hist = g.standard_normal((N, L, J)).astype(np.float32)
    qh = (hist[planted] if planted is not None else g.standard_normal((L, J))).astype(np.float32)
    qh = qh + np.float32(0.01) * g.standard_normal((L, J)).astype(np.float32)
    return q, refs, qh, hist


def _run(q, refs, qh, hist, T, arm=-1, min_cos=0.8, dtype="bf16"):
    cos, top, dist, choice = cgs.ret_select(to_dev(q, dtype), to_dev(refs, dtype), T, to_dev(qh, "f32"),
                                            to_dev(hist, "f32"), arm=arm, min_cos=min_cos)
    torch.cuda.synchronize()
    got = (cos.cpu().numpy(), top.cpu().numpy(), dist.cpu().numpy(), int(choice.item()))
    want = oracle_select(q, refs, T, qh, hist, arm=arm, min_cos=min_cos, dtype=dtype)
    assert np.array_equal(got[0], want[0]), "cosines differ"
    assert np.array_equal(got[1], want[1]), "top-T differs"
    assert np.array_equal(got[2], want[2]), "rerank distances differ"
    assert got[3] == want[3], "choice differs"
    return got


@pytest.mark.parametrize("N,F,T,arm", [(16, 768 * 1152, 4, -1), (20, 768 * 1152, 4, 0), (1, 4096, 1, -1),
                                       (7, 1000, 7, 1), (256, 8192, 12, -1)])
def test_parity(N, F, T, arm):
    say("retrieval", N, F, T, arm)
    q, refs, qh, hist = _case(70 + N, N, F, planted=N // 2)
    got = _run(q, refs, qh, hist, T, arm=arm)
    if T > 1:
        assert got[3] == N // 2   # the planted entry: high cosine and the matching history


def test_fp32_features():
    say("retrieval f32")
    q, refs, qh, hist = _case(80, 10, 6000, dtype="f32", planted=3)
    assert _run(q, refs, qh, hist, 3, dtype="f32")[3] == 3


def test_fallback_below_threshold():
    say("retrieval fallback")
    g = rng(81, 0, "misc")
    q = round_to_bf16_bits(g.standard_normal(50_000))
    refs = round_to_bf16_bits(g.standard_normal((12, 50_000)))   # unrelated: cos ~ 0
    hist = g.standard_normal((12, 4, 14)).astype(np.float32)
    assert _run(q, refs, hist[0], hist, 4)[3] == -1
