"""Plain CPU model of reference retrieval (test infrastructure only; see the
package docstring).

Source: rMuscle (Zhou, Li, Chen, Gu), §4.2 "Retrieving a Relevant Reference"
(visual match: cosine similarity between the flattened current and reference
features, keep the top T) and §5 "Joint-History Retrieval" (rerank by the RMS
joint-angle difference of the aligned state histories, per arm; a dual-arm
task takes the larger arm distance, a single-arm task its active arm) and
"Fallback policy" (visual cosine below 0.8: no reference, dense execution).

Readings (also in the design notes): the cosine is formed from exact
fixed-point sums, each product of two features rounded half-even to an
integer at 2^-24 (the token score's cosine kind), so it is reproducible bit
for bit; ties in the visual rank go to the lower entry index, ties in the
rerank to the better visual rank; the fallback looks at the best match's
cosine.
"""
from __future__ import annotations

import math

import numpy as np

from .cgs_oracle import decode

SCALE = float(2 ** 24)


def _fixed_sum(a, b) -> int:
    """sum over i of rint(2^24 * a_i * b_i) as an exact integer (products exact in float64)."""
    return int(np.rint((a * b) * SCALE).astype(np.int64).sum(dtype=np.int64))


def feature_cosines(query, refs, dtype: str = "bf16") -> np.ndarray:
    q = decode(query, dtype).reshape(-1)
    r = decode(refs, dtype).reshape(len(refs), -1)
    s_qq = _fixed_sum(q, q)
    keys = np.empty(len(r), dtype=np.float64)
    for n in range(len(r)):
        s_rr, s_qr = _fixed_sum(r[n], r[n]), _fixed_sum(q, r[n])
        den = float(s_qq) * float(s_rr)
        keys[n] = float(s_qr) / math.sqrt(den) if den > 0.0 else 0.0
    return keys


def history_distance(q_hist, c_hist, arm: int) -> float:
    """RMS joint difference over the history, per arm (J/2 joints each); arm = -1
    takes the larger arm distance.  Plain left-to-right float64 sums."""
    L, J = len(q_hist), len(q_hist[0])
    half = J // 2
    best = 0.0
    for a in (0, 1):
        if arm >= 0 and a != arm:
            continue
        s = 0.0
        for l in range(L):
            for j in range(a * half, (a + 1) * half):
                df = float(q_hist[l][j]) - float(c_hist[l][j])
                s += df * df
        best = max(best, math.sqrt(s / (L * half)))
    return best


def ret_select(query, refs, T: int, q_hist, r_hist, arm: int = -1, min_cos: float = 0.8,
               dtype: str = "bf16"):
    """Returns (cos [N], top [T], dist [T], choice) with choice = -1 for the fallback."""
    keys = feature_cosines(query, refs, dtype)
    top = sorted(range(len(keys)), key=lambda n: (-keys[n], n))[:T]
    dist = [history_distance(q_hist, r_hist[n], arm) for n in top]
    choice = -1
    if top and keys[top[0]] >= min_cos:
        best = min(range(len(top)), key=lambda i: (dist[i], i))
        choice = top[best]
    return keys, np.array(top, dtype=np.int32), np.array(dist), choice
