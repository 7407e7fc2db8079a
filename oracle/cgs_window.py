"""Plain CPU model of the sliding GPU working set and the reconstruction
budget (test infrastructure only; see the package docstring).

Source: rMuscle (Zhou, Li, Chen, Gu), §4.2 "Sliding Window Prefetching"
(Figure 12): the working set covers, for each of T candidate episodes, the
current matched position and the next L positions; entries shared by
consecutive windows are kept, entries that leave are released, only newly
entering positions are reconstructed.  §4.2 Eq. 5 with Table 2 bounds how
many new entries are reconstructed per window:
    N_prep = min(N_cand, floor(M_free / M_entry), floor((T_avl - T_trans) / T_rec)).

Readings where the pages leave a step open (each listed in the design notes):
  * candidates that exceed N_prep are taken nearest position first, then in
    the episodes' rank order; the rest stay candidates for the next window;
  * the slot capacity of the working set also bounds N_prep;
  * a new entry takes the lowest-numbered free slot, and slots released in an
    advance are free for the entries admitted by the same advance.
Everything here is Python sets, dicts and ``sorted``.
"""
from __future__ import annotations

import math


def prep_budget(n_cand, m_free, m_entry, t_avl, t_trans, t_rec):
    """Eq. 5, clamped at zero."""
    n = min(n_cand, math.floor(m_free / m_entry), math.floor((t_avl - t_trans) / t_rec))
    return max(0, int(n))


def window_entries(episodes, positions, lengths, L):
    """The window as {(episode, position): (offset, rank)}."""
    out = {}
    for rank, (e, p, n) in enumerate(zip(episodes, positions, lengths)):
        for off in range(L + 1):
            if p + off < n:
                out[(e, p + off)] = (off, rank)
    return out


class WindowModel:
    """Resident entries -> slot, over `slots` slots."""

    def __init__(self, slots):
        self.slots = slots
        self.where = {}

    def advance(self, episodes, positions, lengths, L, budget=None):
        """Returns (entered [(episode, position, slot)], left slots ascending, n_candidates)."""
        win = window_entries(episodes, positions, lengths, L)
        left = sorted(s for key, s in self.where.items() if key not in win)
        self.where = {key: s for key, s in self.where.items() if key in win}
        cands = sorted((key for key in win if key not in self.where), key=lambda k: win[k])
        used = set(self.where.values())
        free = [s for s in range(self.slots) if s not in used]
        n = min(len(cands), len(free))
        if budget is not None:
            n = min(n, prep_budget(len(cands), *budget))
        entered = []
        for key, s in zip(cands[:n], free):
            self.where[key] = s
            entered.append((key[0], key[1], s))
        return entered, left, len(cands)


def denoise_schedule(words, ff: int):
    """The denoising schedule of a cache entry's stored masks (rMuscle §4.1,
    "Anchors with Mask Recomputation"; §5 builds a group mask from the
    group's steps).  words[l][t]: the bit-packed mask of layer l at step t.

    Reading: a step whose masks hold every neuron in all layers is a dense
    anchor step; any other step updates the latest anchor with its own masks;
    an update before any anchor is an error.  An update's "mask" is the first
    update step holding the same masks in every layer.  Returns (kind, anchor,
    mask) lists as cgs_denoise_schedule defines them."""
    from .cgs_oracle import mask_indices
    L, T = len(words), len(words[0])
    lists = [[tuple(mask_indices(words[l][t], ff).tolist()) for t in range(T)] for l in range(L)]
    kind, anchor, mask = [], [], []
    n_anchor = 0
    for t in range(T):
        if all(len(lists[l][t]) == ff for l in range(L)):
            kind.append(0)
            anchor.append(n_anchor)
            mask.append(-1)
            n_anchor += 1
            continue
        if n_anchor == 0:
            raise ValueError("an update step before the first anchor")
        kind.append(1)
        anchor.append(n_anchor - 1)
        first = t
        for u in range(t):
            if kind[u] == 1 and all(lists[l][u] == lists[l][t] for l in range(L)):
                first = u
                break
        mask.append(first)
    return kind, anchor, mask
