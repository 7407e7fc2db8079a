// Sliding GPU working set of expanded reference entries and the
// reconstruction budget (rMuscle §4.2: "Sliding Window Prefetching", Figure 12,
// and the cache-entry budget of Eq. 5 with the parameters of Table 2).
//
// The working set holds a fixed number of device slots, each one expanded
// entry (the per-layer FFN inputs and outputs that ref_rebuild_dense writes).
// A window is the current matched position and the next L positions of each
// of T candidate episodes.  On every advance the entries that left the window
// release their slots, and up to N_prep of the window's entries that are not
// resident yet are given free slots, nearest position first; the caller then
// rebuilds exactly those.  Entries shared by consecutive windows stay put.
// Host logic only: no device memory is touched here.
#include <algorithm>
#include <climits>
#include <cmath>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/cgs.h"

struct cgs_window {
  std::vector<int64_t> slot_key;            // packed (episode, position) per slot, -1 = free
  std::unordered_map<int64_t, int> where;   // packed key -> slot
};

namespace {

int64_t pack(int ep, int pos) {
  return (static_cast<int64_t>(ep) << 32) | static_cast<int64_t>(static_cast<uint32_t>(pos));
}

struct Cand {
  int ep, pos, off, rank;
};

}  // namespace

extern "C" int cgs_prep_budget(int n_cand, double m_free, double m_entry, double t_avl, double t_trans,
                               double t_rec) {
  if (n_cand < 0 || !(m_entry > 0.0) || !(t_rec > 0.0) || !(m_free >= 0.0) || std::isnan(t_avl) ||
      std::isnan(t_trans))
    return -1;
  double n = static_cast<double>(n_cand);
  n = std::min(n, std::floor(m_free / m_entry));
  n = std::min(n, std::floor((t_avl - t_trans) / t_rec));
  return n <= 0.0 ? 0 : static_cast<int>(n);
}

extern "C" cgs_window* cgs_window_create(int slots) {
  if (slots <= 0 || slots > (1 << 20)) return nullptr;
  cgs_window* w = new cgs_window;
  w->slot_key.assign(static_cast<size_t>(slots), -1);
  return w;
}

extern "C" void cgs_window_destroy(cgs_window* w) { delete w; }

extern "C" int cgs_window_slot(const cgs_window* w, int episode, int position) {
  if (!w) return -1;
  auto it = w->where.find(pack(episode, position));
  return it == w->where.end() ? -1 : it->second;
}

extern "C" int cgs_window_resident(const cgs_window* w) {
  return w ? static_cast<int>(w->where.size()) : -1;
}

extern "C" int cgs_window_advance(cgs_window* w, int T, const int32_t* episode, const int32_t* position,
                                  const int32_t* length, int L, const cgs_budget* budget, int32_t* enter_ep,
                                  int32_t* enter_pos, int32_t* enter_slot, int32_t* n_enter,
                                  int32_t* leave_slot, int32_t* n_leave, int32_t* n_cand) {
  if (!w || !n_enter || !n_leave || !enter_ep || !enter_pos || !enter_slot || !leave_slot)
    return CGS_ERR_ARG;
  if (T < 0 || L < 0) return CGS_ERR_SHAPE;
  if (T > 0 && (!episode || !position || !length)) return CGS_ERR_ARG;
  if (budget && cgs_prep_budget(0, budget->m_free, budget->m_entry, budget->t_avl, budget->t_trans,
                                budget->t_rec) < 0)
    return CGS_ERR_ARG;
  std::unordered_set<int> seen;
  for (int r = 0; r < T; ++r) {
    if (episode[r] < 0 || position[r] < 0 || length[r] < 0) return CGS_ERR_SHAPE;
    if (!seen.insert(episode[r]).second) return CGS_ERR_ARG;  // an episode listed twice
  }
  // the window, in (offset, episode rank) order
  std::vector<Cand> win;
  std::unordered_set<int64_t> in_win;
  for (int off = 0; off <= L; ++off)
    for (int r = 0; r < T; ++r) {
      const long long q = static_cast<long long>(position[r]) + off;
      if (q >= length[r] || q > INT_MAX) continue;
      win.push_back({episode[r], static_cast<int>(q), off, r});
      in_win.insert(pack(episode[r], static_cast<int>(q)));
    }
  // release what left the window (ascending slot order)
  int nl = 0;
  for (size_t s = 0; s < w->slot_key.size(); ++s) {
    const int64_t k = w->slot_key[s];
    if (k >= 0 && !in_win.count(k)) {
      w->where.erase(k);
      w->slot_key[s] = -1;
      leave_slot[nl++] = static_cast<int32_t>(s);
    }
  }
  // candidates: window entries not resident, nearest first
  std::vector<Cand> cand;
  for (const Cand& c : win)
    if (!w->where.count(pack(c.ep, c.pos))) cand.push_back(c);
  int free_slots = 0;
  for (int64_t k : w->slot_key) free_slots += (k < 0);
  int n_prep = std::min(static_cast<int>(cand.size()), free_slots);
  if (budget) {
    n_prep = std::min(n_prep, cgs_prep_budget(static_cast<int>(cand.size()), budget->m_free, budget->m_entry,
                                              budget->t_avl, budget->t_trans, budget->t_rec));
  }
  int ne = 0;
  size_t s = 0;
  for (int i = 0; i < n_prep; ++i) {
    while (w->slot_key[s] >= 0) ++s;
    const int64_t k = pack(cand[i].ep, cand[i].pos);
    w->slot_key[s] = k;
    w->where[k] = static_cast<int>(s);
    enter_ep[ne] = cand[i].ep;
    enter_pos[ne] = cand[i].pos;
    enter_slot[ne] = static_cast<int32_t>(s);
    ++ne;
  }
  *n_enter = ne;
  *n_leave = nl;
  if (n_cand) *n_cand = static_cast<int32_t>(cand.size());
  return CGS_OK;
}

extern "C" int cgs_denoise_schedule(int L, int T, int ff, const int32_t* counts, const uint64_t* words,
                                    int32_t* kind_out, int32_t* anchor_out, int32_t* mask_out) {
  if (L < 1 || L > 64 || T < 1 || T > 64 || ff < 1 || ff > 65536) return CGS_ERR_SHAPE;
  if (!counts || !words || !kind_out || !anchor_out || !mask_out) return CGS_ERR_ARG;
  const int nw = (ff + 63) / 64;
  const uint64_t last = (ff % 64) ? (~0ull >> (64 - ff % 64)) : ~0ull;  // bits of the last word inside ff
  auto mask_word = [&](int l, int t, int j) {
    const uint64_t v = words[(static_cast<size_t>(l) * T + t) * nw + j];
    return j == nw - 1 ? (v & last) : v;
  };
  for (int l = 0; l < L; ++l)
    for (int t = 0; t < T; ++t) {
      long long bits = 0;
      for (int j = 0; j < nw; ++j) bits += __builtin_popcountll(mask_word(l, t, j));
      if (bits != counts[l * T + t]) return CGS_ERR_ARG;
    }
  auto same = [&](int t1, int t2) {
    for (int l = 0; l < L; ++l)
      for (int j = 0; j < nw; ++j)
        if (mask_word(l, t1, j) != mask_word(l, t2, j)) return false;
    return true;
  };
  int anchors = 0;
  for (int t = 0; t < T; ++t) {
    bool full = true;
    for (int l = 0; l < L && full; ++l) full = counts[l * T + t] == ff;
    if (full) {
      kind_out[t] = 0;
      anchor_out[t] = anchors++;
      mask_out[t] = -1;
      continue;
    }
    if (anchors == 0) return CGS_ERR_SHAPE;  // an update needs an anchor before it
    kind_out[t] = 1;
    anchor_out[t] = anchors - 1;
    mask_out[t] = t;
    for (int u = 0; u < t; ++u)
      if (kind_out[u] == 1 && mask_out[u] == u && same(u, t)) {
        mask_out[t] = u;
        break;
      }
  }
  return CGS_OK;
}
