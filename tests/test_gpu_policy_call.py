"""Consecutive whole policy calls through the sliding working set, checked
against the oracle on every call (rMuscle §4.2: sliding window prefetching,
asynchronous online reconstruction, retrieving a relevant reference; §5:
joint-history retrieval and fallback, group neuron masks kept with each cache
entry; §4.1: the Context Cache prefill and the anchored masked denoise).

The repository holds reference episodes; each entry is a compact residual-
stream input of 768 x 2048 (bf16), its retrieval features (768 x 1152) and
joint history, and its bit-packed neuron masks, one per expert layer and
denoising step (18 x 4 masks of 4096 bits).  Each entry's masks are the
oracle's coverage cut (84.4%) of seeded contribution scores; entries at even
positions hold the one-group schedule [all, G, G, G] (one anchor), at odd
positions the two-group schedule [all, G1, all, G2] (anchors at steps 0 and
2).  The working set is the pages' 2-D window: T = 4 candidate episodes, the
matched position and the next L = 4 of each, 20 slots.

Per call: the window advances every episode by one position (native planner
against the plain model); the entering entries are moved to the device (input,
features, history, masks), expanded by the 17-layer dense rebuild (up to four
entries in one prefill over their rows), their masks
turned back into index lists on the GPU and their update steps' weight rows
gathered into compact buffers.  Retrieval among the 20 slots picks the call's
entry; the 17-layer selective prefill (rho_p 0.3) runs against it, then the
4-step denoise whose schedule and masks come from that entry, as one chain of
72 layers.

Checks, every call: admissions equal the model's; retrieval bit-exact with
the chosen slot the call's entry; the slot's mask words, index lists and
counts equal the stored masks read by the oracle; the schedule equals the
oracle's; every prefill layer's selection is the oracle's on the GPU's own
inputs, copied rows are the cached bits, sampled recomputed rows within the
bound; every denoise layer (anchor and update) within the bound of the oracle
on its own inputs and anchor state, and each next input the RMSNorm of the
residual carried by the GPU's outputs (teacher forcing).
"""
import math

import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import act_tokens, ctx_layer_inputs, ffn_weight_pool, ffn_weights, rng, timestep_embedding
from gpu_helpers import assert_close, bits, dev, ffn_dev, say, to_dev
from oracle.cgs_retrieval import ret_select as oracle_select
from oracle.cgs_window import WindowModel, denoise_schedule

pytestmark = pytest.mark.gpu

L_VLM, P, D, FF = 17, 768, 2048, 16384
L_EXP, S, DE, FFE, STEPS = 18, 50, 1024, 4096, 4
EPISODES, EP_LEN, LOOKAHEAD, CALLS = 4, 14, 4, 8
SLOTS = EPISODES * (LOOKAHEAD + 1)
FEAT, HIST_L, JOINTS, TOP_T = 768 * 1152, 4, 14, 4
RHO_P, N_CHANGED, COVERAGE = 0.3, 231, 0.844
NW = (FFE + 63) // 64


def _entry_id(e, q):
    return e * EP_LEN + q


def _entry_masks(e, q):
    """Stored masks of entry (e, q): words [L_EXP][STEPS][NW] (uint64), counts
    [L_EXP][STEPS].  Each group mask is the oracle's coverage cut of seeded
    heavy-tailed contribution scores."""
    two = q % 2 == 1
    full = np.arange(FFE)
    words = np.empty((L_EXP, STEPS, NW), dtype=np.uint64)
    counts = np.empty((L_EXP, STEPS), dtype=np.int32)
    for l in range(L_EXP):
        groups = []
        for gi in range(2 if two else 1):
            g = rng(50 + gi, _entry_id(e, q) * L_EXP + l, "misc")
            s = np.exp(g.standard_normal(FFE)) * np.abs(g.standard_normal(FFE) * g.standard_normal(FFE))
            groups.append(O.mask_coverage(s, COVERAGE))
        steps = [full, groups[0], full, groups[1]] if two else [full, groups[0], groups[0], groups[0]]
        for t, m in enumerate(steps):
            words[l, t] = O.mask_bits(m, FFE)
            counts[l, t] = len(m)
    return words, counts


class _Store:
    """The host repository, drawn lazily per entry."""

    def __init__(self):
        self.entries, self.masks = {}, {}
        g = rng(46, 0, "misc")
        self.feats = np.empty((EPISODES, EP_LEN, FEAT), dtype=np.uint16)
        self.hist = np.empty((EPISODES, EP_LEN, HIST_L, JOINTS), dtype=np.float32)
        self.queries = {}
        c = np.float32(math.sqrt(1 - 0.98 ** 2))
        for e in range(EPISODES):
            f = g.standard_normal(FEAT, dtype=np.float32)
            for q in range(EP_LEN):
                f = np.float32(0.98) * f + c * g.standard_normal(FEAT, dtype=np.float32)
                self.feats[e, q] = O.round_to_bf16_bits(f)
                if e == 0 and q < CALLS:
                    self.queries[q] = O.round_to_bf16_bits(f + np.float32(0.1) * g.standard_normal(FEAT, dtype=np.float32))
            traj = np.cumsum(0.05 * g.standard_normal((EP_LEN + HIST_L, JOINTS)), axis=0)
            self.hist[e] = np.stack([traj[q:q + HIST_L] for q in range(EP_LEN)])
        self.qhist = {q: (self.hist[0, q] + 0.005 * g.standard_normal((HIST_L, JOINTS))).astype(np.float32)
                      for q in range(CALLS)}

    def entry(self, e, q):
        k = (e, q)
        if k not in self.entries:
            self.entries[k] = ctx_layer_inputs(45, _entry_id(e, q), P, D, N_CHANGED, 1.3333, 0.1752)
            self.masks[k] = _entry_masks(e, q)
        return self.entries[k], self.masks[k]


@pytest.fixture(scope="module")
def calls():
    say("policy calls: setup")
    store = _Store()
    vlm = ffn_weight_pool(44, L_VLM, D, FF)
    W = [ffn_dev(w) for w in vlm]
    exp = [ffn_weights(41, l, DE, FFE, down_layout="fd", down_lognormal_sigma=1.5) for l in range(L_EXP)]
    WE = [ffn_dev(w) for w in exp]
    act = act_tokens(41, 0, S, DE)
    a0 = O.decode(act["x"], "bf16")
    temb = [timestep_embedding(1.0 - s / STEPS, DE) for s in range(STEPS + 1)]
    dtemb = [temb[s + 1] - temb[s] for s in range(STEPS)]
    temb0_d, dtemb_d = to_dev(temb[0].astype(np.float32), "f32"), [to_dev(v.astype(np.float32), "f32") for v in dtemb]
    a0_d = to_dev(a0.astype(np.float32), "f32")
    full = torch.arange(FFE, dtype=torch.int32, device=dev())

    xbar = torch.empty(SLOTS, L_VLM, P, D, dtype=torch.bfloat16, device=dev())
    ybar = torch.empty_like(xbar)
    slot_feat = torch.empty(SLOTS, FEAT, dtype=torch.bfloat16, device=dev())
    slot_hist = torch.empty(SLOTS, HIST_L, JOINTS, dtype=torch.float32, device=dev())
    slot_words = torch.empty(SLOTS, L_EXP, STEPS, NW, dtype=torch.int64, device=dev())
    slot_idx = torch.empty(SLOTS, L_EXP, STEPS, FFE, dtype=torch.int32, device=dev())
    slot_cnt = torch.empty(SLOTS, L_EXP, STEPS, dtype=torch.int32, device=dev())
    y_anc = torch.empty(2, L_EXP, S, DE, dtype=torch.float32, device=dev())
    h_anc = torch.empty(2, L_EXP, FFE, S, dtype=torch.float32, device=dev())
    ych = torch.empty(STEPS * L_EXP, S, DE, dtype=torch.bfloat16, device=dev())
    xch = torch.empty(STEPS * L_EXP + 1, S, DE, dtype=torch.bfloat16, device=dev())
    r_act = torch.empty(S, DE, dtype=torch.float32, device=dev())
    slot_entry, slot_chain, slot_sched = [None] * SLOTS, [None] * SLOTS, [None] * SLOTS

    def admit_batch(batch):
        """The entering entries, up to 4 at a time: one dense rebuild over all
        their rows, then each entry's own preparation."""
        r0 = torch.stack([to_dev(store.entry(e, q)[0]["x"]) for e, q, _ in batch]).contiguous()
        cgs.ref_rebuild_dense_batch(W, r0, [xbar[s_] for _, _, s_ in batch], [ybar[s_] for _, _, s_ in batch])
        for e, q, slot in batch:
            admit(e, q, slot)

    def admit(e, q, slot):
        entry, (words, counts) = store.entry(e, q)
        slot_feat[slot] = to_dev(store.feats[e, q])
        slot_hist[slot] = to_dev(store.hist[e, q], "f32")
        slot_words[slot] = torch.from_numpy(words.view(np.int64)).to(dev())
        cgs.act_mask_indices(slot_words[slot], FFE, idx_out=slot_idx[slot], count_out=slot_cnt[slot])
        kind, anchor, mask = cgs.denoise_schedule(counts, words, FFE)
        compact = {}
        for t in range(STEPS):
            if kind[t] == 1 and mask[t] == t:
                compact[t] = [cgs.act_gather_rows(WE[l], slot_idx[slot, l, t, :counts[l, t]]) for l in range(L_EXP)]
        chain = []
        for t in range(STEPS):
            a = anchor[t]
            for l in range(L_EXP):
                i = t * L_EXP + l
                bias = dtemb_d[t] if l == L_EXP - 1 else None
                if kind[t] == 0:
                    chain.append(cgs.MaskedLayer(WE[l], full, bias=bias, y_out=ych[i], y_f32_out=y_anc[a, l],
                                                 h_out=h_anc[a, l]))
                else:
                    m = mask[t]
                    chain.append(cgs.MaskedLayer(compact[m][l], slot_idx[slot, l, m, :counts[l, m]],
                                                 y_anchor=y_anc[a, l], h_anchor=h_anc[a, l], bias=bias,
                                                 y_out=ych[i]))
        slot_entry[slot], slot_chain[slot] = (e, q), cgs.MaskedChain(chain, S, FFE)
        slot_sched[slot] = (kind, anchor, mask)

    window, model = cgs.Window(SLOTS), WindowModel(SLOTS)
    k = cgs.ratio_to_count(RHO_P, P)
    r = torch.empty(P, D, dtype=torch.float32, device=dev())
    xs = torch.empty(L_VLM, P, D, dtype=torch.bfloat16, device=dev())
    ys = torch.empty_like(xs)
    idx = torch.empty(L_VLM, k, dtype=torch.int32, device=dev())
    skey = torch.empty(P, dtype=torch.float64, device=dev())
    eps, lens = list(range(EPISODES)), [EP_LEN] * EPISODES
    out = []
    for q in range(CALLS):
        say("policy call", q)
        rec = {"q": q}
        entered, left, ncand = window.advance(eps, [q] * EPISODES, lens, LOOKAHEAD)
        rec["window"] = ((entered, left, ncand), model.advance(eps, [q] * EPISODES, lens, LOOKAHEAD))
        for b0 in range(0, len(entered), 4):
            admit_batch(entered[b0:b0 + 4])
        cos, top, dist, choice = cgs.ret_select(to_dev(store.queries[q]), slot_feat, TOP_T,
                                                to_dev(store.qhist[q], "f32"), slot_hist, arm=-1, min_cos=0.8)
        torch.cuda.synchronize()
        c = int(choice.item())
        rec["retrieval"] = (cos.cpu().numpy(), c, window.slot(0, q), slot_entry[c] if c >= 0 else None,
                            bits(slot_feat), slot_hist.cpu().numpy())
        if c < 0:
            out.append(rec)
            continue
        # 17-layer selective prefill against the chosen slot
        entry, (words, counts) = store.entry(*slot_entry[c])
        cgs.residual_rmsnorm(r, r_in=to_dev(O.decode(entry["x_ref"], "bf16").astype(np.float32), "f32"), x_out=xs[0])
        for l in range(L_VLM):
            if l == 0:
                cgs.ctx_select(xs[0], xbar[c, 0], k, idx_out=idx[0])
            else:
                cgs.ctx_select_from_keys(skey, k, idx_out=idx[l])
            glue = (r, None, xs[l + 1], xbar[c, l + 1], skey) if l + 1 < L_VLM else (r, None, None)
            cgs.ctx_ffn_recompute(W[l], xs[l], ybar[c, l], idx[l], y_out=ys[l], glue=glue)
        # the denoise the entry's masks define, one chain of 72 layers
        h_anc.fill_(float("nan"))
        cgs.residual_rmsnorm(r_act, r_in=a0_d, bias=temb0_d, x_out=xch[0])
        cgs.act_masked_layers(slot_chain[c], r_act, xch)
        torch.cuda.synchronize()
        rec.update(entry=entry, words=words, counts=counts, sched=slot_sched[c],
                   slot_words=slot_words[c].cpu().numpy(), slot_idx=slot_idx[c].cpu().numpy(),
                   slot_cnt=slot_cnt[c].cpu().numpy(), x=bits(xs), y=bits(ys), idx=idx.cpu().numpy(),
                   xbar=bits(xbar[c]), ybar=bits(ybar[c]), xch=bits(xch), ych=bits(ych),
                   y_anc=y_anc.cpu().numpy(), h_anc=h_anc.cpu().numpy())
        out.append(rec)
    return {"calls": out, "store": store, "vlm": vlm, "exp": exp, "a0": a0, "temb0": temb[0], "dtemb": dtemb,
            "k": k}


@pytest.mark.parametrize("q", range(CALLS))
def test_window_retrieval_and_stored_masks(calls, q):
    rec, store = calls["calls"][q], calls["store"]
    got, want = rec["window"]
    assert got == want, "window admissions"
    assert len(got[0]) == (SLOTS if q == 0 else EPISODES)
    cos, c, slot_q, ent, feat_h, hist_h = rec["retrieval"]
    w_cos, _, _, w_choice = oracle_select(store.queries[q], feat_h, TOP_T, store.qhist[q], hist_h, arm=-1,
                                          min_cos=0.8)
    assert np.array_equal(cos, w_cos) and c == w_choice, "retrieval differs from the oracle"
    assert c == slot_q and ent == (0, q), "the call's own entry must be chosen"
    # the masks moved with the entry and read back on the GPU
    words, counts = rec["words"], rec["counts"]
    assert np.array_equal(rec["slot_words"].view(np.uint64), words)
    assert np.array_equal(rec["slot_cnt"], counts)
    for l in range(L_EXP):
        for t in range(STEPS):
            lst = O.mask_indices(words[l, t], FFE)
            assert np.array_equal(rec["slot_idx"][l, t, : len(lst)], lst), (l, t)
            assert np.all(rec["slot_idx"][l, t, len(lst):] == -1), (l, t)
    assert tuple(map(list, rec["sched"])) == denoise_schedule(words, FFE)
    assert rec["sched"][0] == ([0, 1, 0, 1] if q % 2 else [0, 1, 1, 1])


@pytest.mark.parametrize("q", range(CALLS))
def test_prefill_against_the_chosen_entry(calls, q):
    rec, k, vlm = calls["calls"][q], calls["k"], calls["vlm"]
    x_h, y_h, idx_h, xb_h, yb_h = rec["x"], rec["y"], rec["idx"], rec["xbar"], rec["ybar"]
    assert_close(O.decode(xb_h[0], "bf16"), O.rms_norm(O.decode(rec["entry"]["x"], "bf16")),
                 "rebuilt xbar_0 of the chosen slot", out="bf16")
    for l in range(L_VLM):
        idx_o, _ = O.ctx_select(x_h[l], xb_h[l], k)
        assert np.array_equal(idx_h[l], idx_o), f"call {q} layer {l}: selection"
        keep = np.ones(P, dtype=bool)
        keep[idx_o] = False
        assert np.array_equal(y_h[l][keep], yb_h[l][keep]), f"call {q} layer {l}: copied rows"
    assert np.array_equal(idx_h[0], rec["entry"]["changed"]), "layer 0 must select the planted tokens"
    for l in range(L_VLM):
        sample = idx_h[l][np.linspace(0, k - 1, 6).astype(int)]
        y_o = O.ffn_geglu(O.decode(x_h[l][sample], "bf16"), vlm[l])
        assert_close(O.decode(y_h[l][sample], "bf16"), y_o, f"call {q} layer {l}: recomputed rows", out="bf16")


@pytest.mark.parametrize("q", range(CALLS))
def test_denoise_driven_by_the_entry_masks(calls, q):
    rec, exp = calls["calls"][q], calls["exp"]
    kind, anchor, mask = denoise_schedule(rec["words"], FFE)
    x_h, y_h, y_anc, h_anc = rec["xch"], rec["ych"], rec["y_anc"], rec["h_anc"]
    r = calls["a0"].astype(np.float32).astype(np.float64) + calls["temb0"].astype(np.float32).astype(np.float64)
    assert_close(O.decode(x_h[0], "bf16"), O.rms_norm(r), "x_0", out="bf16")
    for t in range(STEPS):
        a = anchor[t]
        for l in range(L_EXP):
            i = t * L_EXP + l
            if kind[t] == 0:
                y_o, h_o = O.act_ffn_masked(exp[l], x_h[i], np.arange(FFE))
                assert_close(y_anc[a, l], y_o, f"call {q} anchor step {t} layer {l}: y_a")
                assert_close(h_anc[a, l], h_o, f"call {q} anchor step {t} layer {l}: h_a")
            else:
                m = O.mask_indices(rec["words"][l, mask[t]], FFE)
                y_o, _ = O.act_ffn_masked(exp[l], x_h[i], m, y_anc[a, l], h_anc[a, l])
            y = O.decode(y_h[i], "bf16")
            assert_close(y, y_o, f"call {q} step {t} layer {l}: y", out="bf16")
            r = r + y
            if l == L_EXP - 1:
                r = r + calls["dtemb"][t].astype(np.float32).astype(np.float64)
            assert_close(O.decode(x_h[i + 1], "bf16"), O.rms_norm(r), f"call {q} step {t} layer {l}: next input",
                         out="bf16")
