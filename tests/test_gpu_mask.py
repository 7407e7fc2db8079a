"""GPU parity of act_build_mask (rMuscle §3.4 Eq. 1, §5): mask words, index list
and count must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import ffn_weights, rng, synthetic_h_ref
from gpu_helpers import dev, ffn_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _gpu_mask(h, w, mode, K=0, cov=0.0):
    W = ffn_dev(w)
    m, idx, cnt = cgs.act_build_mask(to_dev(np.ascontiguousarray(h, dtype=np.float32), "f32"), W,
                                     mode, K=K, coverage=cov)
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint64), idx.cpu().numpy(), int(cnt.item())


def _check(h, w, mode, K=0, cov=0.0):
    gm, gi, gc = _gpu_mask(h, w, mode, K, cov)
    oi, om = O.act_build_mask(h, w, mode, K=K, coverage=cov)
    ff = w["ff"]
    assert gc == len(oi), f"count {gc} != {len(oi)}"
    assert np.array_equal(gi[:gc], oi), "mask indices differ"
    assert np.all(gi[gc:] == -1)
    assert np.array_equal(gm, om), "mask words differ"
    assert gm.size == (ff + 63) // 64
    return gc


def _setup(seed, T, ff, S, d, sigma=1.5, dtype="bf16"):
    w = ffn_weights(seed, 0, d, ff, dtype=dtype, down_layout="fd", down_lognormal_sigma=sigma)
    h = synthetic_h_ref(seed, 0, T, ff, S, neuron_sigma=0.5)
    return w, h


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("rho", [0.0, 0.001, 0.2, 0.3, 0.5, 1.0])
def test_topk_expert_size(T, rho):
    """Expert of 4096 neurons, d 1024, 50 action tokens, T reference steps."""
    say("mask topk", T, rho)
    w, h = _setup(20, T, 4096, 50, 1024)
    _check(h, w, "topk", K=O.ratio_to_count(rho, 4096))


@pytest.mark.parametrize("cov", [0.0, 0.3, 0.5, 0.844, 0.99, 1.0])
def test_coverage_expert_size(cov):
    say("mask coverage", cov)
    w, h = _setup(21, 4, 4096, 50, 1024)
    n = _check(h, w, "coverage", cov=cov)
    if cov == 0.844:
        say("  coverage 0.844 keeps", n, "of 4096")


@pytest.mark.parametrize("ff,d,S,T", [(1000, 128, 7, 3), (64, 128, 1, 1), (1, 128, 5, 2), (5000, 256, 33, 2)])
def test_ragged(ff, d, S, T):
    say("mask ragged", ff, d, S, T)
    w, h = _setup(22, T, ff, S, d)
    for K in sorted({0, 1, ff // 3, ff}):
        _check(h, w, "topk", K=K)
    for cov in (0.25, 0.844, 1.0):
        _check(h, w, "coverage", cov=cov)


def test_ties_and_zeros():
    """Duplicated neurons (equal scores) and all-zero activations."""
    say("mask ties")
    ff, d, S, T = 512, 128, 8, 2
    w, h = _setup(23, T, ff, S, d, sigma=0.0)
    g = rng(23, 0, "misc")
    src = g.integers(0, 16, ff)
    wd = w["w_down"].copy()
    wd[:] = wd[src]
    w = dict(w, w_down=wd)
    h = np.ascontiguousarray(h[:, src, :])
    for K in (1, 7, 32, 100, 511):
        _check(h, w, "topk", K=K)
    for cov in (0.1, 0.5, 0.9):
        _check(h, w, "coverage", cov=cov)
    hz = np.zeros_like(h)
    _check(hz, w, "topk", K=10)
    assert _check(hz, w, "coverage", cov=0.5) == 0


def test_fp32_weights():
    say("mask fp32")
    w, h = _setup(24, 2, 1024, 16, 256, dtype="f32")
    _check(h, w, "topk", K=256)
    _check(h, w, "coverage", cov=0.844)


@pytest.mark.parametrize("mode,ff,d,S,T", [("coverage", 4096, 1024, 50, 4), ("topk", 4096, 1024, 50, 4),
                                           ("coverage", 5000, 256, 10, 2), ("topk", 200, 128, 70, 3)])
def test_batched_layers_equal_single_layer_builds(mode, ff, d, S, T):
    """act_build_masks over several layers (one launch pair) gives every layer
    exactly what act_build_mask gives it, and the oracle's mask."""
    say("batched masks", mode, ff, d, S, T)
    layers = 5
    ws = [ffn_weights(50 + l, l, d, ff, down_layout="fd", down_lognormal_sigma=1.5) for l in range(layers)]
    hs = [synthetic_h_ref(50 + l, l, T, ff, S, neuron_sigma=0.5) for l in range(layers)]
    K, cov = (max(1, ff // 3), 0.0) if mode == "topk" else (0, 0.844)
    W = [ffn_dev(w) for w in ws]
    H = to_dev(np.ascontiguousarray(np.stack(hs), dtype=np.float32), "f32")
    m, idx, cnt = cgs.act_build_masks(H, W, mode, K=K, coverage=cov)
    torch.cuda.synchronize()
    m, idx, cnt = m.cpu().numpy().view(np.uint64), idx.cpu().numpy(), cnt.cpu().numpy()
    for l in range(layers):
        gm, gi, gc = _gpu_mask(hs[l], ws[l], mode, K, cov)
        assert cnt[l] == gc and np.array_equal(idx[l], gi) and np.array_equal(m[l], gm), f"layer {l}"
        oi, om = O.act_build_mask(hs[l], ws[l], mode, K=K, coverage=cov)
        assert np.array_equal(gi[:gc], oi) and np.array_equal(gm, om), f"layer {l} vs oracle"


@pytest.mark.parametrize("dtype,ff,d", [("bf16", 4096, 1024), ("bf16", 77, 100), ("f32", 300, 256)])
def test_down_norms_match_oracle(dtype, ff, d):
    """act_down_norms: Eq. 1's weight norms of every layer, bit for bit."""
    say("mask norms", dtype, ff, d)
    ws = [ffn_weights(120 + l, 0, d, ff, dtype=dtype, down_layout="fd", down_lognormal_sigma=1.5)
          for l in range(3)]
    nrm = cgs.act_down_norms([ffn_dev(w) for w in ws])
    torch.cuda.synchronize()
    got = nrm.cpu().numpy()
    for l, w in enumerate(ws):
        assert np.array_equal(got[l].view(np.uint64), O.down_weight_norms(w).view(np.uint64)), f"layer {l}"


@pytest.mark.parametrize("mode,K,cov,L,T,ff,S,d", [
    ("topk", 1229, 0.0, 4, 4, 4096, 50, 1024), ("coverage", 0, 0.844, 4, 4, 4096, 50, 1024),
    ("coverage", 0, 1.0, 4, 4, 4096, 50, 1024), ("topk", 20, 0.0, 3, 3, 77, 7, 100),
    ("coverage", 0, 0.5, 2, 2, 130, 100, 128), ("topk", 9, 0.0, 2, 9, 40, 5, 64)])
def test_masks_from_stored_norms_equal_masks_from_weights(mode, K, cov, L, T, ff, S, d):
    """act_build_masks_normed reads only h_ref: its masks, indices and counts
    equal the weight-based build's (and so the oracle's) bit for bit (ragged
    neuron counts; more than 64 tokens or 8 steps take the general kernel)."""
    say("mask normed", mode, K, cov, L, T, ff, S, d)
    ws = [ffn_weights(130 + l, 0, d, ff, down_layout="fd", down_lognormal_sigma=1.5) for l in range(L)]
    Ws = [ffn_dev(w) for w in ws]
    h = np.stack([synthetic_h_ref(130 + l, 0, T, ff, S, neuron_sigma=0.5) for l in range(L)])
    hd = to_dev(np.ascontiguousarray(h, dtype=np.float32), "f32")
    a = cgs.act_build_masks(hd, Ws, mode, K=K, coverage=cov)
    b = cgs.act_build_masks(hd, None, mode, K=K, coverage=cov, norms=cgs.act_down_norms(Ws))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for l in range(L):
        oi, om = O.act_build_mask(h[l], ws[l], mode, K=K, coverage=cov)
        c = int(b[2][l].item())
        assert c == len(oi) and np.array_equal(b[1][l, :c].cpu().numpy(), oi)
        assert np.array_equal(b[0][l].cpu().numpy().view(np.uint64), om)


@pytest.mark.parametrize("ff,n", [(4096, 72), (1, 3), (63, 5), (64, 4), (200, 9), (1000, 2), (65536, 3)])
def test_mask_indices_bit_exact(ff, n):
    """Stored masks read back as neuron lists (§5 keeps each entry's masks as
    bits): random words with every bit pattern, including bits past ff, an
    empty and a full mask; lists, -1 tails and counts equal the oracle's."""
    say("mask indices", ff, n)
    nw = (ff + 63) // 64
    g = rng(47, ff, "misc")
    words = g.integers(-(2 ** 63), 2 ** 63 - 1, size=(n, nw), dtype=np.int64, endpoint=True)
    dens = g.uniform(0.05, 0.95, size=n)
    keep = g.random((n, nw * 64)) < dens[:, None]            # varied densities
    packed = np.packbits(keep, axis=1, bitorder="little").view("<u8").view(np.int64)
    words = np.where(g.random((n, 1)) < 0.3, words, packed)   # some rows fully random
    words[0] = 0
    if n > 1:
        words[1] = -1                                         # every bit set, also past ff
    idx, cnt = cgs.act_mask_indices(torch.from_numpy(words).to(dev()), ff)
    torch.cuda.synchronize()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    for m in range(n):
        want = O.mask_indices(words[m], ff)
        assert cnt_h[m] == len(want), (m, cnt_h[m], len(want))
        assert np.array_equal(idx_h[m][: len(want)], want), m
        assert np.all(idx_h[m][len(want):] == -1), m
    assert cnt_h[0] == 0 and (n < 2 or cnt_h[1] == ff)


def test_mask_indices_read_back_a_built_mask():
    """The words act_build_masks writes come back as the list it wrote."""
    say("mask indices of built masks")
    L, T, S, ff, d = 4, 4, 50, 4096, 256
    ws = [ffn_weights(48, l, d, ff, down_layout="fd", down_lognormal_sigma=1.5) for l in range(L)]
    h = np.stack([synthetic_h_ref(48, l, T, ff, S) for l in range(L)]).astype(np.float32)
    words, idx, cnt = cgs.act_build_masks(to_dev(h, "f32"), [ffn_dev(w) for w in ws], "coverage", coverage=0.844)
    idx2, cnt2 = cgs.act_mask_indices(words, ff)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
