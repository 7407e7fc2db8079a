"""GPU parity at the documented size limits of the selection and mask entry
points (include/cgs.h): token selection over P = 65536 tokens (and d = 4096),
top-k of stored keys over P = 65536, group masks over ff = 65536 neurons and
S·T = 2^14 activations per neuron.  Indices, keys and masks are compared with
the oracle bit for bit; the shapes are chosen small in the other dimensions
so that the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import ctx_layer_inputs, ffn_weights, rng, synthetic_h_ref
from gpu_helpers import dev, ffn_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _select(x, xr, k, kind="rel_rms"):
    P = x.shape[0]
    keys = torch.empty(P, dtype=torch.float64, device=dev())
    idx = cgs.ctx_select(to_dev(x), to_dev(xr), k, kind=kind, key_out=keys)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), keys.cpu().numpy()


@pytest.mark.parametrize("kind", ["rel_rms", "cosine"])
def test_select_max_tokens(kind):
    say("limits: select P = 65536", kind)
    P, d = 65536, 16
    inp = ctx_layer_inputs(80, 0, P, d, P // 8, 1.0, 0.05)
    for k in (1, 21846, P - 1, P):
        gi, gk = _select(inp["x"], inp["x_ref"], k, kind)
        oi, ok = O.ctx_select(inp["x"], inp["x_ref"], k, kind=kind)
        assert np.array_equal(gk.view(np.uint64), ok.view(np.uint64)), f"keys differ (k {k})"
        assert np.array_equal(gi, oi), f"indices differ (k {k})"


def test_select_max_width():
    say("limits: select d = 4096")
    P, d = 300, 4096
    inp = ctx_layer_inputs(81, 0, P, d, 90, 1.0, 0.1)
    gi, gk = _select(inp["x"], inp["x_ref"], 90)
    oi, ok = O.ctx_select(inp["x"], inp["x_ref"], 90)
    assert np.array_equal(gk.view(np.uint64), ok.view(np.uint64))
    assert np.array_equal(gi, oi)


def test_select_from_keys_max_tokens():
    say("limits: top-k of keys P = 65536")
    P = 65536
    keys = np.round(rng(82, 0, "misc").standard_normal(P), 2) + 0.0  # many ties
    kt = torch.from_numpy(keys).to(dev())
    for k in (1, 4097, P // 2, P):
        idx = cgs.ctx_select_from_keys(kt, k)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), O.topk_ascending(keys, k)), f"k {k}"


@pytest.mark.parametrize("mode,K,cov", [("topk", 1, 0.0), ("topk", 32768, 0.0), ("topk", 65536, 0.0),
                                        ("coverage", 0, 0.5), ("coverage", 0, 0.844)])
def test_mask_max_neurons(mode, K, cov):
    say("limits: mask ff = 65536", mode, K, cov)
    T, ff, S, d = 2, 65536, 8, 128
    w = ffn_weights(83, 0, d, ff, down_layout="fd", down_lognormal_sigma=1.0)
    h = synthetic_h_ref(83, 0, T, ff, S, neuron_sigma=0.5)
    W = ffn_dev(w)
    m, idx, cnt = cgs.act_build_mask(to_dev(h, "f32"), W, mode, K=K, coverage=cov)
    torch.cuda.synchronize()
    oi, om = O.act_build_mask(h, w, mode, K=K, coverage=cov)
    c = int(cnt.item())
    assert c == len(oi)
    assert np.array_equal(idx.cpu().numpy()[:c], oi)
    assert np.array_equal(m.cpu().numpy().view(np.uint64), om)


def test_mask_max_activations_per_neuron():
    """S·T = 2^14 activations per neuron (the fixed-point bound of the
    contribution sums), through the general (non-register) load path."""
    say("limits: mask S*T = 2^14")
    T, ff, S, d = 16, 128, 1024, 128
    w = ffn_weights(84, 0, d, ff, down_layout="fd", down_lognormal_sigma=1.0)
    h = synthetic_h_ref(84, 0, T, ff, S, neuron_sigma=0.5)
    W = ffn_dev(w)
    for mode, K, cov in (("topk", 40, 0.0), ("coverage", 0, 0.844)):
        m, idx, cnt = cgs.act_build_mask(to_dev(h, "f32"), W, mode, K=K, coverage=cov)
        torch.cuda.synchronize()
        oi, om = O.act_build_mask(h, w, mode, K=K, coverage=cov)
        c = int(cnt.item())
        assert c == len(oi) and np.array_equal(idx.cpu().numpy()[:c], oi)
        assert np.array_equal(m.cpu().numpy().view(np.uint64), om)


@pytest.mark.parametrize("T,ff,S,d", [(2, 65536, 8, 128), (16, 128, 1024, 128)])
def test_masks_from_stored_norms_at_the_limits(T, ff, S, d):
    """act_build_masks_normed at ff = 65536 and at S*T = 2^14 (the general
    kernel path): bit for bit the weight-based build."""
    say("limits: normed masks", T, ff, S, d)
    w = ffn_weights(85, 0, d, ff, down_layout="fd", down_lognormal_sigma=1.0)
    W = ffn_dev(w)
    h = to_dev(synthetic_h_ref(85, 0, T, ff, S, neuron_sigma=0.5), "f32")[None]
    nrm = cgs.act_down_norms([W])
    for mode, K, cov in (("topk", ff // 3, 0.0), ("coverage", 0, 0.844)):
        a = cgs.act_build_masks(h, [W], mode, K=K, coverage=cov)
        b = cgs.act_build_masks(h, None, mode, K=K, coverage=cov, norms=nrm)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), mode
