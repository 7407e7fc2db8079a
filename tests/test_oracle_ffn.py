"""Pins of the oracle's FFN arithmetic: GeGLU FFN, selective recompute (rMuscle §4.1
Eq. 3), masked anchor update (Eq. 4) and the dense rebuild (§4.2).

Independent references: torch CPU library routines (gelu tanh, linear,
rms_norm, bf16 casting), the pages' entry size, and algebraic identities of
Eq. 3 / Eq. 4.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from cgs_inputs import act_tokens, ffn_weights, f32_to_bf16_bits, random_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _torch_bf16(v64: torch.Tensor) -> torch.Tensor:
    # fp64 -> fp32 -> bf16 (torch's cast path); may differ from a single rounding in
    # rare double-rounding cases, which only moves a result by one bf16 ulp.
    return v64.float().bfloat16().double()


def _torch_ffn(x64, w, act_bf16=True):
    """Independent GeGLU FFN with torch CPU routines (fp64)."""
    dt = w["dtype"]
    wg = _t(O.decode(w["w_gate"], dt))
    wu = _t(O.decode(w["w_up"], dt))
    wd = _t(O.decode(w["w_down"], dt))
    if w["down_layout"] == "fd":
        wd = wd.T.contiguous()            # nn.Linear weight layout [out][in] = [d][ff]
    h = F.gelu(F.linear(_t(x64), wg), approximate="tanh") * F.linear(_t(x64), wu)
    if act_bf16:
        h = _torch_bf16(h)
    return F.linear(h, wd).numpy()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 3,
                        rng.standard_normal(2000) * 1e-38,          # bf16 subnormals
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38]]).astype(np.float32)
    ours = O.round_to_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # exact ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert O.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert O.round_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_gelu_matches_torch():
    g = np.linspace(-8, 8, 4001)
    ref = F.gelu(_t(g), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(g), ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("dtype,layout", [("bf16", "df"), ("bf16", "fd"), ("f32", "df")])
def test_ffn_matches_torch(dtype, layout):
    d, ff, M = 64, 256, 12
    w = ffn_weights(11, 0, d, ff, dtype=dtype, down_layout=layout)
    x = random_bf16(11, 0, "x", (M, d), dtype=dtype)
    x64 = O.decode(x, dtype)
    ours = O.ffn_geglu(x64, w)
    ref = _torch_ffn(x64, w, act_bf16=(dtype == "bf16"))
    scale = np.sqrt(np.mean(ref ** 2))
    # identical up to rare one-ulp double-rounding differences of h
    assert np.max(np.abs(ours - ref)) <= 2e-3 * scale


def test_recompute_ratio_extremes():
    """100% token ratio = dense FFN on every row; 0% returns the cached bits."""
    d, ff, P = 32, 128, 10
    w = ffn_weights(2, 0, d, ff)
    x = random_bf16(2, 0, "x", (P, d))
    y_ref = random_bf16(2, 0, "y_ref", (P, d))
    y, rec = O.ctx_ffn_recompute(w, x, y_ref, np.arange(P))
    assert rec.all()
    np.testing.assert_array_equal(y, O.ffn_geglu(O.decode(x, "bf16"), w))
    ref = _torch_ffn(O.decode(x, "bf16"), w)
    assert np.max(np.abs(y - ref)) <= 2e-3 * np.sqrt(np.mean(ref ** 2))
    y0, rec0 = O.ctx_ffn_recompute(w, x, y_ref, np.zeros(0, dtype=np.int32))
    assert not rec0.any()
    assert np.array_equal(O.round_to_bf16_bits(y0), y_ref)


def test_recompute_mixes_rows():
    """Eq. 3 row by row: selected rows are F(x_p), the others ybar_p."""
    d, ff, P = 32, 128, 9
    w = ffn_weights(3, 0, d, ff)
    x = random_bf16(3, 0, "x", (P, d))
    y_ref = random_bf16(3, 0, "y_ref", (P, d))
    idx = np.array([1, 4, 8], dtype=np.int32)
    y, rec = O.ctx_ffn_recompute(w, x, y_ref, idx)
    dense = _torch_ffn(O.decode(x, "bf16"), w)
    for p in range(P):
        if p in idx:
            assert rec[p]
            np.testing.assert_allclose(y[p], dense[p], rtol=0, atol=2e-3 * np.abs(dense).max())
        else:
            assert not rec[p] and np.array_equal(O.round_to_bf16_bits(y[p]), y_ref[p])
    with pytest.raises(ValueError):
        O.ctx_ffn_recompute(w, x, y_ref, np.array([4, 1]))


# ----------------------------------------------------------------------------
# Eq. 4
# ----------------------------------------------------------------------------
def _act_setup(seed=4, d=64, ff=256, S=8, dtype="bf16"):
    w = ffn_weights(seed, 0, d, ff, dtype=dtype, down_layout="fd")
    t = act_tokens(seed, 0, S, d, noise_sigma=0.3, dtype=dtype)
    return w, t["x"], t["x_pert"]


def test_full_mask_no_anchor_is_dense():
    w, x, _ = _act_setup()
    ff = w["ff"]
    y, h = O.act_ffn_masked(w, x, np.arange(ff))
    ref = _torch_ffn(O.decode(x, "bf16"), w)
    assert np.max(np.abs(y - ref)) <= 2e-3 * np.sqrt(np.mean(ref ** 2))
    assert h.shape == (ff, x.shape[0])


def test_empty_mask_returns_anchor():
    w, x, xp = _act_setup()
    ff = w["ff"]
    ya, ha = O.act_ffn_masked(w, xp, np.arange(ff))
    ya32, ha32 = ya.astype(np.float32), ha.astype(np.float32)
    y, h = O.act_ffn_masked(w, x, np.zeros(0, dtype=np.int32), ya32, ha32)
    assert np.array_equal(y, ya32.astype(np.float64)) and h.shape == (0, x.shape[0])
    y0, _ = O.act_ffn_masked(w, x, np.zeros(0, dtype=np.int32))
    assert np.all(y0 == 0)


def test_anchor_at_same_input_returns_anchor():
    """Eq. 4 with the anchor taken at the same x: the delta vanishes for any mask."""
    w, x, _ = _act_setup()
    ff = w["ff"]
    ya, ha = O.act_ffn_masked(w, x, np.arange(ff))
    idx = np.arange(0, ff, 3)
    y, _ = O.act_ffn_masked(w, x, idx, ya.astype(np.float32), ha.astype(np.float32))
    # only the float32 storage residue of h_a can enter
    assert np.max(np.abs(y - ya.astype(np.float32))) <= 1e-5 * np.abs(ya).max()


def test_full_mask_with_anchor_is_dense_at_new_input():
    """y_a + (h_t - h_a) W_down over all neurons = F(x_t), up to bf16 delta rounding."""
    w, x, xp = _act_setup()
    ff = w["ff"]
    ya, ha = O.act_ffn_masked(w, xp, np.arange(ff))
    y, _ = O.act_ffn_masked(w, x, np.arange(ff), ya.astype(np.float32), ha.astype(np.float32))
    ref = _torch_ffn(O.decode(x, "bf16"), w, act_bf16=False)
    assert np.max(np.abs(y - ref)) <= 1e-2 * np.sqrt(np.mean(ref ** 2))


def test_eq4_splits_over_disjoint_masks():
    """The update is a sum over neurons: disjoint masks add (catches index mix-ups)."""
    w, x, xp = _act_setup()
    ff = w["ff"]
    ya, ha = O.act_ffn_masked(w, xp, np.arange(ff))
    ya32, ha32 = ya.astype(np.float32), ha.astype(np.float32)
    rng = np.random.default_rng(9)
    perm = rng.permutation(ff)
    m1, m2 = np.sort(perm[:70]), np.sort(perm[70:150])
    y1, h1 = O.act_ffn_masked(w, x, m1, ya32, ha32)
    y2, h2 = O.act_ffn_masked(w, x, m2, ya32, ha32)
    y12, h12 = O.act_ffn_masked(w, x, np.sort(np.concatenate([m1, m2])), ya32, ha32)
    np.testing.assert_allclose(y12 - ya32, (y1 - ya32) + (y2 - ya32), rtol=0, atol=1e-10)
    # h rows follow the mask's neuron ids
    _, hall = O.act_ffn_masked(w, x, np.arange(ff))
    np.testing.assert_allclose(h1, hall[m1], rtol=1e-12, atol=1e-14)


def test_masked_rows_only():
    """Zeroing every unmasked weight row leaves the masked FFN unchanged."""
    w, x, _ = _act_setup()
    ff = w["ff"]
    idx = np.arange(5, ff, 7)
    y, _ = O.act_ffn_masked(w, x, idx)
    w2 = dict(w)
    keep = np.zeros(ff, dtype=bool)
    keep[idx] = True
    for key in ("w_gate", "w_up", "w_down"):
        a = w[key].copy()
        a[~keep] = 0
        w2[key] = a
    ref = _torch_ffn(O.decode(x, "bf16"), w2)
    assert np.max(np.abs(y - ref)) <= 2e-3 * np.sqrt(np.mean(ref ** 2))


# ----------------------------------------------------------------------------
# Rebuild
# ----------------------------------------------------------------------------
def test_rms_norm_matches_torch():
    r = np.random.default_rng(1).standard_normal((7, 96)) * 3
    ref = F.rms_norm(_t(r), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(r), ref, rtol=1e-13)


def test_rebuild_chain_matches_torch():
    d, ff, P, L = 64, 192, 16, 3
    layers = [ffn_weights(20, l, d, ff) for l in range(L)]
    r0 = random_bf16(20, 0, "r0", (P, d), std=2.0)
    xb, yb = O.rebuild_dense(layers, r0)
    assert xb.shape == (L, P, d) and xb.dtype == np.uint16 and yb.shape == (L, P, d)
    r = _t(O.decode(r0, "bf16"))
    for l, w in enumerate(layers):
        xn = _torch_bf16(F.rms_norm(r, (d,), eps=1e-6))
        y = torch.from_numpy(_torch_ffn(xn.numpy(), w))
        assert np.max(np.abs(O.decode(xb[l], "bf16") - xn.numpy())) <= 1e-2 * xn.abs().max().item()
        assert np.max(np.abs(yb[l] - y.numpy())) <= 1e-2 * y.pow(2).mean().sqrt().item()
        r = r + _torch_bf16(y)


def test_rebuild_one_layer_is_dense_ffn():
    d, ff, P = 32, 64, 5
    w = ffn_weights(21, 0, d, ff)
    r0 = random_bf16(21, 0, "r0", (P, d))
    xb, yb = O.rebuild_dense([w], r0)
    np.testing.assert_array_equal(yb[0], O.ffn_geglu(O.decode(xb[0], "bf16"), w))


def test_entry_size_matches_pages():
    g = json.load(open(os.path.join(GOLD, "page_constants.json")))["entry"]
    b = O.entry_bytes(g["layers"], g["tokens"], g["d"], g["elem_bytes"])
    assert b == 106_954_752
    assert round(b / 1e6) == g["approx_mb_per_call"]
    assert round(b * g["calls"] / 1e9, 2) == g["approx_gb_per_40_calls"]
