"""GPU parity of act_ffn_masked (rMuscle §4.1, Eq. 4) and of the dense anchor
step: outputs within 1e-2 x RMS of the oracle; anchors for the masked steps
come from the oracle's own dense run (float32), never from the GPU."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import act_tokens, ffn_weights, rng
from gpu_helpers import assert_close, assert_rne_of, bits, dev, ffn_dev, say, to_dev, values

pytestmark = pytest.mark.gpu


def _idx_dev(idx):
    return torch.from_numpy(np.asarray(idx, dtype=np.int32)).to(dev())


def _masked(w, x, idx, ya=None, ha=None, want_h=False):
    dt = w["dtype"]
    S, d = x.shape
    W = ffn_dev(w)
    yf = torch.empty(S, d, dtype=torch.float32, device=dev())
    h = torch.full((w["ff"], S), float("nan"), dtype=torch.float32, device=dev()) if want_h else None
    y = cgs.act_ffn_masked(W, to_dev(x, dt), _idx_dev(idx),
                           y_anchor=None if ya is None else to_dev(ya, "f32"),
                           h_anchor=None if ha is None else to_dev(ha, "f32"),
                           y_f32_out=yf, h_out=h)
    torch.cuda.synchronize()
    return y, yf, h


def _setup(seed, S, d, ff, dtype="bf16", sigma=1.0):
    w = ffn_weights(seed, 0, d, ff, dtype=dtype, down_layout="fd", down_lognormal_sigma=sigma)
    t = act_tokens(seed, 0, S, d, noise_sigma=0.33, dtype=dtype)
    return w, t["x"], t["x_pert"]


def _stored_is_rounding(y, yf, dtype):
    """The dtype output is the fp32 output rounded once (bf16: RNE; f32: equal)."""
    if dtype == "bf16":
        assert_rne_of(bits(y), values(yf), "y")
    else:
        assert torch.equal(y, yf)


@pytest.mark.parametrize("dtype,S,d,ff", [("f32", 16, 256, 1024), ("bf16", 16, 256, 1024),
                                          ("bf16", 50, 1024, 4096), ("bf16", 70, 128, 200),
                                          ("bf16", 16, 256, 2048), ("bf16", 64, 128, 4096),
                                          ("f32", 50, 256, 2048), ("bf16", 100, 256, 2048)])
def test_dense_anchor(dtype, S, d, ff):
    """Full mask, no anchors: the dense FFN, its fp32 output and every h row."""
    say("act dense anchor", dtype, S, d, ff)
    w, x, _ = _setup(10, S, d, ff, dtype)
    y, yf, h = _masked(w, x, np.arange(ff), want_h=True)
    y_o, h_o = O.act_ffn_masked(w, x, np.arange(ff))
    assert_close(values(yf), y_o, "y_f32")
    assert_close(values(y), y_o, "y", out=dtype)
    _stored_is_rounding(y, yf, dtype)
    assert_close(values(h), h_o, "h_out")


@pytest.mark.parametrize("dtype,S,d,ff,rho", [("f32", 16, 256, 1024, 0.25), ("f32", 16, 256, 1024, 1.0),
                                              ("bf16", 16, 256, 1024, 0.25), ("bf16", 50, 1024, 4096, 0.3),
                                              ("bf16", 50, 1024, 4096, 0.01), ("bf16", 70, 128, 200, 0.4),
                                              ("bf16", 50, 1024, 4096, 0.6), ("bf16", 50, 1024, 4096, 1.0),
                                              ("bf16", 100, 256, 2048, 1.0)])
def test_masked_with_anchor(dtype, S, d, ff, rho):
    say("act masked", dtype, S, d, ff, rho)
    w, x, xa = _setup(11, S, d, ff, dtype)
    ya, ha = O.act_ffn_masked(w, xa, np.arange(ff))
    ya32, ha32 = ya.astype(np.float32), ha.astype(np.float32)
    K = O.ratio_to_count(rho, ff)
    idx = np.sort(rng(11, K, "perm").permutation(ff)[:K]).astype(np.int32)
    y, yf, h = _masked(w, x, idx, ya32, ha32, want_h=True)
    y_o, h_o = O.act_ffn_masked(w, x, idx, ya32, ha32)
    assert_close(values(yf), y_o, "y_f32")
    assert_close(values(y), y_o, "y", out=dtype)
    _stored_is_rounding(y, yf, dtype)
    hv = values(h)
    assert_close(hv[idx], h_o, "h_out rows of the mask")
    untouched = np.ones(ff, dtype=bool)
    untouched[idx] = False
    assert np.all(np.isnan(hv[untouched])), "rows outside the mask were written"


def test_empty_mask_returns_anchor():
    say("act empty mask")
    w, x, xa = _setup(12, 50, 1024, 4096)
    ya, ha = O.act_ffn_masked(w, xa, np.arange(4096))
    ya32 = ya.astype(np.float32)
    y, yf, _ = _masked(w, x, np.zeros(0, dtype=np.int32), ya32, ha.astype(np.float32))
    assert np.array_equal(values(yf).astype(np.float32), ya32)
    assert np.array_equal(bits(y), O.round_to_bf16_bits(ya32.astype(np.float64)))
    y0, yf0, _ = _masked(w, x, np.zeros(0, dtype=np.int32))
    assert np.all(values(yf0) == 0) and np.all(values(y0) == 0)


def test_anchor_at_same_input_is_exact():
    """GPU anchor state at the same x: every mask gives back y_a exactly, because
    the masked h equals the anchor's h bit for bit (same kernel, same data)."""
    say("act same input")
    w, x, _ = _setup(13, 50, 1024, 4096)
    ff = 4096
    _, ya, ha = _masked(w, x, np.arange(ff), want_h=True)
    W = ffn_dev(w)
    idx = _idx_dev(np.arange(0, ff, 3))
    yf = torch.empty_like(ya)
    cgs.act_ffn_masked(W, to_dev(x), idx, y_anchor=ya, h_anchor=ha, y_f32_out=yf)
    torch.cuda.synchronize()
    assert torch.equal(yf, ya)


def test_deterministic_repeats():
    w, x, xa = _setup(14, 50, 1024, 4096)
    idx = np.arange(0, 4096, 3, dtype=np.int32)
    a = values(_masked(w, x, idx)[1])
    b = values(_masked(w, x, idx)[1])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("S,d,ff,rho", [(50, 1024, 4096, 0.3), (16, 256, 1024, 1.0)])
def test_fused_glue(S, d, ff, rho):
    """The finish kernel's residual/RMSNorm glue: r += bf16(y) + bias and
    x_next = RMSNorm(r), checked on the GPU's own y (teacher forcing) against
    the oracle's RMSNorm; y itself against the oracle's Eq. 4."""
    say("act glue", S, d, ff, rho)
    w, x, xa = _setup(15, S, d, ff)
    ya, ha = O.act_ffn_masked(w, xa, np.arange(ff))
    ya32, ha32 = ya.astype(np.float32), ha.astype(np.float32)
    K = O.ratio_to_count(rho, ff)
    idx = np.sort(rng(15, K, "perm").permutation(ff)[:K]).astype(np.int32)
    g = rng(15, 1, "misc")
    r0 = g.standard_normal((S, d)).astype(np.float32)
    bias = g.standard_normal(d).astype(np.float32)
    r = to_dev(r0, "f32")
    xn = torch.empty(S, d, dtype=torch.bfloat16, device=dev())
    y = cgs.act_ffn_masked(ffn_dev(w), to_dev(x), _idx_dev(idx), y_anchor=to_dev(ya32, "f32"),
                           h_anchor=to_dev(ha32, "f32"), glue=(r, to_dev(bias, "f32"), xn))
    torch.cuda.synchronize()
    y_o, _ = O.act_ffn_masked(w, x, idx, ya32, ha32)
    assert_close(values(y), y_o, "y", out="bf16")
    r_exp = r0.astype(np.float64) + values(y) + bias.astype(np.float64)
    assert_close(values(r), r_exp, "residual")
    assert_close(values(xn), O.rms_norm(r_exp), "x_next", out="bf16")
