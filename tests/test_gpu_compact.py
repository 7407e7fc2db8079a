"""GPU checks of the compact-weight variant of the Action Cache path (rMuscle
§4.1: a group's selected neuron weights prepared once into compact buffers and
reused by its masked steps; §5: gathered on a side stream).  act_gather_rows
must copy the mask's rows bit for bit; act_ffn_masked_compact must give
exactly the bits of act_ffn_masked on the full weights (same arithmetic, only
the weight addresses differ), which the oracle parity of act_ffn_masked
covers, and is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import act_tokens, ffn_weights, rng
from gpu_helpers import assert_close, bits, dev, ffn_dev, say, to_dev, values

pytestmark = pytest.mark.gpu


def _idx(ff, K, seed):
    return np.sort(rng(seed, K, "perm").permutation(ff)[:K]).astype(np.int32)


@pytest.mark.parametrize("dtype,d,ff,K", [("bf16", 1024, 4096, 1229), ("f32", 256, 1024, 256),
                                          ("bf16", 128, 200, 1), ("bf16", 128, 200, 200)])
def test_gather_rows_bit_exact(dtype, d, ff, K):
    say("gather rows", dtype, d, ff, K)
    w = ffn_weights(40, 0, d, ff, dtype=dtype, down_layout="fd")
    idx = _idx(ff, K, 40)
    wc = cgs.act_gather_rows(ffn_dev(w), torch.from_numpy(idx).to(dev()))
    torch.cuda.synchronize()
    for name, t in (("w_gate", wc.w_gate), ("w_up", wc.w_up), ("w_down", wc.w_down)):
        assert np.array_equal(bits(t), np.asarray(w[name])[idx]), name


@pytest.mark.parametrize("dtype,S,d,ff,rho", [("bf16", 50, 1024, 4096, 0.3), ("bf16", 16, 256, 1024, 1.0),
                                              ("bf16", 50, 1024, 4096, 0.6),
                                              ("f32", 16, 256, 1024, 0.25), ("bf16", 70, 128, 200, 0.4),
                                              ("bf16", 50, 1024, 4096, 0.01)])
def test_compact_equals_in_place_gather(dtype, S, d, ff, rho):
    say("compact vs in place", dtype, S, d, ff, rho)
    w = ffn_weights(41, 0, d, ff, dtype=dtype, down_layout="fd", down_lognormal_sigma=1.5)
    t = act_tokens(41, 0, S, d, noise_sigma=0.33, dtype=dtype)
    ya, ha = O.act_ffn_masked(w, t["x_pert"], np.arange(ff))
    ya32, ha32 = to_dev(ya.astype(np.float32), "f32"), to_dev(ha.astype(np.float32), "f32")
    K = O.ratio_to_count(rho, ff)
    idx_h = _idx(ff, K, 41)
    idx = torch.from_numpy(idx_h).to(dev())
    W = ffn_dev(w)
    x = to_dev(t["x"], dtype)
    outs = []
    for compact in (False, True):
        yf = torch.empty(S, d, dtype=torch.float32, device=dev())
        h = torch.full((ff, S), float("nan"), dtype=torch.float32, device=dev())
        r = to_dev(rng(41, 1, "misc").standard_normal((S, d)).astype(np.float32), "f32")
        xn = torch.empty_like(x)
        if compact:
            y = cgs.act_ffn_masked_compact(cgs.act_gather_rows(W, idx), x, idx, y_anchor=ya32, h_anchor=ha32,
                                           y_f32_out=yf, h_out=h, glue=(r, None, xn))
        else:
            y = cgs.act_ffn_masked(W, x, idx, y_anchor=ya32, h_anchor=ha32, y_f32_out=yf, h_out=h,
                                   glue=(r, None, xn))
        torch.cuda.synchronize()
        outs.append([y, yf, h, r, xn])
    for a, b, name in zip(outs[0], outs[1], ("y", "y_f32", "h_out", "r", "x_next")):
        assert np.array_equal(bits(a), bits(b), equal_nan=True) if name == "h_out" else torch.equal(a, b), name
    y_o, _ = O.act_ffn_masked(w, t["x"], idx_h, ya.astype(np.float32), ha.astype(np.float32))
    assert_close(values(outs[1][1]), y_o, "y_f32")


def test_compact_without_index_or_anchor():
    """No anchors, no h_out: idx may be NULL; a plain masked FFN of the compact rows."""
    say("compact no idx")
    S, d, ff, K = 50, 1024, 4096, 1000
    w = ffn_weights(42, 0, d, ff, down_layout="fd")
    x = to_dev(act_tokens(42, 0, S, d)["x"])
    idx_h = _idx(ff, K, 42)
    idx = torch.from_numpy(idx_h).to(dev())
    W = ffn_dev(w)
    y1 = cgs.act_ffn_masked(W, x, idx)
    y2 = cgs.act_ffn_masked_compact(cgs.act_gather_rows(W, idx), x, None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y_o, _ = O.act_ffn_masked(w, bits(x), idx_h)
    assert_close(values(y2), y_o, "y", out="bf16")


def test_compact_empty_mask():
    say("compact empty")
    S, d = 50, 1024
    ya = rng(43, 0, "misc").standard_normal((S, d)).astype(np.float32)
    wc = cgs.FFN(torch.empty(0, d, dtype=torch.bfloat16, device=dev()),
                 torch.empty(0, d, dtype=torch.bfloat16, device=dev()),
                 torch.empty(0, d, dtype=torch.bfloat16, device=dev()), "fd")
    x = to_dev(act_tokens(43, 0, S, d)["x"])
    y = cgs.act_ffn_masked_compact(wc, x, None, y_anchor=to_dev(ya, "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), O.round_to_bf16_bits(ya.astype(np.float64)))


def _joint_case(seed, S, d, ff, k, K):
    w = ffn_weights(seed, 0, d, ff, down_layout="fd", down_lognormal_sigma=1.5)
    t = act_tokens(seed, 0, S, d, noise_sigma=0.33)
    ya, ha = O.act_ffn_masked(w, t["x_pert"], np.arange(ff))
    tok = np.sort(rng(seed, 1, "perm").permutation(S)[:k]).astype(np.int32)
    idx = _idx(ff, K, seed)
    return w, t["x"], ya.astype(np.float32), ha.astype(np.float32), tok, idx


@pytest.mark.parametrize("S,d,ff,k,K", [(306, 1024, 4096, 127, 1229), (50, 1024, 4096, 50, 1229),
                                        (70, 128, 200, 33, 80), (40, 256, 1024, 1, 1024)])
def test_joint_token_and_neuron_sparsity(S, d, ff, k, K):
    """Eq. 4 on the selected rows, the anchor output elsewhere (oracle parity);
    all rows selected = act_ffn_masked_compact bit for bit."""
    say("joint", S, d, ff, k, K)
    w, x, ya, ha, tok, idx = _joint_case(44, S, d, ff, k, K)
    W = ffn_dev(w)
    idx_d = torch.from_numpy(idx).to(dev())
    wc = cgs.act_gather_rows(W, idx_d)
    yf = torch.empty(S, d, dtype=torch.float32, device=dev())
    y = cgs.act_ffn_joint(wc, to_dev(x), torch.from_numpy(tok).to(dev()), idx_d, to_dev(ya, "f32"),
                          to_dev(ha, "f32"), y_f32_out=yf)
    torch.cuda.synchronize()
    y_o = O.act_ffn_joint(w, x, tok, idx, ya, ha)
    assert_close(values(yf), y_o, "y_f32")
    assert_close(values(y), y_o, "y", out="bf16")
    rest = np.setdiff1d(np.arange(S), tok)
    assert np.array_equal(values(yf)[rest], ya[rest]), "unselected rows must keep the anchor output"
    if k == S:
        y2 = cgs.act_ffn_masked_compact(wc, to_dev(x), idx_d, y_anchor=to_dev(ya, "f32"), h_anchor=to_dev(ha, "f32"))
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


def test_joint_no_rows_and_glue():
    say("joint empty + glue")
    S, d, ff = 60, 1024, 4096
    w, x, ya, ha, _, idx = _joint_case(45, S, d, ff, 0, 1000)
    W = ffn_dev(w)
    idx_d = torch.from_numpy(idx).to(dev())
    wc = cgs.act_gather_rows(W, idx_d)
    y = cgs.act_ffn_joint(wc, to_dev(x), None, idx_d, to_dev(ya, "f32"), to_dev(ha, "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), O.round_to_bf16_bits(ya.astype(np.float64)))
    # glue over every row, selected or not
    tok = np.arange(0, S, 4, dtype=np.int32)
    r0 = rng(45, 2, "misc").standard_normal((S, d)).astype(np.float32)
    r = to_dev(r0, "f32")
    xn = torch.empty(S, d, dtype=torch.bfloat16, device=dev())
    y = cgs.act_ffn_joint(wc, to_dev(x), torch.from_numpy(tok).to(dev()), idx_d, to_dev(ya, "f32"),
                          to_dev(ha, "f32"), glue=(r, None, xn))
    torch.cuda.synchronize()
    r_exp = r0.astype(np.float64) + values(y)
    assert_close(values(r), r_exp, "residual")
    assert_close(values(xn), O.rms_norm(r_exp), "x_next", out="bf16")


@pytest.mark.parametrize("dtype,d,ff", [("bf16", 1024, 4096), ("f32", 256, 1024)])
def test_gather_rows_layers_bit_exact(dtype, d, ff):
    """All layers of a mask group gathered in one launch: every layer's rows
    are the weights' rows idx, bit for bit (a layer with an empty mask and one
    with every neuron included)."""
    say("gather rows layers", dtype, d, ff)
    Ks = [ff * 3 // 10, 0, 37, ff, 1]
    ws = [ffn_weights(43, l, d, ff, dtype=dtype, down_layout="fd") for l in range(len(Ks))]
    idxs = [_idx(ff, K, 43 + l) for l, K in enumerate(Ks)]
    W = [ffn_dev(w) for w in ws]
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    outs = [cgs.FFN(*(torch.full((K, d), 7, dtype=dt, device=dev()) for _ in range(3)), layout="fd") for K in Ks]
    cgs.act_gather_rows_layers(W, [torch.from_numpy(i).to(dev()) for i in idxs], outs)
    torch.cuda.synchronize()
    for l, (w, idx, out) in enumerate(zip(ws, idxs, outs)):
        for name, t in (("w_gate", out.w_gate), ("w_up", out.w_up), ("w_down", out.w_down)):
            assert np.array_equal(bits(t), np.asarray(w[name])[idx]), (l, name)
