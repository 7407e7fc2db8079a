"""Checked mode (cgs_set_validate): entry points verify their documented
device-data preconditions and return CGS_ERR_DATA before launching anything.
Every bad input here stays inside its allocation (an out-of-range index
points into padding rows of the buffer), so the calls would be memory-safe
even unchecked.  Valid inputs give the same results checked and unchecked."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
from cgs_inputs import act_tokens, ctx_layer_inputs, ffn_weights, random_bf16, rng, synthetic_h_ref
from gpu_helpers import dev, ffn_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def checked():
    prev = cgs.set_validate(True)
    try:
        yield
    finally:
        cgs.set_validate(prev)
        cgs.set_validate(False)


def _i32(a):
    return torch.tensor(a, dtype=torch.int32, device=dev())


def _data_error(fn):
    with pytest.raises(cgs.CgsError) as e:
        fn()
    assert e.value.status == cgs.CGS_ERR_DATA, str(e.value)


def test_set_validate_returns_previous_setting():
    prev = cgs.set_validate(True)
    try:
        assert cgs.set_validate(True) is True
        assert cgs.set_validate(False) is True
        assert cgs.set_validate(False) is False
    finally:
        cgs.set_validate(prev)


def test_ctx_index_lists(checked):
    say("validate ctx indices")
    P, pad, d, ff = 64, 8, 256, 512
    W = ffn_dev(ffn_weights(70, 0, d, ff))
    # padding rows on both sides: indices -1 and P still address rows of the buffer
    xb = to_dev(random_bf16(70, 0, "x", (P + 2 * pad, d)))
    yb = to_dev(random_bf16(70, 0, "y_ref", (P + 2 * pad, d)))
    x, y_ref = xb[pad:pad + P], yb[pad:pad + P]
    good = _i32([1, 5, 9, 40])
    y_checked = cgs.ctx_ffn_recompute(W, x, y_ref, good)
    cgs.set_validate(False)
    y_plain = cgs.ctx_ffn_recompute(W, x, y_ref, good)
    cgs.set_validate(True)
    torch.cuda.synchronize()
    assert torch.equal(y_checked, y_plain)
    for bad in ([5, 1, 9, 40], [1, 5, 5, 40], [1, 5, 9, P], [-1, 5, 9, 40]):
        _data_error(lambda: cgs.ctx_ffn_recompute(W, x, y_ref, _i32(bad)))


def test_ctx_value_ranges(checked):
    say("validate ctx ranges")
    P, d = 32, 256
    inp = ctx_layer_inputs(71, 0, P, d, 8, 1.0, 0.02)
    x, xr = to_dev(inp["x"]), to_dev(inp["x_ref"])
    cgs.ctx_select(x, xr, 8)
    big = x.clone()
    big[3, 7] = 5000.0
    _data_error(lambda: cgs.ctx_select(big, xr, 8))
    keys = torch.rand(P, dtype=torch.float64, device=dev())
    cgs.ctx_select_from_keys(keys, 8)
    keys[5] = float("nan")
    _data_error(lambda: cgs.ctx_select_from_keys(keys, 8))


def test_act_index_lists(checked):
    say("validate act indices")
    S, d, ff = 16, 256, 1024
    w = ffn_weights(72, 0, d, ff, down_layout="fd")
    W = ffn_dev(w)
    x = to_dev(act_tokens(72, 0, S, d)["x"])
    good = _i32(list(range(0, ff, 7)))
    cgs.act_ffn_masked(W, x, good)
    cw = cgs.act_gather_rows(W, good)
    cgs.act_ffn_masked_compact(cw, x, good)
    _data_error(lambda: cgs.act_ffn_masked(W, x, _i32([3, 3, 9])))
    _data_error(lambda: cgs.act_ffn_masked(W, x, _i32([9, 3])))
    _data_error(lambda: cgs.act_gather_rows(W, _i32([9, 3])))
    # joint mode: token rows must ascend too
    ya = torch.zeros(S, d, dtype=torch.float32, device=dev())
    ha = torch.zeros(ff, S, dtype=torch.float32, device=dev())
    cgs.act_ffn_joint(cw, x, _i32([0, 2, 5]), good, ya, ha)
    _data_error(lambda: cgs.act_ffn_joint(cw, x, _i32([2, 0, 5]), good, ya, ha))
    torch.cuda.synchronize()


def test_mask_value_ranges(checked):
    say("validate mask ranges")
    T, ff, S, d = 2, 256, 8, 128
    w = ffn_weights(73, 0, d, ff, down_layout="fd")
    W = ffn_dev(w)
    h = to_dev(synthetic_h_ref(73, 0, T, ff, S), "f32")
    cgs.act_build_mask(h, W, "topk", K=32)
    hb = h.clone()
    hb[1, 5, 3] = float(2 ** 24)
    _data_error(lambda: cgs.act_build_mask(hb, W, "topk", K=32))
    wd = W.w_down.clone()
    wd[7, 11] = 40.0
    Wb = cgs.FFN(W.w_gate, W.w_up, wd, "fd")
    _data_error(lambda: cgs.act_build_mask(h, Wb, "coverage", coverage=0.5))
    torch.cuda.synchronize()


def test_stored_norms_must_be_finite_and_non_negative(checked):
    say("validate norms")
    T, ff, S, d = 2, 256, 8, 128
    W = ffn_dev(ffn_weights(74, 0, d, ff, down_layout="fd"))
    h = to_dev(synthetic_h_ref(74, 0, T, ff, S), "f32")[None]
    nrm = cgs.act_down_norms([W])
    cgs.act_build_masks(h, None, "topk", K=32, norms=nrm)
    bad = nrm.clone()
    bad[0, 9] = -1.0
    _data_error(lambda: cgs.act_build_masks(h, None, "topk", K=32, norms=bad))
    bad[0, 9] = float("inf")
    _data_error(lambda: cgs.act_build_masks(h, None, "topk", K=32, norms=bad))
    torch.cuda.synchronize()


def test_checked_call_refused_under_graph_capture(checked):
    """A checked call reads its verdict back to the host, which a stream under
    graph capture cannot do: it refuses (CGS_ERR_UNSUPPORTED) before enqueuing
    anything, and the capture stays valid (the graph replays what else was
    captured)."""
    say("validate under capture")
    keys = torch.arange(64, dtype=torch.float64, device=dev())
    idx = torch.zeros(8, dtype=torch.int32, device=dev())
    out = torch.zeros(4, device=dev())
    cgs.ctx_select_from_keys(keys, 8, idx_out=idx)  # checked, outside capture: fine
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == list(range(56, 64))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out.add_(1.0)
            with pytest.raises(cgs.CgsError) as e:
                cgs.ctx_select_from_keys(keys, 8, idx_out=idx)
            assert e.value.status == cgs.CGS_ERR_UNSUPPORTED, str(e.value)
    g.replay()
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [1.0] * 4
