"""The no-allocation variant of the compact masked update (rMuscle §4.1, Eq. 4
on a mask's compact weights), for callers that cannot allocate device memory.
act_ffn_masked_compact_noalloc keeps its intermediates in the library's
per-GPU scratch array instead of a caller workspace; its outputs must be the
bits of act_ffn_masked_compact on the same inputs, and within the parity
tolerance of the oracle.  Calls follow each other with shrinking inputs, so
anything the scratch kept from a larger call would show."""
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


def _case(seed, S, d, ff, K, dtype="bf16"):
    w = ffn_weights(seed, 0, d, ff, dtype=dtype, down_layout="fd", down_lognormal_sigma=1.5)
    t = act_tokens(seed, 0, S, d, noise_sigma=0.33, dtype=dtype)
    ya, ha = O.act_ffn_masked(w, t["x_pert"], np.arange(ff))
    idx_h = _idx(ff, K, seed)
    return w, t, ya.astype(np.float32), ha.astype(np.float32), idx_h


def _run(fn, wc, x, idx, ya, ha, S, d, ff, seed):
    y = torch.empty_like(x)
    yf = torch.empty(S, d, dtype=torch.float32, device=dev())
    h = torch.full((ff, S), float("nan"), dtype=torch.float32, device=dev())
    r = to_dev(rng(seed, 1, "misc").standard_normal((S, d)).astype(np.float32), "f32")
    xn = torch.empty_like(x)
    fn(wc, x, idx, y, ya, ha, yf, h, (r, None, xn))
    torch.cuda.synchronize()
    return [y, yf, h, r, xn]


def _with_ws(wc, x, idx, y, ya, ha, yf, h, glue):
    cgs.act_ffn_masked_compact(wc, x, idx, y_anchor=ya, h_anchor=ha, y_out=y, y_f32_out=yf, h_out=h, glue=glue)


def _no_alloc(wc, x, idx, y, ya, ha, yf, h, glue):
    cgs.act_ffn_masked_compact_noalloc(wc, x, idx, y, y_anchor=ya, h_anchor=ha, y_f32_out=yf, h_out=h, glue=glue)


# the largest call the scratch holds (64 tokens, a dense-size 4096-neuron
# mask), then the 18-layer expert's 50-token step with a 0.3 mask, then a
# ragged small one
SHAPES = [(70, 64, 1024, 4096, 4096), (71, 50, 1024, 4096, 1229), (72, 5, 256, 1024, 37)]


def test_no_alloc_matches_the_workspace_entry_point_on_successive_calls():
    for seed, S, d, ff, K in SHAPES:
        say("no-alloc", seed, S, d, ff, K)
        w, t, ya, ha, idx_h = _case(seed, S, d, ff, K)
        W = ffn_dev(w)
        idx = torch.from_numpy(idx_h).to(dev())
        wc = cgs.act_gather_rows(W, idx)
        x = to_dev(t["x"])
        ya_d, ha_d = to_dev(ya, "f32"), to_dev(ha, "f32")
        ref = _run(_with_ws, wc, x, idx, ya_d, ha_d, S, d, ff, seed)
        got = _run(_no_alloc, wc, x, idx, ya_d, ha_d, S, d, ff, seed)
        for a, b, name in zip(ref, got, ("y", "y_f32", "h_out", "r", "x_next")):
            assert np.array_equal(bits(a), bits(b), equal_nan=True), (seed, name)
        y_o, _ = O.act_ffn_masked(w, t["x"], idx_h, ya, ha)
        assert_close(values(got[1]), y_o, "y_f32")
        assert_close(values(got[0]), y_o, "y", out="bf16")


def test_no_alloc_refuses_masks_past_the_scratch():
    S, d, ff = 64, 1024, 16384
    assert cgs.lib().cgs_act_ffn_masked_workspace(S, ff, d, ff) > cgs.NOALLOC_SCRATCH_BYTES
    shape = (ff, d)
    wc = cgs.FFN(*(torch.zeros(shape, dtype=torch.bfloat16, device=dev()) for _ in range(3)), layout="fd")
    x = torch.zeros(S, d, dtype=torch.bfloat16, device=dev())
    with pytest.raises(cgs.CgsError, match="workspace"):
        cgs.act_ffn_masked_compact_noalloc(wc, x, None, torch.empty_like(x))
