"""Per-launch kernel timing (cgs_profile_*): eager launches are bracketed
once per site; launches captured into a HIP graph are not recorded, and nor
are the graph's replays; overflow of the launch buffer is reported."""
import pytest
import torch

import cache_guided_sparse_amd as cgs
from cgs_inputs import ctx_layer_inputs, ffn_weights, random_bf16
from gpu_helpers import dev, ffn_dev, say, to_dev

pytestmark = pytest.mark.gpu

SITES = ("ctx.score", "ctx.topk", "ctx.glu", "ctx.down", "ctx.finish")


def _layer():
    P, d, ff, k = 128, 256, 1024, 40
    inp = ctx_layer_inputs(90, 0, P, d, k, 1.0, 0.05)
    W = ffn_dev(ffn_weights(90, 0, d, ff))
    x, xr, yr = to_dev(inp["x"]), to_dev(inp["x_ref"]), to_dev(random_bf16(90, 0, "y_ref", (P, d)))
    idx = torch.empty(k, dtype=torch.int32, device=dev())
    y = torch.empty_like(yr)

    def run():
        cgs.ctx_select(x, xr, k, idx_out=idx)
        cgs.ctx_ffn_recompute(W, x, yr, idx, y_out=y)
    return run


def test_eager_launches_counted_captured_ones_not():
    say("profile eager vs captured")
    run = _layer()
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cgs.profile_start("ctx.", 64)
    try:
        run()
        with torch.cuda.graph(g):
            run()
        g.replay()
        g.replay()
        run()
        torch.cuda.synchronize()
    finally:
        cgs.profile_stop()
    for site in SITES:
        ms, n = cgs.profile_result(site)
        assert n == 2, (site, n)
        assert ms > 0.0
    ms, n = cgs.profile_result()
    assert n == 2 * len(SITES)


def test_filter_and_overflow():
    say("profile filter and overflow")
    run = _layer()
    cgs.profile_start("ctx.glu", 64)
    try:
        run()
        run()
        torch.cuda.synchronize()
    finally:
        cgs.profile_stop()
    assert cgs.profile_result()[1] == 2
    assert cgs.profile_result("ctx.down")[1] == 0
    cgs.profile_start("ctx.", 3)
    try:
        run()
        torch.cuda.synchronize()
    finally:
        cgs.profile_stop()
    with pytest.raises(cgs.CgsError) as e:
        cgs.profile_result()
    assert e.value.status == 2  # CGS_ERR_SHAPE: launches beyond the buffer were dropped
