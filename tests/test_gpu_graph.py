"""HIP-graph capture of the library's layer chains (as the benchmark runs them):
every replay, with eager work and synchronisations in between, must reproduce
the eager run bit for bit.  The eager run itself is checked against the oracle
by the other GPU tests; here the graph path is compared with it."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
from cgs_inputs import act_tokens, ctx_layer_inputs, ffn_weights, random_bf16
from gpu_helpers import dev, ffn_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _replays_match(run, reset, outputs, replays=3):
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(replays):
        reset()
        # unrelated eager work between replays
        junk = torch.randn(1 << 16, device=dev()).sum()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager run"
        assert torch.isfinite(junk)


def test_act_masked_chain_graph():
    say("graph act chain")
    S, d, ff, L = 50, 1024, 4096, 3
    ws = [ffn_weights(30, l, d, ff, down_layout="fd", down_lognormal_sigma=1.5) for l in range(L)]
    W = [ffn_dev(w) for w in ws]
    a0 = to_dev(act_tokens(30, 0, S, d)["x"])
    r = torch.empty(S, d, dtype=torch.float32, device=dev())
    x = torch.empty(S, d, dtype=torch.bfloat16, device=dev())
    y = torch.empty_like(x)
    ya = torch.empty(L, S, d, dtype=torch.float32, device=dev())
    ha = torch.empty(L, ff, S, dtype=torch.float32, device=dev())
    full = torch.arange(ff, dtype=torch.int32, device=dev())
    mask = torch.arange(0, ff, 3, dtype=torch.int32, device=dev())
    bias = torch.linspace(-1, 1, d, device=dev())

    def reset():
        cgs.residual_rmsnorm(r, r_in=a0.float().contiguous(), x_out=x)

    reset()
    for l in range(L):  # anchors (eager, outside the graph)
        cgs.act_ffn_masked(W[l], x, full, y_out=y, y_f32_out=ya[l], h_out=ha[l], glue=(r, None, x))

    def run():
        for l in range(L):
            cgs.act_ffn_masked(W[l], x, mask, y_anchor=ya[l], h_anchor=ha[l], y_out=y,
                               glue=(r, bias if l == L - 1 else None, x))

    _replays_match(run, reset, [y, r, x])


@pytest.mark.parametrize("fused_score", [False, True])
def test_ctx_chain_graph(fused_score):
    say("graph ctx chain", fused_score)
    P, d, ff, L, k = 300, 256, 512, 3, 90
    ws = [ffn_weights(31, l, d, ff) for l in range(L)]
    W = [ffn_dev(w) for w in ws]
    cur = to_dev(ctx_layer_inputs(31, 0, P, d, k, 1.3333, 0.1752)["x"])
    xr = [to_dev(random_bf16(31, l, "x", (P, d))) for l in range(L)]
    yr = [to_dev(random_bf16(31, l, "y_ref", (P, d))) for l in range(L)]
    r = torch.empty(P, d, dtype=torch.float32, device=dev())
    x = torch.empty(P, d, dtype=torch.bfloat16, device=dev())
    y = torch.empty_like(x)
    idx = torch.empty(k, dtype=torch.int32, device=dev())
    keys = torch.empty(P, dtype=torch.float64, device=dev())

    def reset():
        cgs.residual_rmsnorm(r, r_in=cur.float().contiguous(), x_out=x)

    def run():
        for l in range(L):
            if l == 0 or not fused_score:
                cgs.ctx_select(x, xr[l], k, idx_out=idx)
            else:
                cgs.ctx_select_from_keys(keys, k, idx_out=idx)
            if fused_score and l + 1 < L:
                glue = (r, None, x, xr[l + 1], keys)
            else:
                glue = (r, None, x if l + 1 < L else None)
            cgs.ctx_ffn_recompute(W[l], x, yr[l], idx, y_out=y, glue=glue)

    _replays_match(run, reset, [y, r, x, idx])
    assert np.all(np.diff(idx.cpu().numpy()) > 0)
