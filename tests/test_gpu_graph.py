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


def test_act_masked_layers_graph():
    """A whole two-group denoise (dense anchor, update, dense anchor, update;
    3 layers a step) enqueued by one act_masked_layers call inside a graph:
    every replay reproduces the eager chain bit for bit, anchor state included."""
    say("graph act_masked_layers")
    S, d, ff, L = 50, 1024, 4096, 3
    ws = [ffn_weights(31, l, d, ff, down_layout="fd", down_lognormal_sigma=1.5) for l in range(L)]
    W = [ffn_dev(w) for w in ws]
    a0 = to_dev(act_tokens(31, 0, S, d)["x"]).float().contiguous()
    full = torch.arange(ff, dtype=torch.int32, device=dev())
    masks = [torch.arange(o, ff, 3, dtype=torch.int32, device=dev()) for o in (0, 1)]
    cw = [[cgs.act_gather_rows(W[l], m) for l in range(L)] for m in masks]
    ya = torch.empty(2, L, S, d, dtype=torch.float32, device=dev())
    ha = torch.empty(2, L, ff, S, dtype=torch.float32, device=dev())
    ych = torch.empty(4 * L, S, d, dtype=torch.bfloat16, device=dev())
    bias = torch.linspace(-1, 1, d, device=dev())
    layers = []
    for t in range(4):
        g = t // 2
        for l in range(L):
            b = bias if l == L - 1 else None
            if t % 2 == 0:
                layers.append(cgs.MaskedLayer(W[l], full, bias=b, y_out=ych[t * L + l], y_f32_out=ya[g, l],
                                              h_out=ha[g, l]))
            else:
                layers.append(cgs.MaskedLayer(cw[g][l], masks[g], y_anchor=ya[g, l], h_anchor=ha[g, l], bias=b,
                                              y_out=ych[t * L + l]))
    chain = cgs.MaskedChain(layers, S, ff)
    r = torch.empty(S, d, dtype=torch.float32, device=dev())
    x = torch.empty(4 * L + 1, S, d, dtype=torch.bfloat16, device=dev())

    def reset():
        cgs.residual_rmsnorm(r, r_in=a0, x_out=x[0])

    def run():
        cgs.act_masked_layers(chain, r, x)

    _replays_match(run, reset, [x, ych, r, ya, ha])


def test_act_masked_layers_fp32_and_empty_masks():
    """fp32 weights and activations through act_masked_layers, with an empty
    mask (K = 0: y = y_a) among the layers: every layer's bits equal the
    per-layer act_ffn_masked_compact calls'."""
    say("act_masked_layers fp32")
    S, d, ff, L = 16, 256, 1024, 3
    ws = [ffn_weights(32, l, d, ff, dtype="f32", down_layout="fd") for l in range(L)]
    W = [ffn_dev(w) for w in ws]
    a0 = to_dev(act_tokens(32, 0, S, d, dtype="f32")["x"], "f32")
    full = torch.arange(ff, dtype=torch.int32, device=dev())
    masks = [torch.arange(0, ff, 4, dtype=torch.int32, device=dev()),
             torch.empty(0, dtype=torch.int32, device=dev()),
             torch.arange(5, ff, 7, dtype=torch.int32, device=dev())]
    cw = [cgs.act_gather_rows(W[l], masks[l]) for l in range(L)]
    ya = torch.empty(L, S, d, dtype=torch.float32, device=dev())
    ha = torch.empty(L, ff, S, dtype=torch.float32, device=dev())
    outs = []
    for mode in ("chain", "calls"):
        r = torch.empty(S, d, dtype=torch.float32, device=dev())
        x = torch.empty(2 * L + 1, S, d, dtype=torch.float32, device=dev())
        y = torch.empty(2 * L, S, d, dtype=torch.float32, device=dev())
        cgs.residual_rmsnorm(r, r_in=a0, x_out=x[0])
        if mode == "chain":
            layers = [cgs.MaskedLayer(W[l], full, y_out=y[l], y_f32_out=ya[l], h_out=ha[l]) for l in range(L)]
            layers += [cgs.MaskedLayer(cw[l], masks[l], y_anchor=ya[l], h_anchor=ha[l], y_out=y[L + l])
                       for l in range(L)]
            cgs.act_masked_layers(cgs.MaskedChain(layers, S, ff), r, x)
        else:
            for l in range(L):
                cgs.act_ffn_masked_compact(W[l], x[l], full, y_out=y[l], y_f32_out=ya[l], h_out=ha[l],
                                           glue=(r, None, x[l + 1]))
            for l in range(L):
                cgs.act_ffn_masked_compact(cw[l], x[L + l], masks[l], y_anchor=ya[l], h_anchor=ha[l],
                                           y_out=y[L + l], glue=(r, None, x[L + l + 1]))
        torch.cuda.synchronize()
        outs.append((x.clone(), y.clone(), r.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    # the empty mask's layer is the anchor output rounded to the dtype (fp32: itself)
    assert torch.equal(outs[0][1][L + 1], ya[1])
