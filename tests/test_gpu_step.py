"""GPU parity of act_denoise_step: every layer of a masked denoising step
(rMuscle §4.1, Eq. 4, with the residual / RMSNorm glue between layers) in one
persistent launch, and of act_gather_rows_t, the compact weights it reads.

Teacher forcing: layer l is checked on the GPU's own input x_l (written by
the kernel): y_l against the oracle's Eq. 4 of that input (fp32 output at the
plain bound, bf16 output as its round-to-nearest-even), the residual against
r_l + round(y_l) (+ bias) and x_{l+1} against RMSNorm of it."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import act_tokens, ffn_weights, rng
from gpu_helpers import assert_close, assert_rne_of, bits, dev, ffn_dev, say, to_dev, values

pytestmark = pytest.mark.gpu


def _f32(a):
    return to_dev(np.ascontiguousarray(a, dtype=np.float32), "f32")


def _mask(seed, l, ff, K):
    return np.sort(rng(seed, l, "perm").permutation(ff)[:K]).astype(np.int32)


def _setup(seed, L, S, d, ff, Ks, anchors=True, bias_last=True):
    """Weights, masks, anchor state (the oracle's dense FFN of a perturbed
    input, as fp32), the residual start r0 and its RMSNorm x0."""
    layers, masks, ya, ha = [], [], [], []
    for l in range(L):
        w = ffn_weights(seed, l, d, ff, down_layout="fd", down_lognormal_sigma=1.5)
        layers.append(w)
        masks.append(_mask(seed, l, ff, Ks[l]))
        if anchors:
            xp = act_tokens(seed, l, S, d, noise_sigma=0.3)["x_pert"]
            y0, h0 = O.act_ffn_masked(w, xp, np.arange(ff))
            ya.append(y0.astype(np.float32))
            ha.append(h0.astype(np.float32))
        else:
            ya.append(None)
            ha.append(None)
    r0 = (2.0 * rng(seed, 0, "r0").standard_normal((S, d))).astype(np.float32)
    bias = rng(seed, 1, "r0").standard_normal(d).astype(np.float32) if bias_last else None
    return layers, masks, ya, ha, r0, bias


def _run_step(layers, masks, ya, ha, r0, bias, want_h=False):
    """act_denoise_step on the GPU; returns host copies of x, per-layer y (bf16
    bits and fp32), h_out (if asked), the final r and the status word."""
    L = len(layers)
    S, d = r0.shape
    ff = layers[0]["ff"]
    W = [ffn_dev(w) for w in layers]
    r = _f32(r0)
    x = torch.empty(L + 1, S, d, dtype=torch.bfloat16, device=dev())
    cgs.residual_rmsnorm(r, r_in=r.clone(), x_out=x[0])
    ys = torch.empty(L, S, d, dtype=torch.bfloat16, device=dev())
    yf = torch.empty(L, S, d, dtype=torch.float32, device=dev())
    hs = torch.full((L, ff, S), float("nan"), dtype=torch.float32, device=dev()) if want_h else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev())
    step_layers = []
    for l in range(L):
        K = len(masks[l])
        idx = torch.from_numpy(masks[l]).to(dev())
        cw = cgs.act_gather_rows_t(W[l], idx if K < ff else None, K=K)
        step_layers.append(cgs.StepLayer(
            cw, idx=idx if K < ff else None,
            y_anchor=None if ya[l] is None else _f32(ya[l]), h_anchor=None if ha[l] is None else _f32(ha[l]),
            bias=_f32(bias) if (bias is not None and l == L - 1) else None,
            y_out=ys[l], y_f32_out=yf[l], h_out=hs[l] if want_h else None))
    r_start = r.clone()
    cgs.act_denoise_step(step_layers, r, x, ff, status=status)
    torch.cuda.synchronize()
    out = {"x": bits(x), "y": bits(ys), "yf": yf.cpu().numpy(), "r": r.cpu().numpy(),
           "r0": r_start.cpu().numpy(), "status": int(status.item())}
    if want_h:
        out["h"] = hs.cpu().numpy()
    return out


def _check_teacher_forced(layers, masks, ya, ha, bias, out, h_rows=None):
    L = len(layers)
    r = out["r0"].astype(np.float64)
    assert out["status"] == 0, f"status {out['status']}"
    for l in range(L):
        x_l = out["x"][l]
        y_o, h_o = O.act_ffn_masked(layers[l], x_l, masks[l], ya[l], ha[l])
        assert_close(out["yf"][l], y_o, f"layer {l}: y (fp32)")
        assert_close(O.decode(out["y"][l], "bf16"), y_o, f"layer {l}: y", out="bf16")
        assert_rne_of(out["y"][l], out["yf"][l], f"layer {l}")
        if "h" in out and len(masks[l]):
            assert_close(out["h"][l][masks[l]], h_o, f"layer {l}: h rows of the mask")
        r = r + O.decode(out["y"][l], "bf16")
        if bias is not None and l == L - 1:
            r = r + bias.astype(np.float64)
        assert_close(O.decode(out["x"][l + 1], "bf16"), O.rms_norm(r), f"layer {l}: next input", out="bf16")
    assert_close(out["r"], r, "final residual", tol=1e-5)


@pytest.mark.parametrize("S,d,ff,Ks", [(16, 256, 1024, [256, 0, 1024, 100]), (50, 1024, 4096, [1251, 819, 4096]),
                                      (1, 256, 512, [37, 512]), (64, 1024, 4096, [1638, 2048, 31]),
                                      (33, 512, 2048, [600, 2048]),
                                      # mask sizes changing from layer to layer, with K splits left
                                      # empty (1088 and 919 use 7 of the 8): each down tile resets
                                      # its previous partials only once their row finishes read them
                                      (50, 1024, 4096, [1634, 1088, 1300, 919, 823, 1516])])
def test_masked_step_teacher_forced(S, d, ff, Ks):
    say("step", S, d, ff, Ks)
    layers, masks, ya, ha, r0, bias = _setup(70, len(Ks), S, d, ff, Ks)
    out = _run_step(layers, masks, ya, ha, r0, bias, want_h=True)
    _check_teacher_forced(layers, masks, ya, ha, bias, out)


def test_dense_anchor_step():
    """K = ff, no anchors: every layer is the dense FFN; y_f32 and h_out are the
    anchor state the masked steps read."""
    say("step dense anchor")
    S, d, ff = 50, 1024, 4096
    layers, masks, ya, ha, r0, bias = _setup(71, 3, S, d, ff, [ff, ff, ff], anchors=False)
    out = _run_step(layers, masks, ya, ha, r0, bias, want_h=True)
    _check_teacher_forced(layers, masks, ya, ha, bias, out)


def test_full_expert_step_18_layers():
    """The action expert's shapes: 18 layers, 50 tokens, d 1024, ff 4096, masks of
    20-40% of the neurons; the dense anchor step by the same kernel, then a
    masked step from a perturbed input against that anchor state."""
    say("step 18 layers")
    L, S, d, ff = 18, 50, 1024, 4096
    Ks = [int(k) for k in rng(72, 0, "misc").integers(int(0.2 * ff), int(0.4 * ff), size=L)]
    layers, masks, _, _, r0, bias = _setup(72, L, S, d, ff, Ks, anchors=False)
    dense = [np.arange(ff, dtype=np.int32)] * L
    anc = _run_step(layers, dense, [None] * L, [None] * L, r0, bias, want_h=True)
    _check_teacher_forced(layers, dense, [None] * L, [None] * L, bias, anc)
    ya = [anc["yf"][l] for l in range(L)]
    ha = [anc["h"][l] for l in range(L)]
    r1 = (r0 + 0.3 * rng(72, 2, "r0").standard_normal(r0.shape)).astype(np.float32)
    out = _run_step(layers, masks, ya, ha, r1, bias, want_h=True)
    _check_teacher_forced(layers, masks, ya, ha, bias, out)


def test_zero_mask_gives_the_anchor_output():
    """K = 0 in every layer: y = round(y_a) bit for bit."""
    say("step K = 0")
    S, d, ff = 16, 256, 1024
    layers, masks, ya, ha, r0, bias = _setup(73, 2, S, d, ff, [0, 0])
    out = _run_step(layers, masks, ya, ha, r0, bias)
    for l in range(2):
        assert np.array_equal(out["yf"][l], ya[l])
        assert np.array_equal(out["y"][l], O.round_to_bf16_bits(ya[l].astype(np.float64)))


def test_repeats_and_graph_replays_are_bit_identical():
    """Fixed summation orders: the same step twice eagerly, and replays of a
    captured HIP graph with eager work in between, give the same bits."""
    say("step determinism and graph")
    S, d, ff = 50, 1024, 4096
    Ks = [1200, 1500]
    layers, masks, ya, ha, r0, bias = _setup(74, 2, S, d, ff, Ks)
    a = _run_step(layers, masks, ya, ha, r0, bias)
    b = _run_step(layers, masks, ya, ha, r0, bias)
    for k in ("x", "y", "yf", "r"):
        assert np.array_equal(a[k], b[k]), k
    W = [ffn_dev(w) for w in layers]
    r = _f32(r0)
    x = torch.empty(3, S, d, dtype=torch.bfloat16, device=dev())
    cgs.residual_rmsnorm(r, r_in=r.clone(), x_out=x[0])
    r_start = r.clone()
    sl = []
    for l in range(2):
        idx = torch.from_numpy(masks[l]).to(dev())
        sl.append(cgs.StepLayer(cgs.act_gather_rows_t(W[l], idx), idx=idx, y_anchor=_f32(ya[l]),
                                h_anchor=_f32(ha[l]), bias=_f32(bias) if l == 1 else None))
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    cgs.act_denoise_step(sl, r, x, ff, status=status)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.copy_(r_start)
        cgs.act_denoise_step(sl, r, x, ff, status=status)
    for rep in range(4):
        x[1:].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(bits(x), a["x"]), f"replay {rep}: x"
        assert np.array_equal(r.cpu().numpy(), a["r"]), f"replay {rep}: r"
        cgs.residual_rmsnorm(torch.empty_like(r), r_in=r, x_out=torch.empty_like(x[0]))  # eager work between


def test_wait_limit_turns_a_stall_into_a_status():
    """A wait limit of 0 (set from the host) makes the first unsatisfied wait
    give up: the launch ends with CGS_ERR_TIMEOUT in the status word instead of
    waiting; with the limit restored the same call succeeds."""
    say("step wait limit")
    S, d, ff = 16, 256, 1024
    layers, masks, ya, ha, r0, bias = _setup(75, 3, S, d, ff, [300, 400, 500])
    prev = cgs.set_step_wait_limit(0)
    try:
        out = _run_step(layers, masks, ya, ha, r0, bias)
    finally:
        cgs.set_step_wait_limit(prev)
    assert out["status"] == cgs.CGS_ERR_TIMEOUT
    out = _run_step(layers, masks, ya, ha, r0, bias)
    _check_teacher_forced(layers, masks, ya, ha, bias, out)


@pytest.mark.parametrize("d,ff,K,ldk", [(1024, 4096, 1251, 1280), (256, 1024, 0, 32), (256, 1024, 1024, 1024),
                                         (1024, 4096, 37, 64)])
def test_gather_rows_t_bit_exact(d, ff, K, ldk):
    say("gather_t", d, ff, K, ldk)
    w = ffn_weights(76, 0, d, ff, down_layout="fd")
    idx_h = _mask(76, 0, ff, K)
    W = ffn_dev(w)
    c = cgs.act_gather_rows_t(W, torch.from_numpy(idx_h).to(dev()), K=K, ldk=ldk)
    torch.cuda.synchronize()
    assert np.array_equal(bits(c.w_gate), w["w_gate"][idx_h])
    assert np.array_equal(bits(c.w_up), w["w_up"][idx_h])
    want = np.zeros((d, ldk), dtype=np.uint16)
    want[:, :K] = w["w_down"][idx_h].T
    assert np.array_equal(bits(c.w_down_t), want)
