"""GPU parity of ctx_ffn_recompute (rMuscle §4.1, Eq. 3): recomputed rows within
1e-2 x RMS of the oracle, every other row bit-identical to the cached output."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import ctx_layer_inputs, ffn_weights, random_bf16, rng
from gpu_helpers import assert_close, bits, dev, ffn_dev, say, to_dev, values

pytestmark = pytest.mark.gpu


def _recompute(w, x, y_ref, idx):
    dt = w["dtype"]
    W = ffn_dev(w)
    y = cgs.ctx_ffn_recompute(W, to_dev(x, dt), to_dev(y_ref, dt),
                              torch.from_numpy(np.asarray(idx, dtype=np.int32)).to(dev()))
    torch.cuda.synchronize()
    return y


def _check_full(w, x, y_ref, idx):
    y = _recompute(w, x, y_ref, idx)
    y_o, rec = O.ctx_ffn_recompute(w, x, y_ref, idx)
    assert_close(values(y)[rec], y_o[rec], "recomputed rows", out=w["dtype"])
    assert np.array_equal(bits(y)[~rec], np.asarray(y_ref)[~rec]), "copied rows differ"
    return y


@pytest.mark.parametrize("rho", [0.0, 0.25, 1.0])
def test_tiny_fp32(rho):
    say("ctx tiny fp32", rho)
    P, d, ff = 64, 256, 1024
    inp = ctx_layer_inputs(0, 0, P, d, 16, 1.0, 0.02, dtype="f32")
    w = ffn_weights(0, 0, d, ff, dtype="f32")
    y_ref = O.ffn_geglu(O.decode(inp["x_ref"], "f32"), w).astype(np.float32)
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], O.ratio_to_count(rho, P), "f32")
    _check_full(w, inp["x"], y_ref, idx)


@pytest.mark.parametrize("d,k", [(256, 0), (256, 1), (256, 37), (256, 64), (256, 65), (256, 129), (256, 200),
                                 (256, 300), (2048, 0), (2048, 1), (2048, 231), (2048, 300)])
def test_ragged_bf16(d, k):
    """k spans the 64/128/256-row tiles, several M tiles and a ragged tail;
    d = 2048 (one 8-element run per finish thread) takes the finish kernel
    that loads its rows before the index search."""
    say("ctx ragged", d, k)
    P, ff = 300, 512
    w = ffn_weights(1, 0, d, ff)
    x = random_bf16(1, 0, "x", (P, d))
    y_ref = random_bf16(1, 0, "y_ref", (P, d))
    idx = np.sort(rng(1, k, "perm").permutation(P)[:k]).astype(np.int32)
    _check_full(w, x, y_ref, idx)


@pytest.mark.parametrize("d", [256, 2048])
def test_index_list_longer_than_the_staged_search(d):
    """k > 4096 selected rows: the finish kernels search the index list in
    global memory instead of LDS.  Copied rows bit for bit, a sample of
    recomputed rows against the oracle."""
    say("ctx long index list", d)
    P, ff, k = 5000, 512, 4500
    w = ffn_weights(4, 0, d, ff)
    x = random_bf16(4, 0, "x", (P, d))
    y_ref = random_bf16(4, 0, "y_ref", (P, d))
    idx = np.sort(rng(4, k, "perm").permutation(P)[:k]).astype(np.int32)
    y = bits(_recompute(w, x, y_ref, idx))
    rec = np.zeros(P, dtype=bool)
    rec[idx] = True
    assert np.array_equal(y[~rec], y_ref[~rec])
    sample = idx[np.linspace(0, k - 1, 24).astype(int)]
    y_o = O.ffn_geglu(O.decode(x[sample], "bf16"), w)
    assert_close(O.decode(y[sample], "bf16"), y_o, "sampled recomputed rows", out="bf16")


@pytest.mark.parametrize("P,d,ff,dtype", [(96, 256, 512, "bf16"), (768, 2048, 16384, "bf16"),
                                          (3072, 2048, 16384, "bf16"), (12288, 2048, 16384, "bf16"),
                                          (768, 1024, 16384, "f32"), (1152, 2048, 8320, "bf16"),
                                          (2304, 2048, 16384, "bf16")])
def test_dense_equals_rebuild_layer(P, d, ff, dtype):
    """k = P is the dense FFN: equal to one rebuild layer's output at the same
    input, bit for bit.  The gathered rows of the Context Cache path always run
    one tile per workgroup; with more tiles than CUs the rebuild runs them
    persistently, with the same sums: the gate/up projection at 768, 3072 and
    12288 rows (2, 6 and 24 tiles per workgroup; 192 x 256 and 256 x 256
    tiles) and in fp32 (256 x 128 tiles, 3 per workgroup), the down
    projection at 12288 rows (one K split, 2 tiles per workgroup).  Uneven
    shares: 390 tiles (1152 rows, ff 8320; not a multiple of 8, so without the
    XCD renumbering) and 1152 tiles (2304 rows: 9 row tiles in one group), 1 or
    2 and 4 or 5 tiles per workgroup."""
    say("ctx dense vs rebuild", P, d, ff, dtype)
    w = ffn_weights(2, 0, d, ff, dtype=dtype)
    r0 = random_bf16(2, 0, "r0", (P, d), dtype=dtype)
    W = ffn_dev(w)
    xo, yo = cgs.ref_rebuild_dense([W], to_dev(r0, dtype))
    y = cgs.ctx_ffn_recompute(W, xo[0], torch.zeros_like(xo[0]),
                              torch.arange(P, dtype=torch.int32, device=dev()))
    torch.cuda.synchronize()
    raw = np.uint32 if dtype == "f32" else np.uint16
    assert np.array_equal(bits(y).view(raw), bits(yo[0]).view(raw))
    if P > 4096:
        # both paths run the 12288-row down projection persistently: sampled
        # rows against the oracle, teacher-forced on the GPU's own layer input
        sample = np.linspace(0, P - 1, 16).astype(int)
        y_o = O.ffn_geglu(O.decode(bits(xo[0])[sample], dtype), w)
        assert_close(O.decode(bits(yo[0])[sample], dtype), y_o, "sampled rows", out=dtype)


@pytest.mark.parametrize("rho", [0.1, 0.3, 1.0])
def test_full_layer_every_row(rho):
    """One VLM layer at full size (768 x 2048, ff 16384), the configuration the
    benchmark times: every recomputed row against the oracle (k = 77, 231,
    768), every copied row bit for bit, the selection against the oracle's."""
    say("ctx full layer", rho)
    P, d, ff = 768, 2048, 16384
    inp = ctx_layer_inputs(1, 0, P, d, 231, 1.3333, 0.1752)
    w = ffn_weights(1, 0, d, ff)
    y_ref = random_bf16(1, 0, "y_ref", (P, d))
    k = O.ratio_to_count(rho, P)
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], k)
    gidx = cgs.ctx_select(to_dev(inp["x"]), to_dev(inp["x_ref"]), k)
    torch.cuda.synchronize()
    assert np.array_equal(gidx.cpu().numpy(), idx)
    y = _recompute(w, inp["x"], y_ref, idx)
    yb = bits(y)
    rec = np.zeros(P, dtype=bool)
    rec[idx] = True
    assert np.array_equal(yb[~rec], y_ref[~rec])
    y_o = O.ffn_geglu(O.decode(inp["x"], "bf16")[idx], w)
    e = assert_close(O.decode(yb[idx], "bf16"), y_o, "recomputed rows", out="bf16")
    say(f"  k {k}: max error {e:.2e} x rms")


def test_deterministic_repeats():
    P, d, ff = 300, 256, 512
    w = ffn_weights(3, 0, d, ff)
    x = random_bf16(3, 0, "x", (P, d))
    y_ref = random_bf16(3, 0, "y_ref", (P, d))
    idx = np.arange(0, P, 2, dtype=np.int32)
    a = bits(_recompute(w, x, y_ref, idx))
    b = bits(_recompute(w, x, y_ref, idx))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("d,with_bias", [(256, False), (2048, False), (2048, True)])
def test_fused_glue(d, with_bias):
    """Residual/RMSNorm glue in the finish kernel on all P rows (recomputed and
    copied), checked on the GPU's own y against the oracle's RMSNorm."""
    say("ctx glue", d, with_bias)
    P, ff = 300, 512
    inp = ctx_layer_inputs(21, 0, P, d, 90, 1.3333, 0.1752)
    w = ffn_weights(21, 0, d, ff)
    y_ref = random_bf16(21, 0, "y_ref", (P, d))
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], 90)
    r0 = rng(21, 1, "misc").standard_normal((P, d)).astype(np.float32)
    bias = rng(21, 2, "misc").standard_normal(d).astype(np.float32) if with_bias else None
    r = to_dev(r0, "f32")
    xn = torch.empty(P, d, dtype=torch.bfloat16, device=dev())
    y = cgs.ctx_ffn_recompute(ffn_dev(w), to_dev(inp["x"]), to_dev(y_ref),
                              torch.from_numpy(idx).to(dev()),
                              glue=(r, None if bias is None else to_dev(bias, "f32"), xn))
    torch.cuda.synchronize()
    y_o, rec = O.ctx_ffn_recompute(w, inp["x"], y_ref, idx)
    assert_close(values(y)[rec], y_o[rec], "recomputed rows", out="bf16")
    assert np.array_equal(bits(y)[~rec], y_ref[~rec])
    r_exp = r0.astype(np.float64) + values(y)
    if bias is not None:
        r_exp = r_exp + bias.astype(np.float64)
    assert_close(values(r), r_exp, "residual")
    assert_close(values(xn), O.rms_norm(r_exp), "x_next", out="bf16")


@pytest.mark.parametrize("d", [256, 2048])
@pytest.mark.parametrize("kind", ["rel_rms", "cosine"])
def test_fused_next_score(kind, d):
    """The finish kernel's Eq. 2 keys of x_next against the next layer's cached
    input are bit-identical to ctx_select's keys of the same pair and to the
    oracle's; selecting from them gives the oracle's index set."""
    say("ctx fused score", kind, d)
    P, ff, k = 300, 512, 90
    inp = ctx_layer_inputs(22, 0, P, d, k, 1.3333, 0.1752)
    nxt = ctx_layer_inputs(22, 1, P, d, k, 1.3333, 0.1752)
    w = ffn_weights(22, 0, d, ff)
    y_ref = random_bf16(22, 0, "y_ref", (P, d))
    idx, _ = O.ctx_select(inp["x"], inp["x_ref"], k)
    r = to_dev(rng(22, 1, "misc").standard_normal((P, d)).astype(np.float32), "f32")
    xn = torch.empty(P, d, dtype=torch.bfloat16, device=dev())
    xr = to_dev(nxt["x_ref"])
    keys = torch.full((P,), -1.0, dtype=torch.float64, device=dev())
    cgs.ctx_ffn_recompute(ffn_dev(w), to_dev(inp["x"]), to_dev(y_ref), torch.from_numpy(idx).to(dev()),
                          glue=(r, None, xn, xr, keys, kind))
    sel = cgs.ctx_select_from_keys(keys, k)
    keys2 = torch.empty(P, dtype=torch.float64, device=dev())
    sel2 = cgs.ctx_select(xn, xr, k, kind=kind, key_out=keys2)
    torch.cuda.synchronize()
    assert torch.equal(keys, keys2), "fused keys differ from ctx_select's"
    assert torch.equal(sel, sel2)
    idx_o, keys_o = O.ctx_select(bits(xn), nxt["x_ref"], k, kind=kind)
    assert np.array_equal(keys.cpu().numpy(), keys_o)
    assert np.array_equal(sel.cpu().numpy(), idx_o)


@pytest.mark.parametrize("P,k", [(1, 1), (7, 3), (1024, 1), (1024, 1024), (4096, 2731), (5000, 1667)])
def test_select_from_keys(P, k):
    """Top k of stored keys with ties (repeated values) to the lower index,
    on both the one-chunk (P <= 1024) and the general path."""
    say("select from keys", P, k)
    g = rng(23, P, "misc")
    keys = np.round(g.standard_normal(P), 1) + 0.0  # many equal keys, no -0.0
    idx = cgs.ctx_select_from_keys(torch.from_numpy(keys).to(dev()), k)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), O.topk_ascending(keys, k))


def test_concurrent_streams_keep_their_own_scratch():
    """The same entry point on two streams at once (split-K partials in each
    stream's own workspace): each result equals the same call run alone, bit
    for bit."""
    say("ctx two streams")
    P, d, ff, k = 300, 256, 1024, 90
    w = ffn_weights(5, 0, d, ff)
    W = ffn_dev(w)
    ins = []
    for j in range(2):
        x = to_dev(random_bf16(5, j, "x", (P, d)))
        y_ref = to_dev(random_bf16(5, j, "y_ref", (P, d)))
        idx = torch.from_numpy(np.sort(rng(5, j, "perm").permutation(P)[:k]).astype(np.int32)).to(dev())
        ins.append((x, y_ref, idx))
    alone = [cgs.ctx_ffn_recompute(W, *a) for a in ins]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for st in streams:
            st.wait_stream(main)
        ys = []
        for st, a in zip(streams, ins):
            with torch.cuda.stream(st):
                ys.append(cgs.ctx_ffn_recompute(W, *a))
        for st in streams:
            main.wait_stream(st)
        outs.append(ys)
    torch.cuda.synchronize()
    for ys in outs:
        for y, y0 in zip(ys, alone):
            assert torch.equal(y, y0)
