"""GPU parity of ctx_select (rMuscle §4.1, Eq. 2 + top ceil(rho_p P)): selected
indices and score keys must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import ctx_layer_inputs, f32_to_bf16_bits, rng
from gpu_helpers import bits, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _run(x, xr, k, dtype, kind):
    P = x.shape[0]
    keys = torch.empty(P, dtype=torch.float64, device=dev())
    idx = cgs.ctx_select(to_dev(x, dtype), to_dev(xr, dtype), k, kind=kind, key_out=keys)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), keys.cpu().numpy()


def _check(x, xr, k, dtype, kind):
    gi, gk = _run(x, xr, k, dtype, kind)
    oi, ok = O.ctx_select(x, xr, k, dtype, kind)
    assert np.array_equal(gk.view(np.uint64), ok.view(np.uint64)), "score keys differ"
    assert np.array_equal(gi, oi), "selected indices differ"


@pytest.mark.parametrize("kind", ["rel_rms", "cosine"])
@pytest.mark.parametrize("rho", [0.0, 0.25, 1.0])
def test_tiny_fp32(kind, rho):
    say("select tiny fp32", kind, rho)
    inp = ctx_layer_inputs(0, 0, 64, 256, 16, 1.0, 0.02, dtype="f32")
    k = O.ratio_to_count(rho, 64)
    _check(inp["x"], inp["x_ref"], k, "f32", kind)


@pytest.mark.parametrize("kind", ["rel_rms", "cosine"])
@pytest.mark.parametrize("rho", [0.0, 0.1, 0.3, 0.5, 1.0])
def test_full_layer_bf16(kind, rho):
    """One VLM layer: 768 tokens x d 2048, 30% planted at cosine ~0.6."""
    say("select full layer", kind, rho)
    inp = ctx_layer_inputs(1, 0, 768, 2048, 231, 1.3333, 0.1752)
    k = O.ratio_to_count(rho, 768)
    _check(inp["x"], inp["x_ref"], k, "bf16", kind)
    if rho == 0.3:
        gi, _ = _run(inp["x"], inp["x_ref"], k, "bf16", kind)
        assert np.array_equal(gi, inp["changed"])


@pytest.mark.parametrize("P,d", [(1, 64), (3, 8), (100, 12), (1000, 40), (2500, 64), (5000, 16)])
def test_ragged_shapes(P, d):
    """P above the 1024-thread block, d not a multiple of the 8-wide vector path."""
    say("select ragged", P, d)
    inp = ctx_layer_inputs(2, P, P, d, max(1, P // 4), 1.0, 0.1)
    for k in sorted({0, 1, P // 3, P - 1, P}):
        if 0 <= k <= P:
            _check(inp["x"], inp["x_ref"], k, "bf16", "rel_rms")


def test_ties_go_to_lower_index():
    """Many identical rows: equal keys, ties broken toward the lower index."""
    say("select ties")
    g = rng(3, 0, "misc")
    base = g.standard_normal((7, 32)).astype(np.float32)
    x = np.repeat(base, 40, axis=0)[g.permutation(280)]
    xr = x + np.float32(0.5) * g.standard_normal((1, 32)).astype(np.float32)
    xb, rb = f32_to_bf16_bits(x), f32_to_bf16_bits(xr)
    for k in (1, 5, 40, 41, 139, 279):
        _check(xb, rb, k, "bf16", "rel_rms")
    # identical reference: every key is 0 and the first k indices win
    gi, gk = _run(xb, xb, 17, "bf16", "rel_rms")
    assert np.all(gk == 0) and np.array_equal(gi, np.arange(17))


def test_zero_rows_hit_the_floor():
    """x = 0 rows use the fixed-point floor E; a row with x_ref = 0 scores 1."""
    say("select zero rows")
    g = rng(4, 0, "misc")
    x = g.standard_normal((50, 64)).astype(np.float32)
    x[[3, 9]] = 0
    xr = x + np.float32(0.3) * g.standard_normal((50, 64)).astype(np.float32)
    xr[12] = 0
    _check(f32_to_bf16_bits(x), f32_to_bf16_bits(xr), 10, "bf16", "rel_rms")
    _check(f32_to_bf16_bits(x), f32_to_bf16_bits(xr), 10, "bf16", "cosine")


def test_deterministic_repeats():
    inp = ctx_layer_inputs(5, 0, 768, 2048, 231, 1.3333, 0.1752)
    a = _run(inp["x"], inp["x_ref"], 231, "bf16", "rel_rms")
    b = _run(inp["x"], inp["x_ref"], 231, "bf16", "rel_rms")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint64), b[1].view(np.uint64))
