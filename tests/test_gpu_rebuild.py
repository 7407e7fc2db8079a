"""GPU parity of ref_rebuild_dense (rMuscle §4.2) and of the residual/RMSNorm glue.

Teacher forcing: every layer is checked on the GPU's own input of that layer.
ybar_l is compared with the oracle's F_l of the GPU's xbar_l, and xbar_{l+1}
with the oracle's RMSNorm of the residual r_0 + ybar_0 + ... + ybar_l rebuilt
from the GPU's ybar values (the kernel adds the same values in fp32), each at
the single-call tolerance of gpu_helpers.assert_close.  Tokens are independent
rows, so a row sample checks whole rows exactly."""
import numpy as np
import pytest
import torch

import cache_guided_sparse_amd as cgs
import oracle as O
from cgs_inputs import ffn_weights, random_bf16
from gpu_helpers import assert_close, check_rebuild_teacher_forced, dev, ffn_dev, say, to_dev, values

pytestmark = pytest.mark.gpu


def _rebuild(layers, r0, dtype="bf16"):
    xo, yo = cgs.ref_rebuild_dense([ffn_dev(w) for w in layers], to_dev(r0, dtype))
    torch.cuda.synchronize()
    return xo, yo


@pytest.mark.parametrize("dtype,L,P,d,ff", [("bf16", 1, 64, 256, 512), ("bf16", 3, 100, 256, 512),
                                            ("bf16", 4, 300, 128, 256), ("f32", 2, 64, 256, 1024),
                                            ("bf16", 17, 40, 256, 512)])
def test_small_chains(dtype, L, P, d, ff):
    say("rebuild", dtype, L, P, d, ff)
    layers = [ffn_weights(30, l, d, ff, dtype=dtype) for l in range(L)]
    r0 = random_bf16(30, 0, "r0", (P, d), std=2.0, dtype=dtype)
    xo, yo = _rebuild(layers, r0, dtype)
    check_rebuild_teacher_forced(layers, r0, xo, yo, dtype)


def test_full_size_teacher_forced():
    """Entry-rebuild shapes (768 tokens, d 2048, ff 16384) over 3 layers (the
    per-layer launches are those of the 17-layer rebuild): every row of layer
    0, 64 rows of the later layers."""
    say("rebuild full size")
    L, P, d, ff = 3, 768, 2048, 16384
    layers = [ffn_weights(31, l, d, ff) for l in range(L)]
    r0 = random_bf16(31, 0, "r0", (P, d), std=2.0)
    xo, yo = _rebuild(layers, r0)
    rows = np.linspace(0, P - 1, 64).astype(int)
    e = check_rebuild_teacher_forced(layers, r0, xo, yo, "bf16", rows=rows, full_rows_layers=(0,))
    say(f"  worst ybar error {e:.2e} x rms")


def test_residual_rmsnorm_glue():
    say("glue")
    M, d = 37, 384
    g = np.random.default_rng(0)
    r = g.standard_normal((M, d)).astype(np.float32)
    yb = random_bf16(32, 0, "y_ref", (M, d))
    bias = g.standard_normal(d).astype(np.float32)
    rt = to_dev(r, "f32")
    xo = torch.empty(M, d, dtype=torch.bfloat16, device=dev())
    cgs.residual_rmsnorm(rt, y=to_dev(yb), bias=to_dev(bias, "f32"), x_out=xo)
    torch.cuda.synchronize()
    r_o = r.astype(np.float64) + O.decode(yb, "bf16") + bias
    assert_close(values(rt), r_o, "residual", tol=1e-6)
    assert_close(values(xo), O.rms_norm(r_o), "rmsnorm", out="bf16")


@pytest.mark.parametrize("dtype,n,L,P,d,ff", [("bf16", 4, 3, 100, 256, 512), ("f32", 3, 2, 64, 256, 1024),
                                              ("bf16", 1, 2, 40, 128, 256), ("bf16", 4, 2, 768, 2048, 16384)])
def test_batched_rebuild_teacher_forced(dtype, n, L, P, d, ff):
    """n entries rebuilt as one prefill over n P rows (ref_rebuild_dense_batch):
    every entry's outputs land in its own buffers and pass the teacher-forced
    check on their own; the gate/up rows equal the single-entry rebuild's
    within the bound (the down projection's split order differs with the row
    count), and the buffers around each entry's outputs are untouched."""
    say("batched rebuild", dtype, n, L, P, d, ff)
    layers = [ffn_weights(33, l, d, ff, dtype=dtype) for l in range(L)]
    r0s = [random_bf16(33, 1 + e, "r0", (P, d), std=2.0, dtype=dtype) for e in range(n)]
    W = [ffn_dev(w) for w in layers]
    r0 = torch.stack([to_dev(r, dtype) for r in r0s]).contiguous()
    dt = r0.dtype
    # each entry's outputs inside a larger buffer with guard rows around them
    big_x = torch.full((n, L + 2, P, d), 3.0, dtype=dt, device=dev())
    big_y = torch.full((n, L + 2, P, d), 3.0, dtype=dt, device=dev())
    xs = [big_x[e, 1:L + 1] for e in range(n)]
    ys = [big_y[e, 1:L + 1] for e in range(n)]
    cgs.ref_rebuild_dense_batch(W, r0, xs, ys)
    torch.cuda.synchronize()
    rows = None if P * d <= 256 * 1024 else np.linspace(0, P - 1, 12).astype(int)
    for e in range(n):
        check_rebuild_teacher_forced(layers, r0s[e], xs[e], ys[e], dtype, rows=rows)
        assert bool((big_x[e, 0] == 3.0).all() and (big_x[e, L + 1] == 3.0).all()), "x guard rows"
        assert bool((big_y[e, 0] == 3.0).all() and (big_y[e, L + 1] == 3.0).all()), "y guard rows"
    if n > 1 and P * d <= 256 * 1024:
        x1, y1 = cgs.ref_rebuild_dense(W, r0[1])
        torch.cuda.synchronize()
        assert torch.equal(x1[0], xs[1][0]), "x_ref of layer 0 is one RMSNorm of the same input"
        for l in range(L):
            assert_close(values(ys[1][l]), values(y1[l]).astype(np.float64), f"layer {l}: single-entry rebuild",
                         out=dtype)
