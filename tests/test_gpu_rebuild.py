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
