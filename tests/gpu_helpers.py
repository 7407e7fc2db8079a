"""Helpers shared by the GPU parity tests: host <-> device marshalling and the
tolerance check.

Tolerance (the workload's bound for bf16 outputs): max |gpu - oracle| <=
1e-2 x RMS(oracle output of that call), applied to every element.

* float32 outputs are checked literally.
* bf16 outputs are the kernel's fp32 value stored with round-to-nearest-even,
  and the bound applies to that computed value: the check is that the stored
  bf16 is the RNE image of some value within the bound, i.e.
      RNE(oracle - a) <= gpu <= RNE(oracle + a),   a = 1e-2 x RMS.
  No looser allowance: a perfectly computed output already misses the
  literal unrounded bound wherever |y| > 2^9 a / 1e-2 (about 2.6 x RMS), since
  the storage rounding alone moves it by up to 2^-9 |y| (pinned on the CPU in
  tests/test_tolerance.py).  Where a kernel also writes the fp32 value, tests
  check that value literally and its bf16 output bit for bit against RNE of it.
"""
import sys

import numpy as np
import torch

import cache_guided_sparse_amd as cgs

TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype="bf16"):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(a).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16 tensor (uint16) or the fp32 values."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def values(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ffn_dev(w: dict) -> cgs.FFN:
    dt = w["dtype"]
    return cgs.FFN(to_dev(w["w_gate"], dt), to_dev(w["w_up"], dt), to_dev(w["w_down"], dt),
                   layout=w["down_layout"])


def bf16_bracket(ref: np.ndarray, a) -> tuple:
    """(RNE(ref - a), RNE(ref + a)) as float64: the bf16 values a result within
    a of ref may be stored as (RNE is monotone)."""
    import oracle as O
    lo = O.decode(O.round_to_bf16_bits(ref - a), "bf16")
    hi = O.decode(O.round_to_bf16_bits(ref + a), "bf16")
    return lo, hi


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL, out: str = "f32"):
    """Max-abs check against the oracle (module docstring); ``out='bf16'`` for
    outputs stored in bf16.  Returns max |gpu - ref| / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    a = tol * rms
    diff = np.abs(gpu - ref)
    if out == "bf16":
        lo, hi = bf16_bracket(ref, a)
        bad = (gpu < lo) | (gpu > hi)
    else:
        bad = diff > a
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; max abs err "
                           f"{float(diff.max()):.3e}, rms {rms:.3e}")
    return float(diff.max()) / rms


def assert_rne_of(bf16_bits: np.ndarray, f32: np.ndarray, what: str):
    """The bf16 output is exactly RNE of the fp32 output of the same call."""
    import oracle as O
    want = O.round_to_bf16_bits(np.asarray(f32, dtype=np.float32).astype(np.float64))
    assert np.array_equal(np.asarray(bf16_bits), want), f"{what}: bf16 output is not RNE of the fp32 output"


def check_rebuild_teacher_forced(layers, r0, xo, yo, dtype="bf16", rows=None, full_rows_layers=()):
    """Teacher-forced check of a dense rebuild, per layer l: xbar_l (every row)
    against RMSNorm(r_l), r_l rebuilt from r_0 and the GPU's ybar_0..l-1, and
    ybar_l (rows `rows`; every row for l in full_rows_layers) against F_l of the
    GPU's own xbar_l.  Returns the largest ybar error / RMS."""
    import oracle as O
    xg = bits(xo) if dtype == "bf16" else values(xo)
    yg = bits(yo) if dtype == "bf16" else values(yo)
    P = xg.shape[1]
    rows = np.arange(P) if rows is None else np.asarray(rows)
    r = O.decode(r0, dtype)
    worst = 0.0
    for l in range(len(layers)):
        sel = np.arange(P) if l in full_rows_layers else rows
        x_all = xg[l] if dtype == "bf16" else xg[l].astype(np.float32)
        assert_close(O.decode(x_all, dtype), O.rms_norm(r), f"xbar layer {l}", out=dtype)
        x_l = x_all[sel]
        y_l = yg[l][sel] if dtype == "bf16" else yg[l][sel].astype(np.float32)
        y_o = O.ffn_geglu(O.decode(x_l, dtype), layers[l])
        worst = max(worst, assert_close(O.decode(y_l, dtype), y_o, f"ybar layer {l}", out=dtype))
        yl_all = yg[l] if dtype == "bf16" else yg[l].astype(np.float32)
        r = r + O.decode(yl_all, dtype)
    return worst
