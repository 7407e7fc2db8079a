"""Helpers shared by the GPU parity tests: host <-> device marshalling and the
tolerance check.

Tolerance: |gpu - oracle| <= 1e-2 x RMS(oracle output) for every element of a
float32 output.  A bf16 output is the rounding of the computed value to bf16,
which by itself moves an element by up to half a bf16 ulp (2^-9 relative); so
for bf16 outputs each element may additionally differ by half an ulp of its
magnitude: |gpu - oracle| <= 1e-2 x RMS + ulp_bf16(max(|gpu|, |oracle|)) / 2.
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


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |v| (8 significant bits)."""
    _, e = np.frexp(np.abs(v))                    # |v| = m 2^e, 0.5 <= m < 1
    return np.ldexp(np.ones_like(v), np.maximum(e, -125) - 9)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL, out: str = "f32"):
    """Max-abs check against the oracle; ``out='bf16'`` for outputs stored in bf16."""
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    diff = np.abs(gpu - ref)
    allow = tol * rms
    if out == "bf16":
        allow = allow + half_ulp_bf16(np.maximum(np.abs(gpu), np.abs(ref)))
    bad = diff > allow
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; max abs err "
                           f"{float(diff.max()):.3e}, rms {rms:.3e}")
    return float(diff.max()) / rms


def assert_close_chain(gpu: np.ndarray, ref: np.ndarray, what: str, depth: int, out: str = "f32"):
    """Outputs of a layer chain run independently on both sides.

    depth 0 (no earlier layer feeds it): the single-call rule above.  depth >= 1:
    earlier layers' bf16 rounding decisions may resolve differently on the two
    sides and shift this layer's input by an ulp here and there, so the check is
    the RMS-relative error ||gpu - ref||_2 / ||ref||_2 <= 1e-2, with a max-abs cap
    of 5e-2 x RMS against localised errors."""
    if depth == 0:
        return assert_close(gpu, ref, what, out=out)
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape and np.all(np.isfinite(gpu)), what
    rms = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    rel = float(np.sqrt(np.mean((gpu - ref) ** 2))) / rms
    mx = float(np.max(np.abs(gpu - ref))) / rms
    assert rel <= TOL, f"{what}: rms-relative error {rel:.3e}"
    assert mx <= 5 * TOL, f"{what}: max abs error {mx:.3e} x rms"
    return rel
