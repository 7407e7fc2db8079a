"""Seeded random draws and bf16 encoding (no selective-FFN arithmetic here)."""
from __future__ import annotations

import numpy as np

# Role tags keep the random streams of different tensors independent.
ROLE = {
    "w_gate": 1, "w_up": 2, "w_down": 3, "w_down_scale": 4,
    "x": 10, "x_noise": 11, "perm": 12, "y_ref": 13,
    "act_x": 20, "act_noise": 21, "h_ref": 22, "h_scale": 23, "temb": 24,
    "r0": 30, "misc": 99,
}


def rng(seed: int, layer: int, role: str | int) -> np.random.Generator:
    tag = ROLE[role] if isinstance(role, str) else int(role)
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(layer), tag]))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # 32-bit sums cannot wrap for finite values (the largest, 0xFF7FFFFF,
    # plus 0x8000 stays below 2^32); NaN patterns are replaced below
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(dtype)


def random_bf16(seed, layer, role, shape, std=1.0, dtype="bf16"):
    g = rng(seed, layer, role)
    return _encode((g.standard_normal(shape, dtype=np.float32) * np.float32(std)), dtype)


def ffn_weights(seed: int, layer: int, d: int, ff: int, dtype: str = "bf16",
                down_layout: str = "df", std: float = 0.02,
                down_lognormal_sigma: float | None = None) -> dict:
    """GeGLU FFN weights, N(0, std).

    w_gate, w_up: [ff][d].  w_down: [d][ff] for ``down_layout='df'`` (the
    Context Cache path) or neuron-major [ff][d] for ``'fd'`` (the Action Cache
    path).  With ``down_lognormal_sigma`` each neuron's down weights are scaled
    by exp(sigma * z_n), z_n ~ N(0,1), so that contribution scores are spread
    the way a trained expert's are (a few heavy neurons, a long light tail).
    """
    wg = rng(seed, layer, "w_gate").standard_normal((ff, d), dtype=np.float32) * np.float32(std)
    wu = rng(seed, layer, "w_up").standard_normal((ff, d), dtype=np.float32) * np.float32(std)
    wd_fd = rng(seed, layer, "w_down").standard_normal((ff, d), dtype=np.float32) * np.float32(std)
    if down_lognormal_sigma:
        z = rng(seed, layer, "w_down_scale").standard_normal(ff).astype(np.float64)
        wd_fd = (wd_fd * np.exp(down_lognormal_sigma * z)[:, None]).astype(np.float32)
    wd = wd_fd if down_layout == "fd" else np.ascontiguousarray(wd_fd.T)
    return {
        "w_gate": _encode(wg, dtype), "w_up": _encode(wu, dtype), "w_down": _encode(wd, dtype),
        "d": d, "ff": ff, "dtype": dtype, "down_layout": down_layout,
    }


def ffn_weight_pool(seed: int, layers: int, d: int, ff: int, std: float = 0.02) -> list:
    """bf16 GeGLU weights of ``layers`` Context Cache layers (w_gate, w_up
    [ff][d], w_down [d][ff]) cut from one shared pool of N(0, std) values.

    The pool holds 2 ff d values; matrix m of layer l is the ff d consecutive
    values that start at a seeded offset (one draw per layer and matrix), so
    every layer gets different weights at the cost of drawing two matrices.
    Used where a deep full-size chain would otherwise spend minutes drawing
    independent weights; the arrays are views of the pool (do not write to them).
    """
    n = ff * d
    vals = rng(seed, 0, "w_gate").standard_normal(2 * n, dtype=np.float32)
    vals *= np.float32(std)
    pool = np.empty(2 * n, dtype=np.uint16)
    step = 1 << 22  # encode in chunks: small temporaries
    for c in range(0, 2 * n, step):
        pool[c: c + step] = f32_to_bf16_bits(vals[c: c + step])
    del vals
    out = []
    for l in range(layers):
        off = rng(seed, l, "w_down_scale").integers(0, n + 1, size=3)
        m = [pool[o: o + n] for o in off]
        out.append({"w_gate": m[0].reshape(ff, d), "w_up": m[1].reshape(ff, d),
                    "w_down": m[2].reshape(d, ff), "d": d, "ff": ff, "dtype": "bf16",
                    "down_layout": "df"})
    return out


def ctx_layer_inputs(seed: int, layer: int, P: int, d: int, n_changed: int,
                     sigma_changed: float, sigma_stable: float, dtype: str = "bf16") -> dict:
    """Current FFN input x ~ N(0,1) and reference input x_ref = x + sigma * N(0,1).

    ``n_changed`` tokens (a seeded permutation) get ``sigma_changed``; the rest
    get ``sigma_stable``.  For x ~ N(0,1) the expected cosine between x and
    x_ref is 1/sqrt(1 + sigma^2): sigma 1.3333 gives ~0.6, 0.1752 gives ~0.985.
    Returns bf16 bits (or f32) plus the planted changed set (sorted).
    """
    x = rng(seed, layer, "x").standard_normal((P, d), dtype=np.float32)
    noise = rng(seed, layer, "x_noise").standard_normal((P, d), dtype=np.float32)
    perm = rng(seed, layer, "perm").permutation(P)
    changed = np.sort(perm[:n_changed]).astype(np.int32)
    sig = np.full(P, sigma_stable, dtype=np.float32)
    sig[changed] = np.float32(sigma_changed)
    xr = x + noise * sig[:, None]
    return {"x": _encode(x, dtype), "x_ref": _encode(xr, dtype), "changed": changed}


def act_tokens(seed: int, layer: int, S: int, d: int, noise_sigma: float = 0.0,
               dtype: str = "bf16", role: str = "act_x") -> dict:
    """Action-token activations x ~ N(0,1) [S][d] and a perturbed copy x + sigma*N."""
    x = rng(seed, layer, role).standard_normal((S, d), dtype=np.float32)
    n = rng(seed, layer, "act_noise").standard_normal((S, d), dtype=np.float32)
    return {"x": _encode(x, dtype), "x_pert": _encode(x + np.float32(noise_sigma) * n, dtype)}


def synthetic_h_ref(seed: int, layer: int, T: int, ff: int, S: int,
                    neuron_sigma: float = 1.0) -> np.ndarray:
    """Stand-in post-GeGLU activations [T][ff][S] fp32 with per-neuron log-normal scale.

    Used where the mask builder is exercised at full size without running a
    dense reference pass: a product of two normals per element (GeGLU-like
    heavy tails) times exp(neuron_sigma * z_n).
    """
    g = rng(seed, layer, "h_ref")
    a = g.standard_normal((T, ff, S), dtype=np.float32)
    b = g.standard_normal((T, ff, S), dtype=np.float32)
    z = rng(seed, layer, "h_scale").standard_normal(ff).astype(np.float32)
    return np.ascontiguousarray((a * b) * np.exp(np.float32(neuron_sigma) * z)[None, :, None],
                                dtype=np.float32)


def timestep_embedding(t_frac: float, d: int) -> np.ndarray:
    """Sinusoidal timestep embedding [d] fp32 (synthetic glue, not part of the FFN)."""
    half = d // 2
    freqs = np.exp(-np.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    ang = 1000.0 * float(t_frac) * freqs
    return np.concatenate([np.sin(ang), np.cos(ang)]).astype(np.float32)
