"""Plain, slow CPU oracle of the cache-guided selective FFN.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library: it decodes bf16 bit patterns itself, does all
FFN arithmetic in float64 with NumPy, and makes every selection with Python's
``sorted``.

Source of the method: Zhou, Li, Chen, Gu, "rMuscle: Robotic Muscle Memory for
Efficient Vision-Language-Action Model Inference" (called "the paper" below).

Selections (token top-k, neuron masks) follow a fixed-point reading of the
paper's real-valued scores: each per-element term is a correctly rounded IEEE
float64 operation (no fused multiply-add) rounded half-to-even to an int64 at a
fixed resolution, and every accumulation is an int64 sum, which is exact and
independent of summation order.  The final key is formed from those integers
with correctly rounded float64 operations.  The real-valued Eq. 1 / Eq. 2
rankings agree with these keys except where two scores lie within the fixed
resolution of each other.

Activations are bf16 between the two projections of the FFN (the hidden
activation h and the masked delta are rounded to bf16 before the down
projection), matching a bf16 model with float accumulation; the oracle rounds
the exact float64 value once, half-to-even.

Pins for every function live in ``tests/test_oracle_*.py``.  No function here
is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-6            # paper §4.1, Eq. 2: epsilon in max(RMS(x), eps)
RMS_NORM_EPS = 1e-6   # synthetic inter-layer RMSNorm (no learned scale)
F_SCORE = 24          # fraction bits of the token-score fixed point
F_ACT = 24            # fraction bits of |h| in the contribution score
F_W = 40              # fraction bits of w^2 in the down-weight norm

__all__ = [
    "EPS", "decode", "round_to_bf16_bits", "round_act", "ratio_to_count",
    "score_floor", "ctx_score_keys", "topk_ascending", "ctx_select",
    "gelu_tanh", "ffn_geglu", "ctx_ffn_recompute", "contribution_scores",
    "down_weight_norms", "mask_topk", "coverage_exponent_bits", "mask_coverage", "act_build_mask", "mask_bits",
    "mask_indices",
    "act_ffn_masked", "act_ffn_joint", "rms_norm", "rebuild_dense", "entry_bytes",
]


# --------------------------------------------------------------------------
# Encoding
# --------------------------------------------------------------------------
def decode(a, dtype: str) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> exact float64 values."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), return uint16 bits."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    fin = np.isfinite(v) & (v != 0)
    _, e = np.frexp(np.where(fin, v, 1.0))          # v = m * 2^e, 0.5 <= |m| < 1
    q_exp = np.maximum(e, -125) - 8                  # bf16 spacing in that binade
    q = np.ldexp(np.ones_like(v), q_exp)
    out[...] = np.where(fin, np.rint(v / q) * q, v)  # exact scaling, round half even
    out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, out), out)
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def round_act(v, dtype: str) -> np.ndarray:
    """Value of an activation materialised in ``dtype`` (bf16 or f32), as float64."""
    if dtype == "bf16":
        return decode(round_to_bf16_bits(v), "bf16")
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Ratios
# --------------------------------------------------------------------------
def ratio_to_count(rho: float, n: int) -> int:
    """ceil(rho * n) as in paper §4.1 (top ceil(rho_p P) tokens) and §5
    (K_l = ceil(rho_n H_l)); a 1e-9 guard absorbs products such as
    0.07 * 100 = 7.000000000000001.  Clamped to [0, n]."""
    k = math.ceil(float(rho) * int(n) - 1e-9)
    return int(min(max(k, 0), int(n)))


# --------------------------------------------------------------------------
# Context Cache: token score (Eq. 2) and top-k selection
# --------------------------------------------------------------------------
def score_floor(d: int) -> int:
    """d * eps^2 in fixed point, rounded up and at least 1: max(1, ceil(d * 2^F / 10^12))."""
    return max(1, -((-d * (1 << F_SCORE)) // 10 ** 12))


def _fixed_sum(terms: np.ndarray, frac_bits: int) -> np.ndarray:
    """Row sums of rint(2^frac_bits * term) as exact int64 (term already fl64)."""
    q = np.rint(np.ldexp(terms, frac_bits))
    if np.any(np.abs(q) >= 2.0 ** 62):
        raise OverflowError("fixed-point term out of range")
    return q.astype(np.int64).sum(axis=-1)


def ctx_score_keys(x, x_ref, dtype: str = "bf16", kind: str = "rel_rms") -> np.ndarray:
    """Per-token change score of paper §4.1, Eq. 2.

    d_p = RMS(x_p - xbar_p) / max(RMS(x_p), eps).  Squaring and multiplying by d
    gives the monotone equivalent d_p^2 = S_diff / max(S_xx, d eps^2), which is
    the key computed here in fixed point:
      Sd = sum_j rint(2^24 fl64((x_j - xbar_j)^2)),  Sx = sum_j rint(2^24 fl64(x_j^2)),
      key = fl64( fl64(Sd) / fl64(max(Sx, E)) ),     E = score_floor(d).
    ``kind='cosine'`` ranks by cosine distance instead:
      key = 1 - q|q| / (Sx Sy) with q = Sxy (key = 1 when Sx Sy = 0);
    larger keys mean larger change in both kinds.
    """
    xd = decode(x, dtype)
    rd = decode(x_ref, dtype)
    if xd.ndim != 2 or xd.shape != rd.shape:
        raise ValueError("x and x_ref must both be [P][d]")
    P, d = xd.shape
    Sx = _fixed_sum(xd * xd, F_SCORE)
    if kind == "rel_rms":
        diff = xd - rd
        Sd = _fixed_sum(diff * diff, F_SCORE)
        den = np.maximum(Sx, score_floor(d))
        return Sd.astype(np.float64) / den.astype(np.float64)
    if kind == "cosine":
        Sy = _fixed_sum(rd * rd, F_SCORE)
        Sxy = _fixed_sum(xd * rd, F_SCORE)
        keys = np.empty(P, dtype=np.float64)
        for p in range(P):
            q = float(Sxy[p])
            den = float(Sx[p]) * float(Sy[p])
            keys[p] = 1.0 if den == 0.0 else 1.0 - (q * abs(q)) / den
        return keys
    raise ValueError(kind)


def topk_ascending(keys, k: int) -> np.ndarray:
    """Indices of the k largest keys (ties go to the lower index), in ascending order.

    Brute force: sort every index by (key descending, index ascending)."""
    keys = np.asarray(keys, dtype=np.float64)
    order = sorted(range(len(keys)), key=lambda p: (-float(keys[p]), p))
    return np.array(sorted(order[:k]), dtype=np.int32)


def ctx_select(x, x_ref, k: int, dtype: str = "bf16", kind: str = "rel_rms"):
    """Paper §4.1: the set P_l(rho_p) of the ceil(rho_p P) tokens with the largest
    Eq. 2 scores; uses FFN inputs only.  Returns (idx ascending int32, keys fp64)."""
    keys = ctx_score_keys(x, x_ref, dtype, kind)
    if not 0 <= k <= len(keys):
        raise ValueError("k out of range")
    return topk_ascending(keys, k), keys


# --------------------------------------------------------------------------
# FFN
# --------------------------------------------------------------------------
def gelu_tanh(g):
    """GELU, tanh form (Hendrycks & Gimpel): 0.5 g (1 + tanh(sqrt(2/pi)(g + 0.044715 g^3)))."""
    g = np.asarray(g, dtype=np.float64)
    return 0.5 * g * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)))


def _weights64(w: dict):
    """Decode FFN weights; returns gate [ff][d], up [ff][d], down neuron-major [ff][d]."""
    dt = w["dtype"]
    wg = decode(w["w_gate"], dt)
    wu = decode(w["w_up"], dt)
    wd = decode(w["w_down"], dt)
    if w["down_layout"] == "df":       # stored [d][ff] (output-major)
        wd = wd.T
    elif w["down_layout"] != "fd":     # stored [ff][d] (neuron-major)
        raise ValueError(w["down_layout"])
    return wg, wu, wd


def ffn_geglu(x64: np.ndarray, w: dict) -> np.ndarray:
    """GeGLU FFN F(x) = (gelu(x W_gate^T) * (x W_up^T)) W_down, float64; the hidden
    activation is materialised in the activation dtype before the down projection."""
    wg, wu, wd = _weights64(w)
    h = gelu_tanh(x64 @ wg.T) * (x64 @ wu.T)
    return round_act(h, w["dtype"]) @ wd


def ctx_ffn_recompute(w: dict, x, y_ref, idx):
    """Paper §4.1, Eq. 3: y_p = F(x_p) for p in the selected set, y_p = ybar_p otherwise.

    Selected rows are returned as float64 (before output rounding); the other
    rows carry the reference bits unchanged.  Returns (y64 [P][d], recomputed
    bool [P]); for unselected rows y64 holds decode(y_ref)."""
    dt = w["dtype"]
    idx = np.asarray(idx, dtype=np.int64)
    P = np.asarray(x).shape[0]
    if len(idx) and (np.any(np.diff(idx) <= 0) or idx[0] < 0 or idx[-1] >= P):
        raise ValueError("idx must be ascending, unique and in [0, P)")
    y = decode(y_ref, dt).copy()
    if len(idx):
        y[idx] = ffn_geglu(decode(x, dt)[idx], w)
    rec = np.zeros(P, dtype=bool)
    rec[idx] = True
    return y, rec


# --------------------------------------------------------------------------
# Action Cache: contribution score (Eq. 1) and group masks (§5)
# --------------------------------------------------------------------------
def down_weight_norms(w: dict) -> np.ndarray:
    """Paper §3.4, Eq. 1: the factor ||W_n||_2 of every neuron n, in fixed point:
      B[n] = sum_j rint(2^40 fl64(w_nj^2)) (int64),  nrm[n] = sqrt(fl64(B[n]))
    (correctly rounded; the common factor 2^20 is immaterial).  Returns nrm [ff] fp64."""
    _, _, wd = _weights64(w)
    B = _fixed_sum(wd * wd, F_W)
    return np.sqrt(B.astype(np.float64))


def contribution_scores(h_ref, w: dict):
    """Paper §3.4, Eq. 1: c_{t,n} = (sum_r |h_{t,r,n}|) * ||W_n||_2, in fixed point.

    h_ref: [T][ff][S] float32 post-GeGLU activations of the group's reference
    steps; W_n: neuron n's down-projection weights.
      A[t,n] = sum_r rint(2^24 |h|)            (int64)
      B[n]   = sum_j rint(2^40 fl64(w_nj^2))   (int64)
      nrm[n] = sqrt(fl64(B[n]))                (correctly rounded)
      c[t,n] = fl64(fl64(A[t,n]) * nrm[n]),   s[n] = fl64(fl64(sum_t A[t,n]) * nrm[n])
    The common factor 2^44 changes neither rankings nor coverage ratios.
    Returns (c [T][ff] fp64, s [ff] fp64)."""
    h = np.asarray(h_ref, dtype=np.float32).astype(np.float64)
    if h.ndim != 3:
        raise ValueError("h_ref must be [T][ff][S]")
    A = _fixed_sum(np.abs(h), F_ACT)                     # [T][ff]
    nrm = down_weight_norms(w)                           # [ff]
    c = A.astype(np.float64) * nrm[None, :]
    s = A.sum(axis=0).astype(np.float64) * nrm
    return c, s


def _desc_order(v) -> list:
    return sorted(range(len(v)), key=lambda n: (-float(v[n]), n))


def mask_topk(c, s, K: int) -> np.ndarray:
    """Paper §5 (constructing group neuron masks): the top K neurons of every step,
    their union within the group, ranked by summed contribution, top K kept.
    Returns ascending neuron indices."""
    c = np.asarray(c, dtype=np.float64)
    ff = c.shape[1]
    if not 0 <= K <= ff:
        raise ValueError("K out of range")
    union = set()
    for t in range(c.shape[0]):
        union.update(_desc_order(c[t])[:K])
    ranked = sorted(union, key=lambda n: (-float(s[n]), n))
    return np.array(sorted(ranked[:K]), dtype=np.int32)


def coverage_exponent_bits(ff: int) -> int:
    """Fixed-point bits below the top score's binade in the coverage cut, so that
    ff terms below 2^(Q+1) sum below 2^62."""
    return 61 - (int(ff) - 1).bit_length()


def mask_coverage(s, tau: float) -> np.ndarray:
    """Coverage cut (paper §3.4, coverage = share of total contribution held by
    the top-ranked neurons): the shortest prefix of neurons ordered by
    (s descending, index ascending) whose share of the total reaches tau.

    In fixed point: e = ilogb(max s) - Q, z_n = rint(s_n 2^-e) (int64), Z = sum z;
    m = smallest m with fl64(sum of the first m z) >= fl64(tau * fl64(Z)).
    Returns ascending neuron indices (empty when every score is 0)."""
    s = np.asarray(s, dtype=np.float64)
    ff = len(s)
    if not 0.0 <= tau <= 1.0:
        raise ValueError("coverage must lie in [0, 1]")
    smax = float(s.max()) if ff else 0.0
    if smax <= 0.0:
        return np.zeros(0, dtype=np.int32)
    e = (math.frexp(smax)[1] - 1) - coverage_exponent_bits(ff)
    z = np.rint(np.ldexp(s, -e)).astype(np.int64)
    Z = int(z.sum())
    thr = float(tau) * float(Z)
    order = _desc_order(s)
    acc = 0
    m = 0
    while float(acc) < thr:
        acc += int(z[order[m]])
        m += 1
    return np.array(sorted(order[:m]), dtype=np.int32)


def mask_bits(idx, ff: int) -> np.ndarray:
    """Bit-packed mask: bit (n mod 64) of word n // 64 set for every n in idx."""
    words = np.zeros((ff + 63) // 64, dtype=np.uint64)
    for n in np.asarray(idx, dtype=np.int64):
        words[n // 64] |= np.uint64(1) << np.uint64(n % 64)
    return words


def mask_indices(words, ff: int) -> np.ndarray:
    """A stored bit-packed mask read back as its neuron list (paper §5: the
    group masks kept with a cache entry; §4.1: a masked step reads the mask's
    neurons): every n < ff whose bit (n mod 64) of word n // 64 is set,
    ascending.  Bits at positions >= ff are not neurons and are ignored."""
    words = [int(w) & ((1 << 64) - 1) for w in np.asarray(words).ravel()]
    kept = []
    for n in range(int(ff)):
        if (words[n // 64] >> (n % 64)) & 1:
            kept.append(n)
    return np.array(kept, dtype=np.int32)


def act_build_mask(h_ref, w: dict, mode: str, K: int = 0, coverage: float = 0.0):
    """Group mask from the reference steps' activations: ``mode='topk'`` is the
    paper's §5 rule with K_l = K, ``mode='coverage'`` keeps top neurons until the
    coverage share is reached.  Returns (idx ascending int32, bit words)."""
    c, s = contribution_scores(h_ref, w)
    if mode == "topk":
        idx = mask_topk(c, s, K)
    elif mode == "coverage":
        idx = mask_coverage(s, coverage)
    else:
        raise ValueError(mode)
    return idx, mask_bits(idx, c.shape[1])


# --------------------------------------------------------------------------
# Action Cache: masked FFN with a dense anchor (Eq. 4)
# --------------------------------------------------------------------------
def act_ffn_masked(w: dict, x, idx, y_anchor=None, h_anchor=None):
    """Paper §4.1, Eq. 4: y_t = y_a + (h_t^M - h_a^M) W^down_M.

    x: [S][d] (post-RMSNorm); idx: the mask M (ascending); y_anchor: [S][d]
    float32 or None; h_anchor: [ff][S] float32 or None.  Only the rows M of
    W_gate, W_up and of the neuron-major W_down enter.  Without anchors this
    is the plain masked FFN, and with M = all neurons the dense FFN (the
    anchor step).  The delta (h_t - h_a) is materialised in the activation
    dtype.  Returns (y float64 [S][d], h float64 [K][S] for the rows of M)."""
    dt = w["dtype"]
    idx = np.asarray(idx, dtype=np.int64)
    wg, wu, wd = _weights64(w)
    xs = decode(x, dt)
    S = xs.shape[0]
    h = gelu_tanh(xs @ wg[idx].T) * (xs @ wu[idx].T)            # [S][K]
    ha = 0.0 if h_anchor is None else \
        np.asarray(h_anchor, dtype=np.float32).astype(np.float64)[idx].T
    delta = round_act(h - ha, dt)
    y = delta @ wd[idx]
    if y_anchor is not None:
        y = np.asarray(y_anchor, dtype=np.float32).astype(np.float64) + y
    if len(idx) == 0:
        y = np.zeros((S, wd.shape[1])) if y_anchor is None else \
            np.asarray(y_anchor, dtype=np.float32).astype(np.float64).copy()
    return y, h.T.copy()


def act_ffn_joint(w: dict, x, tok, idx, y_anchor, h_anchor):
    """Paper §6.1 (visual-token and neuron sparsity together inside the
    denoising loop): Eq. 4 on the rows tok of x with the mask idx and the
    anchor state of those rows; every other row keeps the anchor output.
    Returns y float64 [S][d]."""
    tok = np.asarray(tok, dtype=np.int64)
    ya = np.asarray(y_anchor, dtype=np.float32).astype(np.float64)
    y = ya.copy()
    if len(tok):
        xs = np.asarray(x)[tok]
        ha = np.asarray(h_anchor, dtype=np.float32)[:, tok]
        y[tok], _ = act_ffn_masked(w, xs, idx, np.asarray(y_anchor, dtype=np.float32)[tok], ha)
    return y


# --------------------------------------------------------------------------
# Dense reference rebuild (paper §4.2, asynchronous online reconstruction)
# --------------------------------------------------------------------------
def rms_norm(r64: np.ndarray) -> np.ndarray:
    """RMSNorm without a learned scale: v / sqrt(mean(v^2) + 1e-6), float64."""
    ms = (r64 * r64).sum(axis=-1) / r64.shape[-1]
    return r64 / np.sqrt(ms + RMS_NORM_EPS)[..., None]


def rebuild_dense(layers: list, r0):
    """Expand a compact entry: the dense prefill that produces the reference FFN
    inputs and outputs (xbar_l, ybar_l) of every layer.

    r_0 = entry; xbar_l = act(RMSNorm(r_l)); ybar_l = F_l(xbar_l);
    r_{l+1} = r_l + act(ybar_l).  Returns (xbar bits or f32 [L][P][d], ybar
    float64 [L][P][d])."""
    dt = layers[0]["dtype"]
    r = decode(r0, dt)
    xs, ys = [], []
    for w in layers:
        xn = rms_norm(r)
        if dt == "bf16":
            xb = round_to_bf16_bits(xn)
        else:
            xb = xn.astype(np.float32)
        y = ffn_geglu(decode(xb, dt), w)
        xs.append(xb)
        ys.append(y)
        r = r + round_act(y, dt)
    return np.stack(xs), np.stack(ys)


def entry_bytes(layers: int, P: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes of one expanded reference entry: a (xbar, ybar) pair of [P][d] per layer."""
    return layers * 2 * P * d * elem_bytes
