"""Python binding of libcgs, the cache-guided selective FFN for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libcgs.so``.  PyTorch supplies device memory (tensors) and the
current stream; it computes nothing here.  If the library has not been built
the import succeeds but every call raises, so no path silently falls back.

Entry points mirror ``include/cgs.h``: ``ctx_select``, ``ctx_ffn_recompute``,
``act_build_mask``, ``act_ffn_masked``, ``ref_rebuild_dense`` and the
``residual_rmsnorm`` glue.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcgs.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "cgs.h")

CGS_BF16, CGS_F32 = 0, 1
CGS_SCORE_REL_RMS, CGS_SCORE_COSINE = 0, 1
CGS_MASK_TOPK, CGS_MASK_COVERAGE = 0, 1
CGS_DOWN_DF, CGS_DOWN_FD = 0, 1
CGS_OK, CGS_ERR_ARG, CGS_ERR_SHAPE, CGS_ERR_WORKSPACE = 0, 1, 2, 3
CGS_ERR_UNSUPPORTED, CGS_ERR_LAUNCH, CGS_ERR_DATA, CGS_ERR_TIMEOUT = 4, 5, 6, 7

_KIND = {"rel_rms": CGS_SCORE_REL_RMS, "cosine": CGS_SCORE_COSINE}
_MODE = {"topk": CGS_MASK_TOPK, "coverage": CGS_MASK_COVERAGE}
_LAYOUT = {"df": CGS_DOWN_DF, "fd": CGS_DOWN_FD}


class CgsError(RuntimeError):
    """A libcgs call failed; ``status`` is its cgs_status code (0 when the
    binding itself refused the call)."""

    def __init__(self, msg: str, status: int = 0):
        super().__init__(msg)
        self.status = status


class _Glue(ctypes.Structure):
    _fields_ = [("r", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("x_next", ctypes.c_void_p),
                ("score_ref", ctypes.c_void_p), ("score_key", ctypes.c_void_p),
                ("score_kind", ctypes.c_int32)]


def _glue(glue):
    """Optional residual/RMSNorm glue -> cgs_glue pointer or None.

    ``glue`` = (r, bias, x_next) or (r, bias, x_next, score_ref, score_key[, kind]):
    r += y (+ bias), x_next = RMSNorm(r), and optionally the Eq. 2 keys of x_next
    against score_ref into score_key (float64 [rows])."""
    if glue is None:
        return None
    r, bias, x_next = glue[:3]
    score_ref = glue[3] if len(glue) > 3 else None
    score_key = glue[4] if len(glue) > 4 else None
    kind = _KIND[glue[5]] if len(glue) > 5 else CGS_SCORE_REL_RMS
    if r is None or r.dtype != torch.float32:
        raise CgsError("glue residual r must be a float32 device tensor")
    if score_key is not None and score_key.dtype != torch.float64:
        raise CgsError("glue score_key must be a float64 device tensor")
    return ctypes.byref(_Glue(_ptr(r), _ptr(bias), _ptr(x_next), _ptr(score_ref), _ptr(score_key), kind))


class _Ffn(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("ff", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("down_layout", ctypes.c_int32), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


_lib = None
_vp, _i, _sz, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
_SIGS = {
    "cgs_ratio_to_count": (_i, [_d, _i]),
    "cgs_status_str": (ctypes.c_char_p, [_i]),
    "cgs_version": (_i, []),
    "cgs_set_validate": (_i, [_i]),
    "cgs_ctx_select_workspace": (_sz, [_i, _i]),
    "ctx_select": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "ctx_select_from_keys": (_i, [_vp, _i, _i, _vp, _vp]),
    "cgs_ctx_ffn_recompute_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "ctx_ffn_recompute": (_i, [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "cgs_act_build_mask_workspace": (_sz, [_i, _i, _i, _i]),
    "act_build_mask": (_i, [_vp, _i, _i, _vp, _i, _i, _d, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cgs_act_build_masks_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "act_build_masks": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _d, _vp, _vp, _vp, _vp, _sz, _vp]),
    "act_down_norms": (_i, [_vp, _i, _vp, _vp]),
    "act_build_masks_normed": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _i, _d, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cgs_act_ffn_masked_workspace": (_sz, [_i, _i, _i, _i]),
    "act_ffn_masked": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "act_ffn_masked_compact": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "act_ffn_masked_compact_noalloc": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "act_gather_rows": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp]),
    "act_gather_rows_layers": (_i, [_vp, _i, _vp]),
    "cgs_ref_rebuild_dense_batch_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "ref_rebuild_dense_batch": (_i, [_vp, _i, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "act_mask_indices": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "cgs_denoise_schedule": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "cgs_act_masked_layers_workspace": (_sz, [_i, _i, _i]),
    "act_masked_layers": (_i, [_vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "act_ffn_joint": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cgs_ref_rebuild_dense_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "ref_rebuild_dense": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _sz, _vp]),
    "cgs_residual_rmsnorm": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _vp, _i, _vp]),
    "cgs_ret_select_workspace": (_sz, [_i, ctypes.c_longlong]),
    "ret_select": (_i, [_vp, _vp, _i, ctypes.c_longlong, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                        _sz, _vp]),
    "cgs_prep_budget": (_i, [_i, _d, _d, _d, _d, _d]),
    "cgs_window_create": (_vp, [_i]),
    "cgs_window_destroy": (None, [_vp]),
    "cgs_window_slot": (_i, [_vp, _i, _i]),
    "cgs_window_resident": (_i, [_vp]),
    "cgs_window_advance": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "act_gather_rows_t": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _vp]),
    "cgs_act_denoise_step_workspace": (_sz, [_i, _i, _i, _i]),
    "act_denoise_step": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cgs_set_step_wait_limit": (ctypes.c_longlong, [ctypes.c_longlong]),
    "cgs_profile_start": (_i, [ctypes.c_char_p, _i]),
    "cgs_profile_stop": (_i, []),
    "cgs_profile_result": (_i, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_int)]),
}


def lib():
    """The loaded libcgs (raises CgsError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CgsError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise CgsError(f"{what}: {lib().cgs_status_str(status).decode()} (status {status})", status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CGS_BF16
    if t.dtype == torch.float32:
        return CGS_F32
    raise CgsError(f"unsupported dtype {t.dtype}")


def _expect(t, name: str, dtype=None, shape=None, required: bool = True):
    """Refuse a tensor whose dtype or shape is not what the C call will read
    or write (the kernels size every access from the FFN struct and the counts
    passed, so a mismatch would address memory outside the tensor)."""
    if t is None:
        if required:
            raise CgsError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise CgsError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise CgsError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise CgsError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _expect_index(t, name: str, n=None, required: bool = True):
    """An index list: 1-D int32 (of n entries when n is given)."""
    _expect(t, name, torch.int32, None if n is None else (n,), required)
    if t is not None and t.dim() != 1:
        raise CgsError(f"{name} must be 1-D")


def _expect_glue(glue, rows: int, d: int, dt):
    """Shapes of the residual/RMSNorm glue tensors for `rows` rows of width d."""
    if glue is None:
        return
    r, bias, x_next = glue[:3]
    _expect(r, "glue residual r", torch.float32, (rows, d))
    _expect(bias, "glue bias", torch.float32, (d,), required=False)
    _expect(x_next, "glue x_next", dt, (rows, d), required=False)
    if len(glue) > 3:
        _expect(glue[3], "glue score_ref", dt, (rows, d), required=False)
    if len(glue) > 4:
        _expect(glue[4], "glue score_key", torch.float64, (rows,), required=False)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise CgsError("tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


_ws_cache: dict = {}
_ws_retired: list = []


def workspace(nbytes: int, device, tag: str = "default", stream=None) -> torch.Tensor:
    """A cached workspace of at least nbytes for (device, stream, tag).

    Calls on one stream run in order and may share a buffer; calls on other
    streams get their own, so concurrent streams never share scratch memory.
    A buffer outgrown by a larger request is kept allocated for the life of
    the process: a captured HIP graph, or a kernel still queued, may address
    it.  Growth is geometric, so few buffers are ever retired."""
    dev = torch.device(device)
    skey = _stream(stream) if dev.type == "cuda" else 0
    key = (str(dev), skey, tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        size = max(int(nbytes), 256)
        if buf is not None:
            _ws_retired.append(buf)
            size = max(size, 2 * buf.numel())
        buf = torch.empty(size, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


@dataclass
class FFN:
    """Device weights of one GeGLU FFN: w_gate, w_up [ff][d]; w_down [d][ff]
    (``layout='df'``) or neuron-major [ff][d] (``'fd'``)."""
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    layout: str = "df"

    @property
    def d(self) -> int:
        return self.w_gate.shape[1]

    @property
    def ff(self) -> int:
        return self.w_gate.shape[0]

    @property
    def dtype(self):
        return self.w_gate.dtype

    def cstruct(self) -> _Ffn:
        dt = _dtype_code(self.w_gate)
        if self.w_gate.dim() != 2 or tuple(self.w_up.shape) != tuple(self.w_gate.shape):
            raise CgsError("FFN w_gate and w_up must both be [ff][d]")
        want = (self.ff, self.d) if self.layout == "fd" else (self.d, self.ff)
        if tuple(self.w_down.shape) != want:
            raise CgsError(f"FFN w_down must be {want} for layout {self.layout!r}")
        for t in (self.w_up, self.w_down):
            if _dtype_code(t) != dt:
                raise CgsError("FFN weights must share one dtype")
        return _Ffn(self.d, self.ff, dt, _LAYOUT[self.layout], _ptr(self.w_gate),
                    _ptr(self.w_up), _ptr(self.w_down))


def set_validate(on: bool) -> bool:
    """Checked mode (debugging): calls first verify their documented device-data
    preconditions and raise CgsError (status CGS_ERR_DATA) on a violation;
    synchronises streams, so a checked call on a stream under graph capture
    raises CgsError (CGS_ERR_UNSUPPORTED) before enqueuing anything.  Returns
    the previous setting."""
    return bool(lib().cgs_set_validate(1 if on else 0))


def ratio_to_count(rho: float, n: int) -> int:
    return int(lib().cgs_ratio_to_count(float(rho), int(n)))


def ctx_select(x, x_ref, k: int, kind: str = "rel_rms", idx_out=None, key_out=None,
               ws=None, stream=None):
    """Top-k token indices (ascending int32) by the Eq. 2 drift score."""
    _expect(x, "x")
    if x.dim() != 2:
        raise CgsError("x must be [P][d]")
    P, d = x.shape
    _dtype_code(x)
    _expect(x_ref, "x_ref", x.dtype, (P, d))
    if idx_out is None:
        idx_out = torch.empty(k, dtype=torch.int32, device=x.device)
    _expect_index(idx_out, "idx_out", int(k))
    _expect(key_out, "key_out", torch.float64, (P,), required=False)
    nbytes = lib().cgs_ctx_select_workspace(P, d)
    ws = workspace(nbytes, x.device, "select", stream) if ws is None else ws
    _check(lib().ctx_select(_ptr(x), _ptr(x_ref), P, d, _dtype_code(x), int(k), _KIND[kind],
                            _ptr(idx_out), _ptr(key_out), _ptr(ws), ws.numel(), _stream(stream)),
           "ctx_select")
    return idx_out


def ctx_select_from_keys(keys, k: int, idx_out=None, stream=None):
    """The k highest of precomputed Eq. 2 keys (float64 [P]), indices ascending."""
    _expect(keys, "keys", torch.float64)
    P = int(keys.numel())
    if idx_out is None:
        idx_out = torch.empty(int(k), dtype=torch.int32, device=keys.device)
    _expect_index(idx_out, "idx_out", int(k))
    _check(lib().ctx_select_from_keys(_ptr(keys), P, int(k), _ptr(idx_out), _stream(stream)),
           "ctx_select_from_keys")
    return idx_out


def ctx_ffn_recompute(w: FFN, x, y_ref, idx, y_out=None, glue=None, ws=None, stream=None):
    """Eq. 3: F(x) on the rows idx, the reference outputs elsewhere.  ``glue`` =
    (r, bias, x_next) applies r += y (+ bias), x_next = RMSNorm(r) per row."""
    c = w.cstruct()
    _expect(x, "x", w.dtype)
    if x.dim() != 2 or x.shape[1] != w.d:
        raise CgsError(f"x must be [P][{w.d}]")
    P, d = x.shape
    _expect(y_ref, "y_ref", w.dtype, (P, d))
    _expect_index(idx, "idx")
    k = int(idx.numel())
    if y_out is None:
        y_out = torch.empty_like(y_ref)
    _expect(y_out, "y_out", w.dtype, (P, d))
    _expect_glue(glue, P, d, w.dtype)
    nbytes = lib().cgs_ctx_ffn_recompute_workspace(k, P, d, w.ff, c.dtype)
    ws = workspace(nbytes, x.device, "ctx", stream) if ws is None else ws
    _check(lib().ctx_ffn_recompute(ctypes.byref(c), _ptr(x), _ptr(y_ref), _ptr(idx), k, P,
                                   _ptr(y_out), _glue(glue), _ptr(ws), ws.numel(), _stream(stream)),
           "ctx_ffn_recompute")
    return y_out


def act_build_mask(h_ref, w: FFN, mode: str = "topk", K: int = 0, coverage: float = 0.0,
                   mask_out=None, idx_out=None, count_out=None, ws=None, stream=None):
    """Group mask from the reference steps' activations h_ref [T][ff][S] (fp32).
    Returns (mask words uint64 as int64 tensor, idx int32 [ff], count int32 [1])."""
    c = w.cstruct()
    _expect(h_ref, "h_ref", torch.float32)
    if h_ref.dim() != 3 or h_ref.shape[1] != w.ff:
        raise CgsError(f"h_ref must be [T][{w.ff}][S]")
    T, ff, S = h_ref.shape
    dev = h_ref.device
    if mask_out is None:
        mask_out = torch.empty((ff + 63) // 64, dtype=torch.int64, device=dev)
    if idx_out is None:
        idx_out = torch.empty(ff, dtype=torch.int32, device=dev)
    if count_out is None:
        count_out = torch.empty(1, dtype=torch.int32, device=dev)
    _expect(mask_out, "mask_out", torch.int64, ((ff + 63) // 64,))
    _expect_index(idx_out, "idx_out", ff)
    _expect(count_out, "count_out", torch.int32, (1,))
    nbytes = lib().cgs_act_build_mask_workspace(T, S, ff, w.d)
    ws = workspace(nbytes, dev, "mask", stream) if ws is None else ws
    _check(lib().act_build_mask(_ptr(h_ref), T, S, ctypes.byref(c), _MODE[mode], int(K),
                                float(coverage), _ptr(mask_out), _ptr(idx_out), _ptr(count_out),
                                _ptr(ws), ws.numel(), _stream(stream)), "act_build_mask")
    return mask_out, idx_out, count_out


def act_down_norms(layers, out=None, stream=None):
    """Eq. 1's down-projection norms of each layer's W_down (layout 'fd'),
    float64 [layers][ff]; a property of the weights, computed once."""
    Lr = len(layers)
    ff = layers[0].ff
    arr = (_Ffn * Lr)(*[w.cstruct() for w in layers])
    if out is None:
        out = torch.empty((Lr, ff), dtype=torch.float64, device=layers[0].w_down.device)
    _expect(out, "out", torch.float64, (Lr, ff))
    _check(lib().act_down_norms(arr, Lr, _ptr(out), _stream(stream)), "act_down_norms")
    return out


def act_mask_indices(masks, ff: int, idx_out=None, count_out=None, stream=None):
    """Stored bit-packed masks [..., ceil(ff/64)] int64 (bit i%64 of word i/64
    = neuron i) -> (idx [..., ff] int32 ascending then -1, count [...] int32)."""
    ff = int(ff)
    words = (ff + 63) // 64
    _expect(masks, "masks", torch.int64)
    if masks.dim() < 1 or masks.shape[-1] != words:
        raise CgsError(f"masks must be [..., {words}] int64 words for ff = {ff}")
    lead = tuple(masks.shape[:-1])
    n = 1
    for v in lead:
        n *= int(v)
    if idx_out is None:
        idx_out = torch.empty(lead + (ff,), dtype=torch.int32, device=masks.device)
    if count_out is None:
        count_out = torch.empty(lead, dtype=torch.int32, device=masks.device)
    _expect(idx_out, "idx_out", torch.int32, lead + (ff,))
    _expect(count_out, "count_out", torch.int32, lead)
    _check(lib().act_mask_indices(_ptr(masks), n, ff, _ptr(idx_out), _ptr(count_out), _stream(stream)),
           "act_mask_indices")
    return idx_out, count_out


def act_build_masks(h_ref, layers, mode: str = "topk", K: int = 0, coverage: float = 0.0,
                    mask_out=None, idx_out=None, count_out=None, ws=None, stream=None, norms=None):
    """Group masks of several layers at once: h_ref [layers][T][ff][S] float32,
    layers = list of FFN (layout 'fd'); returns (mask words [layers][words],
    idx [layers][ff], count [layers]).  With ``norms`` (act_down_norms of the
    same weights) the weights are not read and ``layers`` may be None."""
    _expect(h_ref, "h_ref", torch.float32)
    if h_ref.dim() != 4:
        raise CgsError("h_ref must be [layers][T][ff][S]")
    Lr, T, ff, S = h_ref.shape
    if norms is None and layers is not None and any(w.ff != ff for w in layers):
        raise CgsError("act_build_masks: h_ref's ff differs from the layers'")
    if norms is None and (layers is None or len(layers) != Lr):
        raise CgsError("act_build_masks: one FFN per layer of h_ref")
    if norms is not None and tuple(norms.shape) != (Lr, ff):
        raise CgsError("act_build_masks: norms must be [layers][ff]")
    dev = h_ref.device
    words = (ff + 63) // 64
    if mask_out is None:
        mask_out = torch.empty((Lr, words), dtype=torch.int64, device=dev)
    if idx_out is None:
        idx_out = torch.empty((Lr, ff), dtype=torch.int32, device=dev)
    if count_out is None:
        count_out = torch.empty(Lr, dtype=torch.int32, device=dev)
    _expect(mask_out, "mask_out", torch.int64, (Lr, words))
    _expect(idx_out, "idx_out", torch.int32, (Lr, ff))
    _expect(count_out, "count_out", torch.int32, (Lr,))
    nbytes = lib().cgs_act_build_masks_workspace(Lr, T, S, ff, 1)
    ws = workspace(nbytes, dev, "mask", stream) if ws is None else ws
    if norms is not None:
        if norms.dtype != torch.float64:
            raise CgsError("act_build_masks: norms must be float64")
        _check(lib().act_build_masks_normed(_ptr(h_ref), Lr, T, S, _ptr(norms), ff, _MODE[mode], int(K),
                                            float(coverage), _ptr(mask_out), _ptr(idx_out), _ptr(count_out),
                                            _ptr(ws), ws.numel(), _stream(stream)), "act_build_masks_normed")
        return mask_out, idx_out, count_out
    arr = (_Ffn * Lr)(*[w.cstruct() for w in layers])
    _check(lib().act_build_masks(_ptr(h_ref), Lr, T, S, arr, _MODE[mode], int(K), float(coverage),
                                 _ptr(mask_out), _ptr(idx_out), _ptr(count_out), _ptr(ws), ws.numel(),
                                 _stream(stream)), "act_build_masks")
    return mask_out, idx_out, count_out


def _check_act_io(w: FFN, x, y_anchor, h_anchor, y_f32_out, h_out, glue, ff_rows=None):
    """Activation tensors of an Action Cache call: x [S][d] in the weights'
    dtype, the fp32 anchors y_anchor [S][d] and h_anchor [ff][S], y_f32_out
    [S][d], h_out [ff][S].  ff_rows: the neuron rows of the [ff][S] tensors
    (default w.ff; -1 when w is a compact FFN and they span the full FFN's
    neurons, which the call does not know)."""
    _expect(x, "x", w.dtype)
    if x.dim() != 2 or x.shape[1] != w.d:
        raise CgsError(f"x must be [S][{w.d}]")
    S = x.shape[0]
    nf = w.ff if ff_rows is None else ff_rows
    _expect(y_anchor, "y_anchor", torch.float32, (S, w.d), required=False)
    _expect(y_f32_out, "y_f32_out", torch.float32, (S, w.d), required=False)
    for t, name in ((h_anchor, "h_anchor"), (h_out, "h_out")):
        _expect(t, name, torch.float32, None, required=False)
        if t is not None and (t.dim() != 2 or t.shape[1] != S or (nf >= 0 and t.shape[0] != nf)):
            raise CgsError(f"{name} must be [{'ff' if nf < 0 else nf}][{S}] float32")
    _expect_glue(glue, S, w.d, w.dtype)


def act_ffn_masked(w: FFN, x, idx, y_anchor=None, h_anchor=None, y_out=None, y_f32_out=None,
                   h_out=None, glue=None, ws=None, stream=None):
    """Eq. 4 masked update of a dense anchor (dense anchor step when idx covers
    every neuron and no anchors are given).  ``glue`` = (r, bias, x_next)."""
    c = w.cstruct()
    _check_act_io(w, x, y_anchor, h_anchor, y_f32_out, h_out, glue)
    S, d = x.shape
    _expect_index(idx, "idx")
    K = int(idx.numel())
    if y_out is None:
        y_out = torch.empty_like(x)
    _expect(y_out, "y_out", w.dtype, (S, d))
    nbytes = lib().cgs_act_ffn_masked_workspace(S, K, d, w.ff)
    ws = workspace(nbytes, x.device, "act", stream) if ws is None else ws
    _check(lib().act_ffn_masked(ctypes.byref(c), _ptr(x), S, _ptr(idx), K, _ptr(y_anchor),
                                _ptr(h_anchor), _ptr(y_out), _ptr(y_f32_out), _ptr(h_out),
                                _glue(glue), _ptr(ws), ws.numel(), _stream(stream)), "act_ffn_masked")
    return y_out


def act_gather_rows(w: FFN, idx, out: FFN = None, stream=None) -> FFN:
    """Compact FFN of the mask idx: rows idx of w_gate, w_up and the
    neuron-major w_down, each [K][d] (into ``out`` when given)."""
    c = w.cstruct()
    _expect_index(idx, "idx")
    K = int(idx.numel())
    if out is None:
        shape = (K, w.d)
        out = FFN(torch.empty(shape, dtype=w.w_gate.dtype, device=w.w_gate.device),
                  torch.empty(shape, dtype=w.w_gate.dtype, device=w.w_gate.device),
                  torch.empty(shape, dtype=w.w_gate.dtype, device=w.w_gate.device), "fd")
    for t, name in ((out.w_gate, "out.w_gate"), (out.w_up, "out.w_up"), (out.w_down, "out.w_down")):
        _expect(t, name, w.dtype, (K, w.d))
    _check(lib().act_gather_rows(ctypes.byref(c), _ptr(idx), K, _ptr(out.w_gate), _ptr(out.w_up),
                                 _ptr(out.w_down), _stream(stream)), "act_gather_rows")
    return out


def act_ffn_masked_compact(wc: FFN, x, idx, y_anchor=None, h_anchor=None, y_out=None, y_f32_out=None,
                           h_out=None, glue=None, ws=None, stream=None, K=None):
    """Eq. 4 on the compact FFN of a mask (act_gather_rows); idx (original
    neuron ids) addresses h_anchor / h_out rows only and may be None without them."""
    c = wc.cstruct()
    K = wc.ff if K is None else int(K)
    _check_act_io(wc, x, y_anchor, h_anchor, y_f32_out, h_out, glue, ff_rows=-1)
    _expect_index(idx, "idx", K, required=False)
    S, d = x.shape
    if y_out is None:
        y_out = torch.empty_like(x)
    _expect(y_out, "y_out", wc.dtype, (S, d))
    nbytes = lib().cgs_act_ffn_masked_workspace(S, K, d, max(K, 1))
    ws = workspace(nbytes, x.device, "act", stream) if ws is None else ws
    _check(lib().act_ffn_masked_compact(ctypes.byref(c), _ptr(x), S, _ptr(idx), K, _ptr(y_anchor),
                                        _ptr(h_anchor), _ptr(y_out), _ptr(y_f32_out), _ptr(h_out),
                                        _glue(glue), _ptr(ws), ws.numel(), _stream(stream)),
           "act_ffn_masked_compact")
    return y_out


NOALLOC_SCRATCH_BYTES = 8 << 20  # CGS_NOALLOC_SCRATCH_BYTES


def act_ffn_masked_compact_noalloc(wc: FFN, x, idx, y_out, y_anchor=None, h_anchor=None, y_f32_out=None,
                                   h_out=None, glue=None, stream=None, K=None):
    """act_ffn_masked_compact for callers that cannot allocate: no workspace,
    and every output is the caller's (y_out is required).  The library's
    per-GPU scratch holds the intermediates, so calls that overlap in time on
    one GPU race; masks whose workspace would exceed NOALLOC_SCRATCH_BYTES are
    refused (CGS_ERR_WORKSPACE)."""
    c = wc.cstruct()
    K = wc.ff if K is None else int(K)
    _check_act_io(wc, x, y_anchor, h_anchor, y_f32_out, h_out, glue, ff_rows=-1)
    _expect_index(idx, "idx", K, required=False)
    S, d = x.shape
    _expect(y_out, "y_out", wc.dtype, (S, d))
    _check(lib().act_ffn_masked_compact_noalloc(ctypes.byref(c), _ptr(x), S, _ptr(idx), K, _ptr(y_anchor),
                                                _ptr(h_anchor), _ptr(y_out), _ptr(y_f32_out), _ptr(h_out),
                                                _glue(glue), _stream(stream)),
           "act_ffn_masked_compact_noalloc")
    return y_out


class _Rerank(ctypes.Structure):
    _fields_ = [("hist_len", ctypes.c_int32), ("joints", ctypes.c_int32), ("arm", ctypes.c_int32),
                ("min_cos", ctypes.c_double)]


def ret_select(query, refs, T: int, q_hist, r_hist, arm: int = -1, min_cos: float = 0.8,
               cos_out=None, top_out=None, dist_out=None, choice_out=None, ws=None, stream=None):
    """Visual top-T of the prepared entries, joint-history rerank, fallback.
    query [F], refs [N][F] (bf16 or float32), q_hist [L][J], r_hist [N][L][J]
    float32.  Returns (cos [N] f64, top [T] i32, dist [T] f64, choice [1] i32)."""
    _expect(query, "query")
    _dtype_code(query)
    F = int(query.numel())
    _expect(refs, "refs", query.dtype)
    if refs.dim() != 2 or refs.shape[1] != F:
        raise CgsError(f"refs must be [N][{F}]")
    N = refs.shape[0]
    _expect(q_hist, "q_hist", torch.float32)
    if q_hist.dim() != 2:
        raise CgsError("q_hist must be [L][J]")
    L, J = q_hist.shape
    _expect(r_hist, "r_hist", torch.float32, (N, L, J))
    dev = query.device
    if cos_out is None:
        cos_out = torch.empty(N, dtype=torch.float64, device=dev)
    if top_out is None:
        top_out = torch.empty(T, dtype=torch.int32, device=dev)
    if dist_out is None:
        dist_out = torch.empty(T, dtype=torch.float64, device=dev)
    if choice_out is None:
        choice_out = torch.empty(1, dtype=torch.int32, device=dev)
    _expect(cos_out, "cos_out", torch.float64, (N,))
    _expect(top_out, "top_out", torch.int32, (T,))
    _expect(dist_out, "dist_out", torch.float64, (T,))
    _expect(choice_out, "choice_out", torch.int32, (1,))
    nbytes = lib().cgs_ret_select_workspace(N, F)
    ws = workspace(nbytes, dev, "retrieval", stream) if ws is None else ws
    rr = _Rerank(L, J, int(arm), float(min_cos))
    _check(lib().ret_select(_ptr(query), _ptr(refs), N, F, _dtype_code(query), int(T), _ptr(q_hist),
                            _ptr(r_hist), ctypes.byref(rr), _ptr(cos_out), _ptr(top_out), _ptr(dist_out),
                            _ptr(choice_out), _ptr(ws), ws.numel(), _stream(stream)), "ret_select")
    return cos_out, top_out, dist_out, choice_out


class _Budget(ctypes.Structure):
    _fields_ = [("m_free", ctypes.c_double), ("m_entry", ctypes.c_double), ("t_avl", ctypes.c_double),
                ("t_trans", ctypes.c_double), ("t_rec", ctypes.c_double)]


def prep_budget(n_cand: int, m_free: float, m_entry: float, t_avl: float, t_trans: float, t_rec: float) -> int:
    """Eq. 5: the number of new entries to reconstruct."""
    n = lib().cgs_prep_budget(int(n_cand), float(m_free), float(m_entry), float(t_avl), float(t_trans),
                              float(t_rec))
    if n < 0:
        raise CgsError("prep_budget: invalid arguments")
    return n


def denoise_schedule(counts, words, ff: int):
    """The schedule an entry's stored masks imply (cgs_denoise_schedule):
    counts [L][T] int, words [L][T][ceil(ff/64)] int64/uint64 host arrays.
    Returns (kind [T]: 0 anchor / 1 update, anchor [T], mask [T]) as lists."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.int32)
    w = np.ascontiguousarray(words).view(np.uint64)
    if c.ndim != 2 or w.shape != c.shape + ((int(ff) + 63) // 64,):
        raise CgsError("denoise_schedule: counts [L][T] and words [L][T][ceil(ff/64)]")
    L, T = c.shape
    kind, anc, msk = ((ctypes.c_int32 * T)() for _ in range(3))
    _check(lib().cgs_denoise_schedule(L, T, int(ff), c.ctypes.data, w.ctypes.data, kind, anc, msk),
           "cgs_denoise_schedule")
    return list(kind), list(anc), list(msk)


class Window:
    """Sliding GPU working set of `slots` expanded entries (host bookkeeping
    in libcgs; the caller rebuilds the entries an advance admits)."""

    def __init__(self, slots: int):
        self.slots = int(slots)
        self._h = lib().cgs_window_create(self.slots)
        if not self._h:
            raise CgsError("cgs_window_create: invalid slot count")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.cgs_window_destroy(h)

    def slot(self, episode: int, position: int) -> int:
        return lib().cgs_window_slot(self._h, int(episode), int(position))

    def resident(self) -> int:
        return lib().cgs_window_resident(self._h)

    def advance(self, episodes, positions, lengths, L: int, budget=None):
        """One advance; budget = (m_free, m_entry, t_avl, t_trans, t_rec) or None.
        Returns (entered [(episode, position, slot)], left slots, n_candidates)."""
        T = len(episodes)
        arr = lambda v: (ctypes.c_int32 * max(T, 1))(*[int(x) for x in v])
        ep, pos, ln = arr(episodes), arr(positions), arr(lengths)
        out = lambda: (ctypes.c_int32 * self.slots)()
        e_ep, e_pos, e_slot, l_slot = out(), out(), out(), out()
        ne, nl, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        b = ctypes.byref(_Budget(*[float(x) for x in budget])) if budget is not None else None
        _check(lib().cgs_window_advance(self._h, T, ep, pos, ln, int(L), b, e_ep, e_pos, e_slot,
                                        ctypes.byref(ne), l_slot, ctypes.byref(nl), ctypes.byref(nc)),
               "cgs_window_advance")
        entered = [(e_ep[i], e_pos[i], e_slot[i]) for i in range(ne.value)]
        return entered, [l_slot[i] for i in range(nl.value)], nc.value


def act_ffn_joint(wc: FFN, x, tok, idx, y_anchor, h_anchor=None, y_out=None, y_f32_out=None, glue=None,
                  ws=None, stream=None):
    """Token + neuron sparsity: Eq. 4 on the rows tok (ascending) of x with the
    compact weights of the mask idx; every other row keeps y_anchor."""
    c = wc.cstruct()
    _check_act_io(wc, x, y_anchor, h_anchor, y_f32_out, None, glue, ff_rows=-1)
    S, d = x.shape
    _expect_index(tok, "tok", required=False)
    _expect_index(idx, "idx", wc.ff, required=False)
    k = 0 if tok is None else int(tok.numel())
    K = wc.ff
    if y_out is None:
        y_out = torch.empty_like(x)
    _expect(y_out, "y_out", wc.dtype, (S, d))
    nbytes = lib().cgs_act_ffn_masked_workspace(max(k, 1), K, d, max(K, 1))
    ws = workspace(nbytes, x.device, "act", stream) if ws is None else ws
    _check(lib().act_ffn_joint(ctypes.byref(c), _ptr(x), S, _ptr(tok), k, _ptr(idx), K, _ptr(y_anchor),
                               _ptr(h_anchor), _ptr(y_out), _ptr(y_f32_out), _glue(glue), _ptr(ws), ws.numel(),
                               _stream(stream)), "act_ffn_joint")
    return y_out


def ref_rebuild_dense(layers, r0, x_ref_out=None, y_ref_out=None, ws=None, stream=None):
    """Dense rebuild of an entry: returns (x_ref [L][P][d], y_ref [L][P][d])."""
    L = len(layers)
    arr = (_Ffn * L)(*[w.cstruct() for w in layers])
    _expect(r0, "r0", layers[0].dtype)
    if r0.dim() != 2 or r0.shape[1] != layers[0].d:
        raise CgsError(f"r0 must be [P][{layers[0].d}]")
    P, d = r0.shape
    if x_ref_out is None:
        x_ref_out = torch.empty((L, P, d), dtype=r0.dtype, device=r0.device)
    if y_ref_out is None:
        y_ref_out = torch.empty((L, P, d), dtype=r0.dtype, device=r0.device)
    _expect(x_ref_out, "x_ref_out", r0.dtype, (L, P, d))
    _expect(y_ref_out, "y_ref_out", r0.dtype, (L, P, d))
    c0 = arr[0]
    nbytes = lib().cgs_ref_rebuild_dense_workspace(L, P, d, c0.ff, c0.dtype)
    ws = workspace(nbytes, r0.device, "rebuild", stream) if ws is None else ws
    _check(lib().ref_rebuild_dense(arr, L, _ptr(r0), P, _ptr(x_ref_out), _ptr(y_ref_out),
                                   _ptr(ws), ws.numel(), _stream(stream)), "ref_rebuild_dense")
    return x_ref_out, y_ref_out



def ref_rebuild_dense_batch(layers, r0, x_ref_outs, y_ref_outs, ws=None, stream=None):
    """Dense rebuild of n entries in one prefill over their n P rows: r0
    [n][P][d]; x_ref_outs / y_ref_outs: n tensors [L][P][d] each (entry e's
    outputs, as ref_rebuild_dense writes them)."""
    L = len(layers)
    arr = (_Ffn * L)(*[w.cstruct() for w in layers])
    _expect(r0, "r0", layers[0].dtype)
    if r0.dim() != 3 or r0.shape[2] != layers[0].d:
        raise CgsError(f"r0 must be [n][P][{layers[0].d}]")
    n, P, d = r0.shape
    if len(x_ref_outs) != n or len(y_ref_outs) != n:
        raise CgsError("one x_ref and one y_ref output per entry")
    for e in range(n):
        _expect(x_ref_outs[e], f"x_ref_outs[{e}]", r0.dtype, (L, P, d))
        _expect(y_ref_outs[e], f"y_ref_outs[{e}]", r0.dtype, (L, P, d))
    xs = (ctypes.c_void_p * n)(*[_ptr(t) for t in x_ref_outs])
    ys = (ctypes.c_void_p * n)(*[_ptr(t) for t in y_ref_outs])
    c0 = arr[0]
    nbytes = lib().cgs_ref_rebuild_dense_batch_workspace(L, n, P, d, c0.ff, c0.dtype)
    if nbytes == 0:
        raise CgsError("ref_rebuild_dense_batch: unsupported shape")
    ws = workspace(nbytes, r0.device, "rebuild", stream) if ws is None else ws
    _check(lib().ref_rebuild_dense_batch(arr, L, _ptr(r0), n, P, xs, ys, _ptr(ws), ws.numel(), _stream(stream)),
           "ref_rebuild_dense_batch")
    return x_ref_outs, y_ref_outs

def residual_rmsnorm(r, y=None, bias=None, x_out=None, r_in=None, stream=None):
    """r = (r_in or r) + y + bias (fp32); x_out = RMSNorm(r) (eps 1e-6, no scale)."""
    _expect(r, "r", torch.float32)
    if r.dim() != 2:
        raise CgsError("r must be [M][d]")
    M, d = r.shape
    _expect(r_in, "r_in", torch.float32, (M, d), required=False)
    _expect(bias, "bias", torch.float32, (d,), required=False)
    for t, name in ((y, "y"), (x_out, "x_out")):
        _expect(t, name, None, (M, d), required=False)
    ydt = _dtype_code(y) if y is not None else CGS_BF16
    odt = _dtype_code(x_out) if x_out is not None else CGS_BF16
    _check(lib().cgs_residual_rmsnorm(_ptr(r), _ptr(r_in), _ptr(y), ydt, _ptr(bias), M, d,
                                      _ptr(x_out), odt, _stream(stream)), "cgs_residual_rmsnorm")
    return x_out


def profile_start(site_filter: str, max_launches: int = 4096):
    """Time every launch whose site name contains site_filter with HIP events."""
    _check(lib().cgs_profile_start(site_filter.encode(), int(max_launches)), "cgs_profile_start")


def profile_stop():
    _check(lib().cgs_profile_stop(), "cgs_profile_stop")


def profile_result(site: str | None = None):
    """(summed kernel milliseconds, launches) of the recorded launches whose site
    contains ``site`` (None = all)."""
    t = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check(lib().cgs_profile_result(None if site is None else site.encode(), ctypes.byref(t),
                                    ctypes.byref(n)), "cgs_profile_result")
    return t.value, n.value


# --------------------------------------------------------------------------
# One whole masked denoising step in one persistent launch
# --------------------------------------------------------------------------
class _GatherLayer(ctypes.Structure):
    _fields_ = [("w", _Ffn), ("idx", ctypes.c_void_p), ("K", ctypes.c_int32), ("wg_out", ctypes.c_void_p),
                ("wu_out", ctypes.c_void_p), ("wd_out", ctypes.c_void_p)]


def act_gather_rows_layers(ws, idxs, outs, stream=None):
    """act_gather_rows for several layers in one launch: ws (full FFNs, 'fd'),
    idxs (int32 lists), outs (compact FFNs [K][d] to fill), one of each per layer."""
    n = len(ws)
    if not (len(idxs) == len(outs) == n) or n == 0:
        raise CgsError("act_gather_rows_layers: one weight set, index list and output per layer")
    arr = (_GatherLayer * n)()
    for i, (w, idx, out) in enumerate(zip(ws, idxs, outs)):
        if w.layout != "fd" or out.layout != "fd":
            raise CgsError("act_gather_rows_layers: neuron-major ('fd') weights")
        _expect_index(idx, f"layer {i} idx")
        K = int(idx.numel())
        for t, name in ((out.w_gate, "w_gate"), (out.w_up, "w_up"), (out.w_down, "w_down")):
            _expect(t, f"layer {i} out.{name}", w.dtype, (K, w.d))
        arr[i] = _GatherLayer(w.cstruct(), _ptr(idx), K, _ptr(out.w_gate), _ptr(out.w_up), _ptr(out.w_down))
    _check(lib().act_gather_rows_layers(arr, n, _stream(stream)), "act_gather_rows_layers")
    return outs


class _MaskedLayer(ctypes.Structure):
    _fields_ = [("w", _Ffn), ("idx", ctypes.c_void_p), ("y_anchor", ctypes.c_void_p),
                ("h_anchor", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("y_out", ctypes.c_void_p),
                ("y_f32_out", ctypes.c_void_p), ("h_out", ctypes.c_void_p)]


@dataclass
class MaskedLayer:
    """One layer of act_masked_layers: the compact FFN of its mask (or the full
    FFN, with idx = 0..ff-1, for a dense anchor layer), the mask's neuron ids,
    the anchor state, the bias added to r after the layer and optional outputs."""
    w: FFN
    idx: torch.Tensor = None
    y_anchor: torch.Tensor = None
    h_anchor: torch.Tensor = None
    bias: torch.Tensor = None
    y_out: torch.Tensor = None
    y_f32_out: torch.Tensor = None
    h_out: torch.Tensor = None


class MaskedChain:
    """A chain of MaskedLayers checked once and kept as the C array, so that
    replaying it (act_masked_layers) costs one host call.  S: action tokens;
    ff: neurons of the full FFN (the rows of h_anchor / h_out)."""

    def __init__(self, layers, S: int, ff: int):
        if not layers:
            raise CgsError("MaskedChain: no layers")
        self.n, self.S, self.ff = len(layers), int(S), int(ff)
        self.d, self.dtype = layers[0].w.d, layers[0].w.dtype
        self.arr = (_MaskedLayer * self.n)()
        self.kmax = 0
        self._refs = []
        for i, ly in enumerate(layers):
            w = ly.w
            if w.layout != "fd" or w.dtype != self.dtype or w.d != self.d:
                raise CgsError(f"layer {i}: weights must be 'fd' with the chain's d and dtype")
            K = w.ff
            self.kmax = max(self.kmax, K)
            _expect_index(ly.idx, f"layer {i} idx", K, required=False)
            if ly.idx is None and (ly.h_anchor is not None or ly.h_out is not None):
                raise CgsError(f"layer {i}: h_anchor / h_out need idx")
            _expect(ly.y_anchor, f"layer {i} y_anchor", torch.float32, (S, self.d), required=False)
            _expect(ly.h_anchor, f"layer {i} h_anchor", torch.float32, (ff, S), required=False)
            _expect(ly.bias, f"layer {i} bias", torch.float32, (self.d,), required=False)
            _expect(ly.y_out, f"layer {i} y_out", self.dtype, (S, self.d), required=False)
            _expect(ly.y_f32_out, f"layer {i} y_f32_out", torch.float32, (S, self.d), required=False)
            _expect(ly.h_out, f"layer {i} h_out", torch.float32, (ff, S), required=False)
            self.arr[i] = _MaskedLayer(w.cstruct(), _ptr(ly.idx), _ptr(ly.y_anchor), _ptr(ly.h_anchor),
                                       _ptr(ly.bias), _ptr(ly.y_out), _ptr(ly.y_f32_out), _ptr(ly.h_out))
            self._refs.append(ly)
        self.ws_bytes = int(lib().cgs_act_masked_layers_workspace(self.S, self.d, self.kmax))
        if self.ws_bytes == 0:
            raise CgsError("MaskedChain: unsupported shape")


def act_masked_layers(chain, r, x, ws=None, stream=None, ff: int = None):
    """Run a chain of masked / dense layers with the residual glue in one host
    call: x [n+1][S][d] (x[0] read, x[1..n] written), r [S][d] fp32 updated.
    chain: a MaskedChain, or a list of MaskedLayer (then ff is required)."""
    if not isinstance(chain, MaskedChain):
        _expect(r, "r", torch.float32)
        chain = MaskedChain(chain, r.shape[0], ff)
    _expect(r, "r", torch.float32, (chain.S, chain.d))
    _expect(x, "x", chain.dtype, (chain.n + 1, chain.S, chain.d))
    ws = workspace(chain.ws_bytes, r.device, "act", stream) if ws is None else ws
    _check(lib().act_masked_layers(chain.arr, chain.n, chain.S, _ptr(r), _ptr(x), _ptr(ws), ws.numel(),
                                   _stream(stream)), "act_masked_layers")
    return x


class _StepLayer(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down_t", ctypes.c_void_p),
                ("K", ctypes.c_int32), ("ldk", ctypes.c_int32), ("idx", ctypes.c_void_p),
                ("y_anchor", ctypes.c_void_p), ("h_anchor", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("y_out", ctypes.c_void_p), ("y_f32_out", ctypes.c_void_p), ("h_out", ctypes.c_void_p)]


@dataclass
class CompactT:
    """Compact weights of a mask for act_denoise_step: w_gate, w_up [K][d] and
    the down weights transposed, w_down_t [d][ldk] (act_gather_rows_t)."""
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down_t: torch.Tensor

    @property
    def K(self) -> int:
        return self.w_gate.shape[0]

    @property
    def d(self) -> int:
        return self.w_down_t.shape[0]

    @property
    def ldk(self) -> int:
        return self.w_down_t.shape[1]


def act_gather_rows_t(w: FFN, idx=None, K: int = None, ldk: int = None, out: CompactT = None,
                      stream=None) -> CompactT:
    """Rows idx of w_gate / w_up ([K][d]) and the same neurons' down weights
    transposed ([d][ldk], zero past K).  idx None: the first K neurons (K = ff
    by default: the full FFN in the step kernel's layout)."""
    c = w.cstruct()
    if w.layout != "fd" or w.dtype != torch.bfloat16:
        raise CgsError("act_gather_rows_t: bf16 weights with neuron-major w_down ('fd')")
    _expect_index(idx, "idx", required=False)
    K = (w.ff if idx is None else int(idx.numel())) if K is None else int(K)
    if idx is not None and int(idx.numel()) != K:
        raise CgsError("act_gather_rows_t: K differs from the index list")
    ldk = (K + 31) // 32 * 32 if ldk is None else int(ldk)
    dev = w.w_gate.device
    if out is None:
        out = CompactT(torch.empty((K, w.d), dtype=torch.bfloat16, device=dev),
                       torch.empty((K, w.d), dtype=torch.bfloat16, device=dev),
                       torch.empty((w.d, ldk), dtype=torch.bfloat16, device=dev))
    _expect(out.w_gate, "out.w_gate", torch.bfloat16, (K, w.d))
    _expect(out.w_up, "out.w_up", torch.bfloat16, (K, w.d))
    _expect(out.w_down_t, "out.w_down_t", torch.bfloat16, (w.d, ldk))
    _check(lib().act_gather_rows_t(ctypes.byref(c), _ptr(idx), K, _ptr(out.w_gate), _ptr(out.w_up),
                                   _ptr(out.w_down_t), ldk, _stream(stream)), "act_gather_rows_t")
    return out


@dataclass
class StepLayer:
    """One layer of act_denoise_step: compact weights (CompactT), the mask's
    neuron ids (idx, or None for the identity), the anchor state, the bias
    added to r after the layer and optional outputs."""
    w: CompactT
    idx: torch.Tensor = None
    y_anchor: torch.Tensor = None
    h_anchor: torch.Tensor = None
    bias: torch.Tensor = None
    y_out: torch.Tensor = None
    y_f32_out: torch.Tensor = None
    h_out: torch.Tensor = None


def act_denoise_step_workspace(L: int, S: int, d: int, K_max: int) -> int:
    return int(lib().cgs_act_denoise_step_workspace(int(L), int(S), int(d), int(K_max)))


def act_denoise_step(layers, r, x, ff: int, status=None, ws=None, stream=None):
    """All len(layers) masked layers of a denoising step in one persistent
    launch: x [L+1][S][d] bf16 (x[0] the input, x[1..L] written), r [S][d]
    fp32 residual (updated).  status: optional int32 [1] device tensor (0, or
    CGS_ERR_TIMEOUT if a wait inside the kernel gave up)."""
    L = len(layers)
    _expect(r, "r", torch.float32)
    if r.dim() != 2:
        raise CgsError("r must be [S][d]")
    S, d = r.shape
    _expect(x, "x", torch.bfloat16, (L + 1, S, d))
    _expect(status, "status", torch.int32, (1,), required=False)
    arr = (_StepLayer * max(L, 1))()
    kmax = 0
    for i, ly in enumerate(layers):
        cw = ly.w
        K = cw.K
        kmax = max(kmax, K)
        _expect(cw.w_gate, f"layer {i} w_gate", torch.bfloat16, (K, d))
        _expect(cw.w_up, f"layer {i} w_up", torch.bfloat16, (K, d))
        _expect(cw.w_down_t, f"layer {i} w_down_t", torch.bfloat16)
        if cw.w_down_t.dim() != 2 or cw.w_down_t.shape[0] != d:
            raise CgsError(f"layer {i} w_down_t must be [{d}][ldk]")
        _expect_index(ly.idx, f"layer {i} idx", K, required=False)
        _expect(ly.y_anchor, f"layer {i} y_anchor", torch.float32, (S, d), required=False)
        _expect(ly.h_anchor, f"layer {i} h_anchor", torch.float32, (ff, S), required=False)
        _expect(ly.bias, f"layer {i} bias", torch.float32, (d,), required=False)
        _expect(ly.y_out, f"layer {i} y_out", torch.bfloat16, (S, d), required=False)
        _expect(ly.y_f32_out, f"layer {i} y_f32_out", torch.float32, (S, d), required=False)
        _expect(ly.h_out, f"layer {i} h_out", torch.float32, (ff, S), required=False)
        arr[i] = _StepLayer(_ptr(cw.w_gate), _ptr(cw.w_up), _ptr(cw.w_down_t), K, cw.ldk, _ptr(ly.idx),
                            _ptr(ly.y_anchor), _ptr(ly.h_anchor), _ptr(ly.bias), _ptr(ly.y_out),
                            _ptr(ly.y_f32_out), _ptr(ly.h_out))
    nbytes = lib().cgs_act_denoise_step_workspace(L, S, d, kmax)
    ws = workspace(nbytes, r.device, "step", stream) if ws is None else ws
    _check(lib().act_denoise_step(arr, L, S, d, int(ff), _ptr(r), _ptr(x), _ptr(status), _ptr(ws), ws.numel(),
                                  _stream(stream)), "act_denoise_step")
    return x


def set_step_wait_limit(ticks: int) -> int:
    """Time limit of act_denoise_step's internal waits (100 MHz device clock
    ticks) for later launches; returns the previous one."""
    return int(lib().cgs_set_step_wait_limit(int(ticks)))
