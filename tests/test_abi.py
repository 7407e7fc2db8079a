"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before launching anything (no GPU needed)."""
import ctypes
import re

import numpy as np
import pytest

import cache_guided_sparse_amd as cgs
import oracle as O


def _declared_functions():
    src = open(cgs.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:long\s+long|[A-Za-z_][A-Za-z0-9_]*)\s*\*?\s+\**"
                       r"([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_entry_points():
    names = _declared_functions()
    for n in ("ctx_select", "ctx_ffn_recompute", "act_build_mask", "act_ffn_masked",
              "ref_rebuild_dense"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = cgs.lib()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(cgs._SIGS)


def test_ratio_to_count_matches_oracle():
    for rho in np.linspace(0, 1, 101):
        for n in (0, 1, 10, 64, 100, 768, 1024, 4096, 16384):
            assert cgs.ratio_to_count(rho, n) == O.ratio_to_count(rho, n), (rho, n)
    assert cgs.ratio_to_count(0.07, 100) == 7
    assert cgs.ratio_to_count(2.0, 10) == 10 and cgs.ratio_to_count(-1.0, 10) == 0


def test_status_strings_and_version():
    L = cgs.lib()
    assert L.cgs_status_str(0) == b"ok"
    assert L.cgs_status_str(3) == b"workspace too small"
    assert L.cgs_status_str(99) == b"unknown status"
    assert L.cgs_version() >= 100


def test_workspace_queries():
    L = cgs.lib()
    assert L.cgs_ctx_select_workspace(768, 2048) >= 768 * 8
    big = L.cgs_ctx_ffn_recompute_workspace(231, 768, 2048, 16384, 0)
    assert big >= 231 * 16384 * 2 + 231 * 2048 * 4
    assert L.cgs_ctx_ffn_recompute_workspace(0, 768, 2048, 16384, 0) > 0
    assert L.cgs_ctx_ffn_recompute_workspace(231, 768, 2000, 16384, 0) == 0  # unsupported d
    assert L.cgs_act_ffn_masked_workspace(50, 1229, 1024, 4096) >= 64 * 1248 * 2
    assert L.cgs_act_build_mask_workspace(4, 50, 4096, 1024) >= 4 * 4096 * 8
    assert L.cgs_ref_rebuild_dense_workspace(17, 768, 2048, 16384, 0) >= 768 * 2048 * 4


def _ffn(d=256, ff=1024, dtype=0, layout=0, null=False):
    p = None if null else 0x1000
    return cgs._Ffn(d, ff, dtype, layout, p, p, p)


def test_host_validation_without_launch():
    """Bad arguments return a status before anything reaches the GPU."""
    L = cgs.lib()
    buf = ctypes.c_void_p(0x1000)
    # ctx_select: bad dtype / kind / k / d
    assert L.ctx_select(buf, buf, 8, 16, 7, 1, 0, buf, None, buf, 1 << 20, None) == 1
    assert L.ctx_select(buf, buf, 8, 16, 0, 1, 5, buf, None, buf, 1 << 20, None) == 1
    assert L.ctx_select(buf, buf, 8, 16, 0, 9, 0, buf, None, buf, 1 << 20, None) == 2
    assert L.ctx_select(buf, buf, 8, 8192, 0, 1, 0, buf, None, buf, 1 << 20, None) == 2
    assert L.ctx_select(None, buf, 8, 16, 0, 1, 0, buf, None, buf, 1 << 20, None) == 1
    assert L.ctx_select(buf, buf, 8, 16, 0, 1, 0, buf, None, buf, 8, None) == 3
    assert L.ctx_select(buf, buf, 0, 16, 0, 0, 0, None, None, None, 0, None) == 0
    # ctx_ffn_recompute: wrong layout, null weights, unsupported d, k > P, aliasing
    w = _ffn()
    assert L.ctx_ffn_recompute(ctypes.byref(_ffn(layout=1)), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), None, buf, 1 << 30, None) == 1
    assert L.ctx_ffn_recompute(ctypes.byref(_ffn(null=True)), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), None, buf, 1 << 30, None) == 1
    assert L.ctx_ffn_recompute(ctypes.byref(_ffn(d=200)), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), None, buf, 1 << 30, None) == 4
    assert L.ctx_ffn_recompute(ctypes.byref(w), buf, buf, buf, 9, 8, ctypes.c_void_p(0x2000), None, buf, 1 << 30, None) == 2
    assert L.ctx_ffn_recompute(ctypes.byref(w), buf, ctypes.c_void_p(0x2000), buf, 1, 8, ctypes.c_void_p(0x2000), None, buf, 1 << 30, None) == 1
    assert L.ctx_ffn_recompute(ctypes.byref(w), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), None, buf, 16, None) == 3
    # act_ffn_masked: wrong layout, K > ff
    wf = _ffn(layout=1)
    assert L.act_ffn_masked(ctypes.byref(w), buf, 4, buf, 1, None, None, buf, None, None, None, buf, 1 << 30, None) == 1
    assert L.act_ffn_masked(ctypes.byref(wf), buf, 4, buf, 2000, None, None, buf, None, None, None, buf, 1 << 30, None) == 2
    assert L.act_ffn_masked(ctypes.byref(wf), buf, 4, buf, 10, None, None, buf, None, None, None, buf, 4, None) == 3
    # glue without a residual buffer
    g = cgs._Glue(None, None, None)
    assert L.act_ffn_masked(ctypes.byref(wf), buf, 4, buf, 10, None, None, buf, None, None, ctypes.byref(g), buf, 1 << 30, None) == 1
    assert L.ctx_ffn_recompute(ctypes.byref(w), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), ctypes.byref(g), buf, 1 << 30, None) == 1
    # glue score keys without x_next / score_ref, or with an unknown kind
    for g in (cgs._Glue(buf, None, None, buf, buf, 0), cgs._Glue(buf, None, buf, None, buf, 0),
              cgs._Glue(buf, None, buf, buf, buf, 7)):
        assert L.ctx_ffn_recompute(ctypes.byref(w), buf, buf, buf, 1, 8, ctypes.c_void_p(0x2000), ctypes.byref(g), buf, 1 << 30, None) == 1
    # ctx_select_from_keys: k > P, P too large, null keys; empty is a no-op
    assert L.ctx_select_from_keys(buf, 8, 9, buf, None) == 2
    assert L.ctx_select_from_keys(buf, 70000, 1, buf, None) == 2
    assert L.ctx_select_from_keys(None, 8, 1, buf, None) == 1
    assert L.ctx_select_from_keys(None, 8, 0, None, None) == 0
    # act_gather_rows: wrong layout, K > ff, null index; K = 0 is a no-op
    assert L.act_gather_rows(ctypes.byref(w), buf, 4, buf, buf, buf, None) == 1
    assert L.act_gather_rows(ctypes.byref(wf), buf, 2000, buf, buf, buf, None) == 2
    assert L.act_gather_rows(ctypes.byref(wf), None, 4, buf, buf, buf, None) == 1
    assert L.act_gather_rows(ctypes.byref(wf), None, 0, None, None, None, None) == 0
    # act_ffn_joint: y_anchor required, k > S, K != compact rows, selected rows need h_anchor
    wc64 = _ffn(layout=1, ff=64)
    assert L.act_ffn_joint(ctypes.byref(wc64), buf, 8, buf, 2, buf, 64, None, buf, buf, None, None, buf, 1 << 30, None) == 1
    assert L.act_ffn_joint(ctypes.byref(wc64), buf, 8, buf, 9, buf, 64, buf, buf, buf, None, None, buf, 1 << 30, None) == 2
    assert L.act_ffn_joint(ctypes.byref(wc64), buf, 8, buf, 2, buf, 63, buf, buf, buf, None, None, buf, 1 << 30, None) == 2
    assert L.act_ffn_joint(ctypes.byref(wc64), buf, 8, buf, 2, buf, 64, buf, None, buf, None, None, buf, 1 << 30, None) == 1
    # act_build_masks: layer count, mismatched layers
    arr2 = (cgs._Ffn * 2)(_ffn(layout=1), _ffn(layout=1, ff=2048))
    assert L.act_build_masks(buf, 0, 2, 8, ctypes.byref(wf), 0, 4, 0.0, buf, buf, buf, buf, 1 << 30, None) == 2
    assert L.act_build_masks(buf, 65, 2, 8, ctypes.byref(wf), 0, 4, 0.0, buf, buf, buf, buf, 1 << 30, None) == 2
    assert L.act_build_masks(buf, 2, 2, 8, arr2, 0, 4, 0.0, buf, buf, buf, buf, 1 << 30, None) == 2
    assert L.cgs_act_build_masks_workspace(18, 4, 50, 4096, 1024) >= 18 * 4096 * (4 * 8 + 8 + 8 + 4 + 4)
    assert L.cgs_act_build_masks_workspace(0, 4, 50, 4096, 1024) == 0
    # act_ffn_masked_compact: K must equal the compact row count; anchors need idx
    wc = _ffn(layout=1, ff=64)
    assert L.act_ffn_masked_compact(ctypes.byref(wc), buf, 4, buf, 10, None, None, buf, None, None, None, buf, 1 << 30, None) == 2
    assert L.act_ffn_masked_compact(ctypes.byref(wc), buf, 4, None, 64, None, buf, buf, None, None, None, buf, 1 << 30, None) == 1
    assert L.act_ffn_masked_compact(ctypes.byref(wc), buf, 4, None, 64, None, None, buf, None, None, None, buf, 4, None) == 3
    # act_build_mask: bad mode, K, coverage, S*T too large
    assert L.act_build_mask(buf, 2, 8, ctypes.byref(wf), 9, 4, 0.0, buf, buf, buf, buf, 1 << 30, None) == 1
    assert L.act_build_mask(buf, 2, 8, ctypes.byref(wf), 0, 5000, 0.0, buf, buf, buf, buf, 1 << 30, None) == 2
    assert L.act_build_mask(buf, 2, 8, ctypes.byref(wf), 1, 0, 1.5, buf, buf, buf, buf, 1 << 30, None) == 2
    assert L.act_build_mask(buf, 1 << 10, 64, ctypes.byref(wf), 0, 4, 0.0, buf, buf, buf, buf, 1 << 30, None) == 2
    # ref_rebuild_dense: mismatched layers
    arr = (cgs._Ffn * 2)(_ffn(), _ffn(ff=2048))
    assert L.ref_rebuild_dense(arr, 2, buf, 8, buf, buf, buf, 1 << 30, None) == 2
    assert L.ref_rebuild_dense(arr, 0, buf, 8, buf, buf, buf, 1 << 30, None) == 2


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(cgs, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(cgs, "_lib", None)
    with pytest.raises(cgs.CgsError):
        cgs.lib()


def test_checked_mode_switch_and_environment_default():
    """cgs_set_validate returns the previous setting; the initial setting comes
    from CGS_VALIDATE (read in a fresh process, no GPU call is made)."""
    import os
    import subprocess
    import sys
    L = cgs.lib()
    prev = L.cgs_set_validate(1)
    try:
        assert L.cgs_set_validate(0) == 1
        assert L.cgs_set_validate(0) == 0
    finally:
        L.cgs_set_validate(prev)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = "import cache_guided_sparse_amd as c; print(c.lib().cgs_set_validate(0))"
    for env, want in (("1", "1"), ("0", "0"), (None, "0")):
        e = dict(os.environ)
        e.pop("CGS_VALIDATE", None)
        if env is not None:
            e["CGS_VALIDATE"] = env
        out = subprocess.run([sys.executable, "-c", code], cwd=root, env=e, capture_output=True, text=True,
                             timeout=300)
        assert out.returncode == 0, out.stderr
        assert out.stdout.strip().splitlines()[-1] == want
    assert L.cgs_status_str(6) == b"device data break a documented precondition"


def test_workspace_cache_reuses_grows_and_retires():
    """The binding's workspace cache (host logic, on CPU tensors): one buffer
    per (device, stream, op family); a larger request retires the old buffer
    (kept alive) and at least doubles the size."""
    cgs._ws_cache.clear()
    cgs._ws_retired.clear()
    a = cgs.workspace(1000, "cpu", "t")
    assert a.numel() >= 1000 and cgs.workspace(500, "cpu", "t") is a
    b = cgs.workspace(1500, "cpu", "t")
    assert b is not a and b.numel() >= 2 * a.numel()
    assert any(r is a for r in cgs._ws_retired)
    assert cgs.workspace(10, "cpu", "other") is not b
    cgs._ws_cache.clear()
    cgs._ws_retired.clear()


def test_norm_entry_points_validate_before_launch():
    """act_down_norms and act_build_masks_normed return their status before
    any launch: null pointers, layer counts, layouts, shapes, mode, workspace."""
    L = cgs.lib()
    buf = ctypes.c_void_p(0x1000)
    wf = (cgs._Ffn * 2)(_ffn(layout=1), _ffn(layout=1))
    wd = (cgs._Ffn * 1)(_ffn(layout=0))
    assert L.act_down_norms(None, 1, buf, None) == 1
    assert L.act_down_norms(wf, 2, None, None) == 1
    assert L.act_down_norms(wf, 0, buf, None) == 2
    assert L.act_down_norms(wf, 65, buf, None) == 2
    assert L.act_down_norms(wd, 1, buf, None) == 1            # W_down must be neuron-major
    wmix = (cgs._Ffn * 2)(_ffn(layout=1), _ffn(layout=1, d=128))
    assert L.act_down_norms(wmix, 2, buf, None) == 2          # layers of different shapes
    ws = L.cgs_act_build_masks_workspace(2, 4, 50, 1024, 1)
    args = (2, 4, 50, buf, 1024, 0, 10, 0.0, buf, buf, buf, buf, ws, None)
    assert L.act_build_masks_normed(None, *args) == 1
    assert L.act_build_masks_normed(buf, 2, 4, 50, None, 1024, 0, 10, 0.0, buf, buf, buf, buf, ws, None) == 1
    assert L.act_build_masks_normed(buf, 0, 4, 50, buf, 1024, 0, 10, 0.0, buf, buf, buf, buf, ws, None) == 2
    assert L.act_build_masks_normed(buf, 2, 4, 50, buf, 0, 0, 10, 0.0, buf, buf, buf, buf, ws, None) == 2
    assert L.act_build_masks_normed(buf, 2, 4, 50, buf, 1024, 7, 10, 0.0, buf, buf, buf, buf, ws, None) == 1
    assert L.act_build_masks_normed(buf, 2, 4, 50, buf, 1024, 0, 2000, 0.0, buf, buf, buf, buf, ws, None) == 2
    assert L.act_build_masks_normed(buf, 2, 4, 50, buf, 1024, 1, 0, 1.5, buf, buf, buf, buf, ws, None) == 2
    assert L.act_build_masks_normed(buf, 2, 400, 50, buf, 1024, 0, 10, 0.0, buf, buf, buf, buf, ws, None) == 2
    assert L.act_build_masks_normed(buf, 2, 4, 50, buf, 1024, 0, 10, 0.0, buf, buf, buf, buf, 8, None) == 3


def test_binding_refuses_mismatched_tensors(monkeypatch):
    """The binding checks every tensor's dtype and shape against the FFN and
    the counts before a pointer reaches the library (the kernels size their
    accesses from those, so a mismatch would read or write outside the
    tensor).  CPU tensors stand in for device ones: pointers are faked, and
    every case below is refused before any library call that launches."""
    import torch
    monkeypatch.setattr(cgs, "_ptr", lambda t: None if t is None else 0x1000)
    bf, f32 = torch.bfloat16, torch.float32
    d, ff, P, S = 256, 1024, 16, 8

    def z(*shape, dt=bf):
        return torch.zeros(*shape, dtype=dt)

    def refuses(fn, what):
        with pytest.raises(cgs.CgsError, match=what):
            fn()

    W = cgs.FFN(z(ff, d), z(ff, d), z(d, ff), "df")
    x, idx = z(P, d), torch.arange(4, dtype=torch.int32)
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, z(P, d, dt=f32), idx), "y_ref")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x.float(), x, idx), "x must be")
    refuses(lambda: cgs.ctx_ffn_recompute(W, z(P, 128), x, idx), "x must be")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx.long()), "idx")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx.view(2, 2)), "idx")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx, y_out=z(P, d, dt=f32)), "y_out")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx, glue=(z(P, d), None, None)), "glue residual")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx, glue=(z(P, d, dt=f32), None, z(P - 1, d))), "x_next")
    refuses(lambda: cgs.ctx_ffn_recompute(W, x, x, idx, glue=(z(P, d, dt=f32), None, x, x, z(P, dt=f32))),
            "score_key")
    refuses(lambda: cgs.ctx_ffn_recompute(cgs.FFN(W.w_gate, W.w_up, z(ff, d), "df"), x, x, idx), "w_down")
    refuses(lambda: cgs.ctx_select(x, z(P, d, dt=f32), 4), "x_ref")
    refuses(lambda: cgs.ctx_select(x, x, 4, idx_out=torch.zeros(4, dtype=torch.int64)), "idx_out")
    refuses(lambda: cgs.ctx_select(x, x, 4, key_out=z(P, dt=f32)), "key_out")
    refuses(lambda: cgs.ctx_select_from_keys(z(P, dt=f32), 4), "keys")

    Wa = cgs.FFN(z(ff, d), z(ff, d), z(ff, d), "fd")
    xa, full = z(S, d), torch.arange(ff, dtype=torch.int32)
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, y_anchor=z(S, d)), "y_anchor")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, h_anchor=z(S, ff, dt=f32)), "h_anchor")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, h_out=z(ff, S + 1, dt=f32)), "h_out")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, y_f32_out=z(S, d)), "y_f32_out")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full.long()), "idx")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa.float(), full), "x must be")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, y_out=z(S, d, dt=f32)), "y_out")
    refuses(lambda: cgs.act_ffn_masked(Wa, xa, full, glue=(z(S + 1, d, dt=f32), None, xa)), "glue residual")
    Wc = cgs.FFN(z(64, d), z(64, d), z(64, d), "fd")
    refuses(lambda: cgs.act_ffn_masked_compact(Wc, xa, torch.arange(63, dtype=torch.int32)), "idx")
    refuses(lambda: cgs.act_ffn_masked_compact(Wc, xa, full[:64], h_anchor=z(ff, S + 2, dt=f32)), "h_anchor")
    refuses(lambda: cgs.act_ffn_joint(Wc, xa, torch.arange(2, dtype=torch.int64), full[:64], z(S, d, dt=f32)),
            "tok")
    refuses(lambda: cgs.act_gather_rows(Wa, full[:64], out=cgs.FFN(z(64, d), z(64, d), z(63, d), "fd")),
            "w_down")
    refuses(lambda: cgs.ref_rebuild_dense([W], z(P, d, dt=f32)), "r0")
    refuses(lambda: cgs.ref_rebuild_dense([W], x, x_ref_out=z(2, P, d)), "x_ref_out")
    refuses(lambda: cgs.act_build_mask(z(1, ff, S, dt=torch.float64), Wa), "h_ref")
    refuses(lambda: cgs.act_build_mask(z(1, ff + 64, S, dt=f32), Wa), "h_ref")
    refuses(lambda: cgs.act_build_mask(z(1, ff, S, dt=f32), Wa, idx_out=torch.zeros(ff, dtype=torch.int64)),
            "idx_out")
    refuses(lambda: cgs.act_build_masks(z(2, 1, ff, S, dt=f32), [Wa, Wa], count_out=z(3, dt=torch.int32)),
            "count_out")
    refuses(lambda: cgs.act_down_norms([Wa], out=z(1, ff, dt=f32)), "out")
    refuses(lambda: cgs.residual_rmsnorm(z(P, d, dt=f32), y=z(P, d + 8)), "y")
    refuses(lambda: cgs.residual_rmsnorm(z(P, d)), "r must be")
    refuses(lambda: cgs.residual_rmsnorm(z(P, d, dt=f32), bias=z(d + 1, dt=f32)), "bias")
    q = z(1024)
    refuses(lambda: cgs.ret_select(q, z(4, 1000), 2, z(4, 14, dt=f32), z(4, 4, 14, dt=f32)), "refs")
    refuses(lambda: cgs.ret_select(q, z(4, 1024), 2, z(4, 14, dt=f32), z(3, 4, 14, dt=f32)), "r_hist")


def test_operands_past_32_bit_offsets_are_unsupported():
    """The GEMM cores address LDS-DMA sources with 32-bit byte offsets: a
    matrix spanning 2^32 bytes or more is refused before any launch (status
    CGS_ERR_UNSUPPORTED, workspace query 0), one case per operand."""
    L = cgs.lib()
    buf = ctypes.c_void_p(0x1000)
    out = ctypes.c_void_p(0x2000)
    assert L.cgs_ctx_ffn_recompute_workspace(231, 768, 2048, 16384, 0) > 0
    assert L.cgs_ctx_ffn_recompute_workspace(1, 1 << 20, 2048, 1024, 0) == 0        # x: P*d*2 = 2^32
    assert L.cgs_ctx_ffn_recompute_workspace(1, 8, 2048, 1 << 20, 0) == 0           # weights: ff*d*2 = 2^32
    assert L.cgs_ctx_ffn_recompute_workspace(1 << 17, 1 << 17, 128, 1 << 14, 0) == 0  # H: k*ff*2 = 2^32
    assert L.cgs_ref_rebuild_dense_workspace(1, 1 << 18, 128, 1 << 13, 1) == 0       # H: P*ff*4 = 2^33
    assert L.ctx_ffn_recompute(ctypes.byref(_ffn(d=2048, ff=1 << 20)), buf, buf, buf, 1, 8, out, None, buf,
                               1 << 40, None) == 4
    assert L.ctx_ffn_recompute(ctypes.byref(_ffn(d=2048, ff=1024)), buf, buf, buf, 1, 1 << 20, out, None, buf,
                               1 << 40, None) == 4
    arr = (cgs._Ffn * 1)(_ffn(d=2048, ff=1024))
    assert L.ref_rebuild_dense(arr, 1, buf, 1 << 20, buf, out, buf, 1 << 40, None) == 4
    wbig = _ffn(d=1024, ff=1 << 20, layout=1)                                       # W_down: ff*d*4 = 2^32
    assert L.act_ffn_masked(ctypes.byref(wbig), buf, 4, buf, 10, None, None, out, None, None, None, buf,
                            1 << 40, None) == 4
    assert L.act_ffn_masked_compact(ctypes.byref(wbig), buf, 4, buf, 1 << 20, None, None, out, None, None,
                                    None, buf, 1 << 40, None) == 4
    assert L.cgs_act_ffn_masked_workspace(50, 10, 1024, 1 << 20) == 0
    # retrieval: at most 2^24 features (their integer sums stay below 2^63)
    assert L.cgs_ret_select_workspace(16, 1 << 24) > 0
    assert L.cgs_ret_select_workspace(16, (1 << 24) + 8) == 0
    rr = cgs._Rerank(4, 14, -1, 0.8)
    assert L.ret_select(buf, buf, 16, (1 << 24) + 8, 0, 4, buf, buf, ctypes.byref(rr), buf, buf, buf, buf, buf,
                        1 << 30, None) == 2


def test_noalloc_entry_point_refuses_before_any_device_call():
    """The no-allocation variant rejects bad arguments and masks whose
    intermediates exceed its fixed scratch before it touches the device."""
    L = cgs.lib()
    buf = ctypes.c_void_p(0x1000)
    out = ctypes.c_void_p(0x2000)
    assert cgs.NOALLOC_SCRATCH_BYTES == 8 << 20
    # the advertised limit: 64 tokens x 4096 neurons at d = 1024 fit
    assert L.cgs_act_ffn_masked_workspace(64, 4096, 1024, 4096) <= cgs.NOALLOC_SCRATCH_BYTES
    big_k = 16384                      # 64 tokens x 16384 neurons do not
    assert L.cgs_act_ffn_masked_workspace(64, big_k, 1024, big_k) > cgs.NOALLOC_SCRATCH_BYTES
    wc = _ffn(d=1024, ff=big_k, layout=1)
    assert L.act_ffn_masked_compact_noalloc(ctypes.byref(wc), buf, 64, buf, big_k, None, None, out, None,
                                            None, None, None) == 3        # CGS_ERR_WORKSPACE
    w4 = _ffn(d=1024, ff=4096, layout=1)
    assert L.act_ffn_masked_compact_noalloc(ctypes.byref(w4), buf, 64, buf, 4095, None, None, out, None,
                                            None, None, None) == 2        # K != wc->ff
    assert L.act_ffn_masked_compact_noalloc(ctypes.byref(w4), None, 64, buf, 4096, None, None, out, None,
                                            None, None, None) == 1        # x missing
    assert L.act_ffn_masked_compact_noalloc(ctypes.byref(w4), buf, 0, buf, 4096, None, None, out, None,
                                            None, None, None) == 0        # S = 0: nothing to do
    w_odd = _ffn(d=1000, ff=4096, layout=1)
    assert L.act_ffn_masked_compact_noalloc(ctypes.byref(w_odd), buf, 64, buf, 4096, None, None, out, None,
                                            None, None, None) == 4


def test_mask_indices_and_masked_layers_validate_before_launch():
    L = cgs.lib()
    buf = ctypes.c_void_p(0x1000)
    assert L.act_mask_indices(buf, 4, 0, buf, None, None) == 2            # ff = 0
    assert L.act_mask_indices(buf, 4, 65537, buf, None, None) == 2        # ff past 65536
    assert L.act_mask_indices(buf, -1, 64, buf, None, None) == 2
    assert L.act_mask_indices(None, 4, 64, buf, None, None) == 1
    assert L.act_mask_indices(None, 0, 64, None, None, None) == 0         # n = 0: nothing to do
    r, x = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    need = L.cgs_act_masked_layers_workspace(50, 1024, 1300)
    assert need >= L.cgs_act_ffn_masked_workspace(50, 1300, 1024, 1300) + 50 * 1024 * 4
    arr = (cgs._MaskedLayer * 3)()
    for i, K in enumerate((4096, 1300, 0)):
        arr[i].w = _ffn(d=1024, ff=K, layout=1)
        arr[i].idx = 0x4000
    assert L.act_masked_layers(arr, 3, 50, r, x, buf, need, None) == 3            # ws sized for K 1300 < 4096
    assert L.act_masked_layers(arr, 3, 50, None, x, buf, 1 << 40, None) == 1      # r missing
    assert L.act_masked_layers(arr, 0, 50, None, None, None, 0, None) == 0        # n = 0
    arr[1].w = _ffn(d=512, ff=1300, layout=1)
    assert L.act_masked_layers(arr, 3, 50, r, x, buf, 1 << 40, None) == 2         # d differs
    arr[1].w = _ffn(d=1024, ff=1300, layout=0)
    assert L.act_masked_layers(arr, 3, 50, r, x, buf, 1 << 40, None) == 1         # not neuron-major
    arr[1].w = _ffn(d=1024, ff=1300, layout=1)
    arr[1].idx = None
    arr[1].h_anchor = 0x5000
    assert L.act_masked_layers(arr, 3, 50, r, x, buf, 1 << 40, None) == 1         # h_anchor without idx


def test_binding_status_codes_match_the_header():
    """The binding's CGS_* status constants are the header's cgs_status values."""
    import re
    text = open(cgs.HEADER_PATH).read()
    enum = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"\b(CGS_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", text))
    assert enum, "no cgs_status values found in the header"
    for name, value in enum.items():
        assert getattr(cgs, name) == value, name
