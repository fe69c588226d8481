"""C-ABI checks that need no GPU: libmsm.so loads, exports every function that
include/msm.h declares, sizes its workspace, and rejects bad arguments before any
HIP call is made."""
import ctypes
import os
import re

import pytest

from elliptic_curve_scalar_amd import msm as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(msm\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for want in ("msm", "msm_run", "msm_ctx_create", "msm_ctx_destroy", "msm_workspace_bytes",
                 "msm_last_error", "msm_g1_from_scalars", "msm_test_fp", "msm_test_fp_mul",
                 "msm_test_fp_sqr", "msm_test_fp_add", "msm_test_fp_sub", "msm_test_fp_inv",
                 "msm_test_batched_add", "msm_version"):
        assert want in names
    assert set(names) == set(M.SYMBOLS), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    L = M.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert L.msm_version() >= 100


def test_workspace_bytes():
    assert M.workspace_bytes(1 << 16, 13) > 0
    assert M.workspace_bytes(1 << 16, 13) % 256 == 0
    for c in (1, 8, 13, 16):  # n = 0 and tiny n still plan a workspace
        assert M.workspace_bytes(0, c) > 0 and M.workspace_bytes(1, c) > 0
    assert M.workspace_bytes(1 << 16, 0) == 0
    assert M.workspace_bytes(1 << 16, 17) == 0
    assert M.workspace_bytes(M.MSM_MAX_N + 1, 8) == 0
    assert M.workspace_bytes(1 << 20, 16) > M.workspace_bytes(1 << 16, 16)
    assert M.workspace_bytes(1 << 16, 13, 4) == M.workspace_bytes(1 << 16, 13, 32)
    # 2 n ceil(128 / c) bucket entries must fit 32-bit offsets
    assert M.workspace_bytes(M.MSM_MAX_N, 5) > 0
    assert M.workspace_bytes(M.MSM_MAX_N, 4) == 0


def _err(L):
    return L.msm_last_error().decode()


def test_argument_errors_without_gpu():
    L = M.lib()
    out = ctypes.c_void_p(256)
    p = ctypes.c_void_p(512)
    # NULL context
    assert L.msm_run(None, p, p, 16, 13, 8, 0, 0, None, 0, None, out) == M.MSM_ERR_ARG
    assert "ctx" in _err(L)
    # NULL h_out / bad c / bad S / misaligned pointers on the synchronous form
    assert L.msm(p, p, 16, 13, None) == M.MSM_ERR_ARG
    assert L.msm(p, p, 16, 0, out) == M.MSM_ERR_ARG
    assert "1..16" in _err(L)
    assert L.msm(p, p, 16, 17, out) == M.MSM_ERR_ARG
    assert L.msm(ctypes.c_void_p(513), p, 16, 13, out) == M.MSM_ERR_ARG
    assert "aligned" in _err(L)
    assert L.msm(None, p, 16, 13, out) == M.MSM_ERR_ARG
    assert L.msm(p, p, M.MSM_MAX_N + 1, 13, out) == M.MSM_ERR_ARG
    assert L.msm(p, p, M.MSM_MAX_N, 4, out) == M.MSM_ERR_ARG
    assert "32-bit" in _err(L)
    # generator and test hooks
    assert L.msm_g1_from_scalars(None, 4, p, None) == M.MSM_ERR_ARG
    assert L.msm_g1_from_scalars(ctypes.c_void_p(4), 4, p, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp(9, p, p, p, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp(-1, p, p, p, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp(0, p, None, p, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp_mul(p, None, p, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp_sub(None, p, p, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp_inv(p, None, 4, None) == M.MSM_ERR_ARG
    assert L.msm_test_fp_sqr(p, p, M.MSM_MAX_N + 1, None) == M.MSM_ERR_ARG
    assert L.msm_test_batched_add(p, p, p, 4, 5, None) == M.MSM_ERR_ARG
    assert L.msm_test_batched_add(p, ctypes.c_void_p(8), p, 4, 8, None) == M.MSM_ERR_ARG
    assert L.msm_test_glv(None, 4, p, None) == M.MSM_ERR_ARG
    assert L.msm_test_issue_rate(3, 1, 1, p, None) == M.MSM_ERR_ARG
    assert L.msm_test_issue_rate(0, 0, 1, p, None) == M.MSM_ERR_ARG
    assert L.msm_test_issue_rate(0, 1, 0, p, None) == M.MSM_ERR_ARG
    assert L.msm_test_issue_rate(0, 1, 1, None, None) == M.MSM_ERR_ARG
    assert L.msm_test_row(10, p, p, p, 4, 0, None) == M.MSM_ERR_ARG     # unknown op
    assert L.msm_test_row(7, p, None, p, 4, 0, None) == M.MSM_ERR_ARG    # point sum, no b
    assert L.msm_test_row(-1, p, p, p, 4, 0, None) == M.MSM_ERR_ARG
    assert L.msm_test_row(0, p, None, p, 4, 0, None) == M.MSM_ERR_ARG    # binary op, no b
    assert L.msm_test_row(3, p, None, p, 4, 5000, None) == M.MSM_ERR_ARG  # d > 4096
    assert L.msm_test_row(5, p, p, p, 8, 10, None) == M.MSM_ERR_ARG      # probe takes n = 4
    assert L.msm_test_row(1, ctypes.c_void_p(6), p, p, 4, 0, None) == M.MSM_ERR_ARG
    assert L.msm_test_glv(p, 4, ctypes.c_void_p(4), None) == M.MSM_ERR_ARG
    # context creation with a NULL out pointer
    assert L.msm_ctx_create(0, None) == M.MSM_ERR_ARG


def test_run_argument_errors_without_gpu():
    """msm_run checks S, sched, verify, c and the workspace before any HIP call; a
    dummy context pointer is never dereferenced on these paths."""
    L = M.lib()
    out = ctypes.c_void_p(256)
    p = ctypes.c_void_p(512)
    ctx = ctypes.c_void_p(4096)
    assert L.msm_run(ctx, p, p, 16, 13, 5, 0, 0, None, 0, None, out) == M.MSM_ERR_ARG
    assert "S must be" in _err(L)
    for sched in (-1, 2, 7):
        assert L.msm_run(ctx, p, p, 16, 13, 8, sched, 0, None, 0, None, out) == M.MSM_ERR_ARG
        assert "sched" in _err(L)
    for verify in (-1, 2):
        assert L.msm_run(ctx, p, p, 16, 13, 8, 0, verify, None, 0, None, out) == M.MSM_ERR_ARG
        assert "verify" in _err(L)
    assert L.msm_run(ctx, p, p, 16, 0, 8, 0, 0, None, 0, None, out) == M.MSM_ERR_ARG
    assert L.msm_run(ctx, p, p, 16, 13, 8, 1, 1, None, 0, None, None) == M.MSM_ERR_ARG
    assert L.msm_run(ctx, ctypes.c_void_p(520), p, 16, 13, 8, 0, 0, None, 0, None, out) == M.MSM_ERR_ARG
    # a caller workspace below msm_workspace_bytes, or misaligned, is refused
    need = M.workspace_bytes(16, 13)
    ws = ctypes.c_void_p(1 << 20)
    assert L.msm_run(ctx, p, p, 16, 13, 8, 0, 0, ws, need - 1, None, out) == M.MSM_ERR_ARG
    assert "workspace" in _err(L)
    assert L.msm_run(ctx, p, p, 16, 13, 8, 0, 0, ctypes.c_void_p((1 << 20) + 16), need, None,
                     out) == M.MSM_ERR_ARG
    assert M.MSM_ERR_OFF_CURVE == -5 and (M.MSM_SCHED_PAIR_TREE, M.MSM_SCHED_WALKER) == (0, 1)
    # the no-allocation entry point checks the same arguments
    assert L.msm_run_noalloc(None, p, p, 16, 13, 8, 0, 0, None, out) == M.MSM_ERR_ARG
    assert L.msm_run_noalloc(ctx, p, p, 16, 13, 8, 3, 0, None, out) == M.MSM_ERR_ARG
    assert L.msm_run_noalloc(ctx, p, p, 16, 17, 8, 0, 0, None, out) == M.MSM_ERR_ARG
    # context knobs: NULL context and out-of-range values are refused before any use
    assert L.msm_ctx_set_scalar_form(None, 0) == M.MSM_ERR_ARG
    for form in (-1, 2):
        assert L.msm_ctx_set_scalar_form(ctx, form) == M.MSM_ERR_ARG
    assert (M.MSM_SCALARS_INTEGER, M.MSM_SCALARS_MONTGOMERY) == (0, 1)


def test_binding_refuses_host_tensors():
    import torch
    pts = torch.zeros((4, 16), dtype=torch.int32)
    with pytest.raises(ValueError):
        M._dev_ptr(pts, 16, "points")
