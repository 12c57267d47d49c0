"""The C-ABI library without a GPU: it loads, exports every function that
include/*.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from conftest import ROOT

import sparse_spd_selected_amd as ssa


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(selinv_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssa.LIB_PATH):
        ssa.build()
    return ssa.lib()


def test_header_declares_entry_points():
    names = _declared()
    for want in ("selinv_chain_f64", "selinv_chain_f32", "selinv_star_f64", "selinv_star_f32",
                 "selinv_tree_f64", "selinv_tree_f32", "selinv_tree_plan_create",
                 "selinv_tree_plan_destroy", "selinv_chain_workspace_bytes",
                 "selinv_star_workspace_bytes", "selinv_tree_workspace_bytes", "selinv_strerror"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_strerror_and_version(lib):
    assert lib.selinv_strerror(0) == b"ok"
    assert b"tree" in lib.selinv_strerror(2)
    assert b"wait" in lib.selinv_strerror(ssa.WAIT_TIMEOUT)
    assert lib.selinv_strerror(99) == b"unknown status"
    assert lib.selinv_version() >= 100


def test_header_status_codes_match_binding():
    src = open(os.path.join(ROOT, "include", "selinv.h")).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"#define (SELINV_[A-Z_]+) \(?(-?\d+)\)?", src))
    assert codes["SELINV_ERR_WAIT_TIMEOUT"] == ssa.WAIT_TIMEOUT
    assert codes["SELINV_INFO_WAIT_TIMEOUT"] == ssa.INFO_WAIT_TIMEOUT
    assert codes["SELINV_ERR_BAD_PATTERN"] == ssa.BAD_PATTERN
    assert codes["SELINV_ERR_SCRATCH_LIMIT"] == ssa.SCRATCH_LIMIT


def test_raise_info_distinguishes_timeout_from_not_pd(lib):
    import torch
    with pytest.raises(ssa.WaitTimeout):
        ssa._raise_info(torch.tensor([0, -1, 3], dtype=torch.int32), "tree")
    with pytest.raises(ssa.NotPositiveDefinite):
        ssa._raise_info(torch.tensor([0, 0, 3], dtype=torch.int32), "chain")
    ssa._raise_info(torch.zeros(4, dtype=torch.int32), "chain")


def test_workspace_sizes(lib):
    assert lib.selinv_chain_workspace_bytes(8, 4096, 64, 16) >= 4096 * 64 * 136 * 8
    assert lib.selinv_chain_workspace_bytes(8, 3, 5, 4) >= 3 * 5 * 64 * 8  # padded 8x8 state
    assert lib.selinv_chain_workspace_bytes(3, 1, 1, 1) == 0  # bad dtype size
    assert lib.selinv_chain_workspace_bytes(8, 1, 1, 33) == 0  # b > 32
    assert lib.selinv_star_workspace_bytes(4, 2, 0, 4) > 0
    assert lib.selinv_tree_workspace_bytes(None) == 0


def _chain_call(lib, B=1, L=2, b=4, diag=1, lower=1, gd=1, gl=1, ld=1, ws=1, wsb=1 << 30):
    # never dereferenced on error paths; an int above 1 is taken as the address
    p = lambda x: ctypes.c_void_p(x if x > 1 else 0x1000) if x else None
    return lib.selinv_chain_f64(B, L, b, p(diag), p(lower), p(gd), p(gl), p(ld), None, p(ws),
                                wsb, None)


def test_chain_argument_validation(lib):
    assert _chain_call(lib, b=0) == ssa.INVALID_ARG
    assert _chain_call(lib, b=33) == ssa.INVALID_ARG
    assert _chain_call(lib, L=0) == ssa.INVALID_ARG
    assert _chain_call(lib, B=-1) == ssa.INVALID_ARG
    assert _chain_call(lib, diag=0) == ssa.INVALID_ARG
    assert _chain_call(lib, lower=0) == ssa.INVALID_ARG
    assert _chain_call(lib, ld=0) == ssa.INVALID_ARG
    assert _chain_call(lib, wsb=16) == ssa.INVALID_ARG
    assert _chain_call(lib, ws=0) == ssa.INVALID_ARG
    assert _chain_call(lib, B=0) == ssa.OK  # empty batch: nothing to do
    # block arrays must be 16-byte aligned, the workspace 256-byte aligned
    assert _chain_call(lib, b=16, diag=0x1008) == ssa.INVALID_ARG
    assert _chain_call(lib, b=3, gl=0x1004) == ssa.INVALID_ARG
    assert _chain_call(lib, ws=0x1010) == ssa.INVALID_ARG


def test_star_argument_validation(lib):
    p = ctypes.c_void_p(0x1000)
    assert lib.selinv_star_f32(1, 2, 0, p, p, p, p, p, p, p, None, p, 1 << 30, None) == \
        ssa.INVALID_ARG
    assert lib.selinv_star_f32(1, 2, 4, p, None, p, p, p, p, p, None, p, 1 << 30, None) == \
        ssa.INVALID_ARG
    assert lib.selinv_star_f32(1, 2, 4, p, p, p, p, p, p, p, None, p, 8, None) == ssa.INVALID_ARG
    q = ctypes.c_void_p(0x1004)
    assert lib.selinv_star_f32(1, 2, 4, p, q, p, p, p, p, p, None, p, 1 << 30, None) == \
        ssa.INVALID_ARG


@pytest.mark.parametrize("parent", [[-1, 0, -1], [0, 0, 1], [-1, 2, 3, 1], [-1, 0, 7],
                                    [-1, 1]])
def test_tree_plan_rejects_invalid_trees(lib, parent):
    a = np.array(parent, np.int32)
    h = ctypes.c_void_p()
    rc = lib.selinv_tree_plan_create(a.ctypes.data, len(a), 4, 8, None, ctypes.byref(h))
    assert rc == ssa.BAD_TREE and not h.value


def test_tree_plan_argument_validation(lib):
    a = np.array([-1, 0], np.int32)
    h = ctypes.c_void_p()
    assert lib.selinv_tree_plan_create(a.ctypes.data, 2, 0, 8, None, ctypes.byref(h)) == \
        ssa.INVALID_ARG
    assert lib.selinv_tree_plan_create(a.ctypes.data, 2, 4, 2, None, ctypes.byref(h)) == \
        ssa.INVALID_ARG
    assert lib.selinv_tree_plan_create(None, 2, 4, 8, None, ctypes.byref(h)) == ssa.INVALID_ARG
    p = ctypes.c_void_p(0x1000)
    assert lib.selinv_tree_f64(None, p, p, p, p, p, None, p, 1 << 30, None) == ssa.INVALID_ARG


def test_python_binding_rejects_cpu_tensors():
    import torch
    d = torch.zeros(1, 2, 4, 4, dtype=torch.float64)
    l = torch.zeros(1, 1, 4, 4, dtype=torch.float64)
    with pytest.raises(ValueError):
        ssa.chain(d, l)
    with pytest.raises(TypeError):
        ssa.chain(d.numpy(), l)


def test_vjp_workspace_sizes(lib):
    # b = 16: packed Sinv and packed GG per block
    assert lib.selinv_chain_vjp_workspace_bytes(8, 4096, 64, 16) >= 4096 * 64 * 272 * 8
    assert lib.selinv_chain_vjp_workspace_bytes(4, 3, 5, 7) >= 3 * 5 * 4 * 49 * 4
    assert lib.selinv_chain_vjp_workspace_bytes(8, 1, 0, 4) == 0  # L < 1
    assert lib.selinv_star_vjp_workspace_bytes(8, 2, 3, 33) == 0
    assert lib.selinv_star_vjp_workspace_bytes(8, 2, 3, 4) >= 5 * 6 * 16 * 8
    assert lib.selinv_tree_vjp_workspace_bytes(None) == 0


def _chain_vjp_call(lib, B=1, L=2, b=4, diag=1, lower=1, gd=1, gl=1, db=1, lb=1, ws=1,
                    wsb=1 << 30):
    p = lambda x: ctypes.c_void_p(x if x > 1 else 0x1000) if x else None
    return lib.selinv_chain_vjp_f64(B, L, b, p(diag), p(lower), p(gd), p(gl), None, p(db),
                                    p(lb), None, p(ws), wsb, None)


def test_chain_vjp_argument_validation(lib):
    assert _chain_vjp_call(lib, b=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, L=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, gd=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, gl=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, lb=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, db=0) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, wsb=64) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, gl=0x1008) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, ws=0x1040) == ssa.INVALID_ARG
    assert _chain_vjp_call(lib, B=0) == ssa.OK


def test_star_and_tree_vjp_argument_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def star(b=4, leaves_bar=p, wsb=1 << 30):
        # center, leaves, coupling, three cotangents, logdet_bar, three outputs, info
        return lib.selinv_star_vjp_f64(1, 2, b, p, p, p, p, p, p, None, p, leaves_bar, p, None,
                                       p, wsb, None)
    assert star(b=0) == ssa.INVALID_ARG
    assert star(leaves_bar=None) == ssa.INVALID_ARG
    assert star(wsb=8) == ssa.INVALID_ARG
    assert lib.selinv_tree_vjp_f64(None, p, p, p, p, None, p, p, None, p, 1 << 30, None) == \
        ssa.INVALID_ARG


def test_tree_graph_argument_validation(lib):
    """The tree graph calls reject a missing plan, handle or output pointer
    before any device work; queries and destroy accept NULL."""
    p = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    for f in (lib.selinv_tree_graph_create_f64, lib.selinv_tree_graph_create_f32):
        assert f(None, p, p, p, p, p, None, p, 1 << 30, ctypes.byref(h)) == ssa.INVALID_ARG
        assert f(None, p, p, p, p, p, None, p, 1 << 30, None) == ssa.INVALID_ARG
    assert not h.value
    assert lib.selinv_tree_graph_launch(None, None) == ssa.INVALID_ARG
    assert lib.selinv_tree_graph_nodes(None) == -1
    lib.selinv_tree_graph_destroy(None)


def test_wait_limit_setting(lib):
    """The dataflow wait bound is a host-side setting (no device work)."""
    old = lib.selinv_wait_limit()
    assert old == 1 << 24
    try:
        lib.selinv_set_wait_limit(12345)
        assert lib.selinv_wait_limit() == 12345
    finally:
        lib.selinv_set_wait_limit(old)
    assert lib.selinv_wait_limit() == old


def test_junction_argument_validation(lib):
    """The junction entry points reject bad arguments before touching a device:
    a null plan, sizes and dtypes out of range, bad patterns (checked by the
    host-only symbolic analysis, which shares the plan's validation)."""
    vp = ctypes.c_void_p
    h = vp()
    e = np.array([[1], [0]], np.int32)
    # plan creation: bad sizes and dtypes are rejected before any device work
    assert lib.selinv_junction_plan_create(0, 1, e.ctypes.data, None, 4, 8, None,
                                           ctypes.byref(h)) == 1
    assert lib.selinv_junction_plan_create(2, 1, e.ctypes.data, None, 33, 8, None,
                                           ctypes.byref(h)) == 1
    assert lib.selinv_junction_plan_create(2, 1, e.ctypes.data, None, 4, 2, None,
                                           ctypes.byref(h)) == 1
    assert lib.selinv_junction_plan_create(2, 1, None, None, 4, 8, None, ctypes.byref(h)) == 1
    assert lib.selinv_junction_plan_create(2, 1, e.ctypes.data, None, 4, 8, None, None) == 1
    # queries on a null plan
    assert lib.selinv_junction_plan_nnz(None) == -1
    assert lib.selinv_junction_plan_levels(None) == -1
    assert lib.selinv_junction_workspace_bytes(None, 4) == 0
    assert lib.selinv_junction_plan_pattern(None, None, None) == 1
    lib.selinv_junction_plan_destroy(None)
    # calls without a plan
    for f in (lib.selinv_junction_f64, lib.selinv_junction_f32):
        assert f(None, 1, None, None, None, None, None, None, None, 0, None) == 1
    # the symbolic analysis: status 4 for bad patterns and orders
    nnz, lev = ctypes.c_int64(), ctypes.c_int32()
    bad = [np.array([[0], [1]], np.int32), np.array([[1, 1], [0, 0]], np.int32),
           np.array([[5], [0]], np.int32)]
    for b in bad:
        assert lib.selinv_junction_symbolic(3, b.shape[1], b.ctypes.data, None, ctypes.byref(nnz),
                                            ctypes.byref(lev), None, 0, None) == 4
    o = np.array([0, 0, 1], np.int32)
    assert lib.selinv_junction_symbolic(3, 1, e.ctypes.data, o.ctypes.data, ctypes.byref(nnz),
                                        ctypes.byref(lev), None, 0, None) == 4
    assert lib.selinv_junction_symbolic(3, 1, e.ctypes.data, None, ctypes.byref(nnz),
                                        ctypes.byref(lev), None, 0, None) == 0
    assert nnz.value == 1 and lev.value == 2
    assert lib.selinv_strerror(4) != b"unknown status"
