"""MI355X batched selected inverse of block-structured SPD matrices.

Python binding of ``libselinv.so`` (C ABI in ``include/selinv.h``).  This
module only marshals arguments: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.

    G_diag, G_lower, logdet = chain(diag, lower)            # block tridiagonal
    G_center, G_leaf, G_cross, logdet = star(center, leaves, coupling)
    G_diag, G_edge, logdet = tree(parent, diag, edge)       # any rooted tree

Shapes and orientations follow the Quickstart section of the
gabp-sparse-inv 0.3.2 page: ``lower[i] = A_{i+1,i}``, ``coupling[j] =
A_{j,0}``, ``edge[v] = A_{parent(v),v}``; leading batch dimensions are allowed
for the chain and star.  ``check=True`` synchronises and raises
``NotPositiveDefinite`` if any Schur pivot failed (the "not positive definite
-> error" convention of the sparsax page), ``WaitTimeout`` if a bounded wait of
the single-launch tree schedule expired (info = -1), and validates the inputs.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
from collections import OrderedDict

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselinv.so")

OK, INVALID_ARG, BAD_TREE, HIP_ERROR, BAD_PATTERN, WAIT_TIMEOUT, SCRATCH_LIMIT = range(7)
INFO_WAIT_TIMEOUT = -1
MAX_B = 32

_lib = None


class SelinvError(RuntimeError):
    """A non-zero status returned by the C ABI."""


class NotPositiveDefinite(SelinvError):
    """A Schur pivot was not positive definite (info > 0)."""


class WaitTimeout(SelinvError):
    """A bounded wait between workgroups of the single-launch tree schedule
    expired (info = -1): the outputs are NaN.  Not a property of the matrix;
    it can happen when other work holds the GPU for longer than the bound
    (set_wait_limit).  Calling again is the remedy."""


def build():
    """Compile libselinv.so in place (hipcc, gfx950)."""
    from . import buildlib as _b
    global _lib
    _lib = None
    return _b.build()


def lib():
    """The loaded C library.  Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libselinv.so is not built (run sparse_spd_selected_amd.build())")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    L.selinv_chain_static_scratch_bytes.argtypes = []
    L.selinv_chain_static_scratch_bytes.restype = sz
    for name in ("selinv_chain_noalloc_f64", "selinv_chain_noalloc_f32"):
        f = getattr(L, name)
        f.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
        f.restype = ctypes.c_int
    L.selinv_tree_schedule.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp]
    L.selinv_tree_schedule.restype = ctypes.c_int
    L.selinv_strerror.argtypes = [ctypes.c_int]
    L.selinv_strerror.restype = ctypes.c_char_p
    L.selinv_version.restype = ctypes.c_int
    L.selinv_chain_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
    L.selinv_chain_workspace_bytes.restype = sz
    L.selinv_star_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
    L.selinv_star_workspace_bytes.restype = sz
    for name in ("selinv_chain_f64", "selinv_chain_f32"):
        f = getattr(L, name)
        f.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    for name in ("selinv_star_f64", "selinv_star_f32"):
        f = getattr(L, name)
        f.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    L.selinv_tree_plan_create.argtypes = [vp, i64, i32, ctypes.c_int, vp, ctypes.POINTER(vp)]
    L.selinv_tree_plan_create.restype = ctypes.c_int
    L.selinv_tree_plan_destroy.argtypes = [vp]
    L.selinv_tree_plan_destroy.restype = None
    L.selinv_tree_plan_levels.argtypes = [vp]
    L.selinv_tree_plan_levels.restype = i32
    L.selinv_tree_workspace_bytes.argtypes = [vp]
    L.selinv_tree_workspace_bytes.restype = sz
    for name in ("selinv_tree_f64", "selinv_tree_f32"):
        f = getattr(L, name)
        f.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    for name in ("selinv_tree_graph_create_f64", "selinv_tree_graph_create_f32"):
        f = getattr(L, name)
        f.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, ctypes.POINTER(vp)]
        f.restype = ctypes.c_int
    L.selinv_set_wait_limit.argtypes = [ctypes.c_uint64]
    L.selinv_set_wait_limit.restype = None
    L.selinv_wait_limit.argtypes = []
    L.selinv_wait_limit.restype = ctypes.c_uint64
    L.selinv_tree_graph_launch.argtypes = [vp, vp]
    L.selinv_tree_graph_launch.restype = ctypes.c_int
    L.selinv_tree_graph_nodes.argtypes = [vp]
    L.selinv_tree_graph_nodes.restype = i64
    L.selinv_tree_graph_destroy.argtypes = [vp]
    L.selinv_tree_graph_destroy.restype = None
    L.selinv_chain_vjp_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
    L.selinv_chain_vjp_workspace_bytes.restype = sz
    L.selinv_star_vjp_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
    L.selinv_star_vjp_workspace_bytes.restype = sz
    L.selinv_tree_vjp_workspace_bytes.argtypes = [vp]
    L.selinv_tree_vjp_workspace_bytes.restype = sz
    for name in ("selinv_chain_vjp_f64", "selinv_chain_vjp_f32"):
        f = getattr(L, name)
        f.argtypes = [i64, i64, i32] + [vp] * 8 + [vp, sz, vp]
        f.restype = ctypes.c_int
    for name in ("selinv_star_vjp_f64", "selinv_star_vjp_f32"):
        f = getattr(L, name)
        f.argtypes = [i64, i64, i32] + [vp] * 11 + [vp, sz, vp]
        f.restype = ctypes.c_int
    for name in ("selinv_tree_vjp_f64", "selinv_tree_vjp_f32"):
        f = getattr(L, name)
        f.argtypes = [vp] * 9 + [vp, sz, vp]
        f.restype = ctypes.c_int
    q = {"selinv_chain_factor_bytes": [ctypes.c_int, i64, i64, i32],
         "selinv_star_factor_bytes": [ctypes.c_int, i64, i64, i32],
         "selinv_star_factor_workspace_bytes": [ctypes.c_int, i64, i64, i32],
         "selinv_star_solve_workspace_bytes": [ctypes.c_int, i64, i64, i32, i64],
         "selinv_tree_factor_bytes": [vp], "selinv_tree_factor_workspace_bytes": [vp],
         "selinv_tree_solve_workspace_bytes": [vp, i64]}
    for name, args in q.items():
        getattr(L, name).argtypes = args
        getattr(L, name).restype = sz
    sigs = {"chain_factor": [i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "chain_solve": [i64, i64, i32, vp, vp, i64, vp, vp, vp],
            "chain_sample": [i64, i64, i32, vp, vp, i64, vp, vp, vp],
            "star_factor": [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "star_solve": [i64, i64, i32, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp],
            "star_sample": [i64, i64, i32, vp, vp, i64, vp, vp, vp, vp, vp],
            "tree_factor": [vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "tree_solve": [vp, vp, vp, i64, vp, vp, vp, sz, vp],
            "tree_sample": [vp, vp, vp, i64, vp, vp, vp, sz, vp]}
    for name, args in sigs.items():
        for sfx in ("f64", "f32"):
            f = getattr(L, "selinv_%s_%s" % (name, sfx))
            f.argtypes = args
            f.restype = ctypes.c_int
    L.selinv_bidiag_workspace_bytes.argtypes = [i64]
    L.selinv_bidiag_workspace_bytes.restype = sz
    L.selinv_nonsym_tree_workspace_bytes.argtypes = [vp]
    L.selinv_nonsym_tree_workspace_bytes.restype = sz
    for sfx in ("f64", "f32"):
        f = getattr(L, "selinv_bidiag_" + sfx)
        f.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
        f = getattr(L, "selinv_nonsym_tree_" + sfx)
        f.argtypes = [vp] * 8 + [vp, sz, vp]
        f.restype = ctypes.c_int
    L.selinv_junction_plan_create.argtypes = [i64, i64, vp, vp, i32, ctypes.c_int, vp,
                                              ctypes.POINTER(vp)]
    L.selinv_junction_plan_create.restype = ctypes.c_int
    L.selinv_junction_plan_destroy.argtypes = [vp]
    L.selinv_junction_plan_destroy.restype = None
    L.selinv_junction_plan_nnz.argtypes = [vp]
    L.selinv_junction_plan_nnz.restype = i64
    L.selinv_junction_plan_levels.argtypes = [vp]
    L.selinv_junction_plan_levels.restype = i32
    L.selinv_junction_plan_pattern.argtypes = [vp, vp, vp]
    L.selinv_junction_plan_pattern.restype = ctypes.c_int
    L.selinv_junction_symbolic.argtypes = [i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.selinv_junction_symbolic.restype = ctypes.c_int
    L.selinv_junction_workspace_bytes.argtypes = [vp, i64]
    L.selinv_junction_workspace_bytes.restype = sz
    for sfx in ("f64", "f32"):
        f = getattr(L, "selinv_junction_" + sfx)
        f.argtypes = [vp, i64] + [vp] * 6 + [vp, sz, vp]
        f.restype = ctypes.c_int
        f = getattr(L, "selinv_junction_logdet_" + sfx)
        f.argtypes = [vp, i64] + [vp] * 4 + [vp, sz, vp]
        f.restype = ctypes.c_int
        f = getattr(L, "selinv_junction_factor_" + sfx)
        f.argtypes = [vp, i64] + [vp] * 5 + [vp, sz, vp]
        f.restype = ctypes.c_int
        f = getattr(L, "selinv_junction_solve_" + sfx)
        f.argtypes = [vp, i64, vp, i64, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
        f = getattr(L, "selinv_junction_sample_" + sfx)
        f.argtypes = [vp, i64, vp, i64, vp, vp, vp]
        f.restype = ctypes.c_int
    L.selinv_junction_solve_workspace_bytes.argtypes = [vp, i64, i64]
    L.selinv_junction_solve_workspace_bytes.restype = sz
    for name in ("selinv_junction_factor_bytes", "selinv_junction_factor_workspace_bytes"):
        getattr(L, name).argtypes = [vp, i64]
        getattr(L, name).restype = sz
    _lib = L
    return L


def _status(rc: int, what: str):
    if rc != OK:
        msg = lib().selinv_strerror(rc).decode()
        raise SelinvError("%s: status %d (%s)" % (what, rc, msg))


def _sfx(t: torch.Tensor) -> str:
    if t.dtype == torch.float64:
        return "f64"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError("selected inverse supports float32 and float64, got %s" % t.dtype)


def _ptr(t):
    return t.data_ptr() if (t is not None and t.numel()) else None


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(t, name, device, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device (got %s)" % (name, t.device))
    if t.device != device or t.dtype != dtype:
        raise ValueError("%s: device/dtype mismatch" % name)
    t = t.contiguous()
    if t.data_ptr() % 16:  # the library takes 16-byte aligned block arrays
        t = t.clone()
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    # 256-byte alignment is guaranteed by the caching allocator (512 B)
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _validate_values(name, t):
    if not torch.isfinite(t).all():
        raise ValueError("%s has non-finite entries" % name)


def _validate_symmetric(name, t):
    if t.numel() and not torch.equal(t, t.transpose(-1, -2)):
        raise ValueError("%s blocks must be exactly symmetric" % name)


def _raise_info(info: torch.Tensor, what: str):
    timed_out = (info == INFO_WAIT_TIMEOUT).nonzero()
    if timed_out.numel():
        idx = tuple(int(i) for i in timed_out[0])
        raise WaitTimeout("%s: %s (matrix %s)" % (
            what, lib().selinv_strerror(WAIT_TIMEOUT).decode(), idx))
    bad = info.nonzero()
    if bad.numel():
        idx = tuple(int(i) for i in bad[0])
        raise NotPositiveDefinite("%s: Schur pivot not positive definite (matrix %s, info=%d)"
                                  % (what, idx, int(info[idx])))


def tree_schedule(parent):
    """The breadth-first level-set schedule of a parent array, computed on the
    host by the library (selinv_tree_schedule): a dict of numpy arrays
    node_at, parent_pos, child_beg, child_end, fail_rank (per position) and
    level_off (levels + 1)."""
    import numpy as np
    parent = np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    n = parent.shape[0]
    out = {k: np.empty(n, np.int32) for k in ("node_at", "parent_pos", "child_beg", "child_end",
                                               "fail_rank")}
    level_off = np.empty(n + 1, np.int64)
    levels = ctypes.c_int32(0)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = lib().selinv_tree_schedule(p(parent), n, p(out["node_at"]), p(out["parent_pos"]),
                                    p(out["child_beg"]), p(out["child_end"]),
                                    p(out["fail_rank"]), p(level_off), ctypes.byref(levels))
    _status(rc, "selinv_tree_schedule")
    out["level_off"] = level_off[:levels.value + 1].copy()
    return out


# ------------------------------------------------------------------ chain
def chain(diag: torch.Tensor, lower: torch.Tensor, check: bool = False, return_info=False):
    """Selected inverse of block-tridiagonal SPD chains.

    diag [..., L, b, b], lower [..., L-1, b, b] with lower[i] = A_{i+1,i}.
    Returns (G_diag [..., L, b, b], G_lower [..., L-1, b, b], logdet [...]
    float64), plus info [...] int32 when return_info.
    """
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    lower = _check_tensor(lower, "lower", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() < 3 or diag.shape[-1] != diag.shape[-2]:
        raise ValueError("diag must be [..., L, b, b]")
    *batch, L, b, _ = diag.shape
    if L < 1 or b < 1 or b > MAX_B:
        raise ValueError("need L >= 1 and 1 <= b <= %d" % MAX_B)
    if tuple(lower.shape) != tuple(batch) + (L - 1, b, b):
        raise ValueError("lower must be [..., L-1, b, b] matching diag")
    if check:
        _validate_values("diag", diag)
        _validate_values("lower", lower)
        _validate_symmetric("diag", diag)
    B = 1
    for s in batch:
        B *= s
    G_diag = torch.empty_like(diag)
    G_lower = torch.empty_like(lower)
    logdet = torch.empty(tuple(batch), dtype=torch.float64, device=dev)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    L_ = lib()
    ws_bytes = L_.selinv_chain_workspace_bytes(diag.element_size(), B, L, b)
    ws = _workspace(ws_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_chain_" + sfx)(
            B, L, b, _ptr(diag), _ptr(lower), _ptr(G_diag), _ptr(G_lower), _ptr(logdet),
            _ptr(info), _ptr(ws), ws_bytes, _stream(dev))
    _status(rc, "selinv_chain_" + sfx)
    if check:
        _raise_info(info, "chain")
    if return_info:
        return G_diag, G_lower, logdet, info
    return G_diag, G_lower, logdet


def chain_noalloc(diag: torch.Tensor, lower: torch.Tensor, return_info=False):
    """chain() through the entry point that allocates no scratch
    (selinv_chain_noalloc_*): the kernels use the library's static per-device
    scratch array instead of a workspace.  Only the outputs are allocated
    here; calls that overlap in time on one device race."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    lower = _check_tensor(lower, "lower", dev, dt)
    if diag.dim() < 3 or diag.shape[-1] != diag.shape[-2]:
        raise ValueError("diag must be [..., L, b, b]")
    *batch, L, b, _ = diag.shape
    if tuple(lower.shape) != tuple(batch) + (L - 1, b, b):
        raise ValueError("lower must be [..., L-1, b, b] matching diag")
    B = 1
    for s_ in batch:
        B *= s_
    G_diag, G_lower = torch.empty_like(diag), torch.empty_like(lower)
    logdet = torch.empty(tuple(batch), dtype=torch.float64, device=dev)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    fn = "selinv_chain_noalloc_" + _sfx(diag)
    with torch.cuda.device(dev):
        rc = getattr(lib(), fn)(B, L, b, _ptr(diag), _ptr(lower), _ptr(G_diag), _ptr(G_lower),
                                _ptr(logdet), _ptr(info), _stream(dev))
    _status(rc, fn)
    return (G_diag, G_lower, logdet, info) if return_info else (G_diag, G_lower, logdet)


# ------------------------------------------------------------------- star
def star(center: torch.Tensor, leaves: torch.Tensor, coupling: torch.Tensor,
         check: bool = False, return_info=False):
    """Selected inverse of block-arrowhead SPD matrices.

    center [..., b, b], leaves [..., K, b, b], coupling [..., K, b, b] with
    coupling[j] = A_{j,0}.  Returns (G_center, G_leaf, G_cross, logdet) with
    G_cross[j] = (A^-1)_{j,0}.
    """
    dt, dev = center.dtype, center.device
    center = _check_tensor(center, "center", dev, dt)
    leaves = _check_tensor(leaves, "leaves", dev, dt)
    coupling = _check_tensor(coupling, "coupling", dev, dt)
    sfx = _sfx(center)
    if center.dim() < 2 or center.shape[-1] != center.shape[-2]:
        raise ValueError("center must be [..., b, b]")
    *batch, b, _ = center.shape
    if leaves.dim() != len(batch) + 3 or tuple(leaves.shape[:len(batch)]) != tuple(batch):
        raise ValueError("leaves must be [..., K, b, b] matching center")
    K = leaves.shape[len(batch)]
    if tuple(leaves.shape) != tuple(batch) + (K, b, b) or coupling.shape != leaves.shape:
        raise ValueError("leaves and coupling must be [..., K, b, b]")
    if b < 1 or b > MAX_B:
        raise ValueError("need 1 <= b <= %d" % MAX_B)
    if check:
        for nm, t in (("center", center), ("leaves", leaves), ("coupling", coupling)):
            _validate_values(nm, t)
        _validate_symmetric("center", center)
        _validate_symmetric("leaves", leaves)
    B = 1
    for s in batch:
        B *= s
    G_center = torch.empty_like(center)
    G_leaf = torch.empty_like(leaves)
    G_cross = torch.empty_like(coupling)
    logdet = torch.empty(tuple(batch), dtype=torch.float64, device=dev)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    L_ = lib()
    ws_bytes = L_.selinv_star_workspace_bytes(center.element_size(), B, K, b)
    ws = _workspace(ws_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_star_" + sfx)(
            B, K, b, _ptr(center), _ptr(leaves), _ptr(coupling), _ptr(G_center), _ptr(G_leaf),
            _ptr(G_cross), _ptr(logdet), _ptr(info), _ptr(ws), ws_bytes, _stream(dev))
    _status(rc, "selinv_star_" + sfx)
    if check:
        _raise_info(info, "star")
    if return_info:
        return G_center, G_leaf, G_cross, logdet, info
    return G_center, G_leaf, G_cross, logdet


# ------------------------------------------------------------------- tree
class TreePlan:
    """A validated level-set schedule for one parent array (owns device
    memory through the C library)."""

    def __init__(self, parent, b: int, dtype: torch.dtype, device):
        import numpy as np
        p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
        self.n = int(p.shape[0])
        self.b = int(b)
        self.dtype = dtype
        self.device = torch.device(device)
        h = ctypes.c_void_p()
        esz = 8 if dtype == torch.float64 else 4
        with torch.cuda.device(self.device):
            rc = lib().selinv_tree_plan_create(p.ctypes.data, self.n, self.b, esz,
                                               _stream(self.device), ctypes.byref(h))
        _status(rc, "selinv_tree_plan_create")
        self._h = h
        self.levels = int(lib().selinv_tree_plan_levels(h))
        self.workspace_bytes = int(lib().selinv_tree_workspace_bytes(h))

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.selinv_tree_plan_destroy(h)
            self._h = None


_PLAN_CACHE: "OrderedDict[tuple, TreePlan]" = OrderedDict()
_PLAN_CACHE_MAX = 8


def tree_plan(parent, b: int, dtype: torch.dtype, device) -> TreePlan:
    """Cached plan keyed by the parent array's content and (n, b, dtype,
    device): repeated calls on one pattern pay only for the numeric work."""
    import numpy as np
    if isinstance(parent, torch.Tensor):
        parent = parent.detach().cpu().numpy()
    p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    key = (hashlib.sha1(p.tobytes()).hexdigest(), p.shape[0], int(b), dtype, str(device))
    plan = _PLAN_CACHE.get(key)
    if plan is None:
        plan = TreePlan(p, b, dtype, device)
        _PLAN_CACHE[key] = plan
        while len(_PLAN_CACHE) > _PLAN_CACHE_MAX:
            _PLAN_CACHE.popitem(last=False)
    else:
        _PLAN_CACHE.move_to_end(key)
    return plan


def tree(parent, diag: torch.Tensor, edge: torch.Tensor, check: bool = False,
         return_info=False, plan: TreePlan | None = None):
    """Selected inverse of a tree-structured SPD matrix.

    parent [n] (root = -1; host array or tensor), diag [n, b, b],
    edge [n, b, b] with edge[v] = A_{parent(v),v}.  Returns (G_diag, G_edge,
    logdet) with G_edge[v] = (A^-1)_{parent(v),v} and a zero root slot.
    """
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    edge = _check_tensor(edge, "edge", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 3 or diag.shape[1] != diag.shape[2] or edge.shape != diag.shape:
        raise ValueError("diag and edge must be [n, b, b]")
    n, b = diag.shape[0], diag.shape[1]
    if plan is None:
        plan = tree_plan(parent, b, dt, dev)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    if check:
        _validate_values("diag", diag)
        _validate_symmetric("diag", diag)
    G_diag = torch.empty_like(diag)
    G_edge = torch.empty_like(edge)
    logdet = torch.empty((), dtype=torch.float64, device=dev)
    info = torch.empty((), dtype=torch.int32, device=dev)
    ws = _workspace(plan.workspace_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_tree_" + sfx)(
            plan.handle, _ptr(diag), _ptr(edge), _ptr(G_diag), _ptr(G_edge), logdet.data_ptr(),
            info.data_ptr(), _ptr(ws), plan.workspace_bytes, _stream(dev))
    _status(rc, "selinv_tree_" + sfx)
    if check:
        _raise_info(info.reshape(1), "tree")
    if return_info:
        return G_diag, G_edge, logdet, info
    return G_diag, G_edge, logdet


def set_wait_limit(ticks: int):
    """Bound of each wait inside the single-launch tree schedules, in ticks of
    the GPU's 100 MHz constant clock (default 2**24).  A call whose wait
    expires reports info = -1 and a NaN log det.  Process-wide; for
    diagnostics and tests of that path."""
    lib().selinv_set_wait_limit(int(ticks))


def wait_limit() -> int:
    return int(lib().selinv_wait_limit())


class TreeGraph:
    """The tree computation for fixed buffers, recorded once as one HIP graph
    (collect levels deepest first, then distribute levels, then the log-det
    reduction) and replayed with a single launch.

    ``diag`` and ``edge`` are the graph's input buffers: change their contents
    in place (``copy_``) between launches.  ``G_diag``, ``G_edge``,
    ``logdet`` and ``info`` are its output buffers, rewritten by every
    ``launch()`` on the current stream.
    """

    def __init__(self, parent, diag: torch.Tensor, edge: torch.Tensor,
                 plan: TreePlan | None = None):
        dt, dev = diag.dtype, diag.device
        sfx = _sfx(diag)
        if diag.dim() != 3 or diag.shape[1] != diag.shape[2] or edge.shape != diag.shape:
            raise ValueError("diag and edge must be [n, b, b]")
        for name, t in (("diag", diag), ("edge", edge)):
            if (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.device != dev
                    or t.dtype != dt or not t.is_contiguous() or t.data_ptr() % 16):
                raise ValueError("%s must be a contiguous, 16-byte aligned tensor on the "
                                 "device and dtype of diag (it is the graph's own buffer)"
                                 % name)
        n, b = diag.shape[0], diag.shape[1]
        if plan is None:
            plan = tree_plan(parent, b, dt, dev)
        if plan.n != n or plan.b != b or plan.dtype != dt:
            raise ValueError("plan does not match (n, b, dtype)")
        self.plan, self.device = plan, dev
        self.diag, self.edge = diag, edge
        self.G_diag = torch.empty_like(diag)
        self.G_edge = torch.empty_like(edge)
        self.logdet = torch.empty((), dtype=torch.float64, device=dev)
        self.info = torch.empty((), dtype=torch.int32, device=dev)
        self._ws = _workspace(plan.workspace_bytes, dev)
        h = ctypes.c_void_p()
        with torch.cuda.device(dev):
            rc = getattr(lib(), "selinv_tree_graph_create_" + sfx)(
                plan.handle, _ptr(diag), _ptr(edge), _ptr(self.G_diag), _ptr(self.G_edge),
                self.logdet.data_ptr(), self.info.data_ptr(), _ptr(self._ws),
                plan.workspace_bytes, ctypes.byref(h))
        _status(rc, "selinv_tree_graph_create_" + sfx)
        self._h = h
        self.nodes = int(lib().selinv_tree_graph_nodes(h))

    def launch(self):
        """Replay the graph on the current stream; returns (G_diag, G_edge,
        logdet), the graph's output buffers."""
        with torch.cuda.device(self.device):
            rc = lib().selinv_tree_graph_launch(self._h, _stream(self.device))
        _status(rc, "selinv_tree_graph_launch")
        return self.G_diag, self.G_edge, self.logdet

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            # no replay may still be pending when the graph is freed
            with torch.cuda.device(self.device):
                torch.cuda.synchronize(self.device)
            _lib.selinv_tree_graph_destroy(h)
            self._h = None


def tree_graph(parent, diag: torch.Tensor, edge: torch.Tensor,
               plan: TreePlan | None = None) -> TreeGraph:
    """Record the tree computation on (diag, edge) as a HIP graph; see
    TreeGraph."""
    return TreeGraph(parent, diag, edge, plan)


# ------------------------------------------------------- reverse mode (VJP)
def _logdet_bar(logdet_bar, batch, dev):
    if logdet_bar is None:
        return None
    t = torch.as_tensor(logdet_bar, dtype=torch.float64, device=dev)
    return _check_tensor(t.expand(tuple(batch)), "logdet_bar", dev, torch.float64)


def chain_vjp(diag, lower, G_diag_bar, G_lower_bar, logdet_bar=None, check=False,
              return_info=False):
    """Cotangents of (diag, lower) for a loss of chain(diag, lower)'s outputs.

    G_diag_bar, G_lower_bar: cotangents of G_diag, G_lower (shapes of
    diag, lower); logdet_bar: cotangent of logdet ([...] or a scalar, float64;
    None = 0).  Returns (diag_bar, lower_bar): diag_bar is the symmetric
    gradient with respect to the symmetric diagonal blocks, lower_bar counts
    both appearances A_{i+1,i} and A_{i,i+1} = lower[i]^T.
    """
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    lower = _check_tensor(lower, "lower", dev, dt)
    gd = _check_tensor(G_diag_bar, "G_diag_bar", dev, dt)
    gl = _check_tensor(G_lower_bar, "G_lower_bar", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() < 3 or diag.shape[-1] != diag.shape[-2]:
        raise ValueError("diag must be [..., L, b, b]")
    *batch, L, b, _ = diag.shape
    if L < 1 or b < 1 or b > MAX_B:
        raise ValueError("need L >= 1 and 1 <= b <= %d" % MAX_B)
    if tuple(lower.shape) != tuple(batch) + (L - 1, b, b):
        raise ValueError("lower must be [..., L-1, b, b] matching diag")
    if gd.shape != diag.shape or gl.shape != lower.shape:
        raise ValueError("cotangents must have the shapes of G_diag and G_lower")
    lb = _logdet_bar(logdet_bar, batch, dev)
    if check:
        _validate_symmetric("diag", diag)
    B = 1
    for s_ in batch:
        B *= s_
    d_bar = torch.empty_like(diag)
    l_bar = torch.empty_like(lower)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    L_ = lib()
    ws_bytes = L_.selinv_chain_vjp_workspace_bytes(diag.element_size(), B, L, b)
    ws = _workspace(ws_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_chain_vjp_" + sfx)(
            B, L, b, _ptr(diag), _ptr(lower), _ptr(gd), _ptr(gl), _ptr(lb), _ptr(d_bar),
            _ptr(l_bar), _ptr(info), _ptr(ws), ws_bytes, _stream(dev))
    _status(rc, "selinv_chain_vjp_" + sfx)
    if check:
        _raise_info(info, "chain_vjp")
    if return_info:
        return d_bar, l_bar, info
    return d_bar, l_bar


def star_vjp(center, leaves, coupling, G_center_bar, G_leaf_bar, G_cross_bar, logdet_bar=None,
             check=False, return_info=False):
    """Cotangents of (center, leaves, coupling) for a loss of star(...)'s
    outputs (G_cross[j] = (A^-1)_{j,0}; coupling_bar counts A_{j,0} and
    A_{0,j} = coupling[j]^T)."""
    dt, dev = center.dtype, center.device
    center = _check_tensor(center, "center", dev, dt)
    leaves = _check_tensor(leaves, "leaves", dev, dt)
    coupling = _check_tensor(coupling, "coupling", dev, dt)
    gc = _check_tensor(G_center_bar, "G_center_bar", dev, dt)
    gleaf = _check_tensor(G_leaf_bar, "G_leaf_bar", dev, dt)
    gx = _check_tensor(G_cross_bar, "G_cross_bar", dev, dt)
    sfx = _sfx(center)
    if center.dim() < 2 or center.shape[-1] != center.shape[-2]:
        raise ValueError("center must be [..., b, b]")
    *batch, b, _ = center.shape
    if leaves.dim() != len(batch) + 3 or tuple(leaves.shape[:len(batch)]) != tuple(batch):
        raise ValueError("leaves must be [..., K, b, b] matching center")
    K = leaves.shape[len(batch)]
    if tuple(leaves.shape) != tuple(batch) + (K, b, b) or coupling.shape != leaves.shape:
        raise ValueError("leaves and coupling must be [..., K, b, b]")
    if gc.shape != center.shape or gleaf.shape != leaves.shape or gx.shape != leaves.shape:
        raise ValueError("cotangents must have the shapes of the outputs")
    if b < 1 or b > MAX_B:
        raise ValueError("need 1 <= b <= %d" % MAX_B)
    lb = _logdet_bar(logdet_bar, batch, dev)
    B = 1
    for s_ in batch:
        B *= s_
    c_bar = torch.empty_like(center)
    lv_bar = torch.empty_like(leaves)
    cp_bar = torch.empty_like(coupling)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    L_ = lib()
    ws_bytes = L_.selinv_star_vjp_workspace_bytes(center.element_size(), B, K, b)
    ws = _workspace(ws_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_star_vjp_" + sfx)(
            B, K, b, _ptr(center), _ptr(leaves), _ptr(coupling), _ptr(gc), _ptr(gleaf), _ptr(gx),
            _ptr(lb), _ptr(c_bar), _ptr(lv_bar), _ptr(cp_bar), _ptr(info), _ptr(ws), ws_bytes,
            _stream(dev))
    _status(rc, "selinv_star_vjp_" + sfx)
    if check:
        _raise_info(info, "star_vjp")
    if return_info:
        return c_bar, lv_bar, cp_bar, info
    return c_bar, lv_bar, cp_bar


def tree_vjp(parent, diag, edge, G_diag_bar, G_edge_bar, logdet_bar=None, check=False,
             return_info=False, plan: TreePlan | None = None):
    """Cotangents of (diag, edge) for a loss of tree(parent, diag, edge)'s
    outputs; edge_bar[v] counts A_{parent(v),v} and its transpose, the root
    slot is zero."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    edge = _check_tensor(edge, "edge", dev, dt)
    gd = _check_tensor(G_diag_bar, "G_diag_bar", dev, dt)
    ge = _check_tensor(G_edge_bar, "G_edge_bar", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 3 or diag.shape[1] != diag.shape[2] or edge.shape != diag.shape:
        raise ValueError("diag and edge must be [n, b, b]")
    if gd.shape != diag.shape or ge.shape != diag.shape:
        raise ValueError("cotangents must be [n, b, b]")
    n, b = diag.shape[0], diag.shape[1]
    if plan is None:
        plan = tree_plan(parent, b, dt, dev)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    lb = _logdet_bar(logdet_bar, (1,), dev)
    d_bar = torch.empty_like(diag)
    e_bar = torch.empty_like(edge)
    info = torch.empty((), dtype=torch.int32, device=dev)
    ws_bytes = int(lib().selinv_tree_vjp_workspace_bytes(plan.handle))
    ws = _workspace(ws_bytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_tree_vjp_" + sfx)(
            plan.handle, _ptr(diag), _ptr(edge), _ptr(gd), _ptr(ge), _ptr(lb), _ptr(d_bar),
            _ptr(e_bar), info.data_ptr(), _ptr(ws), ws_bytes, _stream(dev))
    _status(rc, "selinv_tree_vjp_" + sfx)
    if check:
        _raise_info(info.reshape(1), "tree_vjp")
    if return_info:
        return d_bar, e_bar, info
    return d_bar, e_bar


# ------------------------------------------------- shared-factor siblings
# One collect pass (the block LDL^T factorisation A = L D L^T) kept on the
# device, then any number of solves x = A^{-1} y and Gaussian samples
# x = L^{-T} D^{-1/2} z ~ N(0, A^{-1}) from it; log det comes with the factor
# (or alone, without storing one).  Vectors are [..., n_blocks, b, k].

def _vec(t, name, dev, dt, shape_prefix):
    t = _check_tensor(t, name, dev, dt)
    if tuple(t.shape[:len(shape_prefix)]) != tuple(shape_prefix) or t.dim() != len(shape_prefix) + 1:
        raise ValueError("%s must be %s + (k,)" % (name, tuple(shape_prefix)))
    return t


def _normal_like(shape, dt, dev, generator):
    return torch.randn(shape, dtype=dt, device=dev, generator=generator)


class ChainFactor:
    """Factor of block-tridiagonal chains (see chain_factor)."""

    def __init__(self, lower, factor, logdet, info, shape):
        self.lower, self.factor, self.logdet, self.info = lower, factor, logdet, info
        self.batch, self.L, self.b = shape

    def _apply(self, v, name, sample):
        dev, dt = self.factor.device, self.factor.dtype
        B = 1
        for s_ in self.batch:
            B *= s_
        v = _vec(v, name, dev, dt, tuple(self.batch) + (self.L, self.b))
        k = v.shape[-1]
        x = torch.empty_like(v)
        fn = "selinv_chain_%s_%s" % ("sample" if sample else "solve", _sfx(self.factor))
        with torch.cuda.device(dev):
            rc = getattr(lib(), fn)(B, self.L, self.b, _ptr(self.lower), _ptr(self.factor), k,
                                    _ptr(v), _ptr(x), _stream(dev))
        _status(rc, fn)
        return x

    def solve(self, y):
        """x = A^{-1} y, y [..., L, b, k]."""
        return self._apply(y, "y", False)

    def sample(self, num_samples=None, z=None, generator=None):
        """x = L^{-T} D^{-1/2} z ~ N(0, A^{-1}); z [..., L, b, k] given, or
        drawn with torch.randn (k = num_samples columns)."""
        if z is None:
            z = _normal_like(tuple(self.batch) + (self.L, self.b, num_samples or 1),
                             self.factor.dtype, self.factor.device, generator)
        return self._apply(z, "z", True)


def chain_factor(diag, lower, keep_factor=True):
    """Collect pass of block-tridiagonal chains (diag [..., L, b, b], lower
    [..., L-1, b, b]).  Returns a ChainFactor (logdet, info, solve, sample);
    keep_factor=False computes log det and info only."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    lower = _check_tensor(lower, "lower", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() < 3 or diag.shape[-1] != diag.shape[-2]:
        raise ValueError("diag must be [..., L, b, b]")
    *batch, L, b, _ = diag.shape
    if L < 1 or b < 1 or b > MAX_B:
        raise ValueError("need L >= 1 and 1 <= b <= %d" % MAX_B)
    if tuple(lower.shape) != tuple(batch) + (L - 1, b, b):
        raise ValueError("lower must be [..., L-1, b, b] matching diag")
    B = 1
    for s_ in batch:
        B *= s_
    L_ = lib()
    factor = None
    if keep_factor:
        nbytes = L_.selinv_chain_factor_bytes(diag.element_size(), B, L, b)
        factor = torch.empty(max(nbytes // diag.element_size(), 1), dtype=dt, device=dev)
    logdet = torch.empty(tuple(batch), dtype=torch.float64, device=dev)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_chain_factor_" + sfx)(B, L, b, _ptr(diag), _ptr(lower),
                                                        _ptr(factor), _ptr(logdet), _ptr(info),
                                                        _stream(dev))
    _status(rc, "selinv_chain_factor_" + sfx)
    return ChainFactor(lower, factor, logdet, info, (batch, L, b))


def chain_logdet(diag, lower, return_info=False):
    """log det A of block-tridiagonal chains without storing a factor."""
    f = chain_factor(diag, lower, keep_factor=False)
    return (f.logdet, f.info) if return_info else f.logdet


class StarFactor:
    """Factor of block-arrowhead matrices (see star_factor)."""

    def __init__(self, coupling, factor, logdet, info, shape):
        self.coupling, self.factor, self.logdet, self.info = coupling, factor, logdet, info
        self.batch, self.K, self.b = shape

    def _apply(self, vc, vl, sample):
        dev, dt = self.factor.device, self.factor.dtype
        B = 1
        for s_ in self.batch:
            B *= s_
        vc = _vec(vc, "center vector", dev, dt, tuple(self.batch) + (self.b,))
        vl = _vec(vl, "leaf vector", dev, dt, tuple(self.batch) + (self.K, self.b))
        k = vc.shape[-1]
        if vl.shape[-1] != k:
            raise ValueError("centre and leaf vectors need the same k")
        xc, xl = torch.empty_like(vc), torch.empty_like(vl)
        sfx = _sfx(self.factor)
        with torch.cuda.device(dev):
            if sample:
                rc = getattr(lib(), "selinv_star_sample_" + sfx)(
                    B, self.K, self.b, _ptr(self.coupling), _ptr(self.factor), k, _ptr(vc),
                    _ptr(vl), _ptr(xc), _ptr(xl), _stream(dev))
            else:
                nb = lib().selinv_star_solve_workspace_bytes(vc.element_size(), B, self.K,
                                                             self.b, k)
                ws = _workspace(nb, dev)
                rc = getattr(lib(), "selinv_star_solve_" + sfx)(
                    B, self.K, self.b, _ptr(self.coupling), _ptr(self.factor), k, _ptr(vc),
                    _ptr(vl), _ptr(xc), _ptr(xl), _ptr(ws), nb, _stream(dev))
        _status(rc, "selinv_star_%s_%s" % ("sample" if sample else "solve", sfx))
        return xc, xl

    def solve(self, y_center, y_leaves):
        """x = A^{-1} y split as the centre [..., b, k] and leaves [..., K, b, k]."""
        return self._apply(y_center, y_leaves, False)

    def sample(self, num_samples=None, z_center=None, z_leaves=None, generator=None):
        if z_center is None:
            k = num_samples or 1
            dt, dev = self.factor.dtype, self.factor.device
            z_center = _normal_like(tuple(self.batch) + (self.b, k), dt, dev, generator)
            z_leaves = _normal_like(tuple(self.batch) + (self.K, self.b, k), dt, dev, generator)
        return self._apply(z_center, z_leaves, True)


def star_factor(center, leaves, coupling, keep_factor=True):
    """Collect pass of block-arrowhead matrices; returns a StarFactor."""
    dt, dev = center.dtype, center.device
    center = _check_tensor(center, "center", dev, dt)
    leaves = _check_tensor(leaves, "leaves", dev, dt)
    coupling = _check_tensor(coupling, "coupling", dev, dt)
    sfx = _sfx(center)
    *batch, b, _ = center.shape
    if leaves.dim() != len(batch) + 3 or tuple(leaves.shape[:len(batch)]) != tuple(batch):
        raise ValueError("leaves must be [..., K, b, b] matching center")
    K = leaves.shape[len(batch)]
    if tuple(leaves.shape) != tuple(batch) + (K, b, b) or coupling.shape != leaves.shape:
        raise ValueError("leaves and coupling must be [..., K, b, b]")
    if b < 1 or b > MAX_B:
        raise ValueError("need 1 <= b <= %d" % MAX_B)
    B = 1
    for s_ in batch:
        B *= s_
    L_ = lib()
    factor = None
    if keep_factor:
        nbytes = L_.selinv_star_factor_bytes(center.element_size(), B, K, b)
        factor = torch.empty(max(nbytes // center.element_size(), 1), dtype=dt, device=dev)
    logdet = torch.empty(tuple(batch), dtype=torch.float64, device=dev)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    nb = L_.selinv_star_factor_workspace_bytes(center.element_size(), B, K, b)
    ws = _workspace(nb, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_star_factor_" + sfx)(
            B, K, b, _ptr(center), _ptr(leaves), _ptr(coupling), _ptr(factor), _ptr(logdet),
            _ptr(info), _ptr(ws), nb, _stream(dev))
    _status(rc, "selinv_star_factor_" + sfx)
    return StarFactor(coupling, factor, logdet, info, (batch, K, b))


def star_logdet(center, leaves, coupling, return_info=False):
    f = star_factor(center, leaves, coupling, keep_factor=False)
    return (f.logdet, f.info) if return_info else f.logdet


class TreeFactor:
    """Factor of a tree-structured matrix (see tree_factor)."""

    def __init__(self, plan, edge, factor, logdet, info):
        self.plan, self.edge, self.factor, self.logdet, self.info = plan, edge, factor, logdet, info

    def _apply(self, v, name, sample):
        dev, dt = self.factor.device, self.factor.dtype
        v = _vec(v, name, dev, dt, (self.plan.n, self.plan.b))
        k = v.shape[-1]
        x = torch.empty_like(v)
        sfx = _sfx(self.factor)
        with torch.cuda.device(dev):
            nb = int(lib().selinv_tree_solve_workspace_bytes(self.plan.handle, k))
            ws = _workspace(nb, dev)
            rc = getattr(lib(), "selinv_tree_%s_%s" % ("sample" if sample else "solve", sfx))(
                self.plan.handle, _ptr(self.edge), _ptr(self.factor), k, _ptr(v), _ptr(x),
                _ptr(ws), nb, _stream(dev))
        _status(rc, "selinv_tree_%s_%s" % ("sample" if sample else "solve", sfx))
        return x

    def solve(self, y):
        """x = A^{-1} y, y [n, b, k]."""
        return self._apply(y, "y", False)

    def sample(self, num_samples=None, z=None, generator=None):
        if z is None:
            z = _normal_like((self.plan.n, self.plan.b, num_samples or 1), self.factor.dtype,
                             self.factor.device, generator)
        return self._apply(z, "z", True)


def tree_factor(parent, diag, edge, keep_factor=True, plan: TreePlan | None = None):
    """Collect pass of a tree-structured matrix; returns a TreeFactor."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    edge = _check_tensor(edge, "edge", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 3 or diag.shape[1] != diag.shape[2] or edge.shape != diag.shape:
        raise ValueError("diag and edge must be [n, b, b]")
    n, b = diag.shape[0], diag.shape[1]
    if plan is None:
        plan = tree_plan(parent, b, dt, dev)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    factor = None
    if keep_factor:
        nbytes = int(lib().selinv_tree_factor_bytes(plan.handle))
        factor = torch.empty(max(nbytes // diag.element_size(), 1), dtype=dt, device=dev)
    logdet = torch.empty((), dtype=torch.float64, device=dev)
    info = torch.empty((), dtype=torch.int32, device=dev)
    nb = int(lib().selinv_tree_factor_workspace_bytes(plan.handle))
    ws = _workspace(nb, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_tree_factor_" + sfx)(
            plan.handle, _ptr(diag), _ptr(edge), _ptr(factor), logdet.data_ptr(),
            info.data_ptr(), _ptr(ws), nb, _stream(dev))
    _status(rc, "selinv_tree_factor_" + sfx)
    return TreeFactor(plan, edge, factor, logdet, info)


def tree_logdet(parent, diag, edge, return_info=False):
    f = tree_factor(parent, diag, edge, keep_factor=False)
    return (f.logdet, f.info) if return_info else f.logdet


# ------------------------------------------------- non-symmetric ladder
def bidiag(diag, lower, check=False, return_info=False):
    """Selected inverse of block lower-bidiagonal (non-symmetric) matrices:
    diag [..., L, b, b] = M_ii, lower [..., L-1, b, b] = M_{i+1,i}.  Returns
    (G_diag, G_lower) on M's pattern (the page's selinv_bidiag forward); no
    pivoting, info = 1 + the block whose inverse broke down."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    lower = _check_tensor(lower, "lower", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() < 3 or diag.shape[-1] != diag.shape[-2]:
        raise ValueError("diag must be [..., L, b, b]")
    *batch, L, b, _ = diag.shape
    if L < 1 or b < 1 or b > MAX_B:
        raise ValueError("need L >= 1 and 1 <= b <= %d" % MAX_B)
    if tuple(lower.shape) != tuple(batch) + (L - 1, b, b):
        raise ValueError("lower must be [..., L-1, b, b] matching diag")
    B = 1
    for s_ in batch:
        B *= s_
    G_diag, G_lower = torch.empty_like(diag), torch.empty_like(lower)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=dev)
    nb = lib().selinv_bidiag_workspace_bytes(B)
    ws = _workspace(nb, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_bidiag_" + sfx)(B, L, b, _ptr(diag), _ptr(lower),
                                                     _ptr(G_diag), _ptr(G_lower), _ptr(info),
                                                     _ptr(ws), nb, _stream(dev))
    _status(rc, "selinv_bidiag_" + sfx)
    if check:
        _raise_info(info, "bidiag")
    return (G_diag, G_lower, info) if return_info else (G_diag, G_lower)


def nonsym_tree(parent, diag, up, down, check=False, return_info=False,
                plan: TreePlan | None = None):
    """Selected inverse of a non-symmetric block matrix whose off-diagonal graph
    is a tree: up[v] = M_{parent(v),v}, down[v] = M_{v,parent(v)}.  Returns
    (G_diag, G_up, G_down) with G_up[v] = (M^-1)_{parent(v),v},
    G_down[v] = (M^-1)_{v,parent(v)} and zero root slots."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    up = _check_tensor(up, "up", dev, dt)
    down = _check_tensor(down, "down", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 3 or diag.shape[1] != diag.shape[2] or up.shape != diag.shape or \
            down.shape != diag.shape:
        raise ValueError("diag, up and down must be [n, b, b]")
    n, b = diag.shape[0], diag.shape[1]
    if plan is None:
        plan = tree_plan(parent, b, dt, dev)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    G_diag, G_up, G_down = torch.empty_like(diag), torch.empty_like(up), torch.empty_like(down)
    info = torch.empty((), dtype=torch.int32, device=dev)
    nb = int(lib().selinv_nonsym_tree_workspace_bytes(plan.handle))
    ws = _workspace(nb, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_nonsym_tree_" + sfx)(
            plan.handle, _ptr(diag), _ptr(up), _ptr(down), _ptr(G_diag), _ptr(G_up),
            _ptr(G_down), info.data_ptr(), _ptr(ws), nb, _stream(dev))
    _status(rc, "selinv_nonsym_tree_" + sfx)
    if check:
        _raise_info(info.reshape(1), "nonsym_tree")
    return (G_diag, G_up, G_down, info) if return_info else (G_diag, G_up, G_down)


# ------------------------------------------------------ general sparse SPD
def _edge_index_host(edge_index, n):
    import numpy as np
    if isinstance(edge_index, torch.Tensor):
        edge_index = edge_index.detach().cpu().numpy()
    e = np.ascontiguousarray(np.asarray(edge_index, dtype=np.int32))
    if e.ndim != 2 or e.shape[0] != 2:
        raise ValueError("edge_index must be [2, m]")
    return e


def _order_host(order, n):
    import numpy as np
    if order is None:
        return None
    if isinstance(order, torch.Tensor):
        order = order.detach().cpu().numpy()
    o = np.ascontiguousarray(np.asarray(order, dtype=np.int32))
    if o.shape != (n,):
        raise ValueError("order must have n entries")
    return o


def junction_symbolic(n: int, edge_index, order=None):
    """Host-only symbolic analysis: (order [n], S_index [2, nnz], levels) as
    numpy int32 arrays, the pattern selected_inverse_junction returns."""
    import numpy as np
    e = _edge_index_host(edge_index, n)
    o = _order_host(order, n)
    nnz, lev = ctypes.c_int64(), ctypes.c_int32()
    rc = lib().selinv_junction_symbolic(n, e.shape[1], e.ctypes.data if e.size else None,
                                        o.ctypes.data if o is not None else None,
                                        ctypes.byref(nnz), ctypes.byref(lev), None, 0, None)
    _status(rc, "selinv_junction_symbolic")
    S = np.zeros((2, nnz.value), np.int32)
    out = np.zeros(n, np.int32)
    rc = lib().selinv_junction_symbolic(n, e.shape[1], e.ctypes.data if e.size else None,
                                        o.ctypes.data if o is not None else None, None, None,
                                        S.ctypes.data if S.size else None, nnz.value,
                                        out.ctypes.data)
    _status(rc, "selinv_junction_symbolic")
    return out, S, int(lev.value)


class JunctionPlan:
    """Symbolic analysis of one block pattern (and elimination order) with
    its device tables; owns device memory through the C library."""

    def __init__(self, n: int, edge_index, b: int, dtype: torch.dtype, device, order=None):
        import numpy as np
        e = _edge_index_host(edge_index, n)
        o = _order_host(order, n)
        self.n, self.m, self.b = int(n), int(e.shape[1]), int(b)
        self.dtype = dtype
        self.device = torch.device(device)
        h = ctypes.c_void_p()
        esz = 8 if dtype == torch.float64 else 4
        with torch.cuda.device(self.device):
            rc = lib().selinv_junction_plan_create(
                self.n, self.m, e.ctypes.data if e.size else None,
                o.ctypes.data if o is not None else None, self.b, esz, _stream(self.device),
                ctypes.byref(h))
        _status(rc, "selinv_junction_plan_create")
        self._h = h
        self.nnz = int(lib().selinv_junction_plan_nnz(h))
        self.levels = int(lib().selinv_junction_plan_levels(h))
        S = np.zeros((2, self.nnz), np.int32)
        od = np.zeros(self.n, np.int32)
        _status(lib().selinv_junction_plan_pattern(h, S.ctypes.data if S.size else None,
                                                   od.ctypes.data),
                "selinv_junction_plan_pattern")
        self.S_index = torch.from_numpy(S)
        self.order = torch.from_numpy(od)

    def workspace_bytes(self, B: int) -> int:
        return int(lib().selinv_junction_workspace_bytes(self._h, B))

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.selinv_junction_plan_destroy(h)
            self._h = None


_JPLAN_CACHE: "OrderedDict[tuple, JunctionPlan]" = OrderedDict()


def junction_plan(n: int, edge_index, b: int, dtype: torch.dtype, device,
                  order=None) -> JunctionPlan:
    """Cached plan keyed by the pattern's content, the order and (n, b,
    dtype, device): repeated calls on one pattern pay only for the numeric
    work (the symbolic analysis is done once per pattern)."""
    e = _edge_index_host(edge_index, n)
    o = _order_host(order, n)
    key = (hashlib.sha1(e.tobytes()).hexdigest(), e.shape[1],
           None if o is None else hashlib.sha1(o.tobytes()).hexdigest(), int(n), int(b), dtype,
           str(device))
    plan = _JPLAN_CACHE.get(key)
    if plan is None:
        plan = JunctionPlan(n, e, b, dtype, device, o)
        _JPLAN_CACHE[key] = plan
        while len(_JPLAN_CACHE) > _PLAN_CACHE_MAX:
            _JPLAN_CACHE.popitem(last=False)
    else:
        _JPLAN_CACHE.move_to_end(key)
    return plan


def junction(diag: torch.Tensor, edge_index, edge_val: torch.Tensor, order=None,
             check: bool = False, return_info=False, plan: JunctionPlan | None = None):
    """Selected inverse of general sparse SPD matrices sharing one pattern.

    diag [B, n, b, b] (or [n, b, b]); edge_index [2, m] (host array or
    tensor) with pairs (i, j), i > j; edge_val [B, m, b, b] with
    edge_val[e] = A_{i_e, j_e}; order: optional elimination order (default
    greedy minimum degree).  Returns (G_diag, S_index, G_lower, logdet): the
    selected inverse on the filled pattern S, S_index an int32 CPU tensor
    [2, nnz] (pairs i > j, sorted), G_lower[k] = (A^-1)_{S_index[:, k]}.
    """
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    single = diag.dim() == 3
    if single:
        diag = diag.unsqueeze(0)
        edge_val = edge_val.unsqueeze(0)
    edge_val = _check_tensor(edge_val, "edge_val", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 4 or diag.shape[2] != diag.shape[3]:
        raise ValueError("diag must be [B, n, b, b]")
    B, n, b = diag.shape[0], diag.shape[1], diag.shape[2]
    if plan is None:
        plan = junction_plan(n, edge_index, b, dt, dev, order)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    if edge_val.shape != (B, plan.m, b, b):
        raise ValueError("edge_val must be [B, m, b, b]")
    if check:
        _validate_values("diag", diag)
        _validate_symmetric("diag", diag)
    G_diag = torch.empty_like(diag)
    G_lower = torch.empty((B, plan.nnz, b, b), dtype=dt, device=dev)
    logdet = torch.empty(B, dtype=torch.float64, device=dev)
    info = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = plan.workspace_bytes(B)
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_junction_" + sfx)(
            plan.handle, B, _ptr(diag), _ptr(edge_val) if plan.m else None, _ptr(G_diag),
            _ptr(G_lower) if plan.nnz else None, logdet.data_ptr(), info.data_ptr(), _ptr(ws),
            nbytes, _stream(dev))
    _status(rc, "selinv_junction_" + sfx)
    if check:
        _raise_info(info, "junction")
    if single:
        G_diag, G_lower, logdet, info = G_diag[0], G_lower[0], logdet[0], info[0]
    if return_info:
        return G_diag, plan.S_index, G_lower, logdet, info
    return G_diag, plan.S_index, G_lower, logdet


def junction_logdet(diag, edge_index, edge_val, order=None, check=False, return_info=False,
                    plan: JunctionPlan | None = None):
    """log det A of general sparse SPD matrices sharing one pattern, from the
    sparse block Cholesky factorisation alone (no selected inverse).
    diag [B, n, b, b] (or [n, b, b]) and edge_val as for `junction`."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    single = diag.dim() == 3
    if single:
        diag = diag.unsqueeze(0)
        edge_val = edge_val.unsqueeze(0)
    edge_val = _check_tensor(edge_val, "edge_val", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 4 or diag.shape[2] != diag.shape[3]:
        raise ValueError("diag must be [B, n, b, b]")
    B, n, b = diag.shape[0], diag.shape[1], diag.shape[2]
    if plan is None:
        plan = junction_plan(n, edge_index, b, dt, dev, order)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    if edge_val.shape != (B, plan.m, b, b):
        raise ValueError("edge_val must be [B, m, b, b]")
    if check:
        _validate_values("diag", diag)
        _validate_symmetric("diag", diag)
    logdet = torch.empty(B, dtype=torch.float64, device=dev)
    info = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = plan.workspace_bytes(B)
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        rc = getattr(lib(), "selinv_junction_logdet_" + sfx)(
            plan.handle, B, _ptr(diag), _ptr(edge_val) if plan.m else None, logdet.data_ptr(),
            info.data_ptr(), _ptr(ws), nbytes, _stream(dev))
    _status(rc, "selinv_junction_logdet_" + sfx)
    if check:
        _raise_info(info, "junction")
    if single:
        logdet, info = logdet[0], info[0]
    return (logdet, info) if return_info else logdet


class JunctionFactor:
    """Factor of general sparse SPD matrices on one pattern (see
    junction_factor): log det, info, and the solve / sample sweeps."""

    def __init__(self, plan, B, single, factor, logdet, info):
        self.plan, self.B, self.single = plan, B, single
        self.factor, self.logdet, self.info = factor, logdet, info

    def _apply(self, v, name, sample):
        dev, dt = self.factor.device, self.factor.dtype
        if self.single:
            v = _vec(v, name, dev, dt, (self.plan.n, self.plan.b)).unsqueeze(0)
        else:
            v = _vec(v, name, dev, dt, (self.B, self.plan.n, self.plan.b))
        k = v.shape[-1]
        x = torch.empty_like(v)
        op = "sample" if sample else "solve"
        sfx = _sfx(self.factor)
        with torch.cuda.device(dev):
            if sample:
                rc = getattr(lib(), "selinv_junction_sample_" + sfx)(
                    self.plan.handle, self.B, _ptr(self.factor), k, _ptr(v), _ptr(x),
                    _stream(dev))
            else:
                nb = int(lib().selinv_junction_solve_workspace_bytes(self.plan.handle, self.B, k))
                ws = _workspace(nb, dev)
                rc = getattr(lib(), "selinv_junction_solve_" + sfx)(
                    self.plan.handle, self.B, _ptr(self.factor), k, _ptr(v), _ptr(x), _ptr(ws),
                    nb, _stream(dev))
        _status(rc, "selinv_junction_%s_%s" % (op, sfx))
        return x[0] if self.single else x

    def solve(self, y):
        """x = A^{-1} y, y [B, n, b, k] (or [n, b, k])."""
        return self._apply(y, "y", False)

    def sample(self, num_samples=None, z=None, generator=None):
        """x = L^{-T} D^{-1/2} z ~ N(0, A^{-1}); z drawn here unless given."""
        if z is None:
            shape = (self.plan.n, self.plan.b, num_samples or 1)
            if not self.single:
                shape = (self.B,) + shape
            z = _normal_like(shape, self.factor.dtype, self.factor.device, generator)
        return self._apply(z, "z", True)


def junction_factor(diag, edge_index, edge_val, order=None, plan: JunctionPlan | None = None):
    """Sparse block Cholesky factorisation of general sparse SPD matrices
    sharing one pattern (diag [B, n, b, b] or [n, b, b], edge_val as for
    `junction`), kept for junction_solve / sampling; returns a
    JunctionFactor with .logdet, .info, .solve(y) and .sample(...)."""
    dt, dev = diag.dtype, diag.device
    diag = _check_tensor(diag, "diag", dev, dt)
    single = diag.dim() == 3
    if single:
        diag = diag.unsqueeze(0)
        edge_val = edge_val.unsqueeze(0)
    edge_val = _check_tensor(edge_val, "edge_val", dev, dt)
    sfx = _sfx(diag)
    if diag.dim() != 4 or diag.shape[2] != diag.shape[3]:
        raise ValueError("diag must be [B, n, b, b]")
    B, n, b = diag.shape[0], diag.shape[1], diag.shape[2]
    if plan is None:
        plan = junction_plan(n, edge_index, b, dt, dev, order)
    if plan.n != n or plan.b != b or plan.dtype != dt:
        raise ValueError("plan does not match (n, b, dtype)")
    if edge_val.shape != (B, plan.m, b, b):
        raise ValueError("edge_val must be [B, m, b, b]")
    L_ = lib()
    nbytes = int(L_.selinv_junction_factor_bytes(plan.handle, B))
    factor = torch.empty(max(nbytes // diag.element_size(), 1), dtype=dt, device=dev)
    logdet = torch.empty(B, dtype=torch.float64, device=dev)
    info = torch.empty(B, dtype=torch.int32, device=dev)
    nb = int(L_.selinv_junction_factor_workspace_bytes(plan.handle, B))
    ws = _workspace(nb, dev)
    with torch.cuda.device(dev):
        rc = getattr(L_, "selinv_junction_factor_" + sfx)(
            plan.handle, B, _ptr(diag), _ptr(edge_val) if plan.m else None, _ptr(factor),
            logdet.data_ptr(), info.data_ptr(), _ptr(ws), nb, _stream(dev))
    _status(rc, "selinv_junction_factor_" + sfx)
    if single:
        logdet, info = logdet[0], info[0]
    return JunctionFactor(plan, B, single, factor, logdet, info)


def junction_solve(diag, edge_index, edge_val, y, order=None, plan: JunctionPlan | None = None):
    """x = A^{-1} y on a pattern (one or several right-hand sides, y
    [B, n, b, k] or [n, b, k]); factorises, then solves."""
    return junction_factor(diag, edge_index, edge_val, order, plan).solve(y)
