"""Plain float64 CPU oracle for the block selected inverse (chain, star, tree).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package shares no code with it.

The arithmetic lives in ``oracle.c`` (scalar loops, no BLAS), which states the
recurrences and the passages of the gabp-sparse-inv 0.3.2 project page they
follow.  This module only marshals numpy arrays.  Inputs are float64; a float32
run is checked by widening the float32 inputs it consumed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, INVALID_ARG, BAD_TREE = 0, 1, 2


def compile_oracle(src: str, out: str) -> str:
    """Compile an oracle source to a shared library (plain -O2, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-fno-fast-math", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        compile_oracle(SOURCE, _LIB)
    return _LIB


def load(path: str | None = None):
    """Load the oracle library (or a variant of it at `path`)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None:
        if not os.path.exists(_LIB):
            build(force=False)
        path = _LIB
    lib = ctypes.CDLL(os.path.abspath(path))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_chain.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.oracle_star.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_tree.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_tree_depths.argtypes = [i64, vp, vp]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_tree_vjp.argtypes = [i64, i32, vp, vp, vp, vp, vp, ctypes.c_double, vp, vp]
    lib.oracle_chain_vjp.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_tree_apply.argtypes = [i64, i32, vp, vp, vp, i64, vp, vp, i32]
    lib.oracle_bidiag.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
    lib.oracle_nonsym_tree.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_chain_apply.argtypes = [i64, i64, i32, vp, vp, i64, vp, vp, i32, vp]
    lib.oracle_eliminate.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, i64]
    lib.oracle_junction.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_junction_apply.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, i64, vp, vp, i32,
                                          vp]
    for f in (lib.oracle_chain, lib.oracle_star, lib.oracle_tree, lib.oracle_tree_depths,
              lib.oracle_num_threads, lib.oracle_set_num_threads, lib.oracle_tree_vjp, lib.oracle_chain_vjp,
              lib.oracle_tree_apply, lib.oracle_chain_apply, lib.oracle_bidiag,
              lib.oracle_nonsym_tree, lib.oracle_eliminate, lib.oracle_junction,
              lib.oracle_junction_apply):
        f.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data if a.size else None


class OracleError(RuntimeError):
    pass


def chain(diag, lower, lib=None):
    """Selected inverse of block-tridiagonal chains.

    diag [B,L,b,b], lower [B,L-1,b,b] with lower[i] = A_{i+1,i}.
    Returns (G_diag [B,L,b,b], G_lower [B,L-1,b,b], logdet [B], info [B]).
    """
    lib = lib or load()
    diag, lower = _f64(diag), _f64(lower)
    B, L, b = diag.shape[0], diag.shape[1], diag.shape[2]
    assert lower.shape == (B, L - 1, b, b)
    Gd = np.empty_like(diag)
    Gl = np.empty_like(lower)
    ld = np.empty(B)
    info = np.empty(B, np.int32)
    rc = lib.oracle_chain(B, L, b, _p(diag), _p(lower), _p(Gd), _p(Gl), _p(ld), _p(info))
    if rc:
        raise OracleError("oracle_chain status %d" % rc)
    return Gd, Gl, ld, info


def star(center, leaves, coupling, lib=None):
    """Selected inverse of block-arrowhead matrices.

    center [B,b,b], leaves [B,K,b,b], coupling [B,K,b,b] with
    coupling[j] = A_{j,0}.  Returns (G_center, G_leaf, G_cross, logdet, info)
    with G_cross[j] = (A^-1)_{j,0}.
    """
    lib = lib or load()
    center, leaves, coupling = _f64(center), _f64(leaves), _f64(coupling)
    B, K, b = leaves.shape[0], leaves.shape[1], leaves.shape[2]
    assert center.shape == (B, b, b) and coupling.shape == leaves.shape
    Gc = np.empty_like(center)
    Gl = np.empty_like(leaves)
    Gx = np.empty_like(coupling)
    ld = np.empty(B)
    info = np.empty(B, np.int32)
    rc = lib.oracle_star(B, K, b, _p(center), _p(leaves), _p(coupling), _p(Gc), _p(Gl),
                         _p(Gx), _p(ld), _p(info))
    if rc:
        raise OracleError("oracle_star status %d" % rc)
    return Gc, Gl, Gx, ld, info


def tree(parent, diag, edge, lib=None):
    """Selected inverse of a tree-structured SPD matrix.

    parent [n] (root = -1), diag [n,b,b], edge [n,b,b] with
    edge[v] = A_{parent(v),v}.  Returns (G_diag, G_edge, logdet, info) with
    G_edge[v] = (A^-1)_{parent(v),v} and a zero root slot.
    """
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    diag, edge = _f64(diag), _f64(edge)
    n, b = diag.shape[0], diag.shape[1]
    assert parent.shape == (n,) and edge.shape == diag.shape
    Gd = np.empty_like(diag)
    Ge = np.empty_like(edge)
    ld = np.empty(1)
    info = np.empty(1, np.int32)
    rc = lib.oracle_tree(n, b, _p(parent), _p(diag), _p(edge), _p(Gd), _p(Ge), _p(ld),
                         _p(info))
    if rc:
        raise OracleError("oracle_tree status %d" % rc)
    return Gd, Ge, float(ld[0]), int(info[0])


def tree_depths(parent, lib=None):
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    d = np.empty(parent.shape[0], np.int32)
    rc = lib.oracle_tree_depths(parent.shape[0], _p(parent), _p(d))
    if rc:
        raise OracleError("invalid tree (status %d)" % rc)
    return d


# ------------------------------------------------------------------ VJPs
# Reverse mode of the collect / distribute passes ("Differentiable selected
# inverse" section of the gabp-sparse-inv page: the analytic two-pass
# backward).  Cotangents: gd_bar on each G_vv (only its symmetric part
# matters), an edge cotangent on each G_{p,v}, ld_bar on log det A.  Returns
# the cotangents of the inputs: symmetric d_bar (for symmetric perturbations
# of the diagonal blocks) and the edge blocks' gradients.


def tree_vjp(parent, diag, edge, gd_bar, ge_bar, ld_bar, lib=None):
    """-> (d_bar [n,b,b], e_bar [n,b,b] with a zero root slot)."""
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    diag, edge, gd_bar, ge_bar = _f64(diag), _f64(edge), _f64(gd_bar), _f64(ge_bar)
    n, b = diag.shape[0], diag.shape[1]
    assert edge.shape == diag.shape == gd_bar.shape == ge_bar.shape
    db = np.empty_like(diag)
    eb = np.empty_like(edge)
    rc = lib.oracle_tree_vjp(n, b, _p(parent), _p(diag), _p(edge), _p(gd_bar), _p(ge_bar),
                             float(ld_bar), _p(db), _p(eb))
    if rc:
        raise OracleError("oracle_tree_vjp status %d" % rc)
    return db, eb


def chain_vjp(diag, lower, gd_bar, gl_bar, ld_bar, lib=None):
    """Chains as path trees rooted at their last block.
    -> (d_bar [B,L,b,b], l_bar [B,L-1,b,b], status [B]: 0 or 3 = not PD)."""
    lib = lib or load()
    diag, lower, gd_bar, gl_bar = _f64(diag), _f64(lower), _f64(gd_bar), _f64(gl_bar)
    B, L, b = diag.shape[0], diag.shape[1], diag.shape[2]
    ld_bar = _f64(np.broadcast_to(np.asarray(ld_bar, dtype=np.float64), (B,)))
    db = np.empty_like(diag)
    lb = np.empty_like(lower)
    st = np.empty(B, np.int32)
    rc = lib.oracle_chain_vjp(B, L, b, _p(diag), _p(lower), _p(gd_bar), _p(gl_bar), _p(ld_bar),
                              _p(db), _p(lb), _p(st))
    if rc:
        raise OracleError("oracle_chain_vjp status %d" % rc)
    return db, lb, st


def star_vjp(center, leaves, coupling, gc_bar, gl_bar, gx_bar, ld_bar, lib=None):
    """Stars as depth-1 trees: centre = node 0 (root), leaf j = node j + 1 with
    E_{j+1} = A_{0,j+1} = coupling[j]^T and G_cross[j] = G_{0,j+1}^T.
    -> (c_bar [B,b,b], leaves_bar [B,K,b,b], coupling_bar [B,K,b,b])."""
    center, leaves, coupling = _f64(center), _f64(leaves), _f64(coupling)
    B, K, b = leaves.shape[0], leaves.shape[1], leaves.shape[2]
    ld_bar = np.broadcast_to(np.asarray(ld_bar, dtype=np.float64), (B,))
    parent = np.array([-1] + [0] * K, dtype=np.int32)
    cb = np.empty_like(center)
    lvb = np.empty_like(leaves)
    cpb = np.empty_like(coupling)
    for m in range(B):
        diag = np.concatenate([center[m][None], leaves[m]])
        edge = np.concatenate([np.zeros((1, b, b)), np.swapaxes(coupling[m], -1, -2)])
        gd = np.concatenate([_f64(gc_bar)[m][None], _f64(gl_bar)[m]])
        ge = np.concatenate([np.zeros((1, b, b)), np.swapaxes(_f64(gx_bar)[m], -1, -2)])
        db, eb = tree_vjp(parent, diag, edge, gd, ge, ld_bar[m], lib=lib)
        cb[m], lvb[m] = db[0], db[1:]
        cpb[m] = np.swapaxes(eb[1:], -1, -2)
    return cb, lvb, cpb


# ------------------------------------------------- shared-factor siblings
# Solve A x = y and the Gaussian sampling transform x = L^{-T} D^{-1/2} z from
# the collect's block LDL^T factor (oracle.c states the recurrences).  Vectors
# are [..., n, b, k]; mode "solve" or "sample".

_MODES = {"solve": 0, "sample": 1}


def tree_apply(parent, diag, edge, vec, mode, lib=None):
    """vec [n, b, k] -> out [n, b, k]."""
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    diag, edge, vec = _f64(diag), _f64(edge), _f64(vec)
    n, b = diag.shape[0], diag.shape[1]
    assert edge.shape == diag.shape and vec.shape[:2] == (n, b)
    k = vec.shape[2]
    out = np.empty_like(vec)
    rc = lib.oracle_tree_apply(n, b, _p(parent), _p(diag), _p(edge), k, _p(vec), _p(out),
                               _MODES[mode])
    if rc:
        raise OracleError("oracle_tree_apply status %d" % rc)
    return out


def chain_apply(diag, lower, vec, mode, lib=None):
    """Chains as path trees rooted at their last block.  vec [B, L, b, k]
    -> (out [B, L, b, k], status [B]: 0 or 3 = not PD)."""
    lib = lib or load()
    diag, lower, vec = _f64(diag), _f64(lower), _f64(vec)
    B, L, b = diag.shape[0], diag.shape[1], diag.shape[2]
    assert vec.shape[:3] == (B, L, b)
    k = vec.shape[3]
    out = np.empty_like(vec)
    st = np.empty(B, np.int32)
    rc = lib.oracle_chain_apply(B, L, b, _p(diag), _p(lower), k, _p(vec), _p(out),
                                _MODES[mode], _p(st))
    if rc:
        raise OracleError("oracle_chain_apply status %d" % rc)
    return out, st


def star_apply(center, leaves, coupling, vec_center, vec_leaves, mode, lib=None):
    """Stars as depth-1 trees (centre = node 0, leaf j = node j + 1, edge
    E_{j+1} = coupling[j]^T).  vec_center [B, b, k], vec_leaves [B, K, b, k]
    -> (out_center, out_leaves)."""
    center, leaves, coupling = _f64(center), _f64(leaves), _f64(coupling)
    B, K, b = leaves.shape[0], leaves.shape[1], leaves.shape[2]
    parent = np.array([-1] + [0] * K, dtype=np.int32)
    oc = np.empty_like(_f64(vec_center))
    ol = np.empty_like(_f64(vec_leaves))
    for m in range(B):
        diag = np.concatenate([center[m][None], leaves[m]])
        edge = np.concatenate([np.zeros((1, b, b)), np.swapaxes(coupling[m], -1, -2)])
        vec = np.concatenate([_f64(vec_center)[m][None], _f64(vec_leaves)[m]])
        out = tree_apply(parent, diag, edge, vec, mode, lib=lib)
        oc[m], ol[m] = out[0], out[1:]
    return oc, ol


# ------------------------------------------------- non-symmetric ladder

def bidiag(diag, lower, lib=None):
    """Block lower-bidiagonal M (diag [B,L,b,b], lower [B,L-1,b,b] = M_{i+1,i}).
    -> (G_diag, G_lower, info)."""
    lib = lib or load()
    diag, lower = _f64(diag), _f64(lower)
    B, L, b = diag.shape[0], diag.shape[1], diag.shape[2]
    Gd = np.empty_like(diag)
    Gl = np.empty_like(lower)
    info = np.empty(B, np.int32)
    rc = lib.oracle_bidiag(B, L, b, _p(diag), _p(lower), _p(Gd), _p(Gl), _p(info))
    if rc:
        raise OracleError("oracle_bidiag status %d" % rc)
    return Gd, Gl, info


def nonsym_tree(parent, diag, up, down, lib=None):
    """-> (G_diag, G_up [v] = G_{parent,v}, G_down [v] = G_{v,parent}, info)."""
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    diag, up, down = _f64(diag), _f64(up), _f64(down)
    n, b = diag.shape[0], diag.shape[1]
    Gd, Gu, Gw = np.empty_like(diag), np.empty_like(up), np.empty_like(down)
    info = np.zeros(1, np.int32)
    rc = lib.oracle_nonsym_tree(n, b, _p(parent), _p(diag), _p(up), _p(down), _p(Gd), _p(Gu),
                                _p(Gw), _p(info))
    if rc:
        raise OracleError("oracle_nonsym_tree status %d" % rc)
    return Gd, Gu, Gw, int(info[0])


# -------------------------------------------------------- junction tree

def eliminate(n, edge_index, order=None, lib=None):
    """Symbolic elimination of the block pattern (oracle_eliminate).

    edge_index int32 [2, m], pairs (i, j) with i > j; order: None (greedy
    minimum degree, smallest label on ties) or a permutation of range(n)
    listing the nodes in elimination order.
    -> (order [n], nbr_ptr [n+1], nbr [nnz]): step s eliminates order[s], whose
    later neighbours (labels, ascending) are nbr[nbr_ptr[s]:nbr_ptr[s+1]]."""
    lib = lib or load()
    ei = np.ascontiguousarray(edge_index[0], dtype=np.int32)
    ej = np.ascontiguousarray(edge_index[1], dtype=np.int32)
    oin = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    if oin is not None and oin.shape != (n,):
        raise OracleError("order must have n entries")
    out = np.empty(n, np.int32)
    ptr = np.empty(n + 1, np.int64)
    cap = 4 * ei.shape[0] + n
    while True:
        nbr = np.empty(max(cap, 1), np.int32)
        rc = lib.oracle_eliminate(n, ei.shape[0], _p(ei), _p(ej), _p(oin) if oin is not None else None,
                                  _p(out), _p(ptr), _p(nbr), cap)
        if rc == 3:
            cap = int(ptr[n])
            continue
        if rc:
            raise OracleError("oracle_eliminate status %d" % rc)
        return out, ptr, nbr[:ptr[n]].copy()


def filled_pattern(n, edge_index, order=None, lib=None):
    """The filled (chordal) pattern S of an elimination.

    Returns a dict with the elimination (order, pos, nbr_ptr, nbr), the owner
    node of every slot (col: the label eliminated at the slot's step), and
    the lower pattern S_index int32 [2, nnz]: every pair (i, j), i > j, of S,
    sorted by i then j.  slot[k] is the slot of S entry k and flip[k] says
    that the slot's block (w, v) is the transpose of G_{i,j} (w < v)."""
    order, ptr, nbr = eliminate(n, edge_index, order, lib)
    pos = np.empty(n, np.int64)
    pos[order] = np.arange(n)
    col = np.repeat(order, np.diff(ptr)).astype(np.int64)
    w = nbr.astype(np.int64)
    i, j = np.maximum(w, col), np.minimum(w, col)
    slot = np.lexsort((j, i))
    S_index = np.stack([i[slot], j[slot]]).astype(np.int32)
    return dict(order=order, pos=pos, nbr_ptr=ptr, nbr=nbr, col=col, S_index=S_index,
                slot=slot, flip=(w < col)[slot])


def _slot_values(P, edge_index, edge_val):
    """A on the slots of an elimination: A_{w,v} = edge_val[e] when
    (w, v) = (i_e, j_e), its transpose when (w, v) = (j_e, i_e), zero on
    fill.  edge_val [B, m, b, b] -> [B, nnz, b, b]."""
    B, b = edge_val.shape[0], edge_val.shape[-1]
    ei = np.asarray(edge_index[0], dtype=np.int64)
    ej = np.asarray(edge_index[1], dtype=np.int64)
    nnz = P["nbr"].shape[0]
    key = {(int(a), int(c)): e for e, (a, c) in enumerate(zip(ei, ej))}
    w, v = P["nbr"].astype(np.int64), P["col"]
    Aoff = np.zeros((B, nnz, b, b))
    for t in range(nnz):
        e = key.get((max(w[t], v[t]), min(w[t], v[t])))
        if e is not None:
            Aoff[:, t] = edge_val[:, e] if w[t] > v[t] else np.swapaxes(edge_val[:, e], -1, -2)
    return Aoff


def junction(diag, edge_index, edge_val, order=None, lib=None, pattern=None):
    """Selected inverse of general sparse SPD matrices sharing one pattern.

    diag [B,n,b,b] (or [n,b,b]), edge_index int32 [2,m] with i > j,
    edge_val [B,m,b,b] with edge_val[e] = A_{i_e, j_e}; order as for
    `eliminate`.  -> (G_diag [B,n,b,b], S_index [2,nnz], G_lower [B,nnz,b,b]
    with G_lower[k] = (A^-1)_{S_index[0,k], S_index[1,k]}, logdet [B], info [B]).
    """
    lib = lib or load()
    diag, edge_val = _f64(diag), _f64(edge_val)
    single = diag.ndim == 3
    if single:
        diag, edge_val = diag[None], edge_val[None]
    B, n, b = diag.shape[0], diag.shape[1], diag.shape[2]
    P = pattern or filled_pattern(n, edge_index, order, lib)
    nnz = P["nbr"].shape[0]
    Aoff = _slot_values(P, edge_index, edge_val)
    Gd = np.empty_like(diag)
    Go = np.empty((B, nnz, b, b))
    logdet = np.empty(B)
    info = np.empty(B, np.int32)
    rc = lib.oracle_junction(B, n, b, _p(P["order"]), _p(P["nbr_ptr"]), _p(P["nbr"]), _p(diag),
                             _p(Aoff), _p(Gd), _p(Go), _p(logdet), _p(info))
    if rc:
        raise OracleError("oracle_junction status %d" % rc)
    Gl = Go[:, P["slot"]]
    Gl[:, P["flip"]] = np.swapaxes(Gl[:, P["flip"]], -1, -2)
    if single:
        return Gd[0], P["S_index"], Gl[0], logdet[0], int(info[0])
    return Gd, P["S_index"], Gl, logdet, info


def junction_apply(diag, edge_index, edge_val, vec, mode, order=None, lib=None, pattern=None):
    """Solve (mode "solve": x = A^{-1} y) or the sampling transform (mode
    "sample": x = L^{-T} D^{-1/2} z) on the filled pattern, from the block
    LDL^T of the elimination (oracle_junction_apply).

    diag [B,n,b,b] (or [n,b,b]), edge_index, edge_val and order as for
    `junction`; vec [B,n,b,k] (or [n,b,k]) by label.  -> (x, info)."""
    lib = lib or load()
    diag, edge_val, vec = _f64(diag), _f64(edge_val), _f64(vec)
    single = diag.ndim == 3
    if single:
        diag, edge_val, vec = diag[None], edge_val[None], vec[None]
    B, n, b = diag.shape[0], diag.shape[1], diag.shape[2]
    k = vec.shape[-1]
    if vec.shape != (B, n, b, k):
        raise OracleError("vec must be [B, n, b, k]")
    P = pattern or filled_pattern(n, edge_index, order, lib)
    Aoff = _slot_values(P, edge_index, edge_val)
    out = np.empty_like(vec)
    info = np.empty(B, np.int32)
    md = {"solve": 0, "sample": 1}[mode]
    rc = lib.oracle_junction_apply(B, n, b, _p(P["order"]), _p(P["nbr_ptr"]), _p(P["nbr"]),
                                   _p(diag), _p(Aoff), k, _p(vec), _p(out), md, _p(info))
    if rc:
        raise OracleError("oracle_junction_apply status %d" % rc)
    if single:
        return out[0], int(info[0])
    return out, info
