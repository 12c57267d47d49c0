"""Seeded synthetic SPD block inputs (chain, star, tree) shared by the oracle
tests and the GPU path.

Input construction only: nothing here computes any part of the selected
inverse.  Values come from a counter-based generator (Philox4x32-10, Salmon et
al., SC 2011) so any single matrix of a batch can be regenerated on its own;
``spdgen.c`` states the recipe.  The workload shapes follow the batched
generators of the gabp-sparse-inv 0.3.2 project page (Quickstart section:
``random_spd_chain`` / ``random_spd_star`` / ``random_spd_tree``), with
explicit Gershgorin diagonal loads so that lambda_min(A) >= diag_load.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spdgen.c")
_LIB = os.path.join(_HERE, "libspdgen.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``libspdgen.so`` in place with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        lib.spdgen_chain.argtypes = [u64, i64, i64, i64, i32, dbl, vp, vp]
        lib.spdgen_star.argtypes = [u64, i64, i64, i64, i32, dbl, vp, vp, vp]
        lib.spdgen_random_recursive_tree.argtypes = [u64, i64, vp]
        lib.spdgen_tree.argtypes = [u64, i64, i32, dbl, vp, vp, vp]
        lib.spdgen_normal.argtypes = [u64, ctypes.c_uint32, u64, u64]
        lib.spdgen_normal.restype = dbl
        lib.spdgen_philox4x32_10.argtypes = [vp, vp, vp]
        lib.spdgen_cotangent.argtypes = [u64, ctypes.c_uint32, i64, i64, i64, vp]
        lib.spdgen_nonsym_bidiag.argtypes = [u64, i64, i64, i64, i32, dbl, vp, vp]
        lib.spdgen_nonsym_tree.argtypes = [u64, i64, i32, dbl, vp, vp, vp, vp]
        lib.spdgen_graph.argtypes = [u64, i64, i64, i64, i64, i32, dbl, vp, vp, vp, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    _load().spdgen_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal(seed: int, stream: int, mat: int, e: int) -> float:
    return _load().spdgen_normal(seed, stream, mat, e)


def chain(B: int, L: int, b: int, seed: int = 0, diag_load: float = 2.0, m0: int = 0,
          out=None):
    """Block-tridiagonal SPD chains [m0, m0+B) of a seeded batch.

    Returns ``diag [B,L,b,b]`` and ``lower [B,L-1,b,b]`` (float64) with
    ``lower[i] = A_{i+1,i}``.
    """
    if out is None:
        diag = np.empty((B, L, b, b), np.float64)
        lower = np.empty((B, max(L - 1, 0), b, b), np.float64)
    else:
        diag, lower = out
    _load().spdgen_chain(seed, m0, B, L, b, diag_load, _ptr(diag), _ptr(lower))
    return diag, lower


def star(B: int, K: int, b: int, seed: int = 0, diag_load: float = 2.0, m0: int = 0):
    """Block-arrowhead SPD matrices [m0, m0+B).

    Returns ``center [B,b,b]``, ``leaves [B,K,b,b]`` and ``coupling [B,K,b,b]``
    with ``coupling[j] = A_{j,0}`` (leaf row, centre column).
    """
    center = np.empty((B, b, b), np.float64)
    leaves = np.empty((B, K, b, b), np.float64)
    coupling = np.empty((B, K, b, b), np.float64)
    _load().spdgen_star(seed, m0, B, K, b, diag_load, _ptr(center), _ptr(leaves),
                        _ptr(coupling))
    return center, leaves, coupling


def cotangent(shape, seed: int = 0, k: int = 0, m0: int = 0) -> np.ndarray:
    """Standard normal array of ``shape`` (float64), seeded per leading index:
    row m of the result depends only on (seed, k, m0 + m), so a sample of a
    batch can be regenerated on its own.  ``k`` tells apart several arrays of
    one call (cotangents of different outputs)."""
    shape = tuple(int(x) for x in shape)
    out = np.empty(shape, np.float64)
    count = shape[0] if shape else 1
    per = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    if out.size:
        _load().spdgen_cotangent(seed, k, m0, count, per, _ptr(out))
    return out


def nonsym_bidiag(B: int, L: int, b: int, seed: int = 0, diag_load: float = 2.0, m0: int = 0):
    """Block lower-bidiagonal non-symmetric matrices [m0, m0+B): general
    diagonal blocks and lower[i] = M_{i+1,i}, every scalar row strictly
    diagonally dominant by diag_load."""
    diag = np.empty((B, L, b, b), np.float64)
    lower = np.empty((B, max(L - 1, 0), b, b), np.float64)
    _load().spdgen_nonsym_bidiag(seed, m0, B, L, b, diag_load, _ptr(diag), _ptr(lower))
    return diag, lower


def nonsym_tree(parent, b: int, seed: int = 1, diag_load: float = 2.0):
    """Tree-structured non-symmetric matrix: diag [n,b,b], up[v] = M_{parent,v},
    down[v] = M_{v,parent} (zero root slots), rows diagonally dominant."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    n = parent.shape[0]
    diag = np.empty((n, b, b), np.float64)
    up = np.empty((n, b, b), np.float64)
    down = np.empty((n, b, b), np.float64)
    _load().spdgen_nonsym_tree(seed, n, b, diag_load, _ptr(parent), _ptr(diag), _ptr(up),
                               _ptr(down))
    return diag, up, down


def to_dense_bidiag(diag: np.ndarray, lower: np.ndarray) -> np.ndarray:
    L, b = diag.shape[0], diag.shape[1]
    A = np.zeros((L * b, L * b))
    for i in range(L):
        A[i * b:(i + 1) * b, i * b:(i + 1) * b] = diag[i]
    for i in range(L - 1):
        A[(i + 1) * b:(i + 2) * b, i * b:(i + 1) * b] = lower[i]
    return A


def to_dense_nonsym_tree(parent, diag, up, down) -> np.ndarray:
    n, b = diag.shape[0], diag.shape[1]
    A = np.zeros((n * b, n * b))
    for v in range(n):
        A[v * b:(v + 1) * b, v * b:(v + 1) * b] = diag[v]
        p = int(parent[v])
        if p >= 0:
            A[p * b:(p + 1) * b, v * b:(v + 1) * b] = up[v]
            A[v * b:(v + 1) * b, p * b:(p + 1) * b] = down[v]
    return A


def random_recursive_tree(n: int, seed: int = 1) -> np.ndarray:
    """parent[0] = -1, parent[v] uniform over [0, v)."""
    parent = np.empty(n, np.int32)
    _load().spdgen_random_recursive_tree(seed, n, _ptr(parent))
    return parent


def path_tree(n: int) -> np.ndarray:
    """Path rooted at node 0: parent[v] = v - 1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def star_tree(n: int) -> np.ndarray:
    """Depth-1 tree: node 0 is the root, every other node its child."""
    p = np.zeros(n, np.int32)
    p[0] = -1
    return p


def balanced_tree(n: int, arity: int = 2) -> np.ndarray:
    """Complete `arity`-ary tree in heap order."""
    p = (np.arange(n, dtype=np.int64) - 1) // arity
    p[0] = -1
    return p.astype(np.int32)


def tree(parent: np.ndarray, b: int, seed: int = 1, diag_load: float = 2.0):
    """Tree-structured SPD values for ``parent`` (one matrix).

    Returns ``diag [n,b,b]`` and ``edge [n,b,b]`` with
    ``edge[v] = A_{parent(v),v}`` and a zero root slot.
    """
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    n = parent.shape[0]
    diag = np.empty((n, b, b), np.float64)
    edge = np.empty((n, b, b), np.float64)
    _load().spdgen_tree(seed, n, b, diag_load, _ptr(parent), _ptr(diag), _ptr(edge))
    return diag, edge


def grid_edges(rows: int, cols: int) -> np.ndarray:
    """Edges of the rows x cols grid graph (node r * cols + c), as an int32
    array [2, m] of pairs (i, j) with i > j: for each node its right
    neighbour, then its lower neighbour (the grid_edges helper of the
    gabp-sparse-inv page's junction-tree section)."""
    e = []
    for r in range(rows):
        for c in range(cols):
            v = r * cols + c
            if c + 1 < cols:
                e.append((v + 1, v))
            if r + 1 < rows:
                e.append((v + cols, v))
    return np.array(e, dtype=np.int32).reshape(-1, 2).T.copy()


def random_graph_edges(n: int, extra: int, seed: int = 0) -> np.ndarray:
    """A connected random graph: a random recursive tree on n nodes plus
    `extra` further distinct random pairs; int32 [2, m] with i > j."""
    p = random_recursive_tree(n, seed)
    pairs = {(v, int(p[v])) for v in range(1, n)}
    rng = np.random.default_rng(seed)
    while len(pairs) < n - 1 + extra and len(pairs) < n * (n - 1) // 2:
        i, j = rng.integers(0, n, size=2)
        if i != j:
            pairs.add((int(max(i, j)), int(min(i, j))))
    e = sorted(pairs)
    return np.array(e, dtype=np.int32).reshape(-1, 2).T.copy()


def graph(edge_index: np.ndarray, n: int, b: int, B: int = 1, seed: int = 0,
          diag_load: float = 2.0, m0: int = 0):
    """SPD values on an arbitrary block pattern for a batch of B matrices that
    share it.  ``edge_index`` is int32 [2, m] with rows (i, j), i > j.
    Returns ``diag [B,n,b,b]`` and ``edge_val [B,m,b,b]`` with
    ``edge_val[:, e] = A_{i_e, j_e}``."""
    ei = np.ascontiguousarray(edge_index[0], dtype=np.int32)
    ej = np.ascontiguousarray(edge_index[1], dtype=np.int32)
    assert np.all(ei > ej) and np.all(ej >= 0) and np.all(ei < n)
    m = ei.shape[0]
    diag = np.empty((B, n, b, b), np.float64)
    ev = np.empty((B, m, b, b), np.float64)
    _load().spdgen_graph(seed, m0, B, n, m, b, diag_load, _ptr(ei), _ptr(ej), _ptr(diag),
                         _ptr(ev))
    return diag, ev


def to_dense_graph(edge_index, diag: np.ndarray, edge_val: np.ndarray) -> np.ndarray:
    """Assemble one general block matrix (diag [n,b,b], edge_val [m,b,b])."""
    n, b = diag.shape[0], diag.shape[1]
    A = np.zeros((n * b, n * b))
    for v in range(n):
        A[v * b:(v + 1) * b, v * b:(v + 1) * b] = diag[v]
    for e in range(edge_index.shape[1]):
        i, j = int(edge_index[0, e]), int(edge_index[1, e])
        A[i * b:(i + 1) * b, j * b:(j + 1) * b] = edge_val[e]
        A[j * b:(j + 1) * b, i * b:(i + 1) * b] = edge_val[e].T
    return A


# --------------------------------------------------------------- workloads
# The five synthetic workloads the hot path is measured and checked on.
WORKLOADS = {
    "chain_b4_single": dict(kind="chain", B=1, L=8, b=4, seed=0, diag_load=2.0,
                            dtypes=("f64",)),
    "chain_b16_batched": dict(kind="chain", B=4096, L=64, b=16, seed=0, diag_load=2.0,
                              dtypes=("f64", "f32")),
    "chain_b32_long": dict(kind="chain", B=64, L=16384, b=32, seed=0, diag_load=1.0,
                           dtypes=("f64",)),
    "star_b32": dict(kind="star", B=256, K=1024, b=32, seed=0, diag_load=2.0,
                     dtypes=("f64",)),
    "tree_b8_random": dict(kind="tree", n=262144, b=8, seed=1, diag_load=2.0,
                           dtypes=("f64", "f32")),
    # the non-symmetric ladder at the sizes of the chain and tree workloads
    "bidiag_b16_batched": dict(kind="bidiag", B=4096, L=64, b=16, seed=0, diag_load=2.0,
                               dtypes=("f64", "f32")),
    "nonsym_tree_b8": dict(kind="nonsym_tree", n=262144, b=8, seed=1, diag_load=2.0,
                           dtypes=("f64", "f32")),
    # general sparse SPD: a batch sharing the 64 x 64 grid pattern, b = 8
    "junction_grid64_b8": dict(kind="junction", B=16, rows=64, cols=64, b=8, seed=0,
                               diag_load=2.0, dtypes=("f64", "f32")),
}


def to_dense_chain(diag: np.ndarray, lower: np.ndarray) -> np.ndarray:
    """Assemble one chain (diag [L,b,b], lower [L-1,b,b]) as a dense matrix."""
    L, b = diag.shape[0], diag.shape[1]
    A = np.zeros((L * b, L * b))
    for i in range(L):
        A[i * b:(i + 1) * b, i * b:(i + 1) * b] = diag[i]
    for i in range(L - 1):
        A[(i + 1) * b:(i + 2) * b, i * b:(i + 1) * b] = lower[i]
        A[i * b:(i + 1) * b, (i + 1) * b:(i + 2) * b] = lower[i].T
    return A


def to_dense_star(center: np.ndarray, leaves: np.ndarray, coupling: np.ndarray) -> np.ndarray:
    """Assemble one star; the centre is block 0 and leaf j is block j+1."""
    K, b = leaves.shape[0], leaves.shape[1]
    A = np.zeros(((K + 1) * b, (K + 1) * b))
    A[:b, :b] = center
    for j in range(K):
        s = (j + 1) * b
        A[s:s + b, s:s + b] = leaves[j]
        A[s:s + b, :b] = coupling[j]
        A[:b, s:s + b] = coupling[j].T
    return A


def to_dense_tree(parent: np.ndarray, diag: np.ndarray, edge: np.ndarray) -> np.ndarray:
    """Assemble one tree matrix; node v is block v."""
    n, b = diag.shape[0], diag.shape[1]
    A = np.zeros((n * b, n * b))
    for v in range(n):
        A[v * b:(v + 1) * b, v * b:(v + 1) * b] = diag[v]
        p = int(parent[v])
        if p >= 0:
            A[p * b:(p + 1) * b, v * b:(v + 1) * b] = edge[v]
            A[v * b:(v + 1) * b, p * b:(p + 1) * b] = edge[v].T
    return A
