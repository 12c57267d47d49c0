"""Pins for the oracle's general sparse SPD selected inverse (the junction-tree
section of the gabp-sparse-inv page: elimination to the chordal pattern, then
the multi-neighbour Takahashi recurrence).

Independent references:
  * the hand-derived minimum-degree elimination of the 3 x 3 grid under
    tests/golden/ (order, cliques and fill);
  * numpy's dense inverse and slogdet of the assembled matrix, read on the
    filled pattern, for grids, random graphs, trees and complete graphs, with
    the default order and with explicit orders;
  * the structural nonzeros of numpy's Cholesky factor of the permuted matrix
    (scalar blocks, random values) must be exactly the filled pattern;
  * minimum degree on a tree creates no fill, and then the result must be the
    tree oracle's (pinned on its own); a path is the chain;
  * planted mistakes must break one of the above.

The solve and sampling siblings (oracle_junction_apply) are pinned to
numpy's dense solve of the assembled matrix (solve) and to numpy's Cholesky
factor of the matrix permuted into the elimination order (sample: the
factor's diagonal blocks are the Cholesky factors of the pivots, so
x = L^-T D^-1/2 z is P^T Lc^-T P z for P A P^T = Lc Lc^T), plus
x^T A x = z^T z, the tree reduction and planted mistakes.
"""
import os
import re
import tempfile

import numpy as np
import pytest

import oracle
import spdgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "junction_grid3x3_mindegree.txt")


def blk(M, r, c, b):
    return M[r * b:(r + 1) * b, c * b:(c + 1) * b]


def read_golden():
    order, steps, fill = None, {}, set()
    for line in open(GOLDEN):
        t = line.split()
        if not t or t[0].startswith("#"):
            continue
        if t[0] == "order":
            order = [int(x) for x in t[1:]]
        elif t[0] == "step":
            steps[int(t[1])] = [int(x) for x in t[2:]]
        elif t[0] == "fill":
            fill.add((int(t[1]), int(t[2])))
    return order, steps, fill


def test_golden_grid3x3_min_degree():
    order, steps, fill = read_golden()
    e = spdgen.grid_edges(3, 3)
    o, ptr, nbr = oracle.eliminate(9, e)
    assert list(o) == order
    for s, v in enumerate(o):
        assert list(nbr[ptr[s]:ptr[s + 1]]) == steps[int(v)]
    S = oracle.filled_pattern(9, e)["S_index"]
    got = {(int(i), int(j)) for i, j in S.T}
    grid = {(int(i), int(j)) for i, j in e.T}
    assert got == grid | fill and len(got) == 17


def check_dense(edge_index, n, b, B=2, seed=0, order=None, tol=1e-12):
    d, v = spdgen.graph(edge_index, n, b, B=B, seed=seed)
    Gd, S, Gl, ld, info = oracle.junction(d, edge_index, v, order=order)
    assert (info == 0).all()
    for m in range(B):
        A = spdgen.to_dense_graph(edge_index, d[m], v[m])
        Ai = np.linalg.inv(A)
        sc = np.abs(Ai).max()
        for x in range(n):
            assert np.abs(Gd[m, x] - blk(Ai, x, x, b)).max() <= tol * sc
        for k in range(S.shape[1]):
            assert np.abs(Gl[m, k] - blk(Ai, S[0, k], S[1, k], b)).max() <= tol * sc
        assert abs(ld[m] - np.linalg.slogdet(A)[1]) <= 1e-10 * max(1.0, abs(ld[m]))
    return S


@pytest.mark.parametrize("r,c,b", [(1, 1, 2), (1, 6, 3), (3, 3, 2), (4, 5, 1), (5, 4, 3),
                                   (6, 6, 2)])
def test_grid_dense(r, c, b):
    S = check_dense(spdgen.grid_edges(r, c), r * c, b)
    assert np.all(S[0] > S[1])


@pytest.mark.parametrize("n,extra,b", [(12, 10, 2), (25, 30, 1), (30, 15, 3), (8, 28, 2)])
def test_random_graph_dense(n, extra, b):
    check_dense(spdgen.random_graph_edges(n, extra, seed=n), n, b, seed=n)


def test_complete_graph_fills_nothing_new():
    n = 7
    e = np.array([(i, j) for i in range(n) for j in range(i)], np.int32).T.copy()
    S = check_dense(e, n, 2)
    assert S.shape[1] == n * (n - 1) // 2


@pytest.mark.parametrize("kind", ["natural", "reversed", "random"])
def test_explicit_orders(kind):
    n = 16
    e = spdgen.grid_edges(4, 4)
    order = {"natural": np.arange(n), "reversed": np.arange(n)[::-1],
             "random": np.random.default_rng(1).permutation(n)}[kind]
    check_dense(e, n, 2, order=order)
    o, _, _ = oracle.eliminate(n, e, order)
    assert list(o) == list(order)


@pytest.mark.parametrize("order_kind", ["mindeg", "random"])
def test_pattern_is_the_cholesky_structure(order_kind):
    """b = 1, random values: the structural nonzeros of chol(P A P^T) are S."""
    n = 30
    e = spdgen.random_graph_edges(n, 25, seed=4)
    order = None if order_kind == "mindeg" else np.random.default_rng(2).permutation(n)
    P = oracle.filled_pattern(n, e, order)
    d, v = spdgen.graph(e, n, 1, B=1, seed=3)
    A = spdgen.to_dense_graph(e, d[0], v[0])
    o = P["order"]
    Lc = np.linalg.cholesky(A[np.ix_(o, o)])
    nz = {(max(int(o[r]), int(o[c])), min(int(o[r]), int(o[c])))
          for r in range(n) for c in range(r) if abs(Lc[r, c]) > 1e-13}
    assert nz == {(int(i), int(j)) for i, j in P["S_index"].T}


def test_min_degree_is_greedy():
    """Every step eliminates a node of minimum remaining degree, the smallest
    label among those (checked on the recorded cliques)."""
    n = 40
    e = spdgen.random_graph_edges(n, 40, seed=6)
    o, ptr, nbr = oracle.eliminate(n, e)
    adj = {v: set() for v in range(n)}
    for i, j in e.T:
        adj[int(i)].add(int(j))
        adj[int(j)].add(int(i))
    for s, v in enumerate(o):
        v = int(v)
        best = min(adj, key=lambda u: (len(adj[u]), u))
        assert v == best
        assert sorted(adj[v]) == list(nbr[ptr[s]:ptr[s + 1]])
        for a in adj[v]:
            adj[a] |= adj[v] - {a}
            adj[a].discard(v)
        del adj[v]


@pytest.mark.parametrize("kind", ["random", "star", "balanced"])
def test_tree_has_no_fill_and_is_the_tree_oracle(kind):
    n, b = 40, 3
    parent = {"random": spdgen.random_recursive_tree(n, 2), "star": spdgen.star_tree(n),
              "balanced": spdgen.balanced_tree(n, 2)}[kind]
    d, ed = spdgen.tree(parent, b, seed=5)
    e = np.array([(max(v, int(parent[v])), min(v, int(parent[v])))
                  for v in range(n) if parent[v] >= 0], np.int32).T.copy()
    # edge_val[k] = A_{i,j} with i > j; the tree's edge[v] = A_{parent(v),v}
    ev = np.stack([ed[v] if parent[v] > v else ed[v].T
                   for v in range(n) if parent[v] >= 0])
    for k, v in enumerate(v for v in range(n) if parent[v] >= 0):
        assert (e[0, k], e[1, k]) == (max(v, parent[v]), min(v, parent[v]))
    Gd, S, Gl, ld, info = oracle.junction(d, e, ev)
    assert S.shape[1] == n - 1                                  # no fill
    Td, Te, Tld, Tinfo = oracle.tree(parent, d, ed)
    assert info == 0 and abs(ld - Tld) <= 1e-11 * abs(Tld)
    assert np.abs(Gd - Td).max() <= 1e-12 * np.abs(Td).max()
    look = {(int(i), int(j)): k for k, (i, j) in enumerate(S.T)}
    for v in range(n):
        p = int(parent[v])
        if p < 0:
            continue
        g = Gl[look[(max(v, p), min(v, p))]]
        g = g if p > v else g.T                                 # -> G_{p,v}
        assert np.abs(g - Te[v]).max() <= 1e-12 * np.abs(Te).max()


def test_path_is_the_chain():
    L, b = 9, 2
    d, lo = spdgen.chain(1, L, b, seed=3)
    e = np.array([(i + 1, i) for i in range(L - 1)], np.int32).T.copy()
    Gd, S, Gl, ld, info = oracle.junction(d[0], e, lo[0])
    Cd, Cl, Cld, Cinfo = oracle.chain(d, lo)
    assert S.shape[1] == L - 1 and list(S[0]) == list(range(1, L))
    assert np.abs(Gd - Cd[0]).max() <= 1e-12 * np.abs(Cd).max()
    assert np.abs(Gl - Cl[0]).max() <= 1e-12 * np.abs(Cd).max()
    assert abs(ld - Cld[0]) <= 1e-11 * abs(Cld[0])


def test_not_positive_definite_reports_the_first_node():
    e = spdgen.grid_edges(3, 4)
    d, v = spdgen.graph(e, 12, 2, B=2, seed=1)
    d[1, 6] = -np.eye(2)
    Gd, S, Gl, ld, info = oracle.junction(d, e, v)
    o, _, _ = oracle.eliminate(12, e)
    assert info[0] == 0 and np.isfinite(ld[0])
    assert info[1] == 7 and np.isnan(ld[1])
    assert list(o).index(6) >= 0


def test_bad_input_is_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.eliminate(3, np.array([[0], [1]], np.int32))            # i < j
    with pytest.raises(oracle.OracleError):
        oracle.eliminate(3, np.array([[1, 1], [0, 0]], np.int32))      # repeated
    with pytest.raises(oracle.OracleError):
        oracle.eliminate(3, np.array([[1], [0]], np.int32), order=[0, 0, 1])


MUTANTS = [
    ("skips diagonal update", r"if \(pos\[w1\] < pos\[w2\]\) continue;",
     "if (pos[w1] <= pos[w2]) continue;"),
    ("missing transpose", r"Gwx = T2;", "Gwx = Go + twx * bb;"),
    ("G_vv sign", r"add_to\(bb, Gd \+ v \* bb, T, -1\.0\);", "add_to(bb, Gd + v * bb, T, 1.0);"),
    ("L from unupdated A", r"matmul\(b, Co \+ t \* bb, Di \+ v \* bb, Lo \+ t \* bb\);",
     "matmul(b, A_off + t * bb, Di + v * bb, Lo + t * bb);"),
    ("ties to largest label", r"\(v < 0 \|\| deg\[u\] < deg\[v\]\)", "(v < 0 || deg[u] <= deg[v])"),
    ("no fill", r"adj\[x \* n \+ y\] = adj\[y \* n \+ x\] = 1;", "(void)0;"),
]


@pytest.mark.parametrize("name,pat,rep", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutants_are_caught(name, pat, rep):
    src = open(oracle.SOURCE).read()
    mutated, cnt = re.subn(pat, rep, src)
    assert cnt == 1, "mutation site not found: " + name
    with tempfile.TemporaryDirectory() as td:
        c, so = os.path.join(td, "m.c"), os.path.join(td, "m.so")
        open(c, "w").write(mutated)
        lib = oracle.load(oracle.compile_oracle(c, so))
        order, _, _ = read_golden()
        e = spdgen.grid_edges(3, 3)
        bad = list(oracle.eliminate(9, e, lib=lib)[0]) != order
        e = spdgen.grid_edges(4, 4)
        d, v = spdgen.graph(e, 16, 2, B=1, seed=2)
        try:
            Gd, S, Gl, ld, info = oracle.junction(d[0], e, v[0], lib=lib)
        except oracle.OracleError:
            bad = True
        else:
            Ai = np.linalg.inv(spdgen.to_dense_graph(e, d[0], v[0]))
            for x in range(16):
                bad |= np.abs(Gd[x] - blk(Ai, x, x, 2)).max() > 1e-8
            for k in range(S.shape[1]):
                bad |= np.abs(Gl[k] - blk(Ai, S[0, k], S[1, k], 2)).max() > 1e-8
        assert bad, name


# ------------------------------------------------ solve and sampling siblings
def _perm_blocks(order, b):
    return np.concatenate([np.arange(v * b, (v + 1) * b) for v in order])


def check_apply(edge_index, n, b, k, B=2, seed=0, order=None, lib=None, tol=1e-11):
    """Solve against numpy's dense solve; sample against numpy's Cholesky of
    the matrix permuted into the elimination order.  Returns False on a
    mismatch (for the planted-mistake battery)."""
    d, v = spdgen.graph(edge_index, n, b, B=B, seed=seed)
    rng = np.random.default_rng(seed + 100)
    y = rng.standard_normal((B, n, b, k))
    z = rng.standard_normal((B, n, b, k))
    x, info = oracle.junction_apply(d, edge_index, v, y, "solve", order=order, lib=lib)
    xs, info2 = oracle.junction_apply(d, edge_index, v, z, "sample", order=order, lib=lib)
    if (info != 0).any() or (info2 != 0).any():
        return False
    o = oracle.eliminate(n, edge_index, order, lib=lib)[0]
    p = _perm_blocks(o, b)
    ok = True
    for m in range(B):
        A = spdgen.to_dense_graph(edge_index, d[m], v[m])
        ref = np.linalg.solve(A, y[m].reshape(n * b, k))
        ok &= np.abs(x[m].reshape(n * b, k) - ref).max() <= tol * np.abs(ref).max()
        Lc = np.linalg.cholesky(A[np.ix_(p, p)])
        xp = np.linalg.solve(Lc.T, z[m].reshape(n * b, k)[p])
        ref_s = np.empty_like(xp)
        ref_s[p] = xp
        ok &= np.abs(xs[m].reshape(n * b, k) - ref_s).max() <= tol * np.abs(ref_s).max()
        # x^T A x = z^T z column by column
        X, Z = xs[m].reshape(n * b, k), z[m].reshape(n * b, k)
        q = np.einsum("ic,ij,jc->c", X, A, X)
        ok &= np.allclose(q, (Z * Z).sum(0), rtol=1e-10, atol=0)
    return bool(ok)


@pytest.mark.parametrize("r,c,b,k", [(1, 1, 2, 1), (1, 7, 3, 2), (3, 3, 2, 3), (4, 5, 1, 4),
                                     (5, 4, 3, 1), (6, 6, 2, 5)])
def test_apply_grid_dense(r, c, b, k):
    assert check_apply(spdgen.grid_edges(r, c), r * c, b, k, seed=r * c + b)


@pytest.mark.parametrize("n,extra,b,k", [(20, 30, 2, 3), (40, 80, 1, 2), (12, 40, 4, 1)])
def test_apply_random_graph_dense(n, extra, b, k):
    e = spdgen.random_graph_edges(n, extra, seed=n + extra)
    assert check_apply(e, n, b, k, seed=n)


@pytest.mark.parametrize("kind", ["natural", "reversed", "random"])
def test_apply_explicit_orders(kind):
    n = 16
    order = {"natural": np.arange(n), "reversed": np.arange(n)[::-1].copy(),
             "random": np.random.default_rng(3).permutation(n)}[kind]
    assert check_apply(spdgen.grid_edges(4, 4), n, 2, 3, seed=5, order=order)


def test_apply_no_edges_is_blockwise():
    """No edges: A is block diagonal, x_v = A_vv^-1 y_v and x_v = R_v^-T z_v."""
    n, b, k = 5, 3, 2
    e = np.zeros((2, 0), np.int32)
    d, v = spdgen.graph(e, n, b, B=1, seed=4)
    y = np.random.default_rng(0).standard_normal((1, n, b, k))
    x, info = oracle.junction_apply(d, e, v, y, "solve")
    xs, _ = oracle.junction_apply(d, e, v, y, "sample")
    for u in range(n):
        assert np.allclose(x[0, u], np.linalg.solve(d[0, u], y[0, u]), rtol=1e-12, atol=1e-14)
        R = np.linalg.cholesky(d[0, u])
        assert np.allclose(xs[0, u], np.linalg.solve(R.T, y[0, u]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode", ["solve", "sample"])
def test_apply_tree_is_the_tree_oracle(mode):
    """A tree eliminated children first (deepest level first, the tree
    oracle's order) creates no fill, and its factor is the tree's collect:
    both sweeps must be the tree oracle's (pinned on its own)."""
    n, b, k = 40, 3, 2
    parent = spdgen.random_recursive_tree(n, 2)
    depth = oracle.tree_depths(parent)
    order = np.array(sorted(range(n), key=lambda v: (-depth[v], v)), np.int32)
    e = np.array([(max(v, int(parent[v])), min(v, int(parent[v])))
                  for v in range(n) if parent[v] >= 0], np.int32).T.copy()
    d, ed = spdgen.tree(parent, b, seed=7)
    val = np.stack([ed[v] if parent[v] > v else ed[v].T for v in range(n) if parent[v] >= 0])
    vec = np.random.default_rng(1).standard_normal((n, b, k))
    got, info = oracle.junction_apply(d, e, val, vec, mode, order=order)
    ref = oracle.tree_apply(parent, d, ed, vec, mode)
    assert info == 0
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_apply_not_positive_definite():
    e = spdgen.grid_edges(3, 4)
    d, v = spdgen.graph(e, 12, 2, B=2, seed=1)
    d[1, 6] = -np.eye(2)
    y = np.ones((2, 12, 2, 3))
    for mode in ("solve", "sample"):
        x, info = oracle.junction_apply(d, e, v, y, mode)
        assert info[0] == 0 and np.isfinite(x[0]).all()
        assert info[1] == 7 and np.isnan(x[1]).all()


APPLY_MUTANTS = [
    ("forward update transposed",
     r"acc \+= Lo\[t \* bb \+ i \* b \+ j\] \* u\[v \* bk \+ j \* k \+ c\];",
     "acc += Lo[t * bb + j * b + i] * u[v * bk + j * k + c];"),
    ("backward not transposed",
     r"acc \+= Lo\[t \* bb \+ j \* b \+ i\] \* x\[wl \* bk \+ j \* k \+ c\];",
     "acc += Lo[t * bb + i * b + j] * x[wl * bk + j * k + c];"),
    ("forward update sign", r"u\[wl \* bk \+ i \* k \+ c\] -= acc;",
     "u[wl * bk + i * k + c] += acc;"),
    ("sample with R^-1", r"trsv_LT\(b, k, Rv \+ v \* bb, y \+ v \* bk, w \+ v \* bk\);",
     "trsv_L(b, k, Rv + v * bb, y + v * bk, w + v * bk);"),
    ("pivot solve one-sided", r"trsv_LT\(b, k, Rv \+ v \* bb, t1, w \+ v \* bk\);",
     "memcpy(w + v * bk, t1, sizeof(double) * (size_t)bk);"),
]


@pytest.mark.parametrize("name,pat,rep", APPLY_MUTANTS, ids=[m[0] for m in APPLY_MUTANTS])
def test_apply_mutants_are_caught(name, pat, rep):
    src = open(oracle.SOURCE).read()
    mutated, cnt = re.subn(pat, rep, src)
    assert cnt == 1, "mutation site not found: " + name
    with tempfile.TemporaryDirectory() as td:
        c, so = os.path.join(td, "m.c"), os.path.join(td, "m.so")
        open(c, "w").write(mutated)
        lib = oracle.load(oracle.compile_oracle(c, so))
        with np.errstate(all="ignore"):
            ok = check_apply(spdgen.grid_edges(4, 4), 16, 2, 2, B=1, seed=2, lib=lib)
        assert not ok, name
