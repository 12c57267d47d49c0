"""Pins for the oracle's shared-factor siblings: solve A x = y and the
Gaussian sampling transform x = L^{-T} D^{-1/2} z (the gabp-sparse-inv page's
junction_solve and sample_gaussian_tree passages; log det is the forward
oracle's, pinned elsewhere).

Independent references:
  * numpy's dense solve of the assembled matrix (solve);
  * the sampler applied to the standard basis gives the linear map T itself
    ("verified by the deterministic transform on the standard basis"): T T^T
    must be the dense A^{-1}, and in any children-before-parents order T must
    be upper triangular with a positive diagonal.  Those two facts determine T
    uniquely, so they pin the exact transform, not only its covariance;
  * for a single block, T = (cholesky(A))^{-T} from numpy;
  * planted mistakes in the sweeps must break these pins.
"""
import os
import re
import tempfile

import numpy as np
import pytest

import oracle
import spdgen

rng = np.random.default_rng(77)


def _trees():
    return {"random": spdgen.random_recursive_tree(23, 4), "path": spdgen.path_tree(9),
            "star": spdgen.star_tree(8), "balanced": spdgen.balanced_tree(15, 2)}


@pytest.mark.parametrize("kind", ["random", "path", "star", "balanced"])
@pytest.mark.parametrize("b,k", [(1, 1), (3, 2), (4, 5)])
def test_tree_solve_dense(kind, b, k):
    parent = _trees()[kind]
    n = len(parent)
    d, e = spdgen.tree(parent, b, seed=n + b)
    y = rng.standard_normal((n, b, k))
    x = oracle.tree_apply(parent, d, e, y, "solve")
    A = spdgen.to_dense_tree(parent, d, e)
    ref = np.linalg.solve(A, y.reshape(n * b, k)).reshape(n, b, k)
    assert np.abs(x - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("L,b,k", [(1, 3, 2), (2, 1, 1), (7, 4, 3), (30, 2, 1)])
def test_chain_solve_dense(L, b, k):
    d, l = spdgen.chain(3, L, b, seed=L)
    y = rng.standard_normal((3, L, b, k))
    x, st = oracle.chain_apply(d, l, y, "solve")
    assert (st == 0).all()
    for m in range(3):
        A = spdgen.to_dense_chain(d[m], l[m])
        ref = np.linalg.solve(A, y[m].reshape(L * b, k)).reshape(L, b, k)
        assert np.abs(x[m] - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("K,b,k", [(0, 2, 1), (5, 3, 2)])
def test_star_solve_dense(K, b, k):
    c, lv, cp = spdgen.star(2, K, b, seed=K)
    yc = rng.standard_normal((2, b, k))
    yl = rng.standard_normal((2, K, b, k))
    xc, xl = oracle.star_apply(c, lv, cp, yc, yl, "solve")
    for m in range(2):
        A = spdgen.to_dense_star(c[m], lv[m], cp[m])
        y = np.concatenate([yc[m][None], yl[m]]).reshape((K + 1) * b, k)
        ref = np.linalg.solve(A, y).reshape(K + 1, b, k)
        assert np.abs(xc[m] - ref[0]).max() <= 1e-12 * np.abs(ref).max()
        if K:
            assert np.abs(xl[m] - ref[1:]).max() <= 1e-12 * np.abs(ref).max()


def _children_first_order(parent):
    depth = oracle.tree_depths(parent)
    return sorted(range(len(parent)), key=lambda v: (-depth[v], v))


def _check_transform(T, Ainv, order, b):
    """T T^T = A^{-1}, and T upper triangular with a positive diagonal in the
    given block order."""
    assert np.abs(T @ T.T - Ainv).max() <= 1e-12 * np.abs(Ainv).max()
    perm = np.concatenate([np.arange(v * b, (v + 1) * b) for v in order])
    Tp = T[np.ix_(perm, perm)]
    assert np.abs(np.tril(Tp, -1)).max() <= 1e-13 * np.abs(Tp).max()
    assert (np.diag(Tp) > 0).all()


@pytest.mark.parametrize("kind", ["random", "path", "star", "balanced"])
@pytest.mark.parametrize("b", [1, 3])
def test_tree_sample_transform(kind, b):
    parent = _trees()[kind]
    n = len(parent)
    d, e = spdgen.tree(parent, b, seed=2 * n + b)
    N = n * b
    T = oracle.tree_apply(parent, d, e, np.eye(N).reshape(n, b, N), "sample").reshape(N, N)
    Ainv = np.linalg.inv(spdgen.to_dense_tree(parent, d, e))
    _check_transform(T, Ainv, _children_first_order(parent), b)


def test_chain_and_star_sample_transform():
    d, l = spdgen.chain(2, 6, 3, seed=5)
    N = 18
    T, st = oracle.chain_apply(d, l, np.broadcast_to(np.eye(N).reshape(6, 3, N), (2, 6, 3, N)),
                               "sample")
    for m in range(2):
        Ainv = np.linalg.inv(spdgen.to_dense_chain(d[m], l[m]))
        _check_transform(T[m].reshape(N, N), Ainv, list(range(6)), 3)
    c, lv, cp = spdgen.star(1, 4, 2, seed=1)
    N = 10
    Z = np.eye(N).reshape(5, 2, N)
    tc, tl = oracle.star_apply(c, lv, cp, Z[0][None], Z[1:][None], "sample")
    T = np.concatenate([tc[0][None], tl[0]]).reshape(N, N)
    Ainv = np.linalg.inv(spdgen.to_dense_star(c[0], lv[0], cp[0]))
    _check_transform(T, Ainv, [1, 2, 3, 4, 0], 2)


def test_single_block_sample_is_inverse_transposed_cholesky():
    d, _ = spdgen.tree(np.array([-1], np.int32), 5, seed=3)
    T = oracle.tree_apply(np.array([-1], np.int32), d, np.zeros_like(d),
                          np.eye(5).reshape(1, 5, 5), "sample")[0]
    assert np.allclose(T, np.linalg.inv(np.linalg.cholesky(d[0])).T, atol=1e-14, rtol=0)


def test_not_pd_gives_nan_and_status():
    d, l = spdgen.chain(2, 4, 2, seed=1)
    d[1, 2] = -np.eye(2)
    x, st = oracle.chain_apply(d, l, np.ones((2, 4, 2, 1)), "solve")
    assert list(st) == [0, 3] and np.isnan(x[1]).all() and np.isfinite(x[0]).all()


MUTANTS = [
    ("forward sweep uses X^T", r"s \+= X\[v \* bb \+ i \* b \+ j\] \* u\[v \* bk \+ j \* k \+ c\];",
     "s += X[v * bb + j * b + i] * u[v * bk + j * k + c];"),
    ("backward sweep uses X", r"s \+= X\[v \* bb \+ j \* b \+ i\] \* out\[p \* bk \+ j \* k \+ c\];",
     "s += X[v * bb + i * b + j] * out[p * bk + j * k + c];"),
    ("sample with R^{-1}", r"trsv_LT\(b, k, R \+ v \* bb, in \+ v \* bk, w \+ v \* bk\);",
     "trsv_L(b, k, R + v * bb, in + v * bk, w + v * bk);"),
    ("backward sweep sign", r"out\[v \* bk \+ i \* k \+ c\] = w\[v \* bk \+ i \* k \+ c\] - s;",
     "out[v * bk + i * k + c] = w[v * bk + i * k + c] + s;"),
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
        parent = spdgen.random_recursive_tree(9, 2)
        d, e = spdgen.tree(parent, 2, seed=4)
        A = spdgen.to_dense_tree(parent, d, e)
        N = 18
        y = rng.standard_normal((9, 2, 1))
        x = oracle.tree_apply(parent, d, e, y, "solve", lib=lib)
        solve_ok = np.abs(A @ x.reshape(N, 1) - y.reshape(N, 1)).max() < 1e-10
        T = oracle.tree_apply(parent, d, e, np.eye(N).reshape(9, 2, N), "sample",
                              lib=lib).reshape(N, N)
        cov_ok = np.abs(T @ T.T - np.linalg.inv(A)).max() < 1e-10
        perm = np.concatenate([np.arange(v * 2, v * 2 + 2) for v in _children_first_order(parent)])
        tri_ok = np.abs(np.tril(T[np.ix_(perm, perm)], -1)).max() < 1e-12
        assert not (solve_ok and cov_ok and tri_ok), name
