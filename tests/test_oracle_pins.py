"""Pins of the float64 oracle to results fixed independently of it.

* dense pins: the page's own check -- every on-pattern block equals the
  corresponding block of a dense inverse (the Quickstart section of the
  gabp-sparse-inv 0.3.2 page asserts exactly this against
  torch.linalg.inv(to_dense()) with atol 1e-10); here numpy/LAPACK's inverse
  and slogdet, on non-symmetric random off-diagonal blocks so that any
  orientation mistake shows;
* closed forms: 1-D Laplacian, Usmani's tridiagonal recurrences, Kronecker
  chains, scalar arrowheads, Kronecker stars and trees;
* the hand-derived worked example under tests/golden/.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import pins
from conftest import GOLDEN

TOL_BLOCK = 1e-12  # relative Frobenius per block, oracle vs dense
TOL_LD = 1e-12     # absolute log-det error per diagonal block


# ------------------------------------------------------------------ dense
@pytest.mark.parametrize("B,L,b", [(1, 1, 3), (2, 2, 1), (3, 3, 2), (2, 8, 4), (1, 8, 3),
                                   (2, 5, 8), (1, 30, 1), (1, 12, 5)])
def test_chain_dense(orc, gen, B, L, b):
    d, l = gen.chain(B, L, b, seed=11)
    Gd, Gl, ld, info = orc.chain(d, l)
    assert np.all(info == 0)
    for m in range(B):
        Rd, Rl, Rld, sign = pins.dense_chain_blocks(d[m], l[m])
        assert sign == 1
        assert pins.rel_fro(Gd[m], Rd).max() < TOL_BLOCK
        if L > 1:
            assert pins.rel_fro(Gl[m], Rl).max() < TOL_BLOCK
        assert abs(ld[m] - Rld) < TOL_LD * L


def test_chain_quickstart_example(orc, gen):
    """The Quickstart's chain example: 8 blocks of size 4, seed 0, diagonal
    load 2.0, checked against the dense inverse at atol 1e-10 as the page does."""
    d, l = gen.chain(1, 8, 4, seed=0, diag_load=2.0)
    Gd, Gl, ld, info = orc.chain(d, l)
    Rd, Rl, Rld, _ = pins.dense_chain_blocks(d[0], l[0])
    assert info[0] == 0
    assert np.allclose(Gd[0], Rd, atol=1e-10, rtol=0)
    assert np.allclose(Gl[0], Rl, atol=1e-10, rtol=0)
    assert abs(ld[0] - Rld) < 1e-10


@pytest.mark.parametrize("B,K,b", [(1, 0, 3), (2, 1, 2), (2, 5, 3), (1, 16, 4), (2, 7, 1),
                                   (1, 9, 6)])
def test_star_dense(orc, gen, B, K, b):
    c, lv, cp = gen.star(B, K, b, seed=5)
    Gc, Gl, Gx, ld, info = orc.star(c, lv, cp)
    assert np.all(info == 0)
    for m in range(B):
        Rc, Rl, Rx, Rld, sign = pins.dense_star_blocks(c[m], lv[m], cp[m])
        assert pins.rel_fro(Gc[m], Rc) < TOL_BLOCK
        if K:
            assert pins.rel_fro(Gl[m], Rl).max() < TOL_BLOCK
            assert pins.rel_fro(Gx[m], Rx).max() < TOL_BLOCK
        assert abs(ld[m] - Rld) < TOL_LD * (K + 1)


def _permuted_tree(gen, n, seed):
    """A random tree relabelled by a random permutation: the root is not node
    0 and parents may have larger indices than their children."""
    rng = np.random.default_rng(seed)
    p0 = gen.random_recursive_tree(n, seed)
    perm = rng.permutation(n)  # new label of old node v is perm[v]
    p = np.empty(n, np.int32)
    for v in range(n):
        p[perm[v]] = -1 if p0[v] < 0 else perm[p0[v]]
    return p


@pytest.mark.parametrize("topo,n,b", [("random", 1, 3), ("random", 2, 2), ("random", 30, 3),
                                      ("path", 12, 2), ("star", 10, 3), ("balanced", 31, 2),
                                      ("permuted", 40, 3), ("random", 60, 1),
                                      ("balanced3", 40, 4)])
def test_tree_dense(orc, gen, topo, n, b):
    parent = {"random": lambda: gen.random_recursive_tree(n, 3),
              "path": lambda: gen.path_tree(n),
              "star": lambda: gen.star_tree(n),
              "balanced": lambda: gen.balanced_tree(n, 2),
              "balanced3": lambda: gen.balanced_tree(n, 3),
              "permuted": lambda: _permuted_tree(gen, n, 9)}[topo]()
    d, e = gen.tree(parent, b, seed=4)
    Gd, Ge, ld, info = orc.tree(parent, d, e)
    assert info == 0
    Rd, Re, Rld, sign = pins.dense_tree_blocks(parent, d, e)
    assert pins.rel_fro(Gd, Rd).max() < TOL_BLOCK
    root = int(np.where(parent < 0)[0][0])
    nonroot = np.arange(n) != root
    if n > 1:
        assert pins.rel_fro(Ge[nonroot], Re[nonroot]).max() < TOL_BLOCK
    assert np.all(Ge[root] == 0.0)
    assert abs(ld - Rld) < TOL_LD * n


# ------------------------------------------------------------ closed forms
def test_golden_laplacian3(orc):
    """Hand-derived 3x3 example stored under tests/golden/."""
    rows = {}
    with open(os.path.join(GOLDEN, "laplacian3_inverse.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, idx, val = line.split()
            rows[(kind, idx)] = float(Fraction(val))
    d = np.array([[[[2.0]], [[2.0]], [[2.0]]]])
    l = np.array([[[[-1.0]], [[-1.0]]]])
    Gd, Gl, ld, info = orc.chain(d, l)
    for i in range(3):
        assert abs(Gd[0, i, 0, 0] - rows[("diag", str(i))]) < 1e-15
    for i in range(2):
        assert abs(Gl[0, i, 0, 0] - rows[("lower", str(i))]) < 1e-15
    assert abs(ld[0] - np.log(rows[("det", "-")])) < 1e-15


@pytest.mark.parametrize("L", [1, 2, 7, 100, 1000])
def test_chain_laplacian_closed_form(orc, L):
    d = np.full((1, L, 1, 1), 2.0)
    l = np.full((1, L - 1, 1, 1), -1.0)
    Gd, Gl, ld, info = orc.chain(d, l)
    Ed, El, Eld = pins.laplacian_chain_exact(L)
    assert np.abs(Gd[0, :, 0, 0] - Ed).max() <= 1e-13 * L * max(1.0, Ed.max())
    if L > 1:
        assert np.abs(Gl[0, :, 0, 0] - El).max() <= 1e-13 * L * max(1.0, El.max())
    assert abs(ld[0] - Eld) < 1e-13 * L


@pytest.mark.parametrize("L,seed", [(2, 0), (5, 1), (20, 2), (60, 3)])
def test_chain_usmani_closed_form(orc, L, seed):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(L - 1)
    a = 2.0 + np.abs(np.r_[0.0, c]) + np.abs(np.r_[c, 0.0]) + rng.random(L)
    d = a.reshape(1, L, 1, 1)
    l = c.reshape(1, L - 1, 1, 1)
    Gd, Gl, ld, info = orc.chain(d, l)
    Ed, El, Eld = pins.usmani_chain_exact(a, c)
    assert np.abs(Gd[0, :, 0, 0] / Ed - 1).max() < 1e-13
    assert np.abs(Gl[0, :, 0, 0] - El).max() < 1e-13 * np.abs(El).max()
    assert abs(ld[0] - Eld) < 1e-13 * L


@pytest.mark.parametrize("L,b", [(5, 3), (64, 4), (2000, 2), (300, 8)])
def test_chain_kronecker_closed_form(orc, L, b):
    rng = np.random.default_rng(L + b)
    M = pins.random_spd(b, rng)
    diag, lower, Ed, El, Eld = pins.kron_chain(L, M)
    Gd, Gl, ld, info = orc.chain(diag[None], lower[None])
    scale = np.abs(Ed).max()
    assert np.abs(Gd[0] - Ed).max() < 1e-12 * L * scale
    assert np.abs(Gl[0] - El).max() < 1e-12 * L * scale
    assert abs(ld[0] - Eld) < 1e-12 * L * b


@pytest.mark.parametrize("K,seed", [(1, 0), (8, 1), (200, 2)])
def test_star_arrowhead_closed_form(orc, K, seed):
    rng = np.random.default_rng(seed)
    f = rng.standard_normal(K)
    dl = 1.0 + np.abs(f) + rng.random(K)
    a0 = 1.0 + np.abs(f).sum() + rng.random()
    Gc, Gl, Gx, ld, info = orc.star(np.array([[[a0]]]), dl.reshape(1, K, 1, 1),
                                    f.reshape(1, K, 1, 1))
    E0, Ej, Ex, Eld = pins.arrowhead_exact(a0, dl, f)
    assert abs(Gc[0, 0, 0] / E0 - 1) < 1e-13
    assert np.abs(Gl[0, :, 0, 0] / Ej - 1).max() < 1e-13
    assert np.abs(Gx[0, :, 0, 0] / Ex - 1).max() < 1e-12
    assert abs(ld[0] - Eld) < 1e-13 * (K + 1)


def test_star_kronecker_closed_form(orc):
    """A = T (x) M with T a scalar arrowhead: G = T^-1 (x) M^-1 blockwise."""
    rng = np.random.default_rng(8)
    K, b = 12, 3
    f = rng.standard_normal(K)
    dl = 1.0 + np.abs(f) + rng.random(K)
    a0 = 1.0 + np.abs(f).sum()
    M = pins.random_spd(b, rng)
    Minv = np.linalg.inv(M)
    center = (a0 * M)[None]
    leaves = (dl[:, None, None] * M)[None]
    coupling = (f[:, None, None] * M)[None]
    Gc, Gl, Gx, ld, info = orc.star(center, leaves, coupling)
    E0, Ej, Ex, Eld = pins.arrowhead_exact(a0, dl, f)
    assert np.abs(Gc[0] - E0 * Minv).max() < 1e-13 * abs(E0) * np.abs(Minv).max()
    assert np.abs(Gl[0] - Ej[:, None, None] * Minv).max() < 1e-12
    assert np.abs(Gx[0] - Ex[:, None, None] * Minv).max() < 1e-12
    assert abs(ld[0] - (b * Eld + (K + 1) * np.linalg.slogdet(M)[1])) < 1e-12 * (K + 1) * b


def test_tree_kronecker_closed_form(orc, gen):
    """A = T (x) M with T a scalar tree-structured SPD matrix.  The expected
    blocks come from a dense numpy inverse of the SCALAR matrix T only, so the
    block algebra and edge orientation are pinned independently."""
    rng = np.random.default_rng(3)
    n, b = 80, 3
    parent = gen.random_recursive_tree(n, 2)
    t_edge = rng.standard_normal(n)
    t_edge[0] = 0.0
    t_diag = 1.0 + rng.random(n)
    for v in range(1, n):
        t_diag[v] += abs(t_edge[v])
        t_diag[parent[v]] += abs(t_edge[v])
    T = np.diag(t_diag)
    for v in range(1, n):
        T[parent[v], v] = T[v, parent[v]] = t_edge[v]
    Ti = np.linalg.inv(T)
    M = pins.random_spd(b, rng)
    Minv = np.linalg.inv(M)
    Gd, Ge, ld, info = orc.tree(parent, t_diag[:, None, None] * M, t_edge[:, None, None] * M)
    for v in range(n):
        assert np.abs(Gd[v] - Ti[v, v] * Minv).max() < 1e-12
        if v:
            assert np.abs(Ge[v] - Ti[parent[v], v] * Minv).max() < 1e-12
    Eld = b * np.linalg.slogdet(T)[1] + n * np.linalg.slogdet(M)[1]
    assert abs(ld - Eld) < 1e-12 * n * b
