"""Invariants of the selected inverse, checked on the oracle at sizes where a
dense inverse is no longer the check:

* symmetry and positive definiteness of every G_ii (the oracle does not
  mirror, so symmetry is a real test), and the Loewner bound G_ii >= D_i^-1;
* the block-diagonal residual (A A^-1)_ii = I from on-pattern blocks only
  (the "independent residual checks" of the page's Tests section);
* d log det A = tr(A^-1 dA) along a random on-pattern direction (sparsax
  page, "Gradients & the selected inverse": the log-det gradient is the
  selected inverse);
* root invariance (Quickstart section): path trees reproduce the chain, and
  depth-1 trees the star, block for block; re-rooting a tree changes no block;
* failure path: a non-positive-definite pivot is reported, not hidden.
"""
import numpy as np
import pytest

import pins


def _sym_err(G):
    return pins.rel_fro(G, np.swapaxes(G, -1, -2))


def test_chain_invariants(orc, gen):
    d, l = gen.chain(2, 200, 8, seed=21)
    Gd, Gl, ld, info = orc.chain(d, l)
    assert np.all(info == 0)
    assert _sym_err(Gd).max() < 1e-14
    for m in range(2):
        assert np.linalg.eigvalsh(0.5 * (Gd[m] + np.swapaxes(Gd[m], -1, -2))).min() > 0
        Dinv = np.linalg.inv(d[m])
        lw = np.linalg.eigvalsh(0.5 * (Gd[m] - Dinv + np.swapaxes(Gd[m] - Dinv, -1, -2)))
        assert lw.min() > -1e-12 * np.abs(Gd[m]).max()
        assert pins.chain_residual(d[m], l[m], Gd[m], Gl[m]) < 1e-12


def test_star_invariants(orc, gen):
    c, lv, cp = gen.star(2, 300, 6, seed=2)
    Gc, Gl, Gx, ld, info = orc.star(c, lv, cp)
    assert np.all(info == 0)
    assert _sym_err(Gl).max() < 1e-14 and _sym_err(Gc).max() < 1e-14
    for m in range(2):
        assert pins.star_residual(c[m], lv[m], cp[m], Gc[m], Gl[m], Gx[m]) < 1e-12


def test_tree_invariants(orc, gen):
    p = gen.random_recursive_tree(3000, 7)
    d, e = gen.tree(p, 4, seed=3)
    Gd, Ge, ld, info = orc.tree(p, d, e)
    assert info == 0
    assert _sym_err(Gd).max() < 1e-14
    assert pins.tree_residual(p, d, e, Gd, Ge) < 1e-12
    assert np.linalg.eigvalsh(0.5 * (Gd + np.swapaxes(Gd, -1, -2))).min() > 0


def _fd(f, x, E, eps):
    return (f(x + eps * E) - f(x - eps * E)) / (2 * eps)


def test_logdet_gradient_chain(orc, gen):
    rng = np.random.default_rng(0)
    d, l = gen.chain(1, 40, 5, seed=9)
    Gd, Gl, ld, _ = orc.chain(d, l)
    Ed = rng.standard_normal(d.shape)
    Ed = Ed + np.swapaxes(Ed, -1, -2)
    El = rng.standard_normal(l.shape)
    eps = 1e-5
    fd = (orc.chain(d + eps * Ed, l + eps * El)[2][0] -
          orc.chain(d - eps * Ed, l - eps * El)[2][0]) / (2 * eps)
    an = np.sum(Gd * Ed) + 2 * np.sum(Gl * El)  # <G, dA> over both triangles
    assert abs(fd - an) < 1e-7 * max(1.0, abs(an))


def test_logdet_gradient_star(orc, gen):
    rng = np.random.default_rng(1)
    c, lv, cp = gen.star(1, 30, 4, seed=9)
    Gc, Gl, Gx, ld, _ = orc.star(c, lv, cp)
    Ec = rng.standard_normal(c.shape)
    Ec = Ec + np.swapaxes(Ec, -1, -2)
    El = rng.standard_normal(lv.shape)
    El = El + np.swapaxes(El, -1, -2)
    Ex = rng.standard_normal(cp.shape)
    eps = 1e-5
    fd = (orc.star(c + eps * Ec, lv + eps * El, cp + eps * Ex)[3][0] -
          orc.star(c - eps * Ec, lv - eps * El, cp - eps * Ex)[3][0]) / (2 * eps)
    an = np.sum(Gc * Ec) + np.sum(Gl * El) + 2 * np.sum(Gx * Ex)
    assert abs(fd - an) < 1e-7 * max(1.0, abs(an))


def test_logdet_gradient_tree(orc, gen):
    rng = np.random.default_rng(2)
    p = gen.random_recursive_tree(50, 4)
    d, e = gen.tree(p, 3, seed=5)
    Gd, Ge, ld, _ = orc.tree(p, d, e)
    Ed = rng.standard_normal(d.shape)
    Ed = Ed + np.swapaxes(Ed, -1, -2)
    Ee = rng.standard_normal(e.shape)
    Ee[0] = 0
    eps = 1e-5
    fd = (orc.tree(p, d + eps * Ed, e + eps * Ee)[2] -
          orc.tree(p, d - eps * Ed, e - eps * Ee)[2]) / (2 * eps)
    an = np.sum(Gd * Ed) + 2 * np.sum(Ge * Ee)
    assert abs(fd - an) < 1e-7 * max(1.0, abs(an))


# --------------------------------------------------------- root invariance
def test_path_tree_equals_chain(orc, gen):
    """Chain rooted at its last block vs. the same matrix as a path tree
    rooted at node 0: parent[v] = v-1 and edge[v] = A_{v-1,v} = lower[v-1]^T."""
    L, b = 50, 4
    d, l = gen.chain(1, L, b, seed=13)
    Gd, Gl, ld, _ = orc.chain(d, l)
    p = gen.path_tree(L)
    e = np.zeros((L, b, b))
    e[1:] = np.swapaxes(l[0], -1, -2)
    Td, Te, tld, _ = orc.tree(p, d[0], e)
    assert pins.rel_fro(Td, Gd[0]).max() < 1e-13
    assert pins.rel_fro(Te[1:], np.swapaxes(Gl[0], -1, -2)).max() < 1e-13
    assert abs(tld - ld[0]) < 1e-12 * L


def test_depth1_tree_equals_star(orc, gen):
    K, b = 40, 3
    c, lv, cp = gen.star(1, K, b, seed=3)
    Gc, Gl, Gx, ld, _ = orc.star(c, lv, cp)
    p = gen.star_tree(K + 1)
    d = np.concatenate([c, lv[0]])
    e = np.zeros((K + 1, b, b))
    e[1:] = np.swapaxes(cp[0], -1, -2)  # edge[j+1] = A_{0,j+1} = coupling[j]^T
    Td, Te, tld, _ = orc.tree(p, d, e)
    assert pins.rel_fro(Td[0], Gc[0]) < 1e-13
    assert pins.rel_fro(Td[1:], Gl[0]).max() < 1e-13
    assert pins.rel_fro(Te[1:], np.swapaxes(Gx[0], -1, -2)).max() < 1e-13
    assert abs(tld - ld[0]) < 1e-12 * (K + 1)


def _reroot(parent, edge, r):
    """Same matrix, rooted at r: edges on the path r -> old root flip."""
    parent = parent.copy()
    edge = edge.copy()
    path = [r]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    new_parent = parent.copy()
    new_edge = edge.copy()
    new_parent[r] = -1
    new_edge[r] = 0.0
    for child, up in zip(path[:-1], path[1:]):
        new_parent[up] = child                 # `up` now hangs below `child`
        new_edge[up] = edge[child].T           # A_{child,up} = (A_{up,child})^T
    return new_parent, new_edge, path


def test_reroot_invariance(orc, gen):
    n, b = 400, 3
    p = gen.random_recursive_tree(n, 12)
    d, e = gen.tree(p, b, seed=2)
    Gd, Ge, ld, _ = orc.tree(p, d, e)
    r = n - 1
    p2, e2, path = _reroot(p, e, r)
    Gd2, Ge2, ld2, _ = orc.tree(p2, d, e2)
    assert pins.rel_fro(Gd2, Gd).max() < 1e-13
    flipped = set(path[1:])
    for v in range(n):
        if v == r:
            continue
        if v in flipped:
            child = path[path.index(v) - 1]
            assert pins.rel_fro(Ge2[v], Ge[child].T) < 1e-13
        else:
            assert pins.rel_fro(Ge2[v], Ge[v]) < 1e-13
    assert abs(ld2 - ld) < 1e-12 * n


def test_relabel_invariance(orc, gen):
    n, b = 300, 2
    rng = np.random.default_rng(4)
    p = gen.random_recursive_tree(n, 5)
    d, e = gen.tree(p, b, seed=2)
    Gd, Ge, ld, _ = orc.tree(p, d, e)
    perm = rng.permutation(n)
    p2 = np.where(p < 0, -1, perm[np.maximum(p, 0)]).astype(np.int32)
    P2 = np.empty_like(p2)
    P2[perm] = p2
    d2 = np.empty_like(d)
    e2 = np.empty_like(e)
    d2[perm] = d
    e2[perm] = e
    Gd2, Ge2, ld2, _ = orc.tree(P2, d2, e2)
    assert pins.rel_fro(Gd2[perm], Gd).max() < 1e-13
    assert pins.rel_fro(Ge2[perm][1:], Ge[1:]).max() < 1e-13


# --------------------------------------------------------------- failures
@pytest.mark.parametrize("k", [0, 3, 7])
def test_chain_not_pd_reported(orc, gen, k):
    d, l = gen.chain(3, 8, 4, seed=0)
    d[1, k] = -np.eye(4)
    d[2, k] = np.nan
    Gd, Gl, ld, info = orc.chain(d, l)
    assert list(info) == [0, k + 1, k + 1]
    assert np.isnan(ld[1]) and np.isnan(ld[2]) and np.isfinite(ld[0])
    assert np.all(np.isnan(Gd[1])) and np.all(np.isfinite(Gd[0]))


def test_star_not_pd_reported(orc, gen):
    c, lv, cp = gen.star(3, 6, 3, seed=0)
    lv[1, 4] = -np.eye(3)
    c[2] = -np.eye(3)
    *_, ld, info = orc.star(c, lv, cp)
    assert list(info) == [0, 6, 1]


def test_tree_not_pd_reported(orc, gen):
    p = gen.random_recursive_tree(30, 1)
    d, e = gen.tree(p, 3)
    for v in [0, 5, 29]:
        d2 = d.copy()
        d2[v] = -np.eye(3)
        _, _, ld, info = orc.tree(p, d2, e)
        assert info == v + 1 and np.isnan(ld)


def test_tree_validation(orc, gen):
    d, e = gen.tree(gen.path_tree(4), 2)
    for bad in ([-1, 0, -1, 2], [1, 2, 0, -1][:3] + [0], [-1, 0, 9, 1], [-1, 2, 3, 1],
                [0, 0, 1, 2]):
        with pytest.raises(orc.OracleError):
            orc.tree(np.array(bad, np.int32), d, e)
