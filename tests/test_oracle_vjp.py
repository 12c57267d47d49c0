"""Pins for the oracle's vector-Jacobian product (reverse mode of the collect
and distribute passes; the page's "analytic two-pass backward" of the
differentiable selected inverse).

Independent references:
  * the dense closed form.  G = A^-1 gives dG = -G dA G, so for a loss with
    cotangent Gbar on the selected blocks of G and lbar on log det A,
        Abar = -G Gbar G + lbar G            (G symmetric),
    and for symmetric diagonal perturbations and edge blocks that appear in
    A twice (E at (p, v), E^T at (v, p)):
        Dbar_v = sym(Abar_vv),   Ebar_v = Abar_{p,v} + Abar_{v,p}^T;
  * central finite differences of the forward oracle (no VJP code involved);
  * planted mistakes in the reverse passes must break the closed-form pin.
"""
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import spdgen

rng = np.random.default_rng(20260)


def sym(M):
    return 0.5 * (M + np.swapaxes(M, -1, -2))


def dense_vjp(A, blocks_d, blocks_e, gd, ge, lbar, b):
    """Abar = -G Gbar G + lbar G with Gbar placed at the selected blocks.
    blocks_d: list of v (block index) for each diagonal cotangent;
    blocks_e: list of (p, v) for each edge cotangent (on G_{p,v})."""
    G = np.linalg.inv(A)
    Gbar = np.zeros_like(A)
    for k, v in enumerate(blocks_d):
        Gbar[v * b:(v + 1) * b, v * b:(v + 1) * b] += sym(gd[k])
    for k, (p, v) in enumerate(blocks_e):
        Gbar[p * b:(p + 1) * b, v * b:(v + 1) * b] += ge[k]
    return -G @ Gbar @ G + lbar * G


def blk(M, r, c, b):
    return M[r * b:(r + 1) * b, c * b:(c + 1) * b]


def rel(a, ref):
    return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-300))


@pytest.mark.parametrize("L,b", [(1, 3), (2, 1), (5, 3), (9, 4), (12, 2)])
def test_chain_vjp_dense(L, b):
    d, l = spdgen.chain(3, L, b, seed=L * 10 + b)
    gd = rng.standard_normal(d.shape)
    gl = rng.standard_normal(l.shape)
    lb = rng.standard_normal(3)
    db, lbar, st = oracle.chain_vjp(d, l, gd, gl, lb)
    assert (st == 0).all()
    for m in range(3):
        A = spdgen.to_dense_chain(d[m], l[m])
        Ab = dense_vjp(A, list(range(L)), [(i + 1, i) for i in range(L - 1)], gd[m], gl[m],
                       lb[m], b)
        Db = np.stack([sym(blk(Ab, i, i, b)) for i in range(L)])
        assert rel(db[m], Db) < 1e-11
        if L > 1:
            Cb = np.stack([blk(Ab, i + 1, i, b) + blk(Ab, i, i + 1, b).T for i in range(L - 1)])
            assert rel(lbar[m], Cb) < 1e-11
        assert np.allclose(db[m], np.swapaxes(db[m], -1, -2), atol=0)


@pytest.mark.parametrize("K,b", [(0, 2), (1, 3), (6, 2), (11, 3)])
def test_star_vjp_dense(K, b):
    c, lv, cp = spdgen.star(2, K, b, seed=K + 7)
    gc = rng.standard_normal(c.shape)
    gl = rng.standard_normal(lv.shape)
    gx = rng.standard_normal(cp.shape)
    lb = rng.standard_normal(2)
    cb, lvb, cpb = oracle.star_vjp(c, lv, cp, gc, gl, gx, lb)
    for m in range(2):
        A = spdgen.to_dense_star(c[m], lv[m], cp[m])
        # G_cross[j] = G_{j+1,0}
        Ab = dense_vjp(A, list(range(K + 1)), [(j + 1, 0) for j in range(K)],
                       np.concatenate([gc[m][None], gl[m]]), gx[m], lb[m], b)
        assert rel(cb[m], sym(blk(Ab, 0, 0, b))) < 1e-11
        for j in range(K):
            assert rel(lvb[m, j], sym(blk(Ab, j + 1, j + 1, b))) < 1e-11
            # coupling[j] = A_{j+1,0}
            assert rel(cpb[m, j], blk(Ab, j + 1, 0, b) + blk(Ab, 0, j + 1, b).T) < 1e-11


def permuted_tree(n, seed):
    """A random recursive tree relabelled at random (the root is not node 0)."""
    par = spdgen.random_recursive_tree(n, seed)
    perm = np.random.default_rng(seed).permutation(n)
    out = np.empty(n, np.int32)
    for v in range(n):
        out[perm[v]] = -1 if par[v] < 0 else perm[par[v]]
    return out


@pytest.mark.parametrize("kind,n,b", [("random", 17, 3), ("balanced", 15, 2), ("path", 6, 2),
                                      ("star", 7, 3), ("random", 1, 2), ("permuted", 13, 2)])
def test_tree_vjp_dense(kind, n, b):
    parent = {"random": lambda: spdgen.random_recursive_tree(n, 3),
              "balanced": lambda: spdgen.balanced_tree(n, 3),
              "path": lambda: spdgen.path_tree(n),
              "star": lambda: spdgen.star_tree(n),
              "permuted": lambda: permuted_tree(n, 5)}[kind]()
    if kind == "permuted":
        assert parent[0] != -1
    d, e = spdgen.tree(parent, b, seed=n)
    gd = rng.standard_normal(d.shape)
    ge = rng.standard_normal(e.shape)
    lb = float(rng.standard_normal())
    db, eb = oracle.tree_vjp(parent, d, e, gd, ge, lb)
    A = spdgen.to_dense_tree(parent, d, e)
    edges = [(int(parent[v]), v) for v in range(n) if parent[v] >= 0]
    Ab = dense_vjp(A, list(range(n)), edges, gd, np.stack([ge[v] for _, v in edges])
                   if edges else np.zeros((0, b, b)), lb, b)
    for v in range(n):
        assert rel(db[v], sym(blk(Ab, v, v, b))) < 1e-11
        p = int(parent[v])
        if p >= 0:
            assert rel(eb[v], blk(Ab, p, v, b) + blk(Ab, v, p, b).T) < 1e-11
        else:
            assert not eb[v].any()


def test_chain_vjp_finite_differences():
    """d/dt of L(A + t dA) by central differences of the forward oracle."""
    L, b = 6, 3
    d, l = spdgen.chain(1, L, b, seed=4)
    Wd = rng.standard_normal(d.shape)
    Wl = rng.standard_normal(l.shape)
    w = 0.37

    def loss(dd, ll):
        Gd, Gl, ld, info = oracle.chain(dd, ll)
        assert info[0] == 0
        return float((Wd * Gd).sum() + (Wl * Gl).sum() + w * ld[0])

    dD = sym(rng.standard_normal(d.shape))
    dC = rng.standard_normal(l.shape)
    h = 1e-5
    fd = (loss(d + h * dD, l + h * dC) - loss(d - h * dD, l - h * dC)) / (2 * h)
    db, lbar, _ = oracle.chain_vjp(d, l, Wd, Wl, [w])
    an = float((db * dD).sum() + (lbar * dC).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_tree_vjp_finite_differences():
    n, b = 12, 2
    parent = spdgen.random_recursive_tree(n, 9)
    d, e = spdgen.tree(parent, b, seed=9)
    Wd = rng.standard_normal(d.shape)
    We = rng.standard_normal(e.shape)
    We[parent < 0] = 0.0
    w = -0.8

    def loss(dd, ee):
        Gd, Ge, ld, info = oracle.tree(parent, dd, ee)
        assert info == 0
        return float((Wd * Gd).sum() + (We * Ge).sum() + w * ld)

    dD = sym(rng.standard_normal(d.shape))
    dE = rng.standard_normal(e.shape)
    dE[parent < 0] = 0.0
    h = 1e-5
    fd = (loss(d + h * dD, e + h * dE) - loss(d - h * dD, e - h * dE)) / (2 * h)
    db, eb = oracle.tree_vjp(parent, d, e, Wd, We, w)
    an = float((db * dD).sum() + (eb * dE).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_vjp_of_logdet_is_the_selected_inverse():
    """With only lbar = 1: Dbar = G_diag and Ebar = 2 G_edge (d log det = <A^-1, dA>)."""
    d, l = spdgen.chain(2, 7, 3, seed=2)
    Gd, Gl, _, _ = oracle.chain(d, l)
    db, lbar, _ = oracle.chain_vjp(d, l, np.zeros_like(d), np.zeros_like(l), [1.0, 1.0])
    assert rel(db, sym(Gd)) < 1e-12 and rel(lbar, 2 * Gl) < 1e-12


def test_chain_vjp_not_pd_status():
    d, l = spdgen.chain(2, 5, 2, seed=3)
    d[1, 2] = -np.eye(2)
    db, lbar, st = oracle.chain_vjp(d, l, np.ones_like(d), np.ones_like(l), [1.0, 1.0])
    assert list(st) == [0, 3] and np.isnan(db[1]).all() and np.isfinite(db[0]).all()


# Planted mistakes in the reverse passes: each must fail the dense pin.
MUTANTS = [
    ("GG_p += V_bar X^T", r"add_to\(bb, GG \+ p \* bb, T, 1\.0\);", "add_to(bb, GG + p * bb, T, -1.0);"),
    ("drop X_bar += G_pp^T V_bar",
     r"mm_tn\(b, Gp, Vb, T\);\s+/\* X_bar \+= G_pp\^T V_bar  \*/\n\s+add_to\(bb, Xb \+ v \* bb, T, 1\.0\);",
     "mm_tn(b, Gp, Vb, T);"),
    ("edge cotangent sign", r"add_to\(bb, Vb, ge_bar \+ v \* bb, -1\.0\);",
     "add_to(bb, Vb, ge_bar + v * bb, 1.0);"),
    ("M_bar sign", r"Mb\[e\] = -Sbp\[e\];", "Mb[e] = Sbp[e];"),
    ("logdet term transposed sign", r"-Sbv\[r \* b \+ c\] \+ ld_bar", "Sbv[r * b + c] + ld_bar"),
]


@pytest.mark.parametrize("name,pat,rep", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_vjp_mutants_are_caught(name, pat, rep):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    mutated, k = re.subn(pat, rep, src)
    assert k == 1, "mutation site not found: " + name
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "m.c")
        so = os.path.join(td, "m.so")
        open(c, "w").write(mutated)
        oracle.compile_oracle(c, so)
        lib = oracle.load(so)
        L, b = 6, 3
        d, l = spdgen.chain(1, L, b, seed=11)
        gd = rng.standard_normal(d.shape)
        gl = rng.standard_normal(l.shape)
        db, lbar, st = oracle.chain_vjp(d, l, gd, gl, [0.5], lib=lib)
        A = spdgen.to_dense_chain(d[0], l[0])
        Ab = dense_vjp(A, list(range(L)), [(i + 1, i) for i in range(L - 1)], gd[0], gl[0], 0.5, b)
        Db = np.stack([sym(blk(Ab, i, i, b)) for i in range(L)])
        Cb = np.stack([blk(Ab, i + 1, i, b) + blk(Ab, i, i + 1, b).T for i in range(L - 1)])
        assert rel(db[0], Db) > 1e-6 or rel(lbar[0], Cb) > 1e-6, name
