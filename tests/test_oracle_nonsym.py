"""Pins for the oracle's non-symmetric ladder (the gabp-sparse-inv page's
non-symmetric chain, i.e. the block lower-bidiagonal selected inverse, and the
non-symmetric tree with independent directed edge blocks).

Independent references:
  * numpy's dense inverse of the assembled matrix, read on the pattern;
  * the symmetric case (up = E, down = E^T, symmetric diagonal blocks) must
    reproduce the SPD tree oracle, which has its own pins;
  * planted mistakes must break the dense pin.
"""
import os
import re
import tempfile

import numpy as np
import pytest

import oracle
import spdgen


def blk(M, r, c, b):
    return M[r * b:(r + 1) * b, c * b:(c + 1) * b]


@pytest.mark.parametrize("L,b", [(1, 3), (2, 1), (7, 4), (12, 2)])
def test_bidiag_dense(L, b):
    d, l = spdgen.nonsym_bidiag(3, L, b, seed=L + b)
    Gd, Gl, info = oracle.bidiag(d, l)
    assert (info == 0).all()
    for m in range(3):
        Ai = np.linalg.inv(spdgen.to_dense_bidiag(d[m], l[m]))
        scale = np.abs(Ai).max()
        for i in range(L):
            assert np.abs(Gd[m, i] - blk(Ai, i, i, b)).max() <= 1e-13 * scale
        for i in range(L - 1):
            assert np.abs(Gl[m, i] - blk(Ai, i + 1, i, b)).max() <= 1e-13 * scale


def _trees(n):
    perm = np.random.default_rng(3).permutation(n)
    p0 = spdgen.random_recursive_tree(n, 5)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return {"random": spdgen.random_recursive_tree(n, 2), "path": spdgen.path_tree(n),
            "star": spdgen.star_tree(n), "balanced": spdgen.balanced_tree(n, 2), "perm": p}


@pytest.mark.parametrize("kind", ["random", "path", "star", "balanced", "perm"])
@pytest.mark.parametrize("b", [1, 3])
def test_nonsym_tree_dense(kind, b):
    n = 19
    parent = _trees(n)[kind]
    d, u, w = spdgen.nonsym_tree(parent, b, seed=n + b)
    Gd, Gu, Gw, info = oracle.nonsym_tree(parent, d, u, w)
    assert info == 0
    Ai = np.linalg.inv(spdgen.to_dense_nonsym_tree(parent, d, u, w))
    scale = np.abs(Ai).max()
    for v in range(n):
        assert np.abs(Gd[v] - blk(Ai, v, v, b)).max() <= 1e-13 * scale
        p = int(parent[v])
        if p >= 0:
            assert np.abs(Gu[v] - blk(Ai, p, v, b)).max() <= 1e-13 * scale
            assert np.abs(Gw[v] - blk(Ai, v, p, b)).max() <= 1e-13 * scale
        else:
            assert not Gu[v].any() and not Gw[v].any()


def test_symmetric_case_is_the_spd_tree():
    parent = spdgen.random_recursive_tree(30, 7)
    d, e = spdgen.tree(parent, 3, seed=1)
    Gd, Gu, Gw, info = oracle.nonsym_tree(parent, d, e, np.swapaxes(e, -1, -2).copy())
    Sd, Se, _, _ = oracle.tree(parent, d, e)
    assert info == 0
    assert np.abs(Gd - Sd).max() <= 1e-12 * np.abs(Sd).max()
    assert np.abs(Gu - Se).max() <= 1e-12 * np.abs(Se).max()
    assert np.abs(Gw - np.swapaxes(Se, -1, -2)).max() <= 1e-12 * np.abs(Se).max()


def test_breakdown_reports_the_block():
    d, l = spdgen.nonsym_bidiag(2, 5, 2, seed=3)
    d[1, 3] = 0.0
    Gd, Gl, info = oracle.bidiag(d, l)
    assert list(info) == [0, 4] and np.isnan(Gd[1]).all() and np.isfinite(Gd[0]).all()
    parent = spdgen.random_recursive_tree(20, 1)
    dd, u, w = spdgen.nonsym_tree(parent, 2, seed=1)
    dd[9] = 0.0
    _, _, _, info = oracle.nonsym_tree(parent, dd, u, w)
    assert info == 10  # the only breakdown


MUTANTS = [
    ("collect order", r"matmul\(b, up \+ v \* bb, T, T2\);              /\* up_v S_v\^\{-1\} down_v \*/",
     "matmul(b, T, up + v * bb, T2);"),
    ("G_up sign", r"G_up\[v \* bb \+ e\] = -T2\[e\];", "G_up[v * bb + e] = T2[e];"),
    ("G_diag drops term", r"G_diag\[v \* bb \+ e\] = Sv\[e\] \+ T3\[e\];", "G_diag[v * bb + e] = Sv[e];"),
    ("bidiag order", r"matmul\(b, Gd \+ \(i \+ 1\) \* bb, T, Gl \+ i \* bb\);",
     "matmul(b, T, Gd + (i + 1) * bb, Gl + i * bb);"),
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
        b = 3
        d, l = spdgen.nonsym_bidiag(1, 6, b, seed=2)
        Gd, Gl, _ = oracle.bidiag(d, l, lib=lib)
        Ai = np.linalg.inv(spdgen.to_dense_bidiag(d[0], l[0]))
        bad = any(np.abs(Gl[0, i] - blk(Ai, i + 1, i, b)).max() > 1e-8 for i in range(5))
        parent = spdgen.random_recursive_tree(12, 3)
        dd, u, w = spdgen.nonsym_tree(parent, b, seed=5)
        Td, Tu, Tw, _ = oracle.nonsym_tree(parent, dd, u, w, lib=lib)
        Ti = np.linalg.inv(spdgen.to_dense_nonsym_tree(parent, dd, u, w))
        for v in range(12):
            p = int(parent[v])
            bad |= np.abs(Td[v] - blk(Ti, v, v, b)).max() > 1e-8
            if p >= 0:
                bad |= np.abs(Tu[v] - blk(Ti, p, v, b)).max() > 1e-8
        assert bad, name
