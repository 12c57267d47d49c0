"""The seeded input generator: Philox known answers, determinism, per-matrix
regeneration, exact symmetry and the Gershgorin SPD guarantee."""
import os

import numpy as np
import pytest

from conftest import GOLDEN


def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_philox_known_answers(gen, ctr, key, expect):
    assert list(gen.philox4x32_10(ctr, key)) == expect


def test_normals_moments(gen):
    z = np.array([gen.normal(7, 0, m, e) for m in range(40) for e in range(1000)])
    assert abs(z.mean()) < 0.02
    assert abs(z.var() - 1.0) < 0.03
    # both Box-Muller outputs of a pair are used and differ
    assert gen.normal(7, 0, 0, 0) != gen.normal(7, 0, 0, 1)


def test_chain_regenerates_single_matrix(gen):
    d, l = gen.chain(5, 6, 3, seed=3)
    d2, l2 = gen.chain(1, 6, 3, seed=3, m0=4)
    assert np.array_equal(d[4], d2[0]) and np.array_equal(l[4], l2[0])
    d3, l3 = gen.chain(5, 6, 3, seed=3)
    assert np.array_equal(d, d3) and np.array_equal(l, l3)
    assert not np.array_equal(d[0], d[1])  # distinct values per chain
    d4, _ = gen.chain(5, 6, 3, seed=4)
    assert not np.array_equal(d, d4)


def test_star_regenerates_single_matrix(gen):
    c, lv, cp = gen.star(4, 7, 2, seed=2)
    c2, lv2, cp2 = gen.star(1, 7, 2, seed=2, m0=3)
    assert np.array_equal(c[3], c2[0]) and np.array_equal(lv[3], lv2[0])
    assert np.array_equal(cp[3], cp2[0])


def test_diagonal_blocks_exactly_symmetric(gen):
    d, _ = gen.chain(3, 5, 7)
    assert np.array_equal(d, np.swapaxes(d, -1, -2))
    c, lv, _ = gen.star(2, 5, 5)
    assert np.array_equal(c, np.swapaxes(c, -1, -2))
    assert np.array_equal(lv, np.swapaxes(lv, -1, -2))
    p = gen.random_recursive_tree(40, 1)
    dd, e = gen.tree(p, 4)
    assert np.array_equal(dd, np.swapaxes(dd, -1, -2))
    assert np.all(e[0] == 0.0)


def test_offdiagonal_scale(gen):
    _, l = gen.chain(64, 8, 16)
    assert abs(l.std() - 0.25) < 0.01  # N(0, 1/b) -> std 1/sqrt(b)


@pytest.mark.parametrize("load", [2.0, 1.0, 0.5])
def test_gershgorin_lambda_min(gen, load):
    for b, L in [(1, 30), (3, 9), (4, 8), (8, 6)]:
        d, l = gen.chain(3, L, b, seed=1, diag_load=load)
        for m in range(3):
            lam = np.linalg.eigvalsh(gen.to_dense_chain(d[m], l[m])).min()
            assert lam >= load - 1e-12
    c, lv, cp = gen.star(2, 20, 3, diag_load=load)
    for m in range(2):
        assert np.linalg.eigvalsh(gen.to_dense_star(c[m], lv[m], cp[m])).min() >= load - 1e-12
    p = gen.random_recursive_tree(60, 5)
    dd, e = gen.tree(p, 3, diag_load=load)
    assert np.linalg.eigvalsh(gen.to_dense_tree(p, dd, e)).min() >= load - 1e-12


def test_random_recursive_tree_shape(gen):
    p = gen.random_recursive_tree(5000, 1)
    assert p[0] == -1
    v = np.arange(1, 5000)
    assert np.all(p[1:] >= 0) and np.all(p[1:] < v)
    # parent uniform over [0, v): mean of parent/v close to 1/2
    assert abs((p[1:] / v).mean() - 0.5) < 0.02
    assert np.array_equal(p, gen.random_recursive_tree(5000, 1))


def test_tree_topologies(gen):
    assert list(gen.path_tree(4)) == [-1, 0, 1, 2]
    assert list(gen.star_tree(4)) == [-1, 0, 0, 0]
    assert list(gen.balanced_tree(7, 2)) == [-1, 0, 0, 1, 1, 2, 2]
