"""The product's symbolic analysis of the general sparse SPD path (host C++,
selinv_junction_symbolic) against the oracle's elimination, bit for bit: the
elimination order, the filled pattern S_index and the number of
elimination-tree levels.  Integer work, so the bar is exact equality.  No
GPU needed: the analysis runs on the host."""
import numpy as np
import pytest

import oracle
import spdgen

ssa = pytest.importorskip("sparse_spd_selected_amd")


def levels_from_oracle(n, edge_index, order=None):
    o, ptr, nbr = oracle.eliminate(n, edge_index, order)
    pos = np.empty(n, np.int64)
    pos[o] = np.arange(n)
    level = np.zeros(n, np.int64)
    for s in range(n):
        nb = nbr[ptr[s]:ptr[s + 1]]
        if nb.size:
            p = int(pos[nb].min())
            level[p] = max(level[p], level[s] + 1)
    return int(level.max()) + 1


def check(n, e, order=None):
    P = oracle.filled_pattern(n, e, order)
    o, S, lev = ssa.junction_symbolic(n, e, order)
    assert np.array_equal(o, P["order"])
    assert np.array_equal(S, P["S_index"])
    assert lev == levels_from_oracle(n, e, order)
    return S, lev


@pytest.mark.parametrize("r,c", [(1, 1), (1, 7), (3, 3), (4, 6), (9, 9), (16, 16), (32, 32)])
def test_grids(r, c):
    check(r * c, spdgen.grid_edges(r, c))


def test_grid64_workload_pattern():
    S, lev = check(4096, spdgen.grid_edges(64, 64))
    assert S.shape[1] == 66491


@pytest.mark.parametrize("n,extra,seed", [(20, 30, 1), (60, 100, 2), (200, 150, 3), (7, 21, 4)])
def test_random_graphs(n, extra, seed):
    check(n, spdgen.random_graph_edges(n, extra, seed))


@pytest.mark.parametrize("kind", ["natural", "reversed", "random"])
def test_explicit_orders(kind):
    n = 36
    e = spdgen.grid_edges(6, 6)
    order = {"natural": np.arange(n), "reversed": np.arange(n)[::-1].copy(),
             "random": np.random.default_rng(3).permutation(n)}[kind]
    check(n, e, order)


def test_tree_patterns_have_no_fill():
    for parent in (spdgen.random_recursive_tree(300, 2), spdgen.star_tree(50),
                   spdgen.balanced_tree(127, 2)):
        n = len(parent)
        e = np.array([(max(v, int(parent[v])), min(v, int(parent[v])))
                      for v in range(n) if parent[v] >= 0], np.int32).T.copy()
        S, _ = check(n, e)
        assert S.shape[1] == n - 1


def test_no_edges():
    o, S, lev = ssa.junction_symbolic(5, np.zeros((2, 0), np.int32))
    assert list(o) == [0, 1, 2, 3, 4] and S.shape == (2, 0) and lev == 1


@pytest.mark.parametrize("edges,order", [
    ([[0], [1]], None),                 # i < j
    ([[1, 1], [0, 0]], None),           # repeated edge
    ([[3], [0]], None),                 # out of range (n = 3)
    ([[1], [0]], [0, 0, 1]),            # order is not a permutation
    ([[1], [0]], [0, 1, 5]),
])
def test_bad_patterns_are_rejected(edges, order):
    with pytest.raises(ssa.SelinvError):
        ssa.junction_symbolic(3, np.array(edges, np.int32), order)
