"""The tree level-set schedule (selinv_tree_schedule, the host part of
selinv_tree_plan_create) against brute force on the CPU: depths by walking
up the parent array, levels as contiguous breadth-first ranges, parent
positions, contiguous child ranges in increasing node index, and the
failure ranks of the oracle's elimination order (depth descending, then
index ascending)."""
import numpy as np
import pytest

import spdgen
import sparse_spd_selected_amd as ssa


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(ssa.LIB_PATH):
        ssa.build()


def _depths(parent):
    n = len(parent)
    d = np.full(n, -1, np.int64)
    for v in range(n):
        path, u = [], v
        while u != -1 and d[u] < 0:
            path.append(u)
            u = parent[u]
        base = -1 if u == -1 else d[u]
        for w in reversed(path):
            base += 1
            d[w] = base
    return d


def _perm(p0, seed):
    rng = np.random.default_rng(seed)
    n = len(p0)
    perm = rng.permutation(n)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return p


TOPOLOGIES = {
    "single": lambda: np.array([-1], np.int32),
    "pair": lambda: np.array([1, -1], np.int32),
    "path": lambda: spdgen.path_tree(50),
    "star": lambda: spdgen.star_tree(40),
    "balanced": lambda: spdgen.balanced_tree(127, 2),
    "ternary": lambda: spdgen.balanced_tree(121, 3),
    "random": lambda: spdgen.random_recursive_tree(3000, 4),
    "random_perm": lambda: _perm(spdgen.random_recursive_tree(2000, 5), 6),
    "path_perm": lambda: _perm(spdgen.path_tree(300), 7),
    "workload": lambda: spdgen.random_recursive_tree(262144, 1),
}


@pytest.mark.parametrize("topo", sorted(TOPOLOGIES))
def test_schedule_matches_brute_force(topo):
    parent = np.asarray(TOPOLOGIES[topo](), np.int32)
    n = len(parent)
    sc = ssa.tree_schedule(parent)
    node_at, ppos = sc["node_at"], sc["parent_pos"]
    cb, ce, fr, lo = sc["child_beg"], sc["child_end"], sc["fail_rank"], sc["level_off"]
    depth = _depths(parent)
    H = int(depth.max())
    # a permutation; the root first
    assert sorted(node_at.tolist()) == list(range(n))
    assert parent[node_at[0]] == -1
    pos = np.empty(n, np.int64)
    pos[node_at] = np.arange(n)
    # levels: contiguous ranges of the right depth and size
    assert len(lo) == H + 2 and lo[0] == 0 and lo[-1] == n
    for d in range(H + 1):
        assert (depth[node_at[lo[d]:lo[d + 1]]] == d).all()
        assert lo[d + 1] - lo[d] == int((depth == d).sum())
    # parent positions
    for p in range(n):
        v = node_at[p]
        assert ppos[p] == (-1 if parent[v] < 0 else pos[parent[v]])
    # child ranges: exactly the children, increasing index, in the next level,
    # consecutive from one position to the next
    kids = [[] for _ in range(n)]
    for v in range(n):
        if parent[v] >= 0:
            kids[parent[v]].append(v)
    nxt = 1
    for p in range(n):
        v = node_at[p]
        assert cb[p] == nxt and ce[p] == nxt + len(kids[v])
        assert node_at[cb[p]:ce[p]].tolist() == sorted(kids[v])
        nxt = ce[p]
        if ce[p] > cb[p]:
            assert lo[depth[v] + 1] <= cb[p] and ce[p] <= lo[depth[v] + 2]
    assert nxt == n
    # failure ranks: order (depth descending, index ascending)
    order = sorted(range(n), key=lambda v: (-depth[v], v))
    rank = np.empty(n, np.int64)
    rank[order] = np.arange(n)
    assert (fr == rank[node_at]).all()


@pytest.mark.parametrize("parent", [[-1, -1], [0, 1], [1, 0, -1], [-1, 5], [-1, -2], [0],
                                    [-1, 1], [-1, 2, 1]])
def test_schedule_rejects_invalid_trees(parent):
    with pytest.raises(ssa.SelinvError, match="status 2"):
        ssa.tree_schedule(np.array(parent, np.int32))


def test_schedule_rejects_empty():
    with pytest.raises(ssa.SelinvError, match="status 1"):
        ssa.tree_schedule(np.zeros(0, np.int32))
