"""The tree schedule recorded as one HIP graph (selinv_tree_graph_*).

Every replay must reproduce, bit for bit, the eager call on the same inputs
(same kernels, same fixed summation orders), and the eager results are
checked against the float64 oracle.  Replays are interleaved with input
updates, eager library calls and synchronisations, and a failing input is
followed by a good one, so state left in the workspace by one replay
cannot leak into the next.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import pins
import spdgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"f64": torch.float64, "f32": torch.float32}
TOL = {torch.float64: 1e-10, torch.float32: 2e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ssa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_spd_selected_amd as m
    m.lib()  # fail loudly if not built
    return m


def _to(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dt)


def _same(a, b):
    return torch.equal(a, b) or bool(torch.isnan(a).all() and torch.isnan(b).all())


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("n,b", [(2000, 8), (300, 5), (1, 3), (150, 12)])
def test_tree_graph_replays(ssa, n, b, dt):
    dt = DT[dt]
    parent = spdgen.random_recursive_tree(n, 4)
    inputs = [spdgen.tree(parent, b, seed=s) for s in (1, 2, 3)]
    say("tree graph n=%d b=%d %s" % (n, b, dt))
    diag = _to(inputs[0][0], dt)
    edge = _to(inputs[0][1], dt)
    g = ssa.tree_graph(parent, diag, edge)
    plan = ssa.tree_plan(parent, b, dt, DEV)
    if b <= 8:  # init, one dataflow collect, one dataflow distribute (none for n = 1), 2 reductions
        assert g.nodes == (5 if n > 1 else 4)
    else:  # one collect launch per level, one distribute launch per level below the root
        assert g.nodes >= 2 * plan.levels - 1
    # the eager results of the first input set against the oracle
    Ed, Ee, Eld = ssa.tree(parent, diag, edge)
    torch.cuda.synchronize()
    d64 = inputs[0][0].astype(np.float32).astype(np.float64) if dt == torch.float32 \
        else inputs[0][0]
    e64 = inputs[0][1].astype(np.float32).astype(np.float64) if dt == torch.float32 \
        else inputs[0][1]
    Od, Oe, Old, _ = oracle.tree(parent, d64, e64)
    assert float(pins.rel_fro(Ed.double().cpu().numpy(), Od).max()) <= TOL[dt]
    for rep in range(6):
        d, e = inputs[rep % 3]
        g.diag.copy_(_to(d, dt))
        g.edge.copy_(_to(e, dt))
        Gd, Ge, ld = g.launch()
        Ed, Ee, Eld, Einfo = ssa.tree(parent, _to(d, dt), _to(e, dt), return_info=True)
        torch.cuda.synchronize()
        assert torch.equal(Gd, Ed) and torch.equal(Ge, Ee), "replay %d differs" % rep
        assert _same(ld, Eld) and int(g.info) == int(Einfo) == 0


def test_tree_graph_failure_then_recovery(ssa):
    """A non-PD input replayed through the graph reports info and NaN log det
    as the eager call does; the next replay on a good input is clean."""
    parent = spdgen.random_recursive_tree(400, 6)
    d, e = spdgen.tree(parent, 4, seed=2)
    diag, edge = _to(d, torch.float64), _to(e, torch.float64)
    g = ssa.tree_graph(parent, diag, edge)
    bad = d.copy()
    bad[17] = -np.eye(4)
    for src, want_fail in ((bad, True), (d, False), (bad, True), (d, False)):
        g.diag.copy_(_to(src, torch.float64))
        Gd, Ge, ld = g.launch()
        Ed, Ee, Eld, Einfo = ssa.tree(parent, _to(src, torch.float64), edge, return_info=True)
        torch.cuda.synchronize()
        assert int(g.info) == int(Einfo)
        assert (int(g.info) != 0) == want_fail
        assert _same(ld, Eld)
        if not want_fail:
            assert torch.equal(Gd, Ed) and torch.equal(Ge, Ee)


def test_tree_graph_workload_b8_random(ssa):
    """The random recursive tree of 262144 nodes (seed 1), b = 8, float64:
    two replays equal the eager call bit for bit."""
    parent = spdgen.random_recursive_tree(262144, 1)
    d, e = spdgen.tree(parent, 8, seed=1)
    diag, edge = _to(d, torch.float64), _to(e, torch.float64)
    g = ssa.tree_graph(parent, diag, edge)
    Ed, Ee, Eld = ssa.tree(parent, diag, edge)
    for _ in range(2):
        Gd, Ge, ld = g.launch()
        torch.cuda.synchronize()
        assert torch.equal(Gd, Ed) and torch.equal(Ge, Ee) and _same(ld, Eld)
