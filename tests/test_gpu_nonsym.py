"""GPU parity of the non-symmetric ladder (block lower-bidiagonal selected
inverse and the non-symmetric tree) through the C ABI against the oracle
(oracle.bidiag / oracle.nonsym_tree, pinned to dense inverses) on the same
seeded, row-dominant inputs.

Tolerances: relative Frobenius error per block <= 1e-10 (float64) or 2e-4
(float32).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import pins
import spdgen

pytestmark = pytest.mark.gpu

TOL = {torch.float64: 1e-10, torch.float32: 2e-4}
DT = {"f64": torch.float64, "f32": torch.float32}
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ssa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_spd_selected_amd as m
    m.lib()
    return m


def _to(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dt)


def _as_used(x, dt):
    return x.astype(np.float32).astype(np.float64) if dt == torch.float32 else x


def _cmp(name, got, ref, dt):
    err = pins.rel_fro(got.double().cpu().numpy(), ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dt], "%s rel err %.3e > %.1e" % (name, worst, TOL[dt])
    return worst


def run_bidiag(ssa, B, L, b, dt, seed):
    say("bidiag B=%d L=%d b=%d %s" % (B, L, b, dt))
    d, l = spdgen.nonsym_bidiag(B, L, b, seed=seed)
    Gd, Gl, info = ssa.bidiag(_to(d, dt), _to(l, dt), return_info=True)
    torch.cuda.synchronize()
    Od, Ol, Oinfo = oracle.bidiag(_as_used(d, dt), _as_used(l, dt))
    assert np.array_equal(info.cpu().numpy(), Oinfo) and (Oinfo == 0).all()
    e = _cmp("G_diag", Gd, Od, dt)
    if L > 1:
        e = max(e, _cmp("G_lower", Gl, Ol, dt))
    say("  worst rel err %.2e" % e)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L,b", [(1, 1, 3), (2, 2, 1), (3, 9, 4), (2, 12, 16), (2, 5, 32),
                                   (4, 7, 5), (3, 1, 16), (2, 2, 16), (5, 13, 16)])
def test_bidiag_small(ssa, B, L, b, dt):
    run_bidiag(ssa, B, L, b, DT[dt], seed=B + L + b)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_bidiag_workload_b16(ssa, dt):
    """4096 block lower-bidiagonal matrices of 64 blocks of 16, full oracle."""
    run_bidiag(ssa, 4096, 64, 16, DT[dt], seed=0)


def test_bidiag_breakdown(ssa):
    d, l = spdgen.nonsym_bidiag(3, 6, 4, seed=2)
    d[1, 4] = 0.0
    Gd, Gl, info = ssa.bidiag(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    torch.cuda.synchronize()
    assert list(info.cpu().numpy()) == [0, 5, 0]
    assert torch.isnan(Gd[1]).all() and torch.isnan(Gl[1]).all() and torch.isfinite(Gd[0]).all()


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_bidiag_breakdown_b16(ssa, dt):
    """The b = 16 matrix-core kernel reports the first failing block and
    poisons only that matrix."""
    d, l = spdgen.nonsym_bidiag(3, 7, 16, seed=4)
    d[1, 5] = 0.0
    d[1, 6] = 0.0
    Gd, Gl, info = ssa.bidiag(_to(d, DT[dt]), _to(l, DT[dt]), return_info=True)
    torch.cuda.synchronize()
    assert list(info.cpu().numpy()) == [0, 6, 0]
    assert torch.isnan(Gd[1]).all() and torch.isnan(Gl[1]).all()
    assert torch.isfinite(Gd[0]).all() and torch.isfinite(Gl[2]).all()


def _perm_tree(n, seed):
    rng = np.random.default_rng(seed)
    p0 = spdgen.random_recursive_tree(n, seed)
    perm = rng.permutation(n)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return p


def run_nonsym_tree(ssa, parent, b, dt, seed):
    n = len(parent)
    say("nonsym tree n=%d b=%d %s" % (n, b, dt))
    d, u, w = spdgen.nonsym_tree(parent, b, seed=seed)
    Gd, Gu, Gw, info = ssa.nonsym_tree(parent, _to(d, dt), _to(u, dt), _to(w, dt),
                                       return_info=True)
    torch.cuda.synchronize()
    Od, Ou, Ow, Oinfo = oracle.nonsym_tree(parent, _as_used(d, dt), _as_used(u, dt),
                                           _as_used(w, dt))
    assert int(info) == Oinfo == 0
    e = _cmp("G_diag", Gd, Od, dt)
    root = int(np.where(np.asarray(parent) < 0)[0][0])
    mask = torch.from_numpy(np.arange(n) != root).to(DEV)
    if n > 1:
        e = max(e, _cmp("G_up", Gu[mask], Ou[mask.cpu().numpy()], dt),
                _cmp("G_down", Gw[mask], Ow[mask.cpu().numpy()], dt))
    assert torch.all(Gu[root] == 0) and torch.all(Gw[root] == 0)
    say("  worst rel err %.2e" % e)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("topo,n,b", [("random", 1, 3), ("random", 60, 1), ("path", 40, 4),
                                      ("star", 50, 3), ("balanced", 127, 8), ("perm", 200, 5),
                                      ("random", 80, 16), ("random", 30, 32)])
def test_nonsym_tree_small(ssa, topo, n, b, dt):
    parent = {"random": lambda: spdgen.random_recursive_tree(n, 2),
              "path": lambda: spdgen.path_tree(n), "star": lambda: spdgen.star_tree(n),
              "balanced": lambda: spdgen.balanced_tree(n, 2),
              "perm": lambda: _perm_tree(n, 3)}[topo]()
    run_nonsym_tree(ssa, parent, b, DT[dt], seed=n + b)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_nonsym_tree_workload_b8(ssa, dt):
    """Random recursive tree of 262144 nodes, b = 8, independent directed edges,
    full oracle."""
    run_nonsym_tree(ssa, spdgen.random_recursive_tree(262144, 1), 8, DT[dt], seed=1)


def test_nonsym_tree_symmetric_case_matches_spd_tree(ssa):
    parent = spdgen.random_recursive_tree(300, 4)
    d, e = spdgen.tree(parent, 5, seed=2)
    D, E = _to(d, torch.float64), _to(e, torch.float64)
    Gd, Gu, Gw = ssa.nonsym_tree(parent, D, E, E.transpose(-1, -2).contiguous())
    Sd, Se, _ = ssa.tree(parent, D, E)
    assert float((Gd - Sd).abs().max()) <= 1e-12 * float(Sd.abs().max())
    assert float((Gu - Se).abs().max()) <= 1e-12 * float(Se.abs().max())
    assert float((Gw - Se.transpose(-1, -2)).abs().max()) <= 1e-12 * float(Se.abs().max())


def test_nonsym_tree_breakdown(ssa):
    parent = spdgen.random_recursive_tree(40, 1)
    d, u, w = spdgen.nonsym_tree(parent, 3, seed=1)
    d[11] = 0.0
    Gd, Gu, Gw, info = ssa.nonsym_tree(parent, _to(d, torch.float64), _to(u, torch.float64),
                                       _to(w, torch.float64), return_info=True)
    torch.cuda.synchronize()
    assert int(info) == 12 and torch.isnan(Gd).any()


def test_nonsym_tree_wait_limit_reports_timeout(ssa):
    """Zero wait bound on a path tree: info = -1 instead of a hang; with the
    bound restored the same call matches the oracle."""
    p = spdgen.path_tree(2000)
    d, u, w = spdgen.nonsym_tree(p, 4, seed=6)
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        _, _, _, info = ssa.nonsym_tree(p, _to(d, torch.float64), _to(u, torch.float64),
                                        _to(w, torch.float64), return_info=True)
        torch.cuda.synchronize()
        with pytest.raises(ssa.WaitTimeout):
            ssa.nonsym_tree(p, _to(d, torch.float64), _to(u, torch.float64),
                            _to(w, torch.float64), check=True)
    finally:
        ssa.set_wait_limit(old)
    assert int(info) == -1
    run_nonsym_tree(ssa, p, 4, torch.float64, seed=6)
