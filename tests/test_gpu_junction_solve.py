"""GPU parity of the junction siblings (solve x = A^{-1} y and the sampling
transform x = L^{-T} D^{-1/2} z on the filled pattern, both from the kept
factor) through the C ABI against oracle.junction_apply (pinned to dense
solves and to the Cholesky factor of the permuted matrix) on the same seeded
inputs; z is passed in, so a sample is compared element by element.  The
factor call's log det and failure index are checked against oracle.junction.

Tolerances: max|x - ref| / max|ref| per matrix <= 1e-10 (float64) or 2e-4
(float32), the bar of the chain, star and tree siblings; log det relative
1e-12 (float64) or 1e-5 (float32) as for the junction selected inverse.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import spdgen

pytestmark = pytest.mark.gpu

TOL = {torch.float64: 1e-10, torch.float32: 2e-4}
LDTOL = {torch.float64: 1e-12, torch.float32: 1e-5}
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


def _cmp_vec(name, got, ref, dt):
    g = got.double().cpu().numpy().reshape(ref.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    err = np.abs(g - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-300)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dt], "%s rel err %.3e > %.1e" % (name, worst, TOL[dt])
    return worst


def run(ssa, n, e, b, B, k, dt, seed, order=None, label=""):
    say("junction siblings %s n=%d m=%d b=%d B=%d k=%d %s" % (label, n, e.shape[1], b, B, k, dt))
    d, v = spdgen.graph(e, n, b, B=B, seed=seed)
    y = spdgen.cotangent((B, n, b, k), seed=seed, k=0)
    z = spdgen.cotangent((B, n, b, k), seed=seed, k=1)
    f = ssa.junction_factor(_to(d, dt), e, _to(v, dt), order=order)
    x = f.solve(_to(y, dt))
    xs = f.sample(z=_to(z, dt))
    torch.cuda.synchronize()
    du, vu = _as_used(d, dt), _as_used(v, dt)
    P = oracle.filled_pattern(n, e, order)
    ref, info = oracle.junction_apply(du, e, vu, _as_used(y, dt), "solve", pattern=P)
    ref_s, info_s = oracle.junction_apply(du, e, vu, _as_used(z, dt), "sample", pattern=P)
    _, _, _, Old, Oinfo = oracle.junction(du, e, vu, pattern=P)
    assert (info == 0).all() and (info_s == 0).all()
    assert np.array_equal(f.info.cpu().numpy(), Oinfo)
    ld = f.logdet.cpu().numpy()
    assert np.all(np.abs(ld - Old) <= LDTOL[dt] * np.maximum(1.0, np.abs(Old)))
    e1 = _cmp_vec("solve", x, ref, dt)
    e2 = _cmp_vec("sample", xs, ref_s, dt)
    say("  levels %d, solve err %.2e, sample err %.2e" % (f.plan.levels, e1, e2))


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("r,c,b,B,k", [(1, 1, 3, 2, 1), (1, 9, 2, 1, 3), (3, 3, 2, 2, 1),
                                       (4, 5, 1, 3, 4), (8, 8, 4, 2, 33), (16, 16, 16, 2, 2),
                                       (12, 12, 8, 3, 5)])
def test_grid(ssa, r, c, b, B, k, dt):
    run(ssa, r * c, spdgen.grid_edges(r, c), b, B, k, DT[dt], seed=r * c + b, label="grid")


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("n,extra,b,k", [(30, 40, 3, 2), (100, 150, 2, 1), (12, 60, 8, 17),
                                         (50, 10, 17, 3)])
def test_random_graph(ssa, n, extra, b, k, dt):
    e = spdgen.random_graph_edges(n, extra, seed=n + extra)
    run(ssa, n, e, b, 2, k, DT[dt], seed=n, label="random")


@pytest.mark.parametrize("kind", ["natural", "reversed", "random"])
def test_explicit_order(ssa, kind):
    n = 49
    order = {"natural": np.arange(n), "reversed": np.arange(n)[::-1].copy(),
             "random": np.random.default_rng(2).permutation(n)}[kind]
    run(ssa, n, spdgen.grid_edges(7, 7), 4, 2, 3, torch.float64, seed=3, order=order, label=kind)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_workload_grid64_b8(ssa, dt):
    """The junction workload's batch (16 matrices on the 64 x 64 grid, b = 8),
    one and several right-hand sides, full oracle."""
    run(ssa, 4096, spdgen.grid_edges(64, 64), 8, 16, 1, DT[dt], seed=0, label="grid64")
    run(ssa, 4096, spdgen.grid_edges(64, 64), 8, 4, 8, DT[dt], seed=1, label="grid64")


def test_single_matrix_and_no_edges(ssa):
    """[n, b, b] inputs (no batch axis) and a pattern without edges."""
    e = np.zeros((2, 0), np.int32)
    d, v = spdgen.graph(e, 5, 3, B=1, seed=4)
    y = spdgen.cotangent((1, 5, 3, 2), seed=4, k=0)
    f = ssa.junction_factor(_to(d[0], torch.float64), e, _to(v[0], torch.float64))
    x = f.solve(_to(y[0], torch.float64))
    xs = f.sample(z=_to(y[0], torch.float64))
    ref, _ = oracle.junction_apply(d, e, v, y, "solve")
    ref_s, _ = oracle.junction_apply(d, e, v, y, "sample")
    assert x.shape == (5, 3, 2) and f.logdet.dim() == 0
    _cmp_vec("solve", x[None], ref, torch.float64)
    _cmp_vec("sample", xs[None], ref_s, torch.float64)
    g = spdgen.grid_edges(3, 3)
    d, v = spdgen.graph(g, 9, 2, B=1, seed=1)
    f = ssa.junction_factor(_to(d[0], torch.float64), g, _to(v[0], torch.float64))
    s = f.sample(num_samples=4)
    assert s.shape == (9, 2, 4) and torch.isfinite(s).all()


def test_not_positive_definite_is_reported(ssa):
    e = spdgen.grid_edges(5, 5)
    d, v = spdgen.graph(e, 25, 3, B=3, seed=4)
    d[1, 12] = -np.eye(3)
    f = ssa.junction_factor(_to(d, torch.float64), e, _to(v, torch.float64))
    _, _, _, Old, Oinfo = oracle.junction(d, e, v)
    assert list(f.info.cpu().numpy()) == list(Oinfo) and Oinfo[1] == 13
    assert torch.isnan(f.logdet[1]) and torch.isfinite(f.logdet[[0, 2]]).all()
    y = spdgen.cotangent((3, 25, 3, 2), seed=4, k=0)
    x = f.solve(_to(y, torch.float64))
    ref, _ = oracle.junction_apply(d, e, v, y, "solve")
    _cmp_vec("solve", x[[0, 2]], ref[[0, 2]], torch.float64)


def test_repeated_calls_are_bitwise_identical(ssa):
    e = spdgen.grid_edges(12, 12)
    d, v = spdgen.graph(e, 144, 4, B=3, seed=6)
    y = _to(spdgen.cotangent((3, 144, 4, 3), seed=6, k=0), torch.float64)
    f = ssa.junction_factor(_to(d, torch.float64), e, _to(v, torch.float64))
    a, b_ = f.solve(y), f.solve(y)
    s1, s2 = f.sample(z=y), f.sample(z=y)
    torch.cuda.synchronize()
    assert torch.equal(a, b_) and torch.equal(s1, s2)


def test_solve_wait_limit_gives_nan(ssa):
    """With a zero wait bound the single-launch solve gives up at the first
    unready flag: the call still ends, and every entry of x is NaN (every
    backward workgroup sees the give-up word).  A path pattern eliminated end
    to end makes the chunks a chain, each waiting for the one before it.  With
    the default bound restored, the same solve is exact again."""
    n = 2000
    e = spdgen.grid_edges(1, n)
    d, v = spdgen.graph(e, n, 4, B=1, seed=5)
    y = spdgen.cotangent((1, n, 4, 1), seed=5, k=0)
    f = ssa.junction_factor(_to(d, torch.float64), e, _to(v, torch.float64))
    Y = _to(y, torch.float64)
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        x = f.solve(Y)
        torch.cuda.synchronize()
    finally:
        ssa.set_wait_limit(old)
    assert torch.isnan(x).all()
    ref, _ = oracle.junction_apply(d, e, v, y, "solve")
    _cmp_vec("solve", f.solve(Y), ref, torch.float64)


def test_abi_arguments(ssa):
    """Status codes of the C entry points: k = 0 and B = 0 do nothing; an
    output that aliases the input, a short workspace, a wrong dtype and a
    NULL factor are rejected."""
    e = spdgen.grid_edges(3, 3)
    d, v = spdgen.graph(e, 9, 2, B=1, seed=1)
    f = ssa.junction_factor(_to(d, torch.float64), e, _to(v, torch.float64))
    L = ssa.lib()
    y = torch.ones((1, 9, 2, 1), dtype=torch.float64, device=DEV)
    h, fp, yp = f.plan.handle, f.factor.data_ptr(), y.data_ptr()
    nb = L.selinv_junction_solve_workspace_bytes(h, 1, 1)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    wp = ws.data_ptr()
    assert L.selinv_junction_solve_f64(h, 1, fp, 0, yp, yp, None, 0, None) == ssa.OK
    assert L.selinv_junction_solve_f64(h, 0, fp, 1, yp, yp, None, 0, None) == ssa.OK
    assert L.selinv_junction_solve_f64(h, 1, fp, 1, yp, yp, wp, nb, None) == ssa.INVALID_ARG
    assert L.selinv_junction_solve_f64(h, 1, fp, 1, yp, yp + 8, wp, nb - 1, None) == \
        ssa.INVALID_ARG
    assert L.selinv_junction_sample_f64(h, 1, None, 1, yp, yp + 8, None) == ssa.INVALID_ARG
    assert L.selinv_junction_solve_f32(h, 1, fp, 1, yp, yp + 8, wp, nb, None) == ssa.INVALID_ARG
    assert L.selinv_junction_solve_workspace_bytes(h, 1, 2) > nb > 0
    assert L.selinv_junction_solve_workspace_bytes(h, 1, 0) == 0
    D, V = _to(d, torch.float64), _to(v, torch.float64)
    ld = torch.empty(1, dtype=torch.float64, device=DEV)
    assert L.selinv_junction_factor_f64(h, 1, D.data_ptr(), V.data_ptr(), None, ld.data_ptr(),
                                        None, None, 0, None) == ssa.INVALID_ARG
    assert L.selinv_junction_factor_bytes(h, 2) == 2 * L.selinv_junction_factor_bytes(h, 1) > 0
