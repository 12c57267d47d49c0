"""GPU parity of the shared-factor siblings (log det without a factor, solve
x = A^{-1} y, sample x = L^{-T} D^{-1/2} z) through the C ABI against the
oracle (oracle.chain / star / tree for log det, oracle.chain_apply /
star_apply / tree_apply for the sweeps) on the same seeded inputs; z is
passed in, so a sample is compared element by element.

Tolerances: vectors max|x - ref| / max|ref| per matrix <= 1e-10 (float64) or
2e-4 (float32); |log det error| <= 1e-8 n (float64) or 1e-3 n (float32), n
diagonal blocks.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import par
import spdgen

pytestmark = pytest.mark.gpu

TOL = {torch.float64: 1e-10, torch.float32: 2e-4}
TOL_LD = {torch.float64: 1e-8, torch.float32: 1e-3}
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


def _cmp_vec(name, got, ref, dt, per=1):
    """per: number of leading axes that index matrices"""
    g = got.double().cpu().numpy()
    g = g.reshape(g.shape[:per] + (-1,))
    r = ref.reshape(ref.shape[:per] + (-1,))
    err = np.abs(g - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-300)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dt], "%s rel err %.3e > %.1e" % (name, worst, TOL[dt])
    return worst


def _cmp_ld(got, ref, n, dt):
    d = float(np.abs(np.asarray(got.cpu().numpy(), np.float64) - ref).max())
    assert d <= TOL_LD[dt] * n, "logdet err %.3e" % d


# ---------------------------------------------------------------- chain
@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L,b,k", [(2, 1, 3, 1), (3, 5, 1, 2), (2, 9, 4, 17), (3, 6, 16, 1),
                                     (2, 13, 16, 20), (2, 1, 16, 3), (5, 2, 16, 33),
                                     (2, 4, 17, 3), (2, 7, 32, 2)])
def test_chain_siblings(ssa, B, L, b, k, dt):
    dt = DT[dt]
    say("chain siblings B=%d L=%d b=%d k=%d %s" % (B, L, b, k, dt))
    d, l = spdgen.chain(B, L, b, seed=L + b)
    y = spdgen.cotangent((B, L, b, k), seed=L, k=0)
    z = spdgen.cotangent((B, L, b, k), seed=L, k=1)
    D, C = _to(d, dt), _to(l, dt)
    f = ssa.chain_factor(D, C)
    ld_only, info = ssa.chain_logdet(D, C, return_info=True)
    x = f.solve(_to(y, dt))
    s = f.sample(z=_to(z, dt))
    torch.cuda.synchronize()
    du, lu = _as_used(d, dt), _as_used(l, dt)
    _, _, Old, Oinfo = oracle.chain(du, lu)
    assert np.array_equal(info.cpu().numpy(), Oinfo) and (f.info.cpu().numpy() == 0).all()
    _cmp_ld(ld_only, Old, L, dt)
    assert torch.equal(ld_only, f.logdet)
    Ox, st = oracle.chain_apply(du, lu, _as_used(y, dt), "solve")
    Os, _ = oracle.chain_apply(du, lu, _as_used(z, dt), "sample")
    assert (st == 0).all()
    e1 = _cmp_vec("solve", x, Ox, dt)
    e2 = _cmp_vec("sample", s, Os, dt)
    say("  solve %.2e sample %.2e" % (e1, e2))


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_chain_siblings_workload_b16(ssa, dt):
    """4096 chains of 64 blocks of 16: log det, solve and sample with k = 4,
    every chain checked."""
    dt = DT[dt]
    B, L, b, k = 4096, 64, 16, 4
    d, l = spdgen.chain(B, L, b, seed=0)
    y = spdgen.cotangent((B, L, b, k), seed=0, k=0)
    z = spdgen.cotangent((B, L, b, k), seed=0, k=1)
    f = ssa.chain_factor(_to(d, dt), _to(l, dt))
    x = f.solve(_to(y, dt))
    s = f.sample(z=_to(z, dt))
    torch.cuda.synchronize()
    du, lu = _as_used(d, dt), _as_used(l, dt)
    _, _, Old, _ = oracle.chain(du, lu)
    _cmp_ld(f.logdet, Old, L, dt)
    Ox, _ = oracle.chain_apply(du, lu, _as_used(y, dt), "solve")
    Os, _ = oracle.chain_apply(du, lu, _as_used(z, dt), "sample")
    say("  solve %.2e sample %.2e" % (_cmp_vec("solve", x, Ox, dt),
                                       _cmp_vec("sample", s, Os, dt)))


@pytest.mark.parametrize("b", [4, 16])
def test_chain_factor_not_pd(ssa, b):
    d, l = spdgen.chain(3, 6, b, seed=1)
    d[1, 3] = -np.eye(b)
    ld, info = ssa.chain_logdet(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    assert list(info.cpu().numpy()) == [0, 4, 0]
    assert np.isnan(float(ld[1])) and np.isfinite(float(ld[0]))


def test_chain_sample_deterministic_and_draws(ssa):
    d, l = spdgen.chain(8, 10, 16, seed=3)
    f = ssa.chain_factor(_to(d, torch.float64), _to(l, torch.float64))
    z = _to(spdgen.cotangent((8, 10, 16, 3), seed=1), torch.float64)
    assert torch.equal(f.sample(z=z), f.sample(z=z))
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    a = f.sample(num_samples=2, generator=g)
    assert a.shape == (8, 10, 16, 2) and torch.isfinite(a).all()


# ------------------------------------------------------------------ star
@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,K,b,k", [(1, 0, 3, 2), (2, 5, 4, 1), (2, 33, 8, 18), (2, 9, 32, 3),
                                     (3, 40, 32, 1), (1, 0, 32, 4), (2, 17, 32, 4),
                                     (2, 5, 32, 7)])
def test_star_siblings(ssa, B, K, b, k, dt):
    dt = DT[dt]
    say("star siblings B=%d K=%d b=%d k=%d %s" % (B, K, b, k, dt))
    c, lv, cp = spdgen.star(B, K, b, seed=K + b)
    yc = spdgen.cotangent((B, b, k), seed=K, k=0)
    yl = spdgen.cotangent((B, K, b, k), seed=K, k=1)
    zc = spdgen.cotangent((B, b, k), seed=K, k=2)
    zl = spdgen.cotangent((B, K, b, k), seed=K, k=3)
    f = ssa.star_factor(_to(c, dt), _to(lv, dt), _to(cp, dt))
    ld_only = ssa.star_logdet(_to(c, dt), _to(lv, dt), _to(cp, dt))
    xc, xl = f.solve(_to(yc, dt), _to(yl, dt))
    sc, sl = f.sample(z_center=_to(zc, dt), z_leaves=_to(zl, dt))
    torch.cuda.synchronize()
    cu, lu, pu = _as_used(c, dt), _as_used(lv, dt), _as_used(cp, dt)
    *_, Old, Oinfo = oracle.star(cu, lu, pu)
    _cmp_ld(ld_only, Old, K + 1, dt)
    Oxc, Oxl = oracle.star_apply(cu, lu, pu, _as_used(yc, dt), _as_used(yl, dt), "solve")
    Osc, Osl = oracle.star_apply(cu, lu, pu, _as_used(zc, dt), _as_used(zl, dt), "sample")
    gx = torch.cat([xc.reshape(B, -1), xl.reshape(B, -1)], 1)
    gs = torch.cat([sc.reshape(B, -1), sl.reshape(B, -1)], 1)
    rx = np.concatenate([Oxc.reshape(B, -1), Oxl.reshape(B, -1)], 1)
    rs = np.concatenate([Osc.reshape(B, -1), Osl.reshape(B, -1)], 1)
    say("  solve %.2e sample %.2e" % (_cmp_vec("solve", gx, rx, dt),
                                       _cmp_vec("sample", gs, rs, dt)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_star_siblings_workload_b32(ssa, dt):
    """256 stars of 1024 leaves of 32, k = 1: log det, solve and sample
    checked on every star (host threads over chunks of the batch)."""
    dt = DT[dt]
    B, K, b, k = 256, 1024, 32, 1
    c, lv, cp = spdgen.star(B, K, b, seed=0)
    yc = spdgen.cotangent((B, b, k), seed=0, k=0)
    yl = spdgen.cotangent((B, K, b, k), seed=0, k=1)
    f = ssa.star_factor(_to(c, dt), _to(lv, dt), _to(cp, dt))
    ld_only = ssa.star_logdet(_to(c, dt), _to(lv, dt), _to(cp, dt))
    xc, xl = f.solve(_to(yc, dt), _to(yl, dt))
    sc, sl = f.sample(z_center=_to(yc, dt), z_leaves=_to(yl, dt))
    torch.cuda.synchronize()
    cu, lu, pu = _as_used(c, dt), _as_used(lv, dt), _as_used(cp, dt)
    ycu, ylu = _as_used(yc, dt), _as_used(yl, dt)
    *_, Old, Oinfo = oracle.star(cu, lu, pu)
    assert not Oinfo.any()
    _cmp_ld(ld_only, Old, K + 1, dt)
    _cmp_ld(f.logdet, Old, K + 1, dt)
    for mode, (gc, gl) in (("solve", (xc, xl)), ("sample", (sc, sl))):
        Oc, Ol = par.chunked(lambda *a: oracle.star_apply(*a, mode), B, [cu, lu, pu, ycu, ylu])
        g = torch.cat([gc.reshape(B, -1), gl.reshape(B, -1)], 1)
        r = np.concatenate([Oc.reshape(B, -1), Ol.reshape(B, -1)], 1)
        say("  %s %.2e" % (mode, _cmp_vec(mode, g, r, dt)))


# ------------------------------------------------------------------ tree
def _perm_tree(n, seed):
    rng = np.random.default_rng(seed)
    p0 = spdgen.random_recursive_tree(n, seed)
    perm = rng.permutation(n)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return p


def run_tree(ssa, parent, b, k, dt, seed):
    n = len(parent)
    d, e = spdgen.tree(parent, b, seed=seed)
    y = spdgen.cotangent((n, b, k), seed=seed, k=0)
    z = spdgen.cotangent((n, b, k), seed=seed, k=1)
    f = ssa.tree_factor(parent, _to(d, dt), _to(e, dt))
    ld_only = ssa.tree_logdet(parent, _to(d, dt), _to(e, dt))
    x = f.solve(_to(y, dt))
    s = f.sample(z=_to(z, dt))
    torch.cuda.synchronize()
    du, eu = _as_used(d, dt), _as_used(e, dt)
    _, _, Old, _ = oracle.tree(parent, du, eu)
    _cmp_ld(ld_only.reshape(1), np.array([Old]), n, dt)
    assert int(f.info) == 0
    Ox = oracle.tree_apply(parent, du, eu, _as_used(y, dt), "solve")
    Os = oracle.tree_apply(parent, du, eu, _as_used(z, dt), "sample")
    return _cmp_vec("solve", x[None], Ox[None], dt), _cmp_vec("sample", s[None], Os[None], dt)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("topo,n,b,k", [("random", 1, 3, 1), ("random", 60, 2, 3),
                                        ("path", 30, 4, 1), ("star", 40, 3, 17),
                                        ("balanced", 127, 8, 2), ("perm", 200, 5, 1),
                                        ("random", 50, 16, 2), ("random", 20, 32, 1)])
def test_tree_siblings(ssa, topo, n, b, k, dt):
    parent = {"random": lambda: spdgen.random_recursive_tree(n, 2),
              "path": lambda: spdgen.path_tree(n), "star": lambda: spdgen.star_tree(n),
              "balanced": lambda: spdgen.balanced_tree(n, 2),
              "perm": lambda: _perm_tree(n, 3)}[topo]()
    say("tree siblings %s n=%d b=%d k=%d %s" % (topo, n, b, k, dt))
    say("  solve %.2e sample %.2e" % run_tree(ssa, parent, b, k, DT[dt], seed=n))


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_tree_siblings_workload_b8(ssa, dt):
    """Random recursive tree of 262144 nodes, b = 8, k = 2, full oracle."""
    say("  solve %.2e sample %.2e" % run_tree(ssa, spdgen.random_recursive_tree(262144, 1), 8, 2,
                                               DT[dt], seed=1))


def test_tree_solve_wait_limit_gives_nan(ssa):
    """Zero wait bound on a path tree: the single-launch solve gives up and
    leaves NaN in x rather than a silently wrong result; with the bound
    restored the same solve matches the oracle."""
    p = spdgen.path_tree(2000)
    d, e = spdgen.tree(p, 4, seed=7)
    y = spdgen.cotangent((2000, 4, 1), seed=7, k=0)
    f = ssa.tree_factor(p, _to(d, torch.float64), _to(e, torch.float64))
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        x = f.solve(_to(y, torch.float64))
        torch.cuda.synchronize()
    finally:
        ssa.set_wait_limit(old)
    assert torch.isnan(x).any()
    x = f.solve(_to(y, torch.float64))
    Ox = oracle.tree_apply(p, d, e, y, "solve")
    _cmp_vec("solve", x[None], Ox[None], torch.float64)


def test_tree_sample_wait_limit_gives_nan(ssa):
    """The sampler runs on the same single-launch parents-first schedule:
    with a zero wait bound on a path tree it gives up and leaves NaN in x;
    with the bound restored the same draw matches the oracle."""
    p = spdgen.path_tree(2000)
    d, e = spdgen.tree(p, 4, seed=8)
    z = spdgen.cotangent((2000, 4, 3), seed=8, k=1)
    f = ssa.tree_factor(p, _to(d, torch.float64), _to(e, torch.float64))
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        x = f.sample(z=_to(z, torch.float64))
        torch.cuda.synchronize()
    finally:
        ssa.set_wait_limit(old)
    assert torch.isnan(x).any()
    x = f.sample(z=_to(z, torch.float64))
    Ox = oracle.tree_apply(p, d, e, z, "sample")
    _cmp_vec("sample", x[None], Ox[None], torch.float64)


def test_tree_factor_not_pd(ssa):
    p = spdgen.random_recursive_tree(40, 1)
    d, e = spdgen.tree(p, 3)
    d[7] = -np.eye(3)
    ld, info = ssa.tree_logdet(p, _to(d, torch.float64), _to(e, torch.float64), return_info=True)
    _, _, _, Oinfo = oracle.tree(p, d, e)
    assert int(info) == Oinfo == 8 and np.isnan(float(ld))
