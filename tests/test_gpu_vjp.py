"""GPU parity of the reverse mode (vector-Jacobian products): the HIP path
through the C ABI against the oracle's VJP (oracle.chain_vjp / star_vjp /
tree_vjp, itself pinned to the dense closed form and finite differences) on
the same seeded inputs and cotangents.

Tolerances: relative Frobenius error per block <= 1e-10 (float64) or 2e-4
(float32), as for the forward outputs; a float32 run is compared with the
oracle on its own float32 inputs widened to float64.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import par
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


def _sym_exact(t):
    return torch.equal(t, t.transpose(-1, -2))


# ---------------------------------------------------------------- chain
def chain_case(B, L, b, seed, m0=0, load=2.0):
    d, l = spdgen.chain(B, L, b, seed=seed, diag_load=load, m0=m0)
    gd = spdgen.cotangent(d.shape, seed=seed, k=0, m0=m0)
    gl = spdgen.cotangent(l.shape, seed=seed, k=1, m0=m0)
    lb = spdgen.cotangent((B,), seed=seed, k=2, m0=m0)
    return d, l, gd, gl, lb


def run_chain_vjp(ssa, B, L, b, dt, seed=0, sample=None):
    say("chain_vjp B=%d L=%d b=%d %s" % (B, L, b, dt))
    d, l, gd, gl, lb = chain_case(B, L, b, seed)
    db, lbar, info = ssa.chain_vjp(_to(d, dt), _to(l, dt), _to(gd, dt), _to(gl, dt),
                                   torch.from_numpy(lb).to(DEV), return_info=True)
    torch.cuda.synchronize()
    assert int(info.abs().sum()) == 0
    assert _sym_exact(db)
    sel = list(range(B)) if sample is None else list(sample)
    u = lambda x: _as_used(x[sel], dt)
    Od, Ol, st = oracle.chain_vjp(u(d), u(l), u(gd), u(gl), lb[sel])
    assert (st == 0).all()
    e = _cmp("diag_bar", db[sel], Od, dt)
    if L > 1:
        e = max(e, _cmp("lower_bar", lbar[sel], Ol, dt))
    say("  worst rel err %.2e" % e)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L,b", [(1, 1, 1), (3, 1, 4), (2, 2, 1), (3, 3, 2), (2, 8, 3),
                                   (3, 19, 5), (4, 9, 8), (3, 7, 17), (2, 11, 32),
                                   (2, 1, 16), (3, 2, 16), (2, 3, 16), (5, 12, 16),
                                   (7, 33, 16)])
def test_chain_vjp_small(ssa, B, L, b, dt):
    run_chain_vjp(ssa, B, L, b, DT[dt], seed=B * 100 + L + b)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_chain_vjp_workload_b16_batched(ssa, dt):
    """4096 chains of 64 blocks of 16 in one call; the oracle checks every
    chain."""
    run_chain_vjp(ssa, 4096, 64, 16, DT[dt], seed=0)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L", [(2, 600), (3, 1030)])
def test_chain_vjp_segments(ssa, B, L, dt):
    """b = 32 with few long chains runs the segment-parallel reverse mode
    (4 and 8 segments of uneven length)."""
    run_chain_vjp(ssa, B, L, 32, DT[dt], seed=B + L)


@pytest.mark.timeout(900)
def test_chain_vjp_workload_b32_long(ssa):
    """64 chains of 16384 blocks of 32 (diagonal load 1.0), float64, 128
    segments per chain; the oracle checks every chain, in batches of 16."""
    B, L, b = 64, 16384, 32
    say("chain_vjp long: generating")
    d, l, gd, gl, lb = chain_case(B, L, b, seed=0, load=1.0)
    args = [_to(x, torch.float64) for x in (d, l, gd, gl)]
    say("chain_vjp long: running")
    db, lbar, info = ssa.chain_vjp(*args, torch.from_numpy(lb).to(DEV), return_info=True)
    torch.cuda.synchronize()
    del args
    assert int(info.abs().sum()) == 0
    for m0 in range(0, B, 16):
        sl = slice(m0, m0 + 16)
        Od, Ol, st = oracle.chain_vjp(d[sl], l[sl], gd[sl], gl[sl], lb[sl])
        assert (st == 0).all()
        say("chain_vjp long: chains %d..%d  diag %.2e  lower %.2e" % (
            m0, m0 + 15, _cmp("diag_bar[%d:]" % m0, db[sl], Od, torch.float64),
            _cmp("lower_bar[%d:]" % m0, lbar[sl], Ol, torch.float64)))
        del Od, Ol


def test_chain_vjp_slow_decay_maps_kept(ssa):
    """D_i = (2 + 0.01) M, C_i = -M (M SPD, b = 32), 2 chains of 2048 blocks
    (16 segments of 128 blocks): the products of the X's shrink only by
    about 0.905 per block, so the segment maps are carried to every
    segment's end (on the workload they are dropped after about 28 blocks);
    every chain matches the oracle."""
    rng = np.random.default_rng(22)
    B, L, b = 2, 2048, 32
    d = np.empty((B, L, b, b))
    l = np.empty((B, L - 1, b, b))
    for m in range(B):
        M = pins.random_spd(b, rng, load=1.0)
        d[m] = 2.01 * M
        l[m] = -M
    gd = spdgen.cotangent(d.shape, seed=22, k=0)
    gl = spdgen.cotangent(l.shape, seed=22, k=1)
    lb = spdgen.cotangent((B,), seed=22, k=2)
    db, lbar, info = ssa.chain_vjp(_to(d, torch.float64), _to(l, torch.float64),
                                   _to(gd, torch.float64), _to(gl, torch.float64),
                                   torch.from_numpy(lb).to(DEV), return_info=True)
    torch.cuda.synchronize()
    assert int(info.abs().sum()) == 0
    Od, Ol, st = oracle.chain_vjp(d, l, gd, gl, lb)
    assert (st == 0).all()
    e = max(_cmp("diag_bar", db, Od, torch.float64), _cmp("lower_bar", lbar, Ol, torch.float64))
    say("  worst rel err %.2e" % e)


def test_chain_vjp_segments_not_pd(ssa):
    d, l, gd, gl, lb = chain_case(2, 600, 32, seed=4)
    d[1, 300] = -np.eye(32)
    db, lbar, info = ssa.chain_vjp(_to(d, torch.float64), _to(l, torch.float64),
                                   _to(gd, torch.float64), _to(gl, torch.float64),
                                   torch.from_numpy(lb).to(DEV), return_info=True)
    torch.cuda.synchronize()
    assert list(info.cpu().numpy()) == [0, 301]
    assert torch.isnan(db[1]).all() and torch.isnan(lbar[1]).all()
    Od, Ol, _ = oracle.chain_vjp(d[:1], l[:1], gd[:1], gl[:1], lb[:1])
    _cmp("diag_bar", db[:1], Od, torch.float64)


def test_chain_vjp_logdet_only_is_selected_inverse(ssa):
    """With zero output cotangents and logdet_bar = 1: diag_bar = G_diag and
    lower_bar = 2 G_lower (d log det A = <A^-1, dA>), against the forward
    call on the same GPU."""
    for b in (4, 16):
        d, l = spdgen.chain(6, 10, b, seed=3)
        D, C = _to(d, torch.float64), _to(l, torch.float64)
        Gd, Gl, _ = ssa.chain(D, C)
        db, lbar = ssa.chain_vjp(D, C, torch.zeros_like(D), torch.zeros_like(C), 1.0)
        assert float((db - Gd).abs().max()) <= 1e-12 * float(Gd.abs().max())
        assert float((lbar - 2 * Gl).abs().max()) <= 1e-12 * float(Gl.abs().max())


@pytest.mark.parametrize("b", [3, 16])
def test_chain_vjp_not_pd(ssa, b):
    d, l, gd, gl, lb = chain_case(3, 6, b, seed=9)
    d[1, 4] = -np.eye(b)
    db, lbar, info = ssa.chain_vjp(_to(d, torch.float64), _to(l, torch.float64),
                                   _to(gd, torch.float64), _to(gl, torch.float64),
                                   torch.from_numpy(lb).to(DEV), return_info=True)
    torch.cuda.synchronize()
    assert list(info.cpu().numpy()) == [0, 5, 0]
    assert torch.isnan(db[1]).all() and torch.isnan(lbar[1]).all()
    Od, Ol, _ = oracle.chain_vjp(d[[0, 2]], l[[0, 2]], gd[[0, 2]], gl[[0, 2]], lb[[0, 2]])
    _cmp("diag_bar", db[[0, 2]], Od, torch.float64)
    with pytest.raises(ssa.NotPositiveDefinite):
        ssa.chain_vjp(_to(d, torch.float64), _to(l, torch.float64), _to(gd, torch.float64),
                      _to(gl, torch.float64), check=True)


def test_chain_vjp_default_logdet_bar_and_batch_dims(ssa):
    d, l, gd, gl, _ = chain_case(6, 5, 3, seed=4)
    args = [_to(x, torch.float64) for x in (d, l, gd, gl)]
    a = ssa.chain_vjp(*args)
    b_ = ssa.chain_vjp(*args, logdet_bar=torch.zeros(6, dtype=torch.float64, device=DEV))
    assert all(torch.equal(x, y) for x, y in zip(a, b_))
    c = ssa.chain_vjp(*[x.reshape((2, 3) + tuple(x.shape[1:])) for x in args])
    assert torch.equal(c[0].reshape(a[0].shape), a[0])


# ------------------------------------------------------------------ star
def run_star_vjp(ssa, B, K, b, dt, seed=0, mats=None):
    say("star_vjp B=%d K=%d b=%d %s" % (B, K, b, dt))
    c, lv, cp = spdgen.star(B, K, b, seed=seed)
    gc = spdgen.cotangent(c.shape, seed=seed, k=0)
    gv = spdgen.cotangent(lv.shape, seed=seed, k=1)
    gx = spdgen.cotangent(cp.shape, seed=seed, k=2)
    lb = spdgen.cotangent((B,), seed=seed, k=3)
    cb, vb, xb, info = ssa.star_vjp(_to(c, dt), _to(lv, dt), _to(cp, dt), _to(gc, dt),
                                    _to(gv, dt), _to(gx, dt), torch.from_numpy(lb).to(DEV),
                                    return_info=True)
    torch.cuda.synchronize()
    assert int(info.abs().sum()) == 0
    sel = list(range(B)) if mats is None else list(mats)
    u = lambda x: _as_used(x[sel], dt)
    Oc, Ov, Ox = par.chunked(oracle.star_vjp, len(sel), [u(c), u(lv), u(cp), u(gc), u(gv), u(gx)],
                             [lb[sel]])
    e = _cmp("center_bar", cb[sel], Oc, dt)
    if K:
        e = max(e, _cmp("leaves_bar", vb[sel], Ov, dt), _cmp("coupling_bar", xb[sel], Ox, dt))
    say("  worst rel err %.2e" % e)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,K,b", [(1, 0, 3), (2, 1, 1), (3, 5, 4), (2, 33, 8), (2, 17, 16),
                                   (2, 9, 32), (1, 300, 5)])
def test_star_vjp_small(ssa, B, K, b, dt):
    run_star_vjp(ssa, B, K, b, DT[dt], seed=K + b)


@pytest.mark.timeout(600)
def test_star_vjp_workload_b32(ssa):
    """256 stars of 1024 leaves of 32, float64; the oracle checks every star
    (host threads over chunks of the batch)."""
    run_star_vjp(ssa, 256, 1024, 32, torch.float64, seed=0)


def test_star_vjp_not_pd(ssa):
    c, lv, cp = spdgen.star(3, 6, 3, seed=0)
    lv[1, 4] = -np.eye(3)
    c[2] = -np.eye(3)
    z = lambda x: torch.zeros(x.shape, dtype=torch.float64, device=DEV)
    cb, vb, xb, info = ssa.star_vjp(_to(c, torch.float64), _to(lv, torch.float64),
                                    _to(cp, torch.float64), z(c), z(lv), z(cp), 1.0,
                                    return_info=True)
    assert list(info.cpu().numpy()) == [0, 6, 1]
    assert torch.isnan(vb[1]).all() and torch.isnan(cb[2]).all()
    assert torch.isfinite(vb[0]).all()


# ------------------------------------------------------------------ tree
def _perm_tree(n, seed):
    rng = np.random.default_rng(seed)
    p0 = spdgen.random_recursive_tree(n, seed)
    perm = rng.permutation(n)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return p


def run_tree_vjp(ssa, parent, b, dt, seed=1):
    n = len(parent)
    say("tree_vjp n=%d b=%d %s" % (n, b, dt))
    d, e = spdgen.tree(parent, b, seed=seed)
    gd = spdgen.cotangent(d.shape, seed=seed, k=0)
    ge = spdgen.cotangent(e.shape, seed=seed, k=1)
    lb = float(spdgen.cotangent((1,), seed=seed, k=2)[0])
    db, eb, info = ssa.tree_vjp(parent, _to(d, dt), _to(e, dt), _to(gd, dt), _to(ge, dt), lb,
                                return_info=True)
    torch.cuda.synchronize()
    assert int(info) == 0
    Od, Oe = oracle.tree_vjp(parent, _as_used(d, dt), _as_used(e, dt), _as_used(gd, dt),
                             _as_used(ge, dt), lb)
    err = _cmp("diag_bar", db, Od, dt)
    root = int(np.where(np.asarray(parent) < 0)[0][0])
    mask = np.arange(n) != root
    if n > 1:
        err = max(err, _cmp("edge_bar", eb[torch.from_numpy(mask).to(DEV)], Oe[mask], dt))
    assert torch.all(eb[root] == 0)
    say("  worst rel err %.2e" % err)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("topo,n,b", [("random", 1, 3), ("random", 2, 2), ("random", 50, 1),
                                      ("random", 700, 8), ("path", 40, 4), ("star", 60, 3),
                                      ("balanced", 255, 2), ("perm", 300, 5),
                                      ("random", 100, 16), ("random", 40, 32)])
def test_tree_vjp_small(ssa, topo, n, b, dt):
    parent = {"random": lambda: spdgen.random_recursive_tree(n, 2),
              "path": lambda: spdgen.path_tree(n), "star": lambda: spdgen.star_tree(n),
              "balanced": lambda: spdgen.balanced_tree(n, 2),
              "perm": lambda: _perm_tree(n, 3)}[topo]()
    run_tree_vjp(ssa, parent, b, DT[dt], seed=n)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_tree_vjp_workload_b8_random(ssa, dt):
    """Random recursive tree of 262144 nodes (seed 1), b = 8, full oracle."""
    run_tree_vjp(ssa, spdgen.random_recursive_tree(262144, 1), 8, DT[dt], seed=1)


def test_tree_vjp_not_pd(ssa):
    p = spdgen.random_recursive_tree(64, 1)
    d, e = spdgen.tree(p, 3)
    d[10] = -np.eye(3)
    z = torch.zeros(d.shape, dtype=torch.float64, device=DEV)
    db, eb, info = ssa.tree_vjp(p, _to(d, torch.float64), _to(e, torch.float64), z, z, 1.0,
                                return_info=True)
    _, _, _, Oinfo = oracle.tree(p, d, e)
    assert int(info) == Oinfo != 0
    assert torch.isnan(db).any()


def test_tree_vjp_wait_limit_reports_timeout(ssa):
    """Zero wait bound on a path tree: the single-launch reverse passes give up
    at the first unready flag and report info = -1; with the bound restored
    the same call matches the oracle."""
    p = spdgen.path_tree(2000)
    d, e = spdgen.tree(p, 4, seed=5)
    gd = spdgen.cotangent(d.shape, seed=5, k=0)
    ge = spdgen.cotangent(e.shape, seed=5, k=1)
    args = (_to(d, torch.float64), _to(e, torch.float64), _to(gd, torch.float64),
            _to(ge, torch.float64), 0.5)
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        _, _, info = ssa.tree_vjp(p, *args, return_info=True)
        torch.cuda.synchronize()
        with pytest.raises(ssa.WaitTimeout):
            ssa.tree_vjp(p, *args, check=True)
    finally:
        ssa.set_wait_limit(old)
    assert int(info) == -1
    run_tree_vjp(ssa, p, 4, torch.float64, seed=5)
