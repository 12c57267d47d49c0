"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.

Tolerances: relative Frobenius error per output block <= 1e-10 (float64) or
2e-4 (float32); |log det error| <= 1e-8 n (float64) or 1e-3 n (float32),
n = number of diagonal blocks per matrix.  A float32 run is compared with
the oracle on its own float32 inputs widened to float64.
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
TOL_LD = {torch.float64: 1e-8, torch.float32: 1e-3}
DT = {"f64": torch.float64, "f32": torch.float32}


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


DEV = "cuda:0"


def _to(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dt)


def _as_used(x, dt):
    """The float64 view of exactly the values the GPU consumed."""
    return x.astype(np.float32).astype(np.float64) if dt == torch.float32 else x


def _cmp(name, got, ref, dt):
    err = pins.rel_fro(got.double().cpu().numpy(), ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dt], "%s rel err %.3e > %.1e" % (name, worst, TOL[dt])
    return worst


def _cmp_ld(got, ref, n, dt):
    d = float(np.abs(got.cpu().numpy() - ref).max()) if np.size(ref) else 0.0
    assert d <= TOL_LD[dt] * n, "logdet err %.3e > %.1e" % (d, TOL_LD[dt] * n)
    return d


# ---------------------------------------------------------------- chain
def run_chain(ssa, B, L, b, dt, seed=0, load=2.0):
    d, l = spdgen.chain(B, L, b, seed=seed, diag_load=load)
    say("chain B=%d L=%d b=%d %s" % (B, L, b, dt))
    Gd, Gl, ld, info = ssa.chain(_to(d, dt), _to(l, dt), return_info=True)
    torch.cuda.synchronize()
    Od, Ol, Old, Oinfo = oracle.chain(_as_used(d, dt), _as_used(l, dt))
    assert np.array_equal(info.cpu().numpy(), Oinfo)
    e = max(_cmp("G_diag", Gd, Od, dt), _cmp("G_lower", Gl, Ol, dt) if L > 1 else 0.0)
    _cmp_ld(ld, Old, L, dt)
    return e


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L,b", [(1, 1, 1), (3, 1, 4), (2, 2, 1), (3, 3, 2), (2, 8, 3),
                                   (5, 37, 4), (3, 19, 5), (4, 9, 8), (2, 12, 16), (3, 7, 17),
                                   (2, 6, 31), (2, 11, 32), (1, 200, 1), (65, 5, 16),
                                   (7, 70, 16), (64, 4, 8), (5, 32, 1), (2, 5, 6), (1, 16, 2),
                                   (65, 4, 8)])
def test_chain_small(ssa, B, L, b, dt):
    run_chain(ssa, B, L, b, DT[dt], seed=B * 100 + L)


def test_chain_workload_b4_single(ssa):
    """8 blocks of 4 (seed 0, diagonal load 2.0), float64."""
    run_chain(ssa, 1, 8, 4, torch.float64, seed=0)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_chain_workload_b16_batched(ssa, dt):
    """4096 chains of 64 blocks of 16, full oracle comparison."""
    run_chain(ssa, 4096, 64, 16, DT[dt], seed=0)


@pytest.mark.timeout(900)
def test_chain_workload_b32_long(ssa):
    """64 chains of 16384 blocks of 32 (diagonal load 1.0), float64.  Every
    chain is compared with the oracle (in batches of 16 chains), and every
    chain gets the block-diagonal residual check on the GPU."""
    B, L, b = 64, 16384, 32
    say("chain long: generating")
    d, l = spdgen.chain(B, L, b, seed=0, diag_load=1.0)
    D, C = _to(d, torch.float64), _to(l, torch.float64)
    say("chain long: running")
    Gd, Gl, ld, info = ssa.chain(D, C, return_info=True)
    torch.cuda.synchronize()
    assert int(info.abs().sum()) == 0
    for m0 in range(0, B, 16):
        sl = slice(m0, m0 + 16)
        Od, Ol, Old, Oinfo = oracle.chain(d[sl], l[sl])
        assert not Oinfo.any()
        e = max(_cmp("G_diag[%d:]" % m0, Gd[sl], Od, torch.float64),
                _cmp("G_lower[%d:]" % m0, Gl[sl], Ol, torch.float64))
        _cmp_ld(ld[sl], Old, L, torch.float64)
        say("chain long: chains %d..%d ok, worst rel err %.2e" % (m0, m0 + 15, e))
        del Od, Ol
    del d, l
    # block-diagonal residual on all chains: D_i G_ii + C_{i-1} G_{i-1,i} + C_i^T G_{i+1,i} = I
    eye = torch.eye(b, dtype=torch.float64, device=DEV)
    worst = 0.0
    for m in range(B):
        R = D[m] @ Gd[m]
        R[1:] += C[m] @ Gl[m].transpose(-1, -2)
        R[:-1] += C[m].transpose(-1, -2).contiguous() @ Gl[m]
        worst = max(worst, float((R - eye).abs().max()))
    assert worst < 1e-9, worst


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,L", [(1, 64), (2, 96), (3, 130), (5, 200)])
def test_chain_b32_segments(ssa, B, L, dt):
    """b = 32 with few chains runs the segment-parallel elimination (8 to 25
    segments per chain here, segments of uneven length for L = 130)."""
    run_chain(ssa, B, L, 32, DT[dt], seed=B * 100 + L, load=1.0)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_chain_b32_fill_drop(ssa, dt):
    """8 chains of 8192 blocks of 32 (diagonal load 1.0): 256 segments of 32
    blocks per chain.  The fill block to each segment's left separator decays
    below 2^-100 of the segment's first coupling block after about 28 blocks
    and is dropped from there on (the rest of the segment runs in the plain
    collect and distribute); every chain is compared with the oracle."""
    e = run_chain(ssa, 8, 8192, 32, DT[dt], seed=11, load=1.0)
    say("  worst rel err %.2e" % e)


def test_chain_b32_fill_drop_zero_coupling(ssa):
    """Zero coupling blocks at segment starts (256 segments of 32 blocks per
    chain; the chain splits there, so those segments carry no fill at all and
    (A^-1)_{a,a-1} = 0 exactly)."""
    d, l = spdgen.chain(2, 8192, 32, seed=12, diag_load=1.0)
    for a in (64, 4096, 8128):
        l[:, a - 1] = 0.0
    Gd, Gl, ld, info = ssa.chain(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    torch.cuda.synchronize()
    Od, Ol, Old, Oinfo = oracle.chain(d, l)
    assert not info.any() and not Oinfo.any()
    _cmp("G_diag", Gd, Od, torch.float64)
    for a in (64, 4096, 8128):
        assert not Gl[:, a - 1].any()
    mask = np.ones(8191, bool)
    mask[[63, 4095, 8127]] = False
    _cmp("G_lower", Gl[:, torch.from_numpy(mask).to(DEV)], Ol[:, mask], torch.float64)
    _cmp_ld(ld, Old, 8192, torch.float64)


def test_chain_b32_slow_decay_fill_kept(ssa):
    """D_i = (2 + 0.01) M, C_i = -M (M SPD, b = 32), 2 chains of 20000 blocks
    (400 segments of 50 blocks): the fill shrinks only by about 0.905 per
    block, so it is carried to every segment's end; every chain matches the
    oracle.  (The condition number stays near 400.)"""
    rng = np.random.default_rng(21)
    B, L, b = 2, 20000, 32
    d = np.empty((B, L, b, b))
    l = np.empty((B, L - 1, b, b))
    for m in range(B):
        M = pins.random_spd(b, rng, load=1.0)
        d[m] = 2.01 * M
        l[m] = -M
    Gd, Gl, ld, info = ssa.chain(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    torch.cuda.synchronize()
    Od, Ol, Old, Oinfo = oracle.chain(d, l)
    assert not info.any() and not Oinfo.any()
    e = max(_cmp("G_diag", Gd, Od, torch.float64), _cmp("G_lower", Gl, Ol, torch.float64))
    _cmp_ld(ld, Old, L, torch.float64)
    say("  worst rel err %.2e" % e)


@pytest.mark.parametrize("k", [3, 7, 8, 12, 31, 63])
def test_chain_b32_segments_not_pd_info(ssa, k):
    """One bad block in a segment interior (3, 12), at a separator (7, 31,
    63 with 8 segments of 8 blocks) or first in a segment (8): the reported
    block is the bad one, as in the sequential order."""
    d, l = spdgen.chain(3, 64, 32, seed=5, diag_load=1.0)
    d[1, k] = -np.eye(32)
    d[2, k, 0, 0] = np.nan
    _, _, ld, info = ssa.chain(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    torch.cuda.synchronize()
    _, _, _, Oinfo = oracle.chain(d, l)
    assert list(Oinfo) == [0, k + 1, k + 1]
    assert list(info.cpu().numpy()) == [0, k + 1, k + 1]
    assert np.isnan(ld.cpu().numpy()[1:]).all() and np.isfinite(float(ld[0]))


@pytest.mark.parametrize("k", [0, 5, 7])
def test_chain_not_pd_info(ssa, k):
    d, l = spdgen.chain(3, 8, 4, seed=0)
    d[1, k] = -np.eye(4)
    d[2, k, 0, 0] = np.nan
    _, _, ld, info = ssa.chain(_to(d, torch.float64), _to(l, torch.float64), return_info=True)
    assert list(info.cpu().numpy()) == [0, k + 1, k + 1]
    assert np.isnan(ld.cpu().numpy()[1:]).all() and np.isfinite(float(ld[0]))
    with pytest.raises(ssa.NotPositiveDefinite):
        ssa.chain(_to(d[:2], torch.float64), _to(l[:2], torch.float64), check=True)


def test_chain_deterministic_and_stream(ssa):
    d, l = spdgen.chain(64, 40, 16, seed=5)
    D, C = _to(d, torch.float64), _to(l, torch.float64)
    a = ssa.chain(D, C)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        junk = torch.randn(4096, 4096, device=DEV) @ torch.randn(4096, 4096, device=DEV)
        b_ = ssa.chain(D, C)
    s.synchronize()
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x, y)
    del junk


def test_chain_leading_batch_dims(ssa):
    d, l = spdgen.chain(6, 5, 3, seed=2)
    Gd, Gl, ld = ssa.chain(_to(d, torch.float64).reshape(2, 3, 5, 3, 3),
                           _to(l, torch.float64).reshape(2, 3, 4, 3, 3))
    Od, Ol, Old, _ = oracle.chain(d, l)
    assert ld.shape == (2, 3)
    _cmp("G_diag", Gd.reshape(6, 5, 3, 3), Od, torch.float64)


def test_chain_empty_batch(ssa):
    Gd, Gl, ld = ssa.chain(torch.zeros(0, 4, 3, 3, dtype=torch.float64, device=DEV),
                           torch.zeros(0, 3, 3, 3, dtype=torch.float64, device=DEV))
    assert Gd.shape == (0, 4, 3, 3) and ld.shape == (0,)


# ------------------------------------------------------------------ star
def run_star(ssa, B, K, b, dt, seed=0, mats=None):
    c, lv, cp = spdgen.star(B, K, b, seed=seed)
    say("star B=%d K=%d b=%d %s" % (B, K, b, dt))
    Gc, Gl, Gx, ld, info = ssa.star(_to(c, dt), _to(lv, dt), _to(cp, dt), return_info=True)
    torch.cuda.synchronize()
    sel = slice(None) if mats is None else list(mats)
    c, lv, cp = c[sel], lv[sel], cp[sel]
    Oc, Ol, Ox, Old, Oinfo = oracle.star(_as_used(c, dt), _as_used(lv, dt), _as_used(cp, dt))
    assert np.array_equal(info.cpu().numpy()[sel], Oinfo)
    _cmp("G_center", Gc[sel], Oc, dt)
    if K:
        _cmp("G_leaf", Gl[sel], Ol, dt)
        _cmp("G_cross", Gx[sel], Ox, dt)
    _cmp_ld(ld[sel], Old, K + 1, dt)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("B,K,b", [(1, 0, 3), (2, 1, 1), (3, 5, 4), (2, 33, 8), (2, 70, 16),
                                   (2, 9, 32), (1, 300, 5)])
def test_star_small(ssa, B, K, b, dt):
    run_star(ssa, B, K, b, DT[dt], seed=K + b)


@pytest.mark.timeout(600)
def test_star_workload_b32(ssa):
    """256 stars of 1024 leaves of 32, float64; the oracle checks every star."""
    run_star(ssa, 256, 1024, 32, torch.float64, seed=0)


def test_star_not_pd_info(ssa):
    c, lv, cp = spdgen.star(3, 6, 3, seed=0)
    lv[1, 4] = -np.eye(3)
    c[2] = -np.eye(3)
    *_, ld, info = ssa.star(_to(c, torch.float64), _to(lv, torch.float64),
                            _to(cp, torch.float64), return_info=True)
    assert list(info.cpu().numpy()) == [0, 6, 1]


# ------------------------------------------------------------------ tree
def run_tree(ssa, parent, b, dt, seed=1):
    n = len(parent)
    d, e = spdgen.tree(parent, b, seed=seed)
    say("tree n=%d b=%d %s" % (n, b, dt))
    Gd, Ge, ld, info = ssa.tree(parent, _to(d, dt), _to(e, dt), return_info=True)
    torch.cuda.synchronize()
    Od, Oe, Old, Oinfo = oracle.tree(parent, _as_used(d, dt), _as_used(e, dt))
    assert int(info) == Oinfo
    _cmp("G_diag", Gd, Od, dt)
    root = int(np.where(np.asarray(parent) < 0)[0][0])
    mask = np.arange(n) != root
    if n > 1:
        _cmp("G_edge", Ge[torch.from_numpy(mask).to(DEV)], Oe[mask], dt)
    assert torch.all(Ge[root] == 0)
    _cmp_ld(ld.reshape(1), np.array([Old]), n, dt)


def _perm_tree(n, seed):
    rng = np.random.default_rng(seed)
    p0 = spdgen.random_recursive_tree(n, seed)
    perm = rng.permutation(n)
    p = np.empty(n, np.int32)
    p[perm] = np.where(p0 < 0, -1, perm[np.maximum(p0, 0)])
    return p


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("topo,n,b", [("random", 1, 3), ("random", 2, 2), ("random", 50, 1),
                                      ("random", 700, 8), ("path", 40, 4), ("star", 60, 3),
                                      ("balanced", 255, 2), ("perm", 300, 5),
                                      ("random", 100, 16), ("random", 40, 32)])
def test_tree_small(ssa, topo, n, b, dt):
    parent = {"random": lambda: spdgen.random_recursive_tree(n, 2),
              "path": lambda: spdgen.path_tree(n), "star": lambda: spdgen.star_tree(n),
              "balanced": lambda: spdgen.balanced_tree(n, 2),
              "perm": lambda: _perm_tree(n, 3)}[topo]()
    run_tree(ssa, parent, b, DT[dt], seed=n)


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("n,b", [(16383, 8), (32767, 5)])
def test_tree_wide_and_narrow_levels(ssa, n, b, dt):
    """Balanced binary trees (levels of 1 up to 8192 and 16384 nodes): every
    parent has two children, so every handshake of the single-launch schedule
    has two producers, from one-tile levels to levels of thousands of tiles."""
    run_tree(ssa, spdgen.balanced_tree(n, 2), b, DT[dt], seed=n)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_tree_workload_b8_random(ssa, dt):
    """Random recursive tree of 262144 nodes (seed 1), b = 8, full oracle."""
    run_tree(ssa, spdgen.random_recursive_tree(262144, 1), 8, DT[dt], seed=1)


def test_tree_wait_limit_reports_timeout(ssa):
    """With a zero wait bound the single-launch schedule gives up at the first
    unready flag: the call still ends, with info = -1 and a NaN log det.  A
    path tree makes every tile wait for the one just before it.  With the
    default bound restored, the same call is exact again."""
    p = spdgen.path_tree(3000)
    d, e = spdgen.tree(p, 4, seed=3)
    D, E = _to(d, torch.float64), _to(e, torch.float64)
    old = ssa.wait_limit()
    try:
        ssa.set_wait_limit(0)
        _, _, ld, info = ssa.tree(p, D, E, return_info=True)
        torch.cuda.synchronize()
        with pytest.raises(ssa.WaitTimeout):
            ssa.tree(p, D, E, check=True)
    finally:
        ssa.set_wait_limit(old)
    assert int(info) == ssa.INFO_WAIT_TIMEOUT and np.isnan(float(ld))
    run_tree(ssa, p, 4, torch.float64, seed=3)


def test_tree_not_pd_info(ssa):
    p = spdgen.random_recursive_tree(64, 1)
    d, e = spdgen.tree(p, 3)
    depth = oracle.tree_depths(p)
    for bad in ([5], [0], [10, 40, 63]):
        d2 = d.copy()
        for v in bad:
            d2[v] = -np.eye(3)
        _, _, ld, info = ssa.tree(p, _to(d2, torch.float64), _to(e, torch.float64),
                                  return_info=True)
        _, _, _, Oinfo = oracle.tree(p, d2, e)
        assert int(info) == Oinfo and np.isnan(float(ld))
    assert depth.max() > 1
