"""GPU parity of the general sparse SPD selected inverse (junction tree)
through the C ABI against the oracle (oracle.junction, pinned to dense
inverses, the Cholesky fill structure and the tree / chain oracles) on the
same seeded inputs: the filled pattern exactly, every block of G on it, the
log determinant and the failure index.

Tolerances: relative Frobenius error per block <= 1e-10 (float64) or 2e-4
(float32); log det relative 1e-12 (float64) or 1e-5 (float32).  Fill blocks
of S join nodes far apart in the graph, where A^-1 has decayed by many orders
of magnitude; in float32 such a block's own norm is no meaningful scale, so
for float32 a fill block (i, j) is measured against
sqrt(|G_ii|_F |G_jj|_F), the bound an SPD inverse places on it
(|G_ij|_F <= sqrt(|G_ii|_F |G_jj|_F) up to a factor b^(1/2)); the blocks of
the input pattern keep the per-block relative bound in both precisions.
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


def _cmp(name, got, ref, dt):
    err = pins.rel_fro(got.double().cpu().numpy(), ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dt], "%s rel err %.3e > %.1e" % (name, worst, TOL[dt])
    return worst


def run(ssa, n, e, b, B, dt, seed, order=None, label=""):
    say("junction %s n=%d m=%d b=%d B=%d %s" % (label, n, e.shape[1], b, B, dt))
    d, v = spdgen.graph(e, n, b, B=B, seed=seed)
    Gd, S, Gl, ld, info = ssa.junction(_to(d, dt), e, _to(v, dt), order=order, return_info=True)
    torch.cuda.synchronize()
    Od, OS, Ol, Old, Oinfo = oracle.junction(_as_used(d, dt), e, _as_used(v, dt), order=order)
    assert np.array_equal(S.numpy(), OS)
    assert np.array_equal(info.cpu().numpy(), Oinfo) and (Oinfo == 0).all()
    err = _cmp("G_diag", Gd, Od, dt)
    if OS.shape[1] and dt == torch.float64:
        err = max(err, _cmp("G_lower", Gl, Ol, dt))
    elif OS.shape[1]:
        # blocks of the input pattern: per-block relative Frobenius, as everywhere
        inp = {(int(a), int(c)) for a, c in zip(e[0], e[1])}
        on = np.array([(int(a), int(c)) in inp for a, c in zip(OS[0], OS[1])], bool)
        Glh = Gl.double().cpu().numpy()
        if on.any():
            e1 = float(pins.rel_fro(Glh[:, on], Ol[:, on]).max())
            assert e1 <= TOL[dt], "G_lower (input pattern) rel err %.3e" % e1
            err = max(err, e1)
        # fill blocks: against sqrt(|G_ii| |G_jj|)
        dn = np.sqrt((Od ** 2).sum(axis=(-1, -2)))                 # [B, n]
        scale = np.sqrt(dn[..., OS[0]] * dn[..., OS[1]])           # [B, nnz]
        diff = np.sqrt(((Glh - Ol) ** 2).sum(axis=(-1, -2)))
        e2 = float((diff / scale).max())
        say("  G_lower error against sqrt(|G_ii| |G_jj|): %.2e (per-block relative %.2e; "
            "fill blocks %d of %d)" % (e2, float(pins.rel_fro(Glh, Ol).max()), int((~on).sum()),
                                       on.size))
        assert e2 <= TOL[dt], "G_lower scaled err %.3e" % e2
        err = max(err, e2)
    ldg = ld.cpu().numpy()
    assert np.all(np.abs(ldg - Old) <= LDTOL[dt] * np.maximum(1.0, np.abs(Old)))
    Gd64 = Gd.double().cpu()
    assert torch.equal(Gd64, Gd64.transpose(-1, -2))
    say("  nnz %d, worst rel err %.2e" % (OS.shape[1], err))


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("r,c,b,B", [(1, 1, 3, 2), (1, 9, 2, 1), (3, 3, 2, 2), (4, 5, 1, 3),
                                     (6, 6, 4, 2), (8, 8, 8, 2), (5, 7, 16, 1), (4, 4, 32, 1),
                                     (7, 5, 5, 2)])
def test_grid(ssa, r, c, b, B, dt):
    run(ssa, r * c, spdgen.grid_edges(r, c), b, B, DT[dt], seed=r * c + b, label="grid")


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("n,extra,b", [(30, 40, 3), (100, 150, 2), (12, 60, 8), (50, 10, 17)])
def test_random_graph(ssa, n, extra, b, dt):
    run(ssa, n, spdgen.random_graph_edges(n, extra, seed=n), b, 2, DT[dt], seed=n, label="random")


@pytest.mark.parametrize("kind", ["natural", "reversed", "random"])
def test_explicit_order(ssa, kind):
    n = 49
    order = {"natural": np.arange(n), "reversed": np.arange(n)[::-1].copy(),
             "random": np.random.default_rng(5).permutation(n)}[kind]
    run(ssa, n, spdgen.grid_edges(7, 7), 4, 2, torch.float64, seed=3, order=order, label=kind)


def test_tree_pattern_matches_tree_kernel(ssa):
    parent = spdgen.random_recursive_tree(500, 3)
    n, b = 500, 6
    d, ed = spdgen.tree(parent, b, seed=2)
    kids = [v for v in range(n) if parent[v] >= 0]
    e = np.array([(max(v, int(parent[v])), min(v, int(parent[v]))) for v in kids],
                 np.int32).T.copy()
    ev = np.stack([ed[v] if parent[v] > v else ed[v].T for v in kids])
    Gd, S, Gl, ld = ssa.junction(_to(d, torch.float64), e, _to(ev, torch.float64))
    Td, Te, Tld = ssa.tree(parent, _to(d, torch.float64), _to(ed, torch.float64))
    assert S.shape[1] == n - 1
    sc = float(Td.abs().max())
    assert float((Gd - Td).abs().max()) <= 1e-12 * sc
    assert abs(float(ld) - float(Tld)) <= 1e-11 * abs(float(Tld))
    look = {(int(i), int(j)): k for k, (i, j) in enumerate(S.numpy().T)}
    for v in kids[::7]:
        p = int(parent[v])
        g = Gl[look[(max(v, p), min(v, p))]]
        g = g if p > v else g.T
        assert float((g - Te[v]).abs().max()) <= 1e-12 * sc


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_workload_grid64_b8(ssa, dt):
    """A batch of 16 matrices on the 64 x 64 grid pattern, b = 8, full oracle."""
    run(ssa, 4096, spdgen.grid_edges(64, 64), 8, 16, DT[dt], seed=0, label="grid64")


def test_not_positive_definite(ssa):
    e = spdgen.grid_edges(5, 5)
    d, v = spdgen.graph(e, 25, 3, B=3, seed=4)
    d[1, 12] = -np.eye(3)
    Gd, S, Gl, ld, info = ssa.junction(_to(d, torch.float64), e, _to(v, torch.float64),
                                       return_info=True)
    torch.cuda.synchronize()
    _, _, _, Old, Oinfo = oracle.junction(d, e, v)
    assert list(info.cpu().numpy()) == list(Oinfo) and Oinfo[1] == 13
    assert np.isnan(ld[1].item()) and np.isfinite(ld[0].item()) and np.isfinite(ld[2].item())
    with pytest.raises(ssa.NotPositiveDefinite):
        ssa.junction(_to(d, torch.float64), e, _to(v, torch.float64), check=True)


def test_empty_batch_and_no_edges(ssa):
    e = np.zeros((2, 0), np.int32)
    d, v = spdgen.graph(e, 4, 2, B=2, seed=1)
    Gd, S, Gl, ld = ssa.junction(_to(d, torch.float64), e, _to(v, torch.float64))
    ref = np.linalg.inv(d)
    assert S.shape == (2, 0) and Gl.shape == (2, 0, 2, 2)
    assert np.abs(Gd.cpu().numpy() - ref).max() <= 1e-13 * np.abs(ref).max()
    g = spdgen.grid_edges(2, 2)
    d0 = torch.zeros((0, 4, 2, 2), dtype=torch.float64, device=DEV)
    v0 = torch.zeros((0, 4, 2, 2), dtype=torch.float64, device=DEV)
    Gd, S, Gl, ld = ssa.junction(d0, g, v0)
    assert Gd.shape == (0, 4, 2, 2) and ld.shape == (0,)


def test_repeated_calls_are_bitwise_identical(ssa):
    """Fixed summation orders and no atomics in the arithmetic: two calls on
    the same input agree bit for bit."""
    e = spdgen.grid_edges(12, 12)
    d, v = spdgen.graph(e, 144, 4, B=3, seed=6)
    D, V = _to(d, torch.float64), _to(v, torch.float64)
    a = ssa.junction(D, e, V)
    torch.cuda.synchronize()
    for _ in range(3):
        c = ssa.junction(D, e, V)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, c))


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_logdet_only(ssa, dt):
    """The factorisation alone gives the same log det (bit for bit: the same
    forward kernels) and the same failure index as the full call."""
    e = spdgen.grid_edges(9, 11)
    d, v = spdgen.graph(e, 99, 8, B=3, seed=8)
    d[2, 40] = -np.eye(8)
    D, V = _to(d, DT[dt]), _to(v, DT[dt])
    ld, info = ssa.junction_logdet(D, e, V, return_info=True)
    _, _, _, ld_full, info_full = ssa.junction(D, e, V, return_info=True)
    torch.cuda.synchronize()
    assert torch.equal(info, info_full) and list(info.cpu().numpy())[:2] == [0, 0]
    assert int(info[2]) == 41
    assert torch.equal(ld[:2], ld_full[:2]) and torch.isnan(ld[2])
    _, _, _, Old, Oinfo = oracle.junction(_as_used(d, DT[dt]), e, _as_used(v, DT[dt]))
    assert list(Oinfo) == list(info.cpu().numpy())
    assert np.all(np.abs(ld[:2].cpu().numpy() - Old[:2]) <= LDTOL[DT[dt]] * np.abs(Old[:2]))
