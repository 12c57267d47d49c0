"""The chain entry point that allocates nothing (selinv_chain_noalloc_*,
scratch in the library's static per-device array) against the workspace
entry point (selinv_chain_*) on the same inputs: the same kernels run, so
every output matches to the parity tolerance (in fact bit for bit).  Two
calls in a row, the second on a smaller input, for each kernel family
(b <= 8 short and long chains, b = 16, b = 32 with few long chains), then a
request larger than the static array is refused without a launch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import spdgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.float64: 1e-10, torch.float32: 2e-4}


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


def _noalloc(ssa, D, C):
    """Direct C-ABI call of selinv_chain_noalloc_*; returns the outputs."""
    *batch, L, b, _ = D.shape
    B = int(np.prod(batch)) if batch else 1
    Gd, Gl = torch.empty_like(D), torch.empty_like(C)
    ld = torch.empty(tuple(batch), dtype=torch.float64, device=DEV)
    info = torch.empty(tuple(batch), dtype=torch.int32, device=DEV)
    fn = getattr(ssa.lib(), "selinv_chain_noalloc_" + ("f64" if D.dtype == torch.float64
                                                         else "f32"))
    rc = fn(B, L, b, ctypes.c_void_p(D.data_ptr()), ctypes.c_void_p(C.data_ptr()),
            ctypes.c_void_p(Gd.data_ptr()), ctypes.c_void_p(Gl.data_ptr()),
            ctypes.c_void_p(ld.data_ptr()), ctypes.c_void_p(info.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc
    return Gd, Gl, ld, info


def _rel(a, b):
    num = torch.linalg.matrix_norm(a.double() - b.double())
    den = torch.linalg.matrix_norm(b.double()).clamp_min(1e-300)
    return float((num / den).max()) if num.numel() else 0.0


@pytest.mark.parametrize("dt", [torch.float64, torch.float32])
@pytest.mark.parametrize("first,second", [((3, 20, 4), (2, 7, 4)),          # b <= 8, in LDS
                                          ((70, 40, 6), (65, 33, 6)),       # b <= 8, rows
                                          ((64, 64, 16), (9, 10, 16)),      # b = 16
                                          ((2, 600, 32), (1, 130, 32))])    # b = 32 segments
def test_noalloc_matches_workspace_entry(ssa, dt, first, second):
    for k, (B, L, b) in enumerate((first, second)):
        load = 1.0 if b == 32 else 2.0
        d, l = spdgen.chain(B, L, b, seed=40 + k, diag_load=load)
        D, C = torch.from_numpy(d).to(DEV).to(dt), torch.from_numpy(l).to(DEV).to(dt)
        say("noalloc B=%d L=%d b=%d %s" % (B, L, b, dt))
        Gd, Gl, ld, info = _noalloc(ssa, D, C)
        Rd, Rl, Rld, Rinfo = ssa.chain(D, C, return_info=True)
        torch.cuda.synchronize()
        assert torch.equal(info, Rinfo) and not info.any()
        assert _rel(Gd, Rd) <= TOL[dt] and _rel(Gl, Rl) <= TOL[dt]
        assert float((ld - Rld).abs().max()) <= (1e-8 if dt == torch.float64 else 1e-3) * L
        assert torch.equal(Gd, Rd) and torch.equal(Gl, Rl) and torch.equal(ld, Rld)


def test_noalloc_binding_and_limit(ssa):
    d, l = spdgen.chain(5, 9, 16, seed=3)
    D, C = torch.from_numpy(d).to(DEV), torch.from_numpy(l).to(DEV)
    a = ssa.chain_noalloc(D, C)
    r = ssa.chain(D, C)
    torch.cuda.synchronize()
    for x, y in zip(a, r):
        assert torch.equal(x, y)
    cap = ssa.lib().selinv_chain_static_scratch_bytes()
    assert cap == 256 << 20
    # more chains than the static array can hold state for: refused, nothing launched
    per_chain = ssa.lib().selinv_chain_workspace_bytes(8, 1, 64, 16)
    B = cap // per_chain + 2
    assert ssa.lib().selinv_chain_workspace_bytes(8, B, 64, 16) > cap
    fn = ssa.lib().selinv_chain_noalloc_f64
    p = ctypes.c_void_p(D.data_ptr())  # never dereferenced: the size check comes first
    rc = fn(B, 64, 16, p, p, p, p, p, None, None)
    assert rc == ssa.SCRATCH_LIMIT
