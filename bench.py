"""Benchmark of the selected inverse on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype f64|f32]

One step = one call of the C ABI over one batch of synthetic input already
resident in HBM (all collect, root and distribute work of every matrix).
Default workload: the largest single-GPU configuration, 64 block-tridiagonal
chains of 16384 blocks of 32 in float64 (diagonal load 1.0).  The other
workloads (one chain of 8 blocks of 4; 4096 chains of 64 blocks of 16 in
float64 and float32; 256 stars of 1024 leaves of 32; the random recursive
tree of 262144 nodes, b = 8, float64 and float32) are timed in the same run
and reported compactly under "configs".  Prints ONE JSON line.

Metric: nominal selected-inverse GFLOP/s (7 b^3 per non-root block, b^3 per
root, never the executed count) and block-rows/s; roofline fraction of the
call against MI355X HBM bandwidth (8 TB/s) on compulsory bytes (every input
block read once, every output block written once).  Every workload here has
a compulsory arithmetic intensity below the fp64 / fp32 ridge points, so the
HBM roofline is the binding one; the fraction of the matrix-core peak is
reported beside it.

``--op logdet`` times the log-det-only call (the collect pass without a
stored factor); ``--op solve`` / ``--op sample`` time x = A^{-1} y and
x = L^{-T} D^{-1/2} z with ``--k`` right-hand sides from a factor computed
once before the timed region (nominal 8 b^2 k and 5 b^2 k + b^3 / 3 flop per
block; compulsory bytes = factor + edge blocks + vectors in and out).  For the
junction workload the solve / sample run on the filled pattern: 2 b^2 k per
block of S in each sweep plus the pivot solves; compulsory bytes = the
factor's S blocks and pivot triangles + vectors in and out.

``--op vjp`` times the reverse mode instead (one call = the vector-Jacobian
product of every matrix of the batch, seeded normal cotangents on every
output): nominal 22 b^3 per non-root block and 4 b^3 per root, compulsory
bytes = inputs + cotangents read once, input cotangents written once.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "chain_b32_long"
# the other forward workloads, timed compactly in the default run
OTHER_CONFIGS = (("chain_b4_single", "f64"), ("chain_b16_batched", "f64"),
                 ("chain_b16_batched", "f32"), ("star_b32", "f64"),
                 ("tree_b8_random", "f64"), ("tree_b8_random", "f32"))

HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6
FP32_PEAK_TFLOPS = 157.3


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the HIP library sources; counter-derived traffic is reported
    only when it was measured on exactly these sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_spd_selected_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, dtname):
    """HBM bytes per call from FETCH_SIZE / WRITE_SIZE counter runs (scaled by
    the plain-copy calibration), or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get("%s/%s" % (workload, dtname))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_call")


_JCOUNTS = {}


def junction_counts(cfg):
    """(n, m, nnz, sum_v k_v, sum_v k_v^2) of a junction workload's filled
    pattern, k_v = the number of later neighbours of v, from the library's
    host-side symbolic analysis."""
    key = (cfg["rows"], cfg["cols"])
    if key not in _JCOUNTS:
        import numpy as np
        import spdgen
        import sparse_spd_selected_amd as ssa
        n = cfg["rows"] * cfg["cols"]
        e = spdgen.grid_edges(cfg["rows"], cfg["cols"])
        order, S, _ = ssa.junction_symbolic(n, e)
        pos = np.empty(n, np.int64)
        pos[order] = np.arange(n)
        first = np.where(pos[S[0]] < pos[S[1]], S[0], S[1])      # the earlier node of each pair
        k = np.bincount(first, minlength=n).astype(np.int64)
        _JCOUNTS[key] = (n, e.shape[1], S.shape[1], int(k.sum()), int((k * k).sum()))
    return _JCOUNTS[key]


def nominal_flops(kind, cfg, op="selinv"):
    """Per non-root block: forward 7 b^3 (inverse b^3, X 2 b^3, symmetric M
    b^3, V 2 b^3, symmetric G b^3); reverse mode 22 b^3 (collect: inverse b^3,
    X 2, M 1, W 2, Z 2, N 2, P 3; distribute: Dbar X 2, G Z 2, X^T Q 2, G X 2,
    symmetric X^T V 1).  Per root: b^3 forward, 4 b^3 reverse."""
    b = cfg["b"]
    nblk = block_rows(kind, cfg)
    k = cfg.get("k", 1)
    if kind == "junction" and op in ("solve", "sample"):
        # per S block (w, v): 2 b^2 k in each sweep it enters; per node the
        # pivot solve (two triangular b x b solves, b^2 k each) for a solve,
        # one (R_v^-T) for a sample
        n, m, nnz, sk, sk2 = junction_counts(cfg)
        sweeps, tri = (2, 2) if op == "solve" else (1, 1)
        return cfg["B"] * b * b * k * (2 * sweeps * nnz + tri * n)
    if op == "solve":
        return 8 * b * b * k * nblk
    if op == "sample":
        return (5 * b * b * k + b ** 3 // 3) * nblk
    if kind == "bidiag":  # general inverse 2 b^3 per block, two products per lower block
        return cfg["B"] * (2 * b ** 3 * cfg["L"] + 4 * b ** 3 * (cfg["L"] - 1))
    if kind == "nonsym_tree":  # collect 6 b^3, distribute 10 b^3 per non-root; root 2 b^3
        return 16 * b ** 3 * (cfg["n"] - 1) + 2 * b ** 3
    if kind == "junction" and op == "logdet":  # the factorisation part below
        n, m, nnz, sk, sk2 = junction_counts(cfg)
        return cfg["B"] * b ** 3 * (sk2 + sk + n // 3)
    if kind == "junction":
        # per node with k later neighbours: factor k^2 b^3 (k(k-1)/2 Schur
        # products of 2 b^3 and k symmetric ones of b^3) + k b^3 (triangular
        # scaling) + b^3 / 3 (Cholesky); Takahashi 2 k^2 b^3 (G_NN W) + k b^3
        # (times R^-1) + k b^3 (symmetric W^T G) + b^3 (R^-T X) + b^3 / 3 (R^-1)
        n, m, nnz, sk, sk2 = junction_counts(cfg)
        return cfg["B"] * b ** 3 * (3 * sk2 + 3 * sk + n * 5 // 3)
    per, root = {"selinv": (7, 1), "vjp": (22, 4), "logdet": (4, 1)}[op]
    if kind == "chain":
        return cfg["B"] * (per * b ** 3 * (cfg["L"] - 1) + root * b ** 3)
    if kind == "star":
        return cfg["B"] * (per * b ** 3 * cfg["K"] + root * b ** 3)
    return per * b ** 3 * (cfg["n"] - 1) + root * b ** 3


def compulsory_bytes(kind, cfg, w, op="selinv"):
    """Input blocks read once + output blocks written once + logdet (f64) +
    info (int32) (+ parent indices for the tree).  Reverse mode: inputs and
    output cotangents read once, input cotangents written once, logdet_bar
    (f64) and info."""
    b2 = cfg["b"] ** 2
    if kind == "bidiag":  # diag, lower in; G_diag, G_lower out; info
        return cfg["B"] * (2 * (2 * cfg["L"] - 1) * b2 * w + 4)
    if kind == "nonsym_tree":  # diag, up, down in (root edges skipped); three outputs
        return (3 * cfg["n"] - 2 + 3 * cfg["n"]) * b2 * w + 4 * cfg["n"] + 4
    if kind == "junction":  # diag, edge_val in; G_diag, G_lower (on S) out; logdet, info
        n, m, nnz, sk, sk2 = junction_counts(cfg)
        if op in ("solve", "sample"):  # the factor's S blocks and pivots once, vectors in, out
            b = cfg["b"]
            return cfg["B"] * ((nnz * b2 + n * b * (b + 1) // 2) * w
                               + 2 * n * b * cfg.get("k", 1) * w)
        if op == "logdet":
            return cfg["B"] * ((n + m) * b2 * w + 8 + 4)
        return cfg["B"] * ((2 * n + m + nnz) * b2 * w + 8 + 4)
    if op == "logdet":  # inputs read once, log det and info written
        if kind == "chain":
            return cfg["B"] * ((2 * cfg["L"] - 1) * b2 * w + 12)
        if kind == "star":
            return cfg["B"] * ((2 * cfg["K"] + 1) * b2 * w + 12)
        return (2 * cfg["n"] - 1) * b2 * w + 4 * cfg["n"] + 12
    if op in ("solve", "sample"):  # factor + edge blocks + vectors in and out
        b = cfg["b"]
        pk = (b * (b + 1) // 2 + 3) // 4 * 4
        nblk = block_rows(kind, cfg)
        nedge = nblk - (cfg["B"] if kind in ("chain", "star") else 1)
        return (nblk * pk + nedge * b2 + 2 * nblk * b * cfg.get("k", 1)) * w
    if op == "vjp":
        if kind == "chain":
            return cfg["B"] * ((6 * cfg["L"] - 3) * b2 * w + 8 + 4)
        if kind == "star":
            return cfg["B"] * ((6 * cfg["K"] + 3) * b2 * w + 8 + 4)
        return (6 * cfg["n"] - 2) * b2 * w + 4 * cfg["n"] + 8 + 4
    if kind == "chain":
        return cfg["B"] * ((4 * cfg["L"] - 2) * b2 * w + 8 + 4)
    if kind == "star":
        return cfg["B"] * ((4 * cfg["K"] + 2) * b2 * w + 8 + 4)
    return (4 * cfg["n"] - 1) * b2 * w + 4 * cfg["n"] + 8 + 4


def block_rows(kind, cfg):
    if kind in ("chain", "bidiag"):
        return cfg["B"] * cfg["L"]
    if kind == "junction":
        return cfg["B"] * cfg["rows"] * cfg["cols"]
    if kind == "star":
        return cfg["B"] * (cfg["K"] + 1)
    return cfg["n"]


def make_inputs(kind, cfg, dt, dev):
    import numpy as np
    import torch
    import spdgen
    if kind == "chain":
        d, l = spdgen.chain(cfg["B"], cfg["L"], cfg["b"], seed=cfg["seed"],
                            diag_load=cfg["diag_load"])
        return [torch.from_numpy(x).to(dev).to(dt) for x in (d, l)], None
    if kind == "star":
        arrs = spdgen.star(cfg["B"], cfg["K"], cfg["b"], seed=cfg["seed"],
                           diag_load=cfg["diag_load"])
        return [torch.from_numpy(x).to(dev).to(dt) for x in arrs], None
    if kind == "bidiag":
        d, l = spdgen.nonsym_bidiag(cfg["B"], cfg["L"], cfg["b"], seed=cfg["seed"],
                                    diag_load=cfg["diag_load"])
        return [torch.from_numpy(x).to(dev).to(dt) for x in (d, l)], None
    if kind == "junction":
        e = spdgen.grid_edges(cfg["rows"], cfg["cols"])
        d, v = spdgen.graph(e, cfg["rows"] * cfg["cols"], cfg["b"], B=cfg["B"], seed=cfg["seed"],
                            diag_load=cfg["diag_load"])
        return [torch.from_numpy(x).to(dev).to(dt) for x in (d, v)], e
    parent = spdgen.random_recursive_tree(cfg["n"], cfg["seed"])
    if kind == "nonsym_tree":
        arrs = spdgen.nonsym_tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        return [torch.from_numpy(x).to(dev).to(dt) for x in arrs], np.asarray(parent)
    d, e = spdgen.tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
    return [torch.from_numpy(x).to(dev).to(dt) for x in (d, e)], np.asarray(parent)


def make_cotangents(kind, inputs, cfg, dt, dev):
    """Seeded normal cotangents, one per output (orientation of the outputs:
    the shapes of the inputs), plus logdet_bar."""
    import torch
    import spdgen
    shapes = [tuple(x.shape) for x in inputs]
    bars = [torch.from_numpy(spdgen.cotangent(sh, seed=cfg["seed"], k=i)).to(dev).to(dt)
            for i, sh in enumerate(shapes)]
    nb = 1 if kind == "tree" else cfg["B"]
    lb = torch.from_numpy(spdgen.cotangent((nb,), seed=cfg["seed"], k=len(shapes))).to(dev)
    return bars, lb


def run_gpu(kind, cfg, dtname, steps, warmup, op="selinv", graph=False):
    import torch
    import sparse_spd_selected_amd as ssa
    ssa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    dt = torch.float64 if dtname == "f64" else torch.float32
    inputs, parent = make_inputs(kind, cfg, dt, dev)
    if op in ("solve", "sample"):
        import spdgen
        k = cfg.get("k", 1)
        if kind == "chain":
            f = ssa.chain_factor(*inputs)
            v = spdgen.cotangent((cfg["B"], cfg["L"], cfg["b"], k), seed=cfg["seed"])
            v = torch.from_numpy(v).to(dev).to(dt)
            call = (lambda: f.solve(v)) if op == "solve" else (lambda: f.sample(z=v))
        elif kind == "star":
            f = ssa.star_factor(*inputs)
            vc = torch.from_numpy(spdgen.cotangent((cfg["B"], cfg["b"], k), seed=cfg["seed"],
                                                   k=0)).to(dev).to(dt)
            vl = torch.from_numpy(spdgen.cotangent((cfg["B"], cfg["K"], cfg["b"], k),
                                                   seed=cfg["seed"], k=1)).to(dev).to(dt)
            call = ((lambda: f.solve(vc, vl)) if op == "solve"
                    else (lambda: f.sample(z_center=vc, z_leaves=vl)))
        elif kind == "junction":  # plan and factor once, untimed
            e = parent
            plan = ssa.junction_plan(cfg["rows"] * cfg["cols"], e, cfg["b"], dt, dev)
            f = ssa.junction_factor(inputs[0], e, inputs[1], plan=plan)
            v = torch.from_numpy(spdgen.cotangent((cfg["B"], cfg["rows"] * cfg["cols"], cfg["b"],
                                                   k), seed=cfg["seed"])).to(dev).to(dt)
            call = (lambda: f.solve(v)) if op == "solve" else (lambda: f.sample(z=v))
        else:
            plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
            f = ssa.tree_factor(parent, *inputs, plan=plan)
            v = torch.from_numpy(spdgen.cotangent((cfg["n"], cfg["b"], k),
                                                  seed=cfg["seed"])).to(dev).to(dt)
            call = (lambda: f.solve(v)) if op == "solve" else (lambda: f.sample(z=v))
    elif op == "logdet" and kind == "junction":
        e = parent
        plan = ssa.junction_plan(cfg["rows"] * cfg["cols"], e, cfg["b"], dt, dev)
        call = lambda: ssa.junction_logdet(inputs[0], e, inputs[1], plan=plan)
    elif op == "logdet":
        if kind == "chain":
            call = lambda: ssa.chain_logdet(*inputs)
        elif kind == "star":
            call = lambda: ssa.star_logdet(*inputs)
        else:
            plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
            f0 = ssa.tree_factor(parent, *inputs, keep_factor=False, plan=plan)
            call = lambda: ssa.tree_factor(parent, *inputs, keep_factor=False, plan=plan).logdet
    elif op == "vjp":
        bars, lb = make_cotangents(kind, inputs, cfg, dt, dev)
        if kind == "chain":
            call = lambda: ssa.chain_vjp(*inputs, *bars, lb)
        elif kind == "star":
            call = lambda: ssa.star_vjp(*inputs, *bars, lb)
        else:
            plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
            call = lambda: ssa.tree_vjp(parent, *inputs, *bars, lb, plan=plan)
    elif kind == "chain":
        call = lambda: ssa.chain(*inputs)
    elif kind == "star":
        call = lambda: ssa.star(*inputs)
    elif kind == "bidiag":
        call = lambda: ssa.bidiag(*inputs)
    elif kind == "nonsym_tree":
        plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
        call = lambda: ssa.nonsym_tree(parent, *inputs, plan=plan)
    elif kind == "junction":  # the symbolic plan is built once per pattern, untimed
        e = parent
        plan = ssa.junction_plan(cfg["rows"] * cfg["cols"], e, cfg["b"], dt, dev)
        call = lambda: ssa.junction(inputs[0], e, inputs[1], plan=plan)
    elif graph:  # the level-set schedule recorded once as a HIP graph, untimed
        plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
        g = ssa.tree_graph(parent, *inputs, plan=plan)
        call = g.launch
    else:
        plan = ssa.tree_plan(parent, cfg["b"], dt, dev)
        call = lambda: ssa.tree(parent, *inputs, plan=plan)
    out = None
    for _ in range(warmup):
        out = call()
    torch.cuda.synchronize()
    del out
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        out = call()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [a.elapsed_time(b) for a, b in evs]
    return {"wall_s": wall, "ev_ms": ev_ms}


def cpu_baseline_apply(kind, cfg, op):
    """The oracle's solve / sample (its collect included: the oracle keeps no
    factor) on a bounded sample; value = nominal flops of the sweeps only."""
    import oracle
    import spdgen
    lib = oracle.load()
    k = cfg.get("k", 1)
    if kind == "chain":
        Bs = min(cfg["B"], 1024)
        d, l = spdgen.chain(Bs, cfg["L"], cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        v = spdgen.cotangent((Bs, cfg["L"], cfg["b"], k), seed=cfg["seed"])
        t0 = time.perf_counter()
        oracle.chain_apply(d, l, v, op, lib=lib)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        sample = "%d of %d chains, k = %d, float64, collect + %s" % (Bs, cfg["B"], k, op)
    elif kind == "star":
        Bs = min(cfg["B"], 4)
        c, lv, cp = spdgen.star(Bs, cfg["K"], cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        vc = spdgen.cotangent((Bs, cfg["b"], k), seed=cfg["seed"], k=0)
        vl = spdgen.cotangent((Bs, cfg["K"], cfg["b"], k), seed=cfg["seed"], k=1)
        t0 = time.perf_counter()
        oracle.star_apply(c, lv, cp, vc, vl, op, lib=lib)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        sample = "%d of %d stars, k = %d, float64, collect + %s" % (Bs, cfg["B"], k, op)
    elif kind == "junction":
        Bs = min(cfg["B"], 8)
        n = cfg["rows"] * cfg["cols"]
        e = spdgen.grid_edges(cfg["rows"], cfg["cols"])
        d, val = spdgen.graph(e, n, cfg["b"], B=Bs, seed=cfg["seed"], diag_load=cfg["diag_load"])
        v = spdgen.cotangent((Bs, n, cfg["b"], k), seed=cfg["seed"])
        P = oracle.filled_pattern(n, e, lib=lib)
        t0 = time.perf_counter()
        oracle.junction_apply(d, e, val, v, op, lib=lib, pattern=P)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        sample = ("%d of %d matrices on the %d x %d grid (b=%d), k = %d, float64, "
                  "factorisation + %s, symbolic analysis untimed"
                  % (Bs, cfg["B"], cfg["rows"], cfg["cols"], cfg["b"], k, op))
    else:
        parent = spdgen.random_recursive_tree(cfg["n"], cfg["seed"])
        d, e = spdgen.tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        v = spdgen.cotangent((cfg["n"], cfg["b"], k), seed=cfg["seed"])
        t0 = time.perf_counter()
        oracle.tree_apply(parent, d, e, v, op, lib=lib)
        t = time.perf_counter() - t0
        sub = cfg
        sample = "the whole tree, k = %d, float64, collect + %s, single thread" % (k, op)
    cores = 1 if kind == "tree" else int(lib.oracle_num_threads())
    if kind == "junction":
        cores = min(Bs, cores)
    return {"value": round(nominal_flops(kind, sub, op) / t / 1e9, 3), "unit": "GFLOP/s",
            "cores": cores, "kind": "oracle", "sample": sample, "seconds": round(t, 3),
            "block_rows_per_s": round(block_rows(kind, sub) / t, 1)}


def cpu_baseline_vjp(kind, cfg, op="vjp"):
    """The float64 oracle's VJP, as it stands, on a bounded sample."""
    import oracle
    import spdgen
    lib = oracle.load()
    if kind == "chain":
        Bs = cfg["B"] if cfg["B"] * cfg["L"] * cfg["b"] ** 3 <= 2e9 else max(1, int(2e9 // (cfg["L"] * cfg["b"] ** 3)))
        d, l = spdgen.chain(Bs, cfg["L"], cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        gd = spdgen.cotangent(d.shape, seed=cfg["seed"], k=0)
        gl = spdgen.cotangent(l.shape, seed=cfg["seed"], k=1)
        lb = spdgen.cotangent((Bs,), seed=cfg["seed"], k=2)
        t0 = time.perf_counter()
        oracle.chain_vjp(d, l, gd, gl, lb, lib=lib)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        sample = "%d of %d chains (L=%d, b=%d), float64, reverse mode" % (Bs, cfg["B"], cfg["L"], cfg["b"])
    elif kind == "star":
        Bs = min(cfg["B"], 4)
        c, lv, cp = spdgen.star(Bs, cfg["K"], cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        bars = [spdgen.cotangent(x.shape, seed=cfg["seed"], k=i) for i, x in enumerate((c, lv, cp))]
        lb = spdgen.cotangent((Bs,), seed=cfg["seed"], k=3)
        t0 = time.perf_counter()
        oracle.star_vjp(c, lv, cp, *bars, lb, lib=lib)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        sample = "%d of %d stars (K=%d, b=%d), float64, reverse mode" % (Bs, cfg["B"], cfg["K"], cfg["b"])
    else:
        parent = spdgen.random_recursive_tree(cfg["n"], cfg["seed"])
        d, e = spdgen.tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        gd = spdgen.cotangent(d.shape, seed=cfg["seed"], k=0)
        ge = spdgen.cotangent(e.shape, seed=cfg["seed"], k=1)
        lb = float(spdgen.cotangent((1,), seed=cfg["seed"], k=2)[0])
        t0 = time.perf_counter()
        oracle.tree_vjp(parent, d, e, gd, ge, lb, lib=lib)
        t = time.perf_counter() - t0
        sub = cfg
        sample = "the whole tree (n=%d, b=%d), float64, reverse mode, single thread" % (cfg["n"], cfg["b"])
    gflops = nominal_flops(kind, sub, "vjp") / t / 1e9
    cores = 1 if kind == "tree" else int(lib.oracle_num_threads())
    return {"value": round(gflops, 3), "unit": "GFLOP/s", "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(t, 3),
            "block_rows_per_s": round(block_rows(kind, sub) / t, 1)}


def cpu_baseline(kind, cfg, op="selinv"):
    """The float64 oracle, as it stands, on a bounded sample of the workload
    (for --op logdet too: the oracle has no cheaper log-det path; value is
    then the collect's nominal flops over the full oracle time)."""
    import numpy as np
    import oracle
    import spdgen
    lib = oracle.load()
    if kind == "junction":
        Bs = min(cfg["B"], 8)
        n = cfg["rows"] * cfg["cols"]
        e = spdgen.grid_edges(cfg["rows"], cfg["cols"])
        d, v = spdgen.graph(e, n, cfg["b"], B=Bs, seed=cfg["seed"], diag_load=cfg["diag_load"])
        P = oracle.filled_pattern(n, e, lib=lib)
        t0 = time.perf_counter()
        oracle.junction(d, e, v, lib=lib, pattern=P)
        t = time.perf_counter() - t0
        sub = dict(cfg, B=Bs)
        cores = min(Bs, int(lib.oracle_num_threads()))
        return {"value": round(nominal_flops(kind, sub, op) / t / 1e9, 3), "unit": "GFLOP/s",
                "cores": cores, "kind": "oracle", "seconds": round(t, 3),
                "sample": "%d of %d matrices on the %d x %d grid (b=%d), float64, symbolic "
                          "analysis untimed" % (Bs, cfg["B"], cfg["rows"], cfg["cols"], cfg["b"]),
                "block_rows_per_s": round(block_rows(kind, sub) / t, 1)}
    if kind in ("bidiag", "nonsym_tree"):
        if kind == "bidiag":
            Bs = min(cfg["B"], 1024)
            d, l = spdgen.nonsym_bidiag(Bs, cfg["L"], cfg["b"], seed=cfg["seed"],
                                        diag_load=cfg["diag_load"])
            t0 = time.perf_counter()
            oracle.bidiag(d, l, lib=lib)
            t = time.perf_counter() - t0
            sub = dict(cfg, B=Bs)
            sample = "%d of %d matrices (L=%d, b=%d), float64" % (Bs, cfg["B"], cfg["L"], cfg["b"])
            cores = int(lib.oracle_num_threads())
        else:
            parent = spdgen.random_recursive_tree(cfg["n"], cfg["seed"])
            arrs = spdgen.nonsym_tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
            t0 = time.perf_counter()
            oracle.nonsym_tree(parent, *arrs, lib=lib)
            t = time.perf_counter() - t0
            sub = cfg
            sample = "the whole tree (n=%d, b=%d), float64, single thread" % (cfg["n"], cfg["b"])
            cores = 1
        return {"value": round(nominal_flops(kind, sub, op) / t / 1e9, 3), "unit": "GFLOP/s",
                "cores": cores, "kind": "oracle", "sample": sample, "seconds": round(t, 3),
                "block_rows_per_s": round(block_rows(kind, sub) / t, 1)}
    def timed(fn, min_s=0.0, max_reps=30):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= min_s or reps >= max_reps:
                break
        return (time.perf_counter() - t0) / reps, reps

    nthr = int(lib.oracle_num_threads())
    if kind == "chain":
        per = cfg["L"] * cfg["b"] ** 3
        # all threads: the whole batch when it is small (repeated for ~3 s),
        # else one chain per thread
        Bs = cfg["B"] if cfg["B"] * per <= 4e9 else max(1, min(cfg["B"], nthr))
        B1 = max(1, min(cfg["B"], int(5e8 // per)))  # one thread: ~1-4 s of work
        d, l = spdgen.chain(max(Bs, B1), cfg["L"], cfg["b"], seed=cfg["seed"],
                            diag_load=cfg["diag_load"])
        t, reps = timed(lambda: oracle.chain(d[:Bs], l[:Bs], lib=lib), 3.0)
        old = lib.oracle_set_num_threads(1)
        try:
            t1, _ = timed(lambda: oracle.chain(d[:B1], l[:B1], lib=lib))
        finally:
            lib.oracle_set_num_threads(old)
        sub, sub1 = dict(cfg, B=Bs), dict(cfg, B=B1)
        what = "chains (L=%d, b=%d), float64" % (cfg["L"], cfg["b"])
        sample = "%d of %d %s, mean of %d passes" % (Bs, cfg["B"], what, reps)
        sample1 = "%d of %d %s" % (B1, cfg["B"], what)
        cores = min(nthr, Bs)
    elif kind == "star":
        Bs = min(cfg["B"], nthr)
        arrs = spdgen.star(Bs, cfg["K"], cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        t, _ = timed(lambda: oracle.star(*arrs, lib=lib))
        old = lib.oracle_set_num_threads(1)
        try:
            t1, _ = timed(lambda: oracle.star(*(a[:1] for a in arrs), lib=lib))
        finally:
            lib.oracle_set_num_threads(old)
        sub, sub1 = dict(cfg, B=Bs), dict(cfg, B=1)
        what = "stars (K=%d, b=%d), float64" % (cfg["K"], cfg["b"])
        sample = "%d of %d %s" % (Bs, cfg["B"], what)
        sample1 = "1 of %d %s" % (cfg["B"], what)
        cores = Bs
    else:
        parent = spdgen.random_recursive_tree(cfg["n"], cfg["seed"])
        d, e = spdgen.tree(parent, cfg["b"], seed=cfg["seed"], diag_load=cfg["diag_load"])
        t, _ = timed(lambda: oracle.tree(parent, d, e, lib=lib))
        t1, sub, sub1 = t, cfg, cfg
        sample = sample1 = "the whole tree (n=%d, b=%d), float64" % (cfg["n"], cfg["b"])
        cores = 1  # one tree: the oracle's tree recurrence is sequential
    out = {"value": round(nominal_flops(kind, sub, op) / t / 1e9, 3), "unit": "GFLOP/s",
           "cores": cores, "kind": "oracle", "sample": sample, "seconds": round(t, 3),
           "block_rows_per_s": round(block_rows(kind, sub) / t, 1),
           "one_thread": {"value": round(nominal_flops(kind, sub1, op) / t1 / 1e9, 3),
                          "unit": "GFLOP/s", "cores": 1, "sample": sample1,
                          "seconds": round(t1, 3),
                          "block_rows_per_s": round(block_rows(kind, sub1) / t1, 1)}}
    out.update(host_info())
    return out


def host_info():
    """CPU model, logical CPU count and the CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


def copy_probe(mib, steps):
    """A plain device-to-device copy of known size: one read and one write of
    `mib` MiB per launch, for scaling the HBM traffic counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "launches": max(steps, 1)}), flush=True)


def peak_probe():
    """Achievable peaks on this device, for reading the roofline fractions
    against measured rather than datasheet limits: a device-to-device copy
    (bytes read + written per second) and large float64 / float32 matrix
    products through torch (vendor GEMM)."""
    import torch
    dev = torch.device("cuda:0")
    out = {}

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    n = (1 << 30) // 4  # 1 GiB of float32 each way
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 20)
    out["copy_GBps"] = round(2 * n * 4 / t / 1e9, 1)
    del src, dst
    for name, dt, m in (("gemm_f64_TFLOPs", torch.float64, 8192),
                        ("gemm_f32_TFLOPs", torch.float32, 8192)):
        a = torch.randn(m, m, dtype=dt, device=dev)
        b = torch.randn(m, m, dtype=dt, device=dev)
        c = torch.empty_like(a)
        t = timed(lambda: torch.matmul(a, b, out=c), 10)
        out[name] = round(2 * m ** 3 / t / 1e12, 2)
        del a, b, c
    out["datasheet"] = {"hbm_GBps": HBM_PEAK_GBS, "f64_TFLOPs": FP64_PEAK_TFLOPS,
                        "f32_TFLOPs": FP32_PEAK_TFLOPS}
    print(json.dumps(out), flush=True)


def compact(workload, dtname, steps, warmup):
    """Event-timed forward calls of another workload: median and min call
    time, nominal GFLOP/s, block-rows/s and the HBM roofline fraction on
    compulsory bytes (median call), with the number of calls sized by time
    (the call count is reported)."""
    import spdgen
    import torch
    cfg = dict(spdgen.WORKLOADS[workload])
    kind = cfg.pop("kind")
    cfg.pop("dtypes")
    w = 8 if dtname == "f64" else 4
    # Short calls are timed in steady state: a probe estimates the call time,
    # then at least ~20 ms of warm-up and ~50 ms of timed calls (at most 500).
    probe = run_gpu(kind, cfg, dtname, 3, 1)
    t_ms = max(min(probe["ev_ms"]), 1e-3)
    warm = max(warmup, 3, int(math.ceil(20.0 / t_ms)))
    n = max(steps, 20, min(500, int(math.ceil(50.0 / t_ms))))
    res = run_gpu(kind, cfg, dtname, n, min(warm, 500))
    torch.cuda.empty_cache()
    ev = sorted(res["ev_ms"])
    med = ev[len(ev) // 2]
    F = nominal_flops(kind, cfg)
    nbytes = compulsory_bytes(kind, cfg, w)
    peak_t = FP64_PEAK_TFLOPS if dtname == "f64" else FP32_PEAK_TFLOPS
    return {"ms_median": round(med, 4), "ms_min": round(ev[0], 4), "calls": n,
            "gflops": round(F / (med * 1e-3) / 1e9, 3),
            "block_rows_per_s": round(block_rows(kind, cfg) / (med * 1e-3), 1),
            "hbm_frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "flop_frac": round(F / (med * 1e-3) / 1e12 / peak_t, 4),
            "algorithmic_bytes": nbytes, "nominal_flops": F}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--op", default="selinv",
                    choices=("selinv", "vjp", "logdet", "solve", "sample"),
                    help="selinv: the selected inverse; vjp: its reverse mode; logdet, solve, "
                         "sample: the shared-factor siblings")
    ap.add_argument("--k", type=int, default=1, help="right-hand sides for --op solve/sample")
    ap.add_argument("--dtype", default=None, help="f64 or f32 (default: the workload's first)")
    ap.add_argument("--graph", action="store_true",
                    help="tree workloads: replay the schedule as one recorded HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second-dtype", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the compact timings of the other workloads")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--peak-probe", action="store_true",
                    help="only measure achievable peaks (device copy, float64/float32 GEMM) "
                         "and exit")
    args = ap.parse_args()
    if args.peak_probe:
        peak_probe()
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; --gpus %d is not supported (independent "
              "matrices shard across GPUs with no communication)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import spdgen
    cfg = dict(spdgen.WORKLOADS[args.workload])
    kind = cfg.pop("kind")
    dtypes = cfg.pop("dtypes")
    dtname = args.dtype or dtypes[0]
    w = 8 if dtname == "f64" else 4

    op = args.op
    if op in ("solve", "sample"):
        cfg["k"] = args.k
    if args.graph and (kind != "tree" or op != "selinv"):
        print("bench.py: --graph applies to the tree selected inverse only", file=sys.stderr)
        sys.exit(2)
    res = run_gpu(kind, cfg, dtname, args.steps, args.warmup, op, graph=args.graph)
    ev = sorted(res["ev_ms"])
    ms_mean = sum(res["ev_ms"]) / len(ev)
    ms_step = res["wall_s"] * 1e3 / args.steps
    F = nominal_flops(kind, cfg, op)
    nbytes = compulsory_bytes(kind, cfg, w, op)
    gflops = F / (ms_step * 1e-3) / 1e9
    achieved_gbs = nbytes / (ms_mean * 1e-3) / 1e9
    peak_t = FP64_PEAK_TFLOPS if dtname == "f64" else FP32_PEAK_TFLOPS
    tkey = args.workload if op == "selinv" else args.workload + "+" + op
    what = {"selinv": "selected-inverse", "vjp": "selected-inverse VJP",
            "logdet": "log-det (collect only)", "solve": "shared-factor solve",
            "sample": "shared-factor Gaussian sampling"}[op]
    out = {
        "metric": what + " GFLOP/s and block-rows/s (fp64/fp32), % of MI355X roofline",
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtname,
        "data": "synthetic (seeded Philox SPD blocks)",
        "config": dict({"workload": args.workload, "pattern": kind, "op": op}, **cfg,
                       **({"graph": True} if args.graph else {})),
        "block_rows_per_s": round(block_rows(kind, cfg) / (ms_step * 1e-3), 1),
        "kernel_ms": {"mean": round(ms_mean, 4), "median": round(ev[len(ev) // 2], 4),
                      "min": round(ev[0], 4)},
        "flop_frac_of_peak": round(gflops / (peak_t * 1e3), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "scope": "one call (every launch of the step), HIP events on its stream",
                     "traffic": measured_traffic(tkey, dtname),
                     "algorithmic_bytes": nbytes, "kernel_source_hash": kernel_source_hash()},
    }
    if kind == "junction":
        # about 100 nominal flops per compulsory byte: bound by vector ALU
        # arithmetic (the level kernels run on the vector units)
        tf = F / (ms_mean * 1e-3) / 1e12
        out["roofline"] = {"bound": "alu", "achieved": round(tf, 4), "peak": peak_t,
                           "unit": "TFLOP/s", "frac": round(tf / peak_t, 4),
                           "traffic": measured_traffic(tkey, dtname),
                           "algorithmic_flops": F, "algorithmic_bytes": nbytes,
                           "kernel_source_hash": kernel_source_hash()}
    if not args.no_second_dtype and len(dtypes) > 1 and args.dtype is None:
        other = dtypes[1]
        r2 = run_gpu(kind, cfg, other, args.steps, args.warmup, op, graph=args.graph)
        ms2 = r2["wall_s"] * 1e3 / args.steps
        ev2 = sum(r2["ev_ms"]) / len(r2["ev_ms"])
        w2 = 8 if other == "f64" else 4
        out[other] = {"value": round(F / (ms2 * 1e-3) / 1e9, 3), "unit": "GFLOP/s",
                      "ms_per_step": round(ms2, 4),
                      "block_rows_per_s": round(block_rows(kind, cfg) / (ms2 * 1e-3), 1),
                      "hbm_frac": round(compulsory_bytes(kind, cfg, w2, op) / (ev2 * 1e-3) / 1e9
                                        / HBM_PEAK_GBS, 4)}
    if (op == "selinv" and args.workload == DEFAULT_WORKLOAD and args.dtype is None
            and not args.no_configs):
        out["configs"] = {}
        for wl, dn in OTHER_CONFIGS:
            out["configs"]["%s/%s" % (wl, dn)] = compact(wl, dn, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = {"selinv": cpu_baseline, "vjp": cpu_baseline_vjp,
                               "logdet": cpu_baseline, "solve": cpu_baseline_apply,
                               "sample": cpu_baseline_apply}[op](kind, cfg, op)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
