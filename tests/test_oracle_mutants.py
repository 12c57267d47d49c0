"""Planted mistakes: each case copies oracle.c, applies one plausible bug
(a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
visiting order), compiles the copy on the CPU, and checks that the pins used
for the oracle reject it.  This shows the pins have teeth; the real oracle
must pass the same battery."""
import os

import numpy as np
import pytest

import oracle
import pins
import spdgen

MUTANTS = [
    ("schur_sign", "Sp[r * b + c] -= s;", "Sp[r * b + c] += s;"),
    ("drop_takahashi_term", "Gvv[e] = Sinv[e] - T[e];", "Gvv[e] = Sinv[e];"),
    ("offdiag_sign", "Gpv[e] = -Gpv[e];", "Gpv[e] = Gpv[e];"),
    ("x_not_transposed", "transpose(b, Z, X);     /* X = E S^{-1}             */",
     "memcpy(X, Z, sizeof(double) * b * b);"),
    ("logdet_half", "return 2.0 * s;", "return s;"),
    ("inverse_wwt", "s += W[k * b + r] * W[k * b + c];", "s += W[r * b + k] * W[c * b + k];"),
    ("chol_wrong_row", "s -= R[i * b + k] * R[j * b + k];", "s -= R[i * b + k] * R[i * b + k];"),
    ("trsm_upper", "s -= R[k * b + i] * Y[k * b + c];", "s -= R[i * b + k] * Y[k * b + c];"),
    ("chain_wrong_next_diag", "memcpy(S, D + (i + 1) * bb, sizeof(double) * bb);",
     "memcpy(S, D + i * bb, sizeof(double) * bb);"),
    ("star_coupling_orientation", "transpose(b, F + j * bb, w + 3 * bb);",
     "memcpy(w + 3 * bb, F + j * bb, sizeof(double) * bb);"),
    ("star_cross_orientation", "transpose(b, w + 3 * bb, Gx + j * bb);",
     "memcpy(Gx + j * bb, w + 3 * bb, sizeof(double) * bb);"),
    ("tree_update_self", "S + (int64_t)parent[v] * bb, X + v * bb,", "S + v * bb, X + v * bb,"),
    ("tree_collect_top_down", "for (int32_t d = H; d >= 0 && !fail; --d)",
     "for (int32_t d = 0; d <= H && !fail; ++d)"),
    ("tree_distribute_own_g", "distribute_edge(b, G_diag + (int64_t)parent[v] * bb,",
     "distribute_edge(b, G_diag + (int64_t)(parent[v] >= 0 ? v : 0) * bb,"),
    ("chol_pivot_index", "double d = S[j * b + j];", "double d = S[j * b + (j ? j - 1 : 0)];"),
]


def _battery(lib):
    """Return the names of the pins this oracle build fails."""
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    def chain_dense():
        d, l = spdgen.chain(2, 6, 3, seed=11)
        Gd, Gl, ld, info = oracle.chain(d, l, lib=lib)
        for m in range(2):
            Rd, Rl, Rld, _ = pins.dense_chain_blocks(d[m], l[m])
            if not (pins.rel_fro(Gd[m], Rd).max() < 1e-12 and pins.rel_fro(Gl[m], Rl).max() < 1e-12
                    and abs(ld[m] - Rld) < 1e-11):
                return False
        return True

    def star_dense():
        c, lv, cp = spdgen.star(1, 5, 3, seed=5)
        Gc, Gl, Gx, ld, info = oracle.star(c, lv, cp, lib=lib)
        Rc, Rl, Rx, Rld, _ = pins.dense_star_blocks(c[0], lv[0], cp[0])
        return (pins.rel_fro(Gc[0], Rc) < 1e-12 and pins.rel_fro(Gl[0], Rl).max() < 1e-12
                and pins.rel_fro(Gx[0], Rx).max() < 1e-12 and abs(ld[0] - Rld) < 1e-11)

    def tree_dense():
        p = spdgen.random_recursive_tree(25, 3)
        d, e = spdgen.tree(p, 3, seed=4)
        Gd, Ge, ld, info = oracle.tree(p, d, e, lib=lib)
        Rd, Re, Rld, _ = pins.dense_tree_blocks(p, d, e)
        return (pins.rel_fro(Gd, Rd).max() < 1e-12 and pins.rel_fro(Ge[1:], Re[1:]).max() < 1e-12
                and abs(ld - Rld) < 1e-11)

    def laplacian():
        L = 9
        Gd, Gl, ld, _ = oracle.chain(np.full((1, L, 1, 1), 2.0), np.full((1, L - 1, 1, 1), -1.0),
                                     lib=lib)
        Ed, El, Eld = pins.laplacian_chain_exact(L)
        return (np.abs(Gd[0, :, 0, 0] - Ed).max() < 1e-12 and
                np.abs(Gl[0, :, 0, 0] - El).max() < 1e-12 and abs(ld[0] - Eld) < 1e-12)

    check("chain_dense", chain_dense)
    check("star_dense", star_dense)
    check("tree_dense", tree_dense)
    check("laplacian", laplacian)
    return failed


def _variant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation site for %s not unique/found" % name
    path = os.path.join(str(tmp_path), "oracle_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return oracle.load(oracle.compile_oracle(path, path[:-2] + ".so"))


def test_real_oracle_passes_battery(orc):
    assert _battery(orc.load()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    lib = _variant(tmp_path, name, old, new)
    assert _battery(lib), "planted mistake %s passed every pin" % name
