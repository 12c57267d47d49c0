"""Helpers for pinning the oracle to things other than itself: dense numpy
inverses (LAPACK), closed forms and exact identities.  Used by the oracle pin
tests and by the planted-mistake test, which runs the same checks on
deliberately broken oracle builds."""
from __future__ import annotations

import numpy as np

import spdgen


def rel_fro(a, ref):
    """Relative Frobenius error per block over the trailing two axes."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.sqrt(((a - ref) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((ref ** 2).sum(axis=(-1, -2)))
    return num / np.maximum(den, 1e-300)


def dense_chain_blocks(diag, lower):
    """On-pattern blocks of A^-1 and log det A for one chain, from a dense
    numpy inverse (independent of the oracle)."""
    A = spdgen.to_dense_chain(diag, lower)
    Ai = np.linalg.inv(A)
    sign, ld = np.linalg.slogdet(A)
    L, b = diag.shape[0], diag.shape[1]
    Gd = np.stack([Ai[i * b:(i + 1) * b, i * b:(i + 1) * b] for i in range(L)])
    Gl = np.stack([Ai[(i + 1) * b:(i + 2) * b, i * b:(i + 1) * b] for i in range(L - 1)]) \
        if L > 1 else np.zeros((0, b, b))
    return Gd, Gl, ld, sign


def dense_star_blocks(center, leaves, coupling):
    A = spdgen.to_dense_star(center, leaves, coupling)
    Ai = np.linalg.inv(A)
    sign, ld = np.linalg.slogdet(A)
    K, b = leaves.shape[0], center.shape[0]
    Gc = Ai[:b, :b]
    Gl = np.stack([Ai[(j + 1) * b:(j + 2) * b, (j + 1) * b:(j + 2) * b] for j in range(K)]) \
        if K else np.zeros((0, b, b))
    Gx = np.stack([Ai[(j + 1) * b:(j + 2) * b, :b] for j in range(K)]) \
        if K else np.zeros((0, b, b))
    return Gc, Gl, Gx, ld, sign


def dense_tree_blocks(parent, diag, edge):
    A = spdgen.to_dense_tree(parent, diag, edge)
    Ai = np.linalg.inv(A)
    sign, ld = np.linalg.slogdet(A)
    n, b = diag.shape[0], diag.shape[1]
    Gd = np.stack([Ai[v * b:(v + 1) * b, v * b:(v + 1) * b] for v in range(n)])
    Ge = np.zeros_like(diag)
    for v in range(n):
        p = int(parent[v])
        if p >= 0:
            Ge[v] = Ai[p * b:(p + 1) * b, v * b:(v + 1) * b]
    return Gd, Ge, ld, sign


def laplacian_chain_exact(L):
    """1-D Laplacian tridiag(-1, 2, -1), b = 1: (A^-1)_ij =
    min(i,j)(L+1-max(i,j))/(L+1) (1-based), det A = L+1."""
    i = np.arange(1, L + 1, dtype=np.float64)
    Gd = i * (L + 1 - i) / (L + 1)
    j = np.arange(1, L, dtype=np.float64)  # G_{j+1, j}
    Gl = j * (L - j) / (L + 1)
    return Gd, Gl, np.log(L + 1.0)


def usmani_chain_exact(a, c):
    """Scalar symmetric tridiagonal with diagonal a[0..L-1] and sub-diagonal
    c[0..L-2] (c[i] = A_{i+1,i}).  Usmani's recurrences (1-based):
    theta_0 = 1, theta_1 = a_1, theta_i = a_i theta_{i-1} - c_{i-1}^2 theta_{i-2};
    phi_{L+1} = 1, phi_L = a_L, phi_i = a_i phi_{i+1} - c_i^2 phi_{i+2};
    (A^-1)_ii = theta_{i-1} phi_{i+1} / theta_L,
    (A^-1)_{i+1,i} = -c_i theta_{i-1} phi_{i+2} / theta_L,  det A = theta_L."""
    L = len(a)
    th = np.zeros(L + 1)
    th[0] = 1.0
    th[1] = a[0]
    for i in range(2, L + 1):
        th[i] = a[i - 1] * th[i - 1] - c[i - 2] ** 2 * th[i - 2]
    ph = np.zeros(L + 2)
    ph[L + 1] = 1.0
    ph[L] = a[L - 1]
    for i in range(L - 1, 0, -1):
        ph[i] = a[i - 1] * ph[i + 1] - c[i - 1] ** 2 * ph[i + 2]
    Gd = np.array([th[i - 1] * ph[i + 1] / th[L] for i in range(1, L + 1)])
    Gl = np.array([-c[i - 1] * th[i - 1] * ph[i + 2] / th[L] for i in range(1, L)])
    return Gd, Gl, np.log(th[L])


def arrowhead_exact(a0, d, f):
    """Scalar arrowhead: centre a0, leaves d_j, couplings f_j = A_{j,0}.
    s = a0 - sum f_j^2/d_j; G00 = 1/s; G_{j0} = -f_j/(d_j s);
    G_jj = 1/d_j + f_j^2/(d_j^2 s); log det = ln s + sum ln d_j."""
    s = a0 - np.sum(f * f / d)
    return 1.0 / s, 1.0 / d + f * f / (d * d * s), -f / (d * s), np.log(s) + np.log(d).sum()


def kron_chain(L, M):
    """Chain A = K_L (x) M with K_L = tridiag(-1, 2, -1): D_i = 2M, C_i = -M.
    Exact: G_ij = (K_L^-1)_ij M^-1, log det = b ln(L+1) + L ln det M."""
    b = M.shape[0]
    diag = np.broadcast_to(2.0 * M, (L, b, b)).copy()
    lower = np.broadcast_to(-M, (L - 1, b, b)).copy()
    Minv = np.linalg.inv(M)
    Gd_s, Gl_s, ldK = laplacian_chain_exact(L)
    Gd = Gd_s[:, None, None] * Minv
    Gl = Gl_s[:, None, None] * Minv
    ld = b * ldK + L * np.linalg.slogdet(M)[1]
    return diag, lower, Gd, Gl, ld


def random_spd(b, rng, load=1.0):
    W = rng.standard_normal((b, b))
    return W @ W.T / b + load * np.eye(b)


def chain_residual(diag, lower, Gd, Gl):
    """max over block rows i of |D_i G_ii + C_{i-1} G_{i-1,i} + C_i^T G_{i+1,i} - I|
    using on-pattern blocks only ((A A^-1)_ii = I)."""
    L, b = diag.shape[0], diag.shape[1]
    worst = 0.0
    for i in range(L):
        R = diag[i] @ Gd[i]
        if i >= 1:
            R += lower[i - 1] @ Gl[i - 1].T  # A_{i,i-1} (A^-1)_{i-1,i}
        if i <= L - 2:
            R += lower[i].T @ Gl[i]          # A_{i,i+1} (A^-1)_{i+1,i}
        worst = max(worst, np.abs(R - np.eye(b)).max())
    return worst


def star_residual(center, leaves, coupling, Gc, Gl, Gx):
    b = center.shape[0]
    R0 = center @ Gc + sum(coupling[j].T @ Gx[j] for j in range(leaves.shape[0]))
    worst = np.abs(R0 - np.eye(b)).max()
    for j in range(leaves.shape[0]):
        Rj = leaves[j] @ Gl[j] + coupling[j] @ Gx[j].T
        worst = max(worst, np.abs(Rj - np.eye(b)).max())
    return worst


def tree_residual(parent, diag, edge, Gd, Ge):
    """(A A^-1)_vv = I for every node, from on-pattern blocks only."""
    n, b = diag.shape[0], diag.shape[1]
    R = np.einsum("vij,vjk->vik", diag, Gd)
    for v in range(n):
        p = int(parent[v])
        if p < 0:
            continue
        R[v] += edge[v].T @ Ge[v]          # A_{v,p} (A^-1)_{p,v}
        R[p] += edge[v] @ Ge[v].T          # A_{p,v} (A^-1)_{v,p}
    return np.abs(R - np.eye(b)).max()
