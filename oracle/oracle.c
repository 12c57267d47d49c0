/*
 * oracle.c -- plain, slow float64 reference for the selected inverse of
 * block-structured SPD matrices whose block graph is a tree (chain = path,
 * star = depth 1, general rooted tree).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code; the product path never
 * calls it and shares no code with it.
 *
 * What is computed (gabp-sparse-inv 0.3.2 project page, opening paragraphs
 * and section "Implemented and tested kernels"): only the blocks of A^-1 on
 * A's own block pattern -- every diagonal block and every pattern edge --
 * plus log det A, without forming the dense inverse.  On a tree the method is
 * a two-pass schedule: a collect pass (leaves -> root) that is a block LDL^T /
 * Cholesky elimination, and a distribute pass (root -> leaves) that is the
 * Takahashi back-recursion; the page states the two views agree.  The log
 * determinant comes from the same factorization (same page, "Statement of
 * need" and the tree_logdet / junction_logdet passage in the junction-tree
 * section).
 *
 * Notation.  For a non-root node v with parent p:
 *     E_v = A_{p,v}                     (the off-diagonal block)
 *     S_v = D_v - sum_{children c} E_c S_c^{-1} E_c^T      (Schur pivot)
 *     R_v = chol(S_v),  S_v = R_v R_v^T, R_v lower triangular
 *     X_v = E_v S_v^{-1}
 * collect:    S_p -= E_v S_v^{-1} E_v^T  (= Y^T Y with Y = R_v^{-1} E_v^T)
 * root:       G_rr = S_r^{-1}
 * distribute: G_{p,v} = -G_pp X_v
 *             G_vv    = S_v^{-1} - X_v^T G_{p,v}
 * log det A = sum_v 2 sum_k ln (R_v)_kk.
 *
 * Layouts (Quickstart section of the same page): blocks are b x b,
 * row-major, contiguous.
 *   chain: diag[B][L], lower[B][L-1] with lower[i] = A_{i+1,i};
 *          G_diag[i] = (A^-1)_{ii}, G_lower[i] = (A^-1)_{i+1,i}.
 *          The chain is the path rooted at its last block.
 *   star:  center[B], leaves[B][K], coupling[B][K] with coupling[j] = A_{j,0}
 *          (centre = block 0, leaf j = block j+1);
 *          G_center = (A^-1)_00, G_leaf[j] = (A^-1)_jj, G_cross[j] = (A^-1)_{j,0}.
 *   tree:  parent[n] (root = -1), diag[n], edge[n] with edge[v] = A_{parent(v),v};
 *          G_diag[v] = (A^-1)_vv, G_edge[v] = (A^-1)_{parent(v),v}, root slot 0.
 * Only the lower triangle of each diagonal input block is read.
 *
 * Failure: if a Schur pivot is not positive definite (Cholesky finds a
 * diagonal that is not > 0, NaN included), info = 1 + that block's index in
 * the caller's numbering (chain: block i -> i+1; star: centre -> 1, leaf j ->
 * j+2; tree: node v -> v+1), the matrix's outputs are filled with NaN and its
 * logdet is NaN.  This mirrors the "not positive definite -> error"
 * convention of the sparsax page (Features list).
 *
 * Plain C, scalar loops, no BLAS; OpenMP only across independent matrices.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------ primitives */

/* Cholesky S = R R^T of a symmetric block, reading the lower triangle of S.
 * R is lower triangular with zeros above the diagonal.  Returns 0 on
 * success, 1 if a pivot is not > 0 (NaN included). */
static int chol(int b, const double *S, double *R) {
  memset(R, 0, sizeof(double) * (size_t)b * b);
  for (int j = 0; j < b; ++j) {
    double d = S[j * b + j];
    for (int k = 0; k < j; ++k) d -= R[j * b + k] * R[j * b + k];
    if (!(d > 0.0)) return 1;
    const double rjj = sqrt(d);
    R[j * b + j] = rjj;
    for (int i = j + 1; i < b; ++i) {
      double s = S[i * b + j];
      for (int k = 0; k < j; ++k) s -= R[i * b + k] * R[j * b + k];
      R[i * b + j] = s / rjj;
    }
  }
  return 0;
}

/* Solve R Y = Bm (R lower triangular) by forward substitution, column by
 * column.  Bm, Y are b x b. */
static void trsm_L(int b, const double *R, const double *Bm, double *Y) {
  for (int c = 0; c < b; ++c)
    for (int i = 0; i < b; ++i) {
      double s = Bm[i * b + c];
      for (int k = 0; k < i; ++k) s -= R[i * b + k] * Y[k * b + c];
      Y[i * b + c] = s / R[i * b + i];
    }
}

/* Solve R^T Y = Bm (R lower triangular) by back substitution. */
static void trsm_LT(int b, const double *R, const double *Bm, double *Y) {
  for (int c = 0; c < b; ++c)
    for (int i = b - 1; i >= 0; --i) {
      double s = Bm[i * b + c];
      for (int k = i + 1; k < b; ++k) s -= R[k * b + i] * Y[k * b + c];
      Y[i * b + c] = s / R[i * b + i];
    }
}

/* S^{-1} = R^{-T} R^{-1}: W = R^{-1} by forward substitution on the identity,
 * then the full product W^T W, deliberately NOT symmetrised. */
static void inv_from_chol(int b, const double *R, double *Sinv) {
  double *I = (double *)calloc((size_t)b * b, sizeof(double));
  double *W = (double *)malloc(sizeof(double) * (size_t)b * b);
  for (int i = 0; i < b; ++i) I[i * b + i] = 1.0;
  trsm_L(b, R, I, W);
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += W[k * b + r] * W[k * b + c];
      Sinv[r * b + c] = s;
    }
  free(I);
  free(W);
}

/* ln det S = 2 sum_k ln R_kk */
static double logdet_chol(int b, const double *R) {
  double s = 0.0;
  for (int k = 0; k < b; ++k) s += log(R[k * b + k]);
  return 2.0 * s;
}

static void transpose(int b, const double *Bm, double *T) {
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) T[c * b + r] = Bm[r * b + c];
}

/* Out = P Q */
static void matmul(int b, const double *P, const double *Q, double *Out) {
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += P[r * b + k] * Q[k * b + c];
      Out[r * b + c] = s;
    }
}

/* Out = P^T Q */
static void matmul_tn(int b, const double *P, const double *Q, double *Out) {
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += P[k * b + r] * Q[k * b + c];
      Out[r * b + c] = s;
    }
}

static void fill_nan(double *p, int64_t n) {
  for (int64_t i = 0; i < n; ++i) p[i] = NAN;
}

/* One collect step for a non-root node: from R_v (chol of S_v) and the edge
 * block E = A_{p,v}, subtract E S_v^{-1} E^T from the parent's pivot S_p and
 * return X_v = E S_v^{-1}.  Work arrays: Et, Y, Z (b x b each). */
static void collect_edge(int b, const double *R, const double *E, double *Sp, double *X,
                         double *Et, double *Y, double *Z) {
  transpose(b, E, Et);    /* E^T                      */
  trsm_L(b, R, Et, Y);    /* Y = R^{-1} E^T           */
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += Y[k * b + r] * Y[k * b + c];
      Sp[r * b + c] -= s; /* S_p -= Y^T Y = E S^{-1} E^T */
    }
  trsm_LT(b, R, Y, Z);    /* Z = S^{-1} E^T           */
  transpose(b, Z, X);     /* X = E S^{-1}             */
}

/* One distribute step: G_{p,v} = -G_pp X_v ; G_vv = S_v^{-1} - X_v^T G_{p,v}. */
static void distribute_edge(int b, const double *Gpp, const double *X, const double *R,
                            double *Gpv, double *Gvv, double *Sinv, double *T) {
  matmul(b, Gpp, X, Gpv);
  for (int64_t e = 0; e < (int64_t)b * b; ++e) Gpv[e] = -Gpv[e];
  inv_from_chol(b, R, Sinv);
  matmul_tn(b, X, Gpv, T);
  for (int64_t e = 0; e < (int64_t)b * b; ++e) Gvv[e] = Sinv[e] - T[e];
}

/* ----------------------------------------------------------------- chain */

/* Block-tridiagonal chain (item "Chain" of "Implemented and tested kernels":
 * block LDL^T factorisation plus Takahashi back-recursion; the chain is the
 * path tree rooted at its last block, per the root-invariance remark of the
 * Quickstart section).  Batch loop over B independent matrices. */
ORACLE_API int oracle_chain(int64_t B, int64_t L, int b, const double *diag,
                            const double *lower, double *G_diag, double *G_lower,
                            double *logdet, int32_t *info) {
  if (B < 0 || L < 1 || b < 1 || !diag || !G_diag || !logdet || !info) return 1;
  if (L > 1 && (!lower || !G_lower)) return 1;
  const int64_t bb = (int64_t)b * b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < B; ++m) {
    const double *D = diag + m * L * bb;
    const double *C = lower + m * (L - 1) * bb;
    double *Gd = G_diag + m * L * bb;
    double *Gl = G_lower + m * (L - 1) * bb;
    double *R = (double *)malloc(sizeof(double) * L * bb); /* R_i, i < L   */
    double *X = (double *)malloc(sizeof(double) * L * bb); /* X_i, i < L-1 */
    double *S = (double *)malloc(sizeof(double) * bb);
    double *w = (double *)malloc(sizeof(double) * 4 * bb);
    double ld = 0.0;
    int32_t fail = 0;
    memcpy(S, D, sizeof(double) * bb); /* S_0 = D_0 */
    for (int64_t i = 0; i < L; ++i) {
      if (chol(b, S, R + i * bb)) {
        fail = (int32_t)(i + 1);
        break;
      }
      ld += logdet_chol(b, R + i * bb);
      if (i == L - 1) break;
      /* next pivot starts from D_{i+1}; parent of i is i+1, E_i = lower[i] */
      memcpy(S, D + (i + 1) * bb, sizeof(double) * bb);
      collect_edge(b, R + i * bb, C + i * bb, S, X + i * bb, w, w + bb, w + 2 * bb);
    }
    if (fail) {
      info[m] = fail;
      logdet[m] = NAN;
      fill_nan(Gd, L * bb);
      if (L > 1) fill_nan(Gl, (L - 1) * bb);
    } else {
      info[m] = 0;
      logdet[m] = ld;
      inv_from_chol(b, R + (L - 1) * bb, Gd + (L - 1) * bb); /* root closure */
      for (int64_t i = L - 2; i >= 0; --i)
        distribute_edge(b, Gd + (i + 1) * bb, X + i * bb, R + i * bb, Gl + i * bb,
                        Gd + i * bb, w, w + bb);
    }
    free(R);
    free(X);
    free(S);
    free(w);
  }
  return 0;
}

/* ------------------------------------------------------------------ star */

/* Block arrowhead (item "Star": one centre coupled to K leaves with no
 * leaf-leaf coupling, leaves eliminated first).  The centre is the parent of
 * every leaf, so E_j = A_{0,j} = coupling[j]^T.  Leaves are eliminated in
 * index order. */
ORACLE_API int oracle_star(int64_t B, int64_t K, int b, const double *center,
                           const double *leaves, const double *coupling, double *G_center,
                           double *G_leaf, double *G_cross, double *logdet, int32_t *info) {
  if (B < 0 || K < 0 || b < 1 || !center || !G_center || !logdet || !info) return 1;
  if (K > 0 && (!leaves || !coupling || !G_leaf || !G_cross)) return 1;
  const int64_t bb = (int64_t)b * b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < B; ++m) {
    const double *Dl = leaves + m * K * bb;
    const double *F = coupling + m * K * bb;
    double *Gc = G_center + m * bb;
    double *Gl = G_leaf + m * K * bb;
    double *Gx = G_cross + m * K * bb;
    double *R = (double *)malloc(sizeof(double) * (K + 1) * bb); /* leaves, then centre */
    double *X = (double *)malloc(sizeof(double) * (K > 0 ? K : 1) * bb);
    double *S0 = (double *)malloc(sizeof(double) * bb);
    double *w = (double *)malloc(sizeof(double) * 5 * bb);
    double ld = 0.0;
    int32_t fail = 0;
    memcpy(S0, center + m * bb, sizeof(double) * bb);
    for (int64_t j = 0; j < K; ++j) {
      if (chol(b, Dl + j * bb, R + j * bb)) { /* a leaf has no children: S_j = D_j */
        fail = (int32_t)(j + 2);
        break;
      }
      ld += logdet_chol(b, R + j * bb);
      transpose(b, F + j * bb, w + 3 * bb); /* E_j = A_{0,j} = coupling[j]^T */
      collect_edge(b, R + j * bb, w + 3 * bb, S0, X + j * bb, w, w + bb, w + 2 * bb);
    }
    if (!fail && chol(b, S0, R + K * bb)) fail = 1;
    if (fail) {
      info[m] = fail;
      logdet[m] = NAN;
      fill_nan(Gc, bb);
      if (K > 0) {
        fill_nan(Gl, K * bb);
        fill_nan(Gx, K * bb);
      }
    } else {
      info[m] = 0;
      ld += logdet_chol(b, R + K * bb);
      logdet[m] = ld;
      inv_from_chol(b, R + K * bb, Gc);
      for (int64_t j = 0; j < K; ++j) {
        /* w+3bb receives G_{0,j}; the output wants G_{j,0} = G_{0,j}^T */
        distribute_edge(b, Gc, X + j * bb, R + j * bb, w + 3 * bb, Gl + j * bb, w, w + bb);
        transpose(b, w + 3 * bb, Gx + j * bb);
      }
    }
    free(R);
    free(X);
    free(S0);
    free(w);
  }
  return 0;
}

/* ------------------------------------------------------------------ tree */

/* Validate a parent array and compute depths.  Returns 0 and fills depth[] and
 * *root on success; 2 if the array is not a single rooted tree (not exactly
 * one root, an index out of range, or a cycle). */
static int tree_depths(int64_t n, const int32_t *parent, int32_t *depth, int64_t *root) {
  int64_t r = -1;
  for (int64_t v = 0; v < n; ++v) {
    const int32_t p = parent[v];
    if (p == -1) {
      if (r >= 0) return 2;
      r = v;
    } else if (p < 0 || p >= n || p == v) {
      return 2;
    }
  }
  if (r < 0) return 2;
  for (int64_t v = 0; v < n; ++v) depth[v] = -1;
  depth[r] = 0;
  int64_t *stack = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n + 1));
  for (int64_t v = 0; v < n; ++v) {
    /* walk up until a node of known depth; more than n steps means a cycle */
    int64_t top = 0, u = v;
    while (depth[u] < 0) {
      if (top > n) {
        free(stack);
        return 2;
      }
      stack[top++] = u;
      u = parent[u];
    }
    int32_t d = depth[u];
    while (top > 0) depth[stack[--top]] = ++d;
  }
  free(stack);
  *root = r;
  return 0;
}

/* Arbitrary rooted tree (item "Tree": a parent array and one edge block per
 * non-root node; collect leaves -> root, then distribute root -> leaves).
 * Collect visits depths from the deepest up to 0, nodes of one depth in
 * increasing index (so a parent's children, which share a depth, are
 * subtracted in increasing index); distribute visits depths 1, 2, ... */
ORACLE_API int oracle_tree(int64_t n, int b, const int32_t *parent, const double *diag,
                           const double *edge, double *G_diag, double *G_edge, double *logdet,
                           int32_t *info) {
  if (n < 1 || b < 1 || !parent || !diag || !edge || !G_diag || !G_edge || !logdet || !info)
    return 1;
  const int64_t bb = (int64_t)b * b;
  int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int64_t root = -1;
  if (tree_depths(n, parent, depth, &root)) {
    free(depth);
    return 2;
  }
  int32_t H = 0;
  for (int64_t v = 0; v < n; ++v)
    if (depth[v] > H) H = depth[v];
  /* nodes bucketed by depth, increasing index within a depth */
  int64_t *cnt = (int64_t *)calloc((size_t)H + 2, sizeof(int64_t));
  for (int64_t v = 0; v < n; ++v) cnt[depth[v] + 1]++;
  for (int32_t d = 0; d <= H; ++d) cnt[d + 1] += cnt[d];
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  int64_t *fillp = (int64_t *)malloc(sizeof(int64_t) * ((size_t)H + 1));
  for (int32_t d = 0; d <= H; ++d) fillp[d] = cnt[d];
  for (int64_t v = 0; v < n; ++v) order[fillp[depth[v]]++] = v;

  double *S = (double *)malloc(sizeof(double) * n * bb);
  double *R = (double *)malloc(sizeof(double) * n * bb);
  double *X = (double *)malloc(sizeof(double) * n * bb);
  double *w = (double *)malloc(sizeof(double) * 4 * bb);
  memcpy(S, diag, sizeof(double) * n * bb); /* S_v starts at D_v */
  double ld = 0.0;
  int32_t fail = 0;
  for (int32_t d = H; d >= 0 && !fail; --d)
    for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
      const int64_t v = order[k];
      if (chol(b, S + v * bb, R + v * bb)) {
        fail = (int32_t)(v + 1);
        break;
      }
      ld += logdet_chol(b, R + v * bb);
      if (v != root)
        collect_edge(b, R + v * bb, edge + v * bb, S + (int64_t)parent[v] * bb, X + v * bb,
                     w, w + bb, w + 2 * bb);
    }
  if (fail) {
    *info = fail;
    *logdet = NAN;
    fill_nan(G_diag, n * bb);
    fill_nan(G_edge, n * bb);
  } else {
    *info = 0;
    *logdet = ld;
    inv_from_chol(b, R + root * bb, G_diag + root * bb);
    for (int32_t d = 1; d <= H; ++d)
      for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
        const int64_t v = order[k];
        distribute_edge(b, G_diag + (int64_t)parent[v] * bb, X + v * bb, R + v * bb,
                        G_edge + v * bb, G_diag + v * bb, w, w + bb);
      }
    memset(G_edge + root * bb, 0, sizeof(double) * bb);
  }
  free(depth);
  free(cnt);
  free(order);
  free(fillp);
  free(S);
  free(R);
  free(X);
  free(w);
  return 0;
}

/* ------------------------------------------------- vector-Jacobian product */

/* Reverse mode of the two passes above (the pages' "analytic two-pass
 * backward" of selinv_tree, section "Differentiable selected inverse"): given
 * cotangents Gd_bar[v] on G_vv, Ge_bar[v] on G_{p,v} = G_edge[v] and ld_bar on
 * log det A, return D_bar[v] and E_bar[v] with
 *     dL = sum_v <D_bar[v], dD_v> + sum_{v != root} <E_bar[v], dE_v>
 * for symmetric perturbations dD_v (D_bar is symmetric; the cotangent of G_vv
 * enters through its symmetric part, G_vv being symmetric).  Each forward
 * step is reversed in the opposite order:
 *   forward collect     S_v = D_v - sum_c M_c, Sinv_v = S_v^-1,
 *                       X_v = E_v Sinv_v, M_v = X_v E_v^T, logdet += ln det S_v
 *   forward distribute  V_v = G_pp X_v, G_{p,v} = -V_v, G_vv = Sinv_v + X_v^T V_v
 * Reverse distribute (deepest nodes first; GG_v = total cotangent of G_vv):
 *   Sinv_bar_v += GG_v,  X_bar_v += V_v GG_v^T,  V_bar = X_v GG_v - Ge_bar_v,
 *   GG_p += V_bar X_v^T, X_bar_v += G_pp^T V_bar;   root: Sinv_bar_r += GG_r.
 * Reverse collect (root first; S_bar_p known when v is visited):
 *   M_bar = -S_bar_p,  X_bar_v += M_bar E_v,  E_bar_v = M_bar^T X_v + X_bar_v Sinv_v^T,
 *   Sinv_bar_v += E_v^T X_bar_v,
 *   S_bar_v = -Sinv_v^T Sinv_bar_v Sinv_v^T + ld_bar Sinv_v^T,  D_bar_v = sym(S_bar_v).
 * Returns 0, 2 for an invalid parent array, 3 if a pivot is not positive
 * definite (outputs NaN). */
static void mm_nn(int b, const double *P, const double *Q, double *Out) { matmul(b, P, Q, Out); }
static void mm_nt(int b, const double *P, const double *Q, double *Out) { /* P Q^T */
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += P[r * b + k] * Q[c * b + k];
      Out[r * b + c] = s;
    }
}
static void mm_tn(int b, const double *P, const double *Q, double *Out) { matmul_tn(b, P, Q, Out); }
static void add_to(int64_t n, double *dst, const double *src, double sign) {
  for (int64_t e = 0; e < n; ++e) dst[e] += sign * src[e];
}

static int tree_vjp_core(int64_t n, int b, const int32_t *parent, const double *diag,
                         const double *edge, const double *gd_bar, const double *ge_bar,
                         double ld_bar, double *d_bar, double *e_bar) {
  const int64_t bb = (int64_t)b * b;
  int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int64_t root = -1;
  if (tree_depths(n, parent, depth, &root)) {
    free(depth);
    return 2;
  }
  int32_t H = 0;
  for (int64_t v = 0; v < n; ++v)
    if (depth[v] > H) H = depth[v];
  int64_t *cnt = (int64_t *)calloc((size_t)H + 2, sizeof(int64_t));
  for (int64_t v = 0; v < n; ++v) cnt[depth[v] + 1]++;
  for (int32_t d = 0; d <= H; ++d) cnt[d + 1] += cnt[d];
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  int64_t *fillp = (int64_t *)malloc(sizeof(int64_t) * ((size_t)H + 1));
  for (int32_t d = 0; d <= H; ++d) fillp[d] = cnt[d];
  for (int64_t v = 0; v < n; ++v) order[fillp[depth[v]]++] = v;

  double *S = (double *)malloc(sizeof(double) * n * bb);
  double *R = (double *)malloc(sizeof(double) * n * bb);
  double *X = (double *)calloc((size_t)(n * bb), sizeof(double));
  double *Si = (double *)malloc(sizeof(double) * n * bb);
  double *G = (double *)malloc(sizeof(double) * n * bb);
  double *GG = (double *)malloc(sizeof(double) * n * bb);
  double *Sib = (double *)calloc((size_t)(n * bb), sizeof(double));
  double *Xb = (double *)calloc((size_t)(n * bb), sizeof(double));
  double *Sb = (double *)malloc(sizeof(double) * n * bb);
  double *w = (double *)malloc(sizeof(double) * 6 * bb);
  double *V = w + 3 * bb, *Vb = w + 4 * bb, *T = w + 5 * bb;
  int rc = 0;

  /* forward collect: R_v, X_v */
  memcpy(S, diag, sizeof(double) * n * bb);
  for (int32_t d = H; d >= 0 && !rc; --d)
    for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
      const int64_t v = order[k];
      if (chol(b, S + v * bb, R + v * bb)) {
        rc = 3;
        break;
      }
      const int64_t p = parent[v];
      if (p >= 0) collect_edge(b, R + v * bb, edge + v * bb, S + p * bb, X + v * bb, w, w + bb,
                               w + 2 * bb);
    }
  if (rc) {
    fill_nan(d_bar, n * bb);
    fill_nan(e_bar, n * bb);
  } else {
    for (int64_t v = 0; v < n; ++v) inv_from_chol(b, R + v * bb, Si + v * bb);
    /* forward distribute: G_vv (G_{p,v} = -G_pp X_v is not needed) */
    memcpy(G + root * bb, Si + root * bb, sizeof(double) * bb);
    for (int32_t d = 1; d <= H; ++d)
      for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
        const int64_t v = order[k], p = parent[v];
        mm_nn(b, G + p * bb, X + v * bb, V);          /* V = G_pp X_v */
        mm_tn(b, X + v * bb, V, T);                   /* X^T V        */
        for (int64_t e = 0; e < bb; ++e) G[v * bb + e] = Si[v * bb + e] + T[e];
      }
    /* GG_v = sym(Gd_bar_v) */
    for (int64_t v = 0; v < n; ++v)
      for (int r = 0; r < b; ++r)
        for (int c = 0; c < b; ++c)
          GG[v * bb + r * b + c] =
              0.5 * (gd_bar[v * bb + r * b + c] + gd_bar[v * bb + c * b + r]);
    /* reverse distribute, deepest first */
    for (int32_t d = H; d >= 1; --d)
      for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
        const int64_t v = order[k], p = parent[v];
        const double *Xv = X + v * bb, *Gp = G + p * bb, *GGv = GG + v * bb;
        mm_nn(b, Gp, Xv, V);                          /* V = G_pp X_v           */
        add_to(bb, Sib + v * bb, GGv, 1.0);            /* Sinv_bar += GG_v       */
        mm_nt(b, V, GGv, T);                           /* V GG^T                 */
        add_to(bb, Xb + v * bb, T, 1.0);
        mm_nn(b, Xv, GGv, Vb);                         /* V_bar = X GG - Ge_bar  */
        add_to(bb, Vb, ge_bar + v * bb, -1.0);
        mm_nt(b, Vb, Xv, T);                           /* GG_p += V_bar X^T      */
        add_to(bb, GG + p * bb, T, 1.0);
        mm_tn(b, Gp, Vb, T);                           /* X_bar += G_pp^T V_bar  */
        add_to(bb, Xb + v * bb, T, 1.0);
      }
    add_to(bb, Sib + root * bb, GG + root * bb, 1.0);
    /* reverse collect, root first */
    for (int32_t d = 0; d <= H; ++d)
      for (int64_t k = cnt[d]; k < cnt[d + 1]; ++k) {
        const int64_t v = order[k];
        const double *Sv = Si + v * bb;
        if (v != root) {
          const double *Sbp = Sb + (int64_t)parent[v] * bb, *Ev = edge + v * bb, *Xv = X + v * bb;
          double *Mb = w, *Eb = e_bar + v * bb;
          for (int64_t e = 0; e < bb; ++e) Mb[e] = -Sbp[e];
          mm_nn(b, Mb, Ev, T);                          /* X_bar += M_bar E       */
          add_to(bb, Xb + v * bb, T, 1.0);
          mm_tn(b, Mb, Xv, Eb);                         /* E_bar = M_bar^T X      */
          mm_nt(b, Xb + v * bb, Sv, T);                 /* + X_bar Sinv^T         */
          add_to(bb, Eb, T, 1.0);
          mm_tn(b, Ev, Xb + v * bb, T);                 /* Sinv_bar += E^T X_bar  */
          add_to(bb, Sib + v * bb, T, 1.0);
        }
        /* S_bar = -Sinv^T Sinv_bar Sinv^T + ld_bar Sinv^T */
        double *Sbv = Sb + v * bb;
        mm_tn(b, Sv, Sib + v * bb, T);                  /* Sinv^T Sinv_bar        */
        mm_nt(b, T, Sv, Sbv);                           /* (...) Sinv^T           */
        for (int r = 0; r < b; ++r)
          for (int c = 0; c < b; ++c)
            Sbv[r * b + c] = -Sbv[r * b + c] + ld_bar * Sv[c * b + r];
        for (int r = 0; r < b; ++r)
          for (int c = 0; c < b; ++c)
            d_bar[v * bb + r * b + c] = 0.5 * (Sbv[r * b + c] + Sbv[c * b + r]);
      }
    memset(e_bar + root * bb, 0, sizeof(double) * bb);
  }
  free(depth); free(cnt); free(order); free(fillp);
  free(S); free(R); free(X); free(Si); free(G); free(GG); free(Sib); free(Xb); free(Sb); free(w);
  return rc;
}

ORACLE_API int oracle_tree_vjp(int64_t n, int b, const int32_t *parent, const double *diag,
                               const double *edge, const double *gd_bar, const double *ge_bar,
                               double ld_bar, double *d_bar, double *e_bar) {
  if (n < 1 || b < 1 || !parent || !diag || !edge || !gd_bar || !ge_bar || !d_bar || !e_bar)
    return 1;
  return tree_vjp_core(n, b, parent, diag, edge, gd_bar, ge_bar, ld_bar, d_bar, e_bar);
}

/* Chains as path trees rooted at their last block (parent of i is i + 1,
 * E_i = lower[i], G_edge[i] = G_lower[i]), one matrix after another.
 * status[m] = 0 or 3 (not positive definite). */
ORACLE_API int oracle_chain_vjp(int64_t B, int64_t L, int b, const double *diag,
                                const double *lower, const double *gd_bar, const double *gl_bar,
                                const double *ld_bar, double *d_bar, double *l_bar,
                                int32_t *status) {
  if (B < 0 || L < 1 || b < 1 || !diag || !gd_bar || !ld_bar || !d_bar || !status) return 1;
  if (L > 1 && (!lower || !gl_bar || !l_bar)) return 1;
  const int64_t bb = (int64_t)b * b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < B; ++m) {
    int32_t *par = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
    double *e = (double *)calloc((size_t)(L * bb), sizeof(double));
    double *geb = (double *)calloc((size_t)(L * bb), sizeof(double));
    double *eb = (double *)malloc(sizeof(double) * L * bb);
    for (int64_t i = 0; i < L; ++i) par[i] = i + 1 < L ? (int32_t)(i + 1) : -1;
    if (L > 1) {
      memcpy(e, lower + m * (L - 1) * bb, sizeof(double) * (L - 1) * bb);
      memcpy(geb, gl_bar + m * (L - 1) * bb, sizeof(double) * (L - 1) * bb);
    }
    status[m] = tree_vjp_core(L, b, par, diag + m * L * bb, e, gd_bar + m * L * bb, geb,
                              ld_bar[m], d_bar + m * L * bb, eb);
    if (L > 1) memcpy(l_bar + m * (L - 1) * bb, eb, sizeof(double) * (L - 1) * bb);
    free(par); free(e); free(geb); free(eb);
  }
  return 0;
}

/* ---------------------------------------------- shared-factor siblings */

/* Solve and Gaussian sampling from the factor of the collect pass (the
 * gabp-sparse-inv 0.3.2 page: junction_solve, tree_logdet / junction_logdet and
 * sample_gaussian_tree passages, all reusing "the same factorization").  The
 * collect is a block LDL^T factorisation A = L D L^T with D = blockdiag(S_v)
 * and L_{p,v} = X_v = E_v S_v^{-1}, unit block lower triangular in any
 * children-first order:
 *   solve A x = y:   u = y; children first: u_p -= X_v u_v;
 *                    w_v = S_v^{-1} u_v (two triangular solves, S_v = R_v R_v^T);
 *                    x_root = w_root; parents first: x_v = w_v - X_v^T x_p
 *   sample:          x = L^{-T} D^{-1/2} z with D^{-1/2}_v = R_v^{-T}, the
 *                    upper triangular factor of S_v^{-1}; then
 *                    Cov(x) = L^{-T} D^{-1} L^{-1} = A^{-1} for z ~ N(0, I):
 *                    w_v = R_v^{-T} z_v, then the same parents-first sweep.
 * Vectors are [n][b][k] (k right-hand sides, k fastest).  mode 0 = solve,
 * 1 = sample.  Returns 0, 2 (invalid parent array) or 3 (a pivot is not
 * positive definite: out is NaN). */

/* R Y = Bm, R lower triangular, Y and Bm b x k */
static void trsv_L(int b, int64_t k, const double *R, const double *Bm, double *Y) {
  for (int64_t c = 0; c < k; ++c)
    for (int i = 0; i < b; ++i) {
      double s = Bm[i * k + c];
      for (int t = 0; t < i; ++t) s -= R[i * b + t] * Y[t * k + c];
      Y[i * k + c] = s / R[i * b + i];
    }
}

/* R^T Y = Bm, R lower triangular */
static void trsv_LT(int b, int64_t k, const double *R, const double *Bm, double *Y) {
  for (int64_t c = 0; c < k; ++c)
    for (int i = b - 1; i >= 0; --i) {
      double s = Bm[i * k + c];
      for (int t = i + 1; t < b; ++t) s -= R[t * b + i] * Y[t * k + c];
      Y[i * k + c] = s / R[i * b + i];
    }
}

static int tree_ldl_apply(int64_t n, int b, const int32_t *parent, const double *diag,
                          const double *edge, int64_t k, const double *in, double *out,
                          int mode) {
  const int64_t bb = (int64_t)b * b, bk = (int64_t)b * k;
  int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int64_t root = -1;
  if (tree_depths(n, parent, depth, &root)) {
    free(depth);
    return 2;
  }
  int32_t H = 0;
  for (int64_t v = 0; v < n; ++v)
    if (depth[v] > H) H = depth[v];
  int64_t *cnt = (int64_t *)calloc((size_t)H + 2, sizeof(int64_t));
  for (int64_t v = 0; v < n; ++v) cnt[depth[v] + 1]++;
  for (int32_t d = 0; d <= H; ++d) cnt[d + 1] += cnt[d];
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  int64_t *fillp = (int64_t *)malloc(sizeof(int64_t) * ((size_t)H + 1));
  for (int32_t d = 0; d <= H; ++d) fillp[d] = cnt[d];
  for (int64_t v = 0; v < n; ++v) order[fillp[depth[v]]++] = v;

  double *S = (double *)malloc(sizeof(double) * n * bb);
  double *R = (double *)malloc(sizeof(double) * n * bb);
  double *X = (double *)calloc((size_t)(n * bb), sizeof(double));
  double *w = (double *)malloc(sizeof(double) * n * bk);
  double *u = (double *)malloc(sizeof(double) * n * bk);
  double *t = (double *)malloc(sizeof(double) * bk);
  double *ws = (double *)malloc(sizeof(double) * 3 * bb);
  int rc = 0;
  /* collect: R_v and X_v, deepest level first */
  memcpy(S, diag, sizeof(double) * n * bb);
  for (int32_t d = H; d >= 0 && !rc; --d)
    for (int64_t q = cnt[d]; q < cnt[d + 1]; ++q) {
      const int64_t v = order[q], p = parent[v];
      if (chol(b, S + v * bb, R + v * bb)) {
        rc = 3;
        break;
      }
      if (p >= 0) collect_edge(b, R + v * bb, edge + v * bb, S + p * bb, X + v * bb, ws,
                               ws + bb, ws + 2 * bb);
    }
  if (rc) {
    fill_nan(out, n * bk);
  } else {
    if (mode == 0) {
      memcpy(u, in, sizeof(double) * n * bk);
      for (int32_t d = H; d >= 1; --d) /* L u = y, children first */
        for (int64_t q = cnt[d]; q < cnt[d + 1]; ++q) {
          const int64_t v = order[q], p = parent[v];
          for (int i = 0; i < b; ++i)
            for (int64_t c = 0; c < k; ++c) {
              double s = 0.0;
              for (int j = 0; j < b; ++j) s += X[v * bb + i * b + j] * u[v * bk + j * k + c];
              u[p * bk + i * k + c] -= s;
            }
        }
      for (int64_t v = 0; v < n; ++v) { /* D w = u */
        trsv_L(b, k, R + v * bb, u + v * bk, t);
        trsv_LT(b, k, R + v * bb, t, w + v * bk);
      }
    } else {
      for (int64_t v = 0; v < n; ++v) trsv_LT(b, k, R + v * bb, in + v * bk, w + v * bk);
    }
    /* L^T x = w, parents first */
    memcpy(out + root * bk, w + root * bk, sizeof(double) * bk);
    for (int32_t d = 1; d <= H; ++d)
      for (int64_t q = cnt[d]; q < cnt[d + 1]; ++q) {
        const int64_t v = order[q], p = parent[v];
        for (int i = 0; i < b; ++i)
          for (int64_t c = 0; c < k; ++c) {
            double s = 0.0;
            for (int j = 0; j < b; ++j) s += X[v * bb + j * b + i] * out[p * bk + j * k + c];
            out[v * bk + i * k + c] = w[v * bk + i * k + c] - s;
          }
      }
  }
  free(depth); free(cnt); free(order); free(fillp);
  free(S); free(R); free(X); free(w); free(u); free(t); free(ws);
  return rc;
}

ORACLE_API int oracle_tree_apply(int64_t n, int b, const int32_t *parent, const double *diag,
                                 const double *edge, int64_t k, const double *in, double *out,
                                 int mode) {
  if (n < 1 || b < 1 || k < 0 || !parent || !diag || !edge || !in || !out) return 1;
  if (mode != 0 && mode != 1) return 1;
  return tree_ldl_apply(n, b, parent, diag, edge, k, in, out, mode);
}

/* Chains as path trees rooted at the last block, one matrix after another;
 * status[m] = 0 or 3. */
ORACLE_API int oracle_chain_apply(int64_t B, int64_t L, int b, const double *diag,
                                  const double *lower, int64_t k, const double *in, double *out,
                                  int mode, int32_t *status) {
  if (B < 0 || L < 1 || b < 1 || k < 0 || !diag || !in || !out || !status) return 1;
  if (L > 1 && !lower) return 1;
  if (mode != 0 && mode != 1) return 1;
  const int64_t bb = (int64_t)b * b, bk = (int64_t)b * k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < B; ++m) {
    int32_t *par = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
    double *e = (double *)calloc((size_t)(L * bb), sizeof(double));
    for (int64_t i = 0; i < L; ++i) par[i] = i + 1 < L ? (int32_t)(i + 1) : -1;
    if (L > 1) memcpy(e, lower + m * (L - 1) * bb, sizeof(double) * (L - 1) * bb);
    status[m] = tree_ldl_apply(L, b, par, diag + m * L * bb, e, k, in + m * L * bk,
                               out + m * L * bk, mode);
    free(par);
    free(e);
  }
  return 0;
}

/* ------------------------------------------------- non-symmetric ladder */

/* Inverse of a general b x b block by Gaussian elimination on [A | I]
 * without pivoting (the page's non-symmetric kernels eliminate "with no
 * pivoting", safe while block-diagonally dominant).  Returns 0, or 1 if a
 * pivot is zero or not finite. */
static int gen_inverse(int b, const double *A, double *Ainv) {
  const int w = 2 * b;
  double *M = (double *)malloc(sizeof(double) * (size_t)b * w);
  int rc = 0;
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < w; ++c) M[r * w + c] = c < b ? A[r * b + c] : (c - b == r ? 1.0 : 0.0);
  for (int k = 0; k < b && !rc; ++k) {
    const double d = M[k * w + k];
    if (d == 0.0 || !isfinite(d)) {
      rc = 1;
      break;
    }
    for (int c = 0; c < w; ++c) M[k * w + c] /= d;
    for (int r = 0; r < b; ++r) {
      if (r == k) continue;
      const double f = M[r * w + k];
      for (int c = 0; c < w; ++c) M[r * w + c] -= f * M[k * w + c];
    }
  }
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) Ainv[r * b + c] = M[r * w + b + c];
  free(M);
  return rc;
}

/* Block lower-bidiagonal M (item "Non-symmetric chain" of "Implemented and
 * tested kernels"): fully local, G_ii = M_ii^{-1},
 * G_{i+1,i} = -M_{i+1,i+1}^{-1} M_{i+1,i} M_ii^{-1}.  info[m] = 0, or 1 + the
 * smallest block index whose inverse breaks down (the matrix's outputs are
 * then NaN). */
ORACLE_API int oracle_bidiag(int64_t B, int64_t L, int b, const double *diag,
                             const double *lower, double *G_diag, double *G_lower,
                             int32_t *info) {
  if (B < 0 || L < 1 || b < 1 || !diag || !G_diag || !info) return 1;
  if (L > 1 && (!lower || !G_lower)) return 1;
  const int64_t bb = (int64_t)b * b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < B; ++m) {
    double *Gd = G_diag + m * L * bb, *Gl = G_lower + m * (L - 1) * bb;
    double *T = (double *)malloc(sizeof(double) * bb);
    int32_t fail = 0;
    for (int64_t i = 0; i < L && !fail; ++i)
      if (gen_inverse(b, diag + (m * L + i) * bb, Gd + i * bb)) fail = (int32_t)(i + 1);
    if (fail) {
      fill_nan(Gd, L * bb);
      if (L > 1) fill_nan(Gl, (L - 1) * bb);
    } else {
      for (int64_t i = 0; i + 1 < L; ++i) {
        matmul(b, lower + (m * (L - 1) + i) * bb, Gd + i * bb, T); /* M_{i+1,i} M_ii^{-1} */
        matmul(b, Gd + (i + 1) * bb, T, Gl + i * bb);
        for (int64_t e = 0; e < bb; ++e) Gl[i * bb + e] = -Gl[i * bb + e];
      }
    }
    info[m] = fail;
    free(T);
  }
  return 0;
}

/* Non-symmetric tree (item "Non-symmetric tree"): a general block matrix
 * whose off-diagonal graph is a tree, with independent directed edge blocks
 * up[v] = M_{p,v} and down[v] = M_{v,p}.  Two-sided block elimination,
 * children first, no pivoting:
 *   collect:    S_v = M_vv - sum_children up_c S_c^{-1} down_c
 *   root:       G_rr = S_r^{-1}
 *   distribute: G_{p,v} = -G_pp up_v S_v^{-1},  G_{v,p} = -S_v^{-1} down_v G_pp,
 *               G_vv = S_v^{-1} + S_v^{-1} down_v G_pp up_v S_v^{-1}
 * (in the symmetric case up_v = E_v, down_v = E_v^T this is the tree kernel
 * above).  Order as in oracle_tree; info = v + 1 for the first breakdown in
 * that order. */
ORACLE_API int oracle_nonsym_tree(int64_t n, int b, const int32_t *parent, const double *diag,
                                  const double *up, const double *down, double *G_diag,
                                  double *G_up, double *G_down, int32_t *info) {
  if (n < 1 || b < 1 || !parent || !diag || !up || !down || !G_diag || !G_up || !G_down || !info)
    return 1;
  const int64_t bb = (int64_t)b * b;
  int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int64_t root = -1;
  if (tree_depths(n, parent, depth, &root)) {
    free(depth);
    return 2;
  }
  int32_t H = 0;
  for (int64_t v = 0; v < n; ++v)
    if (depth[v] > H) H = depth[v];
  int64_t *cnt = (int64_t *)calloc((size_t)H + 2, sizeof(int64_t));
  for (int64_t v = 0; v < n; ++v) cnt[depth[v] + 1]++;
  for (int32_t d = 0; d <= H; ++d) cnt[d + 1] += cnt[d];
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  int64_t *fillp = (int64_t *)malloc(sizeof(int64_t) * ((size_t)H + 1));
  for (int32_t d = 0; d <= H; ++d) fillp[d] = cnt[d];
  for (int64_t v = 0; v < n; ++v) order[fillp[depth[v]]++] = v;
  double *S = (double *)malloc(sizeof(double) * n * bb);
  double *Si = (double *)malloc(sizeof(double) * n * bb);
  double *T = (double *)malloc(sizeof(double) * 3 * bb);
  double *T2 = T + bb, *T3 = T + 2 * bb;
  memcpy(S, diag, sizeof(double) * n * bb);
  int32_t fail = 0;
  for (int32_t lev = H; lev >= 0 && !fail; --lev)  /* deepest level first */
    for (int64_t q = cnt[lev]; q < cnt[lev + 1]; ++q) {
      const int64_t v = order[q], p = parent[v];
      if (gen_inverse(b, S + v * bb, Si + v * bb)) {
        fail = (int32_t)(v + 1);
        break;
      }
      if (p >= 0) {
        matmul(b, Si + v * bb, down + v * bb, T);  /* S_v^{-1} down_v */
        matmul(b, up + v * bb, T, T2);              /* up_v S_v^{-1} down_v */
        for (int64_t e = 0; e < bb; ++e) S[p * bb + e] -= T2[e];
      }
    }
  if (fail) {
    fill_nan(G_diag, n * bb);
    fill_nan(G_up, n * bb);
    fill_nan(G_down, n * bb);
  } else {
    memcpy(G_diag + root * bb, Si + root * bb, sizeof(double) * bb);
    memset(G_up + root * bb, 0, sizeof(double) * bb);
    memset(G_down + root * bb, 0, sizeof(double) * bb);
    for (int32_t d = 1; d <= H; ++d)
      for (int64_t q = cnt[d]; q < cnt[d + 1]; ++q) {
        const int64_t v = order[q], p = parent[v];
        const double *Gp = G_diag + p * bb, *Sv = Si + v * bb;
        matmul(b, up + v * bb, Sv, T);   /* up_v S_v^{-1} */
        matmul(b, Gp, T, T2);            /* G_pp up_v S_v^{-1} = -G_{p,v} */
        for (int64_t e = 0; e < bb; ++e) G_up[v * bb + e] = -T2[e];
        matmul(b, Sv, down + v * bb, T); /* S_v^{-1} down_v */
        matmul(b, T, Gp, T3);            /* S_v^{-1} down_v G_pp = -G_{v,p} */
        for (int64_t e = 0; e < bb; ++e) G_down[v * bb + e] = -T3[e];
        matmul(b, T, T2, T3);            /* S_v^{-1} down_v G_pp up_v S_v^{-1} */
        for (int64_t e = 0; e < bb; ++e) G_diag[v * bb + e] = Sv[e] + T3[e];
      }
  }
  *info = fail;
  free(depth); free(cnt); free(order); free(fillp);
  free(S); free(Si); free(T);
  return 0;
}

/* ------------------------------------------------------- junction tree
 * General sparse SPD (gabp-sparse-inv page, junction-tree section): an
 * arbitrary block pattern is eliminated node by node in an elimination order
 * (default: greedy minimum degree); eliminating v joins all of v's remaining
 * neighbours into a clique, so the pattern grows to its chordal completion S
 * = pattern(L + L^T).  The selected inverse on S then follows from the block
 * LDL^T factor by the multi-neighbour Takahashi recurrence.
 *
 * Symbolic part.  The elimination graph is a dense n x n byte matrix; the
 * degree of a node is its number of remaining neighbours.  Minimum degree
 * picks, at every step, the remaining node of smallest degree, the smallest
 * label among ties.  For step s (node v = order[s]) the labels of v's
 * remaining neighbours at that moment, ascending, are nbr[nbr_ptr[s] ..
 * nbr_ptr[s+1]): the later nodes w with (w, v) in S.  Returns 0, 2 for bad
 * input (an edge out of range, i <= j, a repeated edge, an order that is not
 * a permutation), 3 if `cap` is too small (nbr_ptr[n] then holds the size
 * needed; nothing else is meaningful). */
ORACLE_API int oracle_eliminate(int64_t n, int64_t m, const int32_t *ei, const int32_t *ej,
                                const int32_t *order_in, int32_t *order_out, int64_t *nbr_ptr,
                                int32_t *nbr, int64_t cap) {
  if (n < 1 || n > 16384 || m < 0) return 2;
  unsigned char *adj = (unsigned char *)calloc((size_t)(n * n), 1);
  unsigned char *gone = (unsigned char *)calloc((size_t)n, 1);
  int64_t *deg = (int64_t *)calloc((size_t)n, sizeof(int64_t));
  int32_t *nb = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int rc = 0;
  for (int64_t e = 0; e < m && !rc; ++e) {
    const int64_t i = ei[e], j = ej[e];
    if (j < 0 || i <= j || i >= n || adj[i * n + j]) {
      rc = 2;
      break;
    }
    adj[i * n + j] = adj[j * n + i] = 1;
    deg[i]++;
    deg[j]++;
  }
  int64_t fill = 0;
  nbr_ptr[0] = 0;
  for (int64_t s = 0; s < n && !rc; ++s) {
    int64_t v = -1;
    if (order_in) {
      v = order_in[s];
      if (v < 0 || v >= n || gone[v]) {
        rc = 2;
        break;
      }
    } else {
      for (int64_t u = 0; u < n; ++u)
        if (!gone[u] && (v < 0 || deg[u] < deg[v])) v = u;
    }
    gone[v] = 1;
    order_out[s] = (int32_t)v;
    int64_t k = 0;
    for (int64_t u = 0; u < n; ++u)
      if (adj[v * n + u]) nb[k++] = (int32_t)u;
    for (int64_t a = 0; a < k; ++a) {
      if (fill + a < cap) nbr[fill + a] = nb[a];
      for (int64_t c = a + 1; c < k; ++c) {
        const int64_t x = nb[a], y = nb[c];
        if (!adj[x * n + y]) {
          adj[x * n + y] = adj[y * n + x] = 1;
          deg[x]++;
          deg[y]++;
        }
      }
    }
    for (int64_t a = 0; a < k; ++a) {
      adj[v * n + nb[a]] = adj[nb[a] * n + v] = 0;
      deg[nb[a]]--;
    }
    fill += k;
    nbr_ptr[s + 1] = fill;
  }
  if (!rc && fill > cap) rc = 3;
  free(adj);
  free(gone);
  free(deg);
  free(nb);
  return rc;
}

/* Slot of the block (w, x) of S, x eliminated before w: its index in the
 * neighbour list of x's elimination step; -1 if absent. */
static int64_t junction_slot(const int64_t *nbr_ptr, const int32_t *nbr, const int32_t *pos,
                             int32_t w, int32_t x) {
  const int64_t s = pos[x];
  for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t)
    if (nbr[t] == w) return t;
  return -1;
}

/* Numeric part, for a batch of B matrices on the pattern of one elimination
 * (order, nbr_ptr, nbr from oracle_eliminate).  Slot t of the neighbour list
 * of step s holds the block (w, v) of S with w = nbr[t] and v = order[s].
 *   diag   [B][n]   A_vv by label;  Aoff [B][nnz]  A_{w,v} per slot (zero
 *                   where (w, v) is fill)
 *   G_diag [B][n]   (A^-1)_vv by label;  G_off [B][nnz]  (A^-1)_{w,v} per slot
 *   logdet [B], info [B] (0, or 1 + the label of the first node in the
 *                   elimination order whose Schur pivot is not positive
 *                   definite; logdet is then NaN).
 * Block LDL^T, right-looking, in the elimination order: the pivot of v is
 * D_v = C_vv (the fully updated diagonal block), L_{w,v} = C_{w,v} D_v^-1 for
 * every later neighbour w, and every pair (w1, w2) of later neighbours
 * receives C_{w1,w2} -= L_{w1,v} D_v L_{w2,v}^T (= L_{w1,v} C_{w2,v}^T).
 * Takahashi, in reverse elimination order, with N = the later neighbours of v:
 *   G_{w,v} = - sum_{x in N} G_{w,x} L_{x,v}        (w in N)
 *   G_vv    = D_v^-1 - sum_{w in N} L_{w,v}^T G_{w,v}
 * where G_{w,x} for w before x is G_{x,w}^T.  Every block read lies in S
 * because N is a clique of S; returns 4 if the given pattern is not closed
 * that way (not the output of an elimination), else 0. */
/* The block LDL^T of one matrix in the elimination order (right-looking):
 * on return Cd holds the pivots D_v by label, Rv their Cholesky factors
 * (D_v = R_v R_v^T), Di their inverses and Lo the multipliers
 * L_{w,v} = C_{w,v} D_v^-1 by slot; Co is the working copy of the
 * off-diagonal blocks.  *fail = 0 or 1 + the label of the first node whose
 * pivot is not positive definite (its Di and Rv are NaN); *ld = log det A
 * when *fail == 0.  Returns 1 if the pattern is not closed under elimination
 * (a block the Schur update needs is missing), else 0. */
static int junction_ldl(int64_t n, int b, const int32_t *order, const int64_t *nbr_ptr,
                        const int32_t *nbr, const int32_t *pos, const double *A_diag,
                        const double *A_off, double *Cd, double *Co, double *Lo, double *Di,
                        double *Rv, double *T, int32_t *fail, double *ld) {
  const int64_t bb = (int64_t)b * b, nnz = nbr_ptr[n];
  int bad_pattern = 0;
  memcpy(Cd, A_diag, sizeof(double) * (size_t)(n * bb));
  if (nnz) memcpy(Co, A_off, sizeof(double) * (size_t)(nnz * bb));
  *fail = 0;
  *ld = 0.0;
  for (int64_t s = 0; s < n; ++s) {
    const int32_t v = order[s];
    /* the pivot: D_v = R R^T, its inverse and its log det */
    if (chol(b, Cd + v * bb, Rv + v * bb)) {
      if (!*fail) *fail = v + 1;
      fill_nan(Di + v * bb, bb);
      fill_nan(Rv + v * bb, bb);
    } else {
      inv_from_chol(b, Rv + v * bb, Di + v * bb);
      *ld += logdet_chol(b, Rv + v * bb);
    }
    for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t)
      matmul(b, Co + t * bb, Di + v * bb, Lo + t * bb);            /* L_{w,v} */
    /* Schur update of every pair of later neighbours */
    for (int64_t t1 = nbr_ptr[s]; t1 < nbr_ptr[s + 1]; ++t1)
      for (int64_t t2 = nbr_ptr[s]; t2 < nbr_ptr[s + 1]; ++t2) {
        const int32_t w1 = nbr[t1], w2 = nbr[t2];
        if (pos[w1] < pos[w2]) continue;
        mm_nt(b, Lo + t1 * bb, Co + t2 * bb, T);                     /* L_{w1,v} C_{w2,v}^T */
        const int64_t t12 = w1 == w2 ? 0 : junction_slot(nbr_ptr, nbr, pos, w1, w2);
        if (t12 < 0) {                          /* not a chordal pattern */
          bad_pattern = 1;
          continue;
        }
        add_to(bb, w1 == w2 ? Cd + w1 * bb : Co + t12 * bb, T, -1.0);
      }
  }
  return bad_pattern;
}

/* Numeric part, for a batch of B matrices on the pattern of one elimination
 * (order, nbr_ptr, nbr from oracle_eliminate).  Slot t of the neighbour list
 * of step s holds the block (w, v) of S with w = nbr[t] and v = order[s].
 *   diag   [B][n]   A_vv by label;  Aoff [B][nnz]  A_{w,v} per slot (zero
 *                   where (w, v) is fill)
 *   G_diag [B][n]   (A^-1)_vv by label;  G_off [B][nnz]  (A^-1)_{w,v} per slot
 *   logdet [B], info [B] (0, or 1 + the label of the first node in the
 *                   elimination order whose Schur pivot is not positive
 *                   definite; logdet is then NaN).
 * Block LDL^T, right-looking, in the elimination order (junction_ldl): the
 * pivot of v is D_v = C_vv (the fully updated diagonal block),
 * L_{w,v} = C_{w,v} D_v^-1 for every later neighbour w, and every pair
 * (w1, w2) of later neighbours receives C_{w1,w2} -= L_{w1,v} D_v L_{w2,v}^T
 * (= L_{w1,v} C_{w2,v}^T).
 * Takahashi, in reverse elimination order, with N = the later neighbours of v:
 *   G_{w,v} = - sum_{x in N} G_{w,x} L_{x,v}        (w in N)
 *   G_vv    = D_v^-1 - sum_{w in N} L_{w,v}^T G_{w,v}
 * where G_{w,x} for w before x is G_{x,w}^T.  Every block read lies in S
 * because N is a clique of S; returns 4 if the given pattern is not closed
 * that way (not the output of an elimination), else 0. */
ORACLE_API int oracle_junction(int64_t B, int64_t n, int b, const int32_t *order,
                               const int64_t *nbr_ptr, const int32_t *nbr, const double *diag,
                               const double *Aoff, double *G_diag, double *G_off, double *logdet,
                               int32_t *info) {
  const int64_t bb = (int64_t)b * b, nnz = nbr_ptr[n];
  int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  for (int64_t s = 0; s < n; ++s) pos[order[s]] = (int32_t)s;
  int bad_pattern = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t mat = 0; mat < B; ++mat) {
    double *Cd = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *Co = (double *)malloc(sizeof(double) * (size_t)((nnz ? nnz : 1) * bb));
    double *Lo = (double *)malloc(sizeof(double) * (size_t)((nnz ? nnz : 1) * bb));
    double *Di = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *Rv = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *T = (double *)malloc(sizeof(double) * bb);
    double *T2 = (double *)malloc(sizeof(double) * bb);
    double *Gd = G_diag + mat * n * bb, *Go = G_off + mat * nnz * bb;
    int32_t fail = 0;
    double ld = 0.0;
    if (junction_ldl(n, b, order, nbr_ptr, nbr, pos, diag + mat * n * bb, Aoff + mat * nnz * bb,
                     Cd, Co, Lo, Di, Rv, T, &fail, &ld))
      bad_pattern = 1;
    /* Takahashi, reverse elimination order */
    for (int64_t s = n - 1; s >= 0; --s) {
      const int32_t v = order[s];
      for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t) {
        const int32_t w = nbr[t];
        memset(Go + t * bb, 0, sizeof(double) * bb);
        for (int64_t u = nbr_ptr[s]; u < nbr_ptr[s + 1]; ++u) {
          const int32_t x = nbr[u];
          const double *Gwx;
          const int64_t twx = w == x ? 0 : pos[w] > pos[x] ? junction_slot(nbr_ptr, nbr, pos, w, x)
                                                           : junction_slot(nbr_ptr, nbr, pos, x, w);
          if (twx < 0) {
            bad_pattern = 1;
            continue;
          }
          if (w == x) {
            Gwx = Gd + w * bb;
          } else if (pos[w] > pos[x]) {
            Gwx = Go + twx * bb;
          } else {
            transpose(b, Go + twx * bb, T2);
            Gwx = T2;
          }
          matmul(b, Gwx, Lo + u * bb, T);                             /* G_{w,x} L_{x,v} */
          add_to(bb, Go + t * bb, T, -1.0);
        }
      }
      memcpy(Gd + v * bb, Di + v * bb, sizeof(double) * bb);
      for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t) {
        mm_tn(b, Lo + t * bb, Go + t * bb, T);                        /* L_{w,v}^T G_{w,v} */
        add_to(bb, Gd + v * bb, T, -1.0);
      }
    }
    logdet[mat] = fail ? NAN : ld;
    info[mat] = fail;
    free(Cd); free(Co); free(Lo); free(Di); free(Rv); free(T); free(T2);
  }
  free(pos);
  return bad_pattern ? 4 : 0;
}

/* Solve and Gaussian sampling on the filled pattern, from the same block
 * LDL^T (gabp-sparse-inv page, junction-tree section: junction_solve for one
 * or several right-hand sides, and Gaussian sampling, both reusing the
 * factorisation of the selected inverse):
 *   solve A x = y:  u = y; in elimination order, for every later neighbour
 *                   w of v: u_w -= L_{w,v} u_v; then w_v = D_v^-1 u_v (two
 *                   triangular solves with R_v); in reverse order:
 *                   x_v = w_v - sum_{w in N(v)} L_{w,v}^T x_w
 *   sample:         w_v = R_v^-T z_v (D_v = R_v R_v^T), then the same reverse
 *                   sweep, x = L^-T D^-1/2 z: Cov(x) = L^-T D^-1 L^-1 = A^-1
 *                   for z ~ N(0, I).
 * in, out [B][n][b][k] by label (k right-hand sides, k fastest); mode 0 =
 * solve, 1 = sample; info [B] as for oracle_junction, and a matrix that
 * fails gets NaN in out.  Returns 0, 1 for a bad argument, 4 for a pattern
 * that is not closed under elimination. */
ORACLE_API int oracle_junction_apply(int64_t B, int64_t n, int b, const int32_t *order,
                                     const int64_t *nbr_ptr, const int32_t *nbr,
                                     const double *diag, const double *Aoff, int64_t k,
                                     const double *in, double *out, int mode, int32_t *info) {
  if (B < 0 || n < 1 || b < 1 || k < 0 || (mode != 0 && mode != 1)) return 1;
  const int64_t bb = (int64_t)b * b, bk = (int64_t)b * k, nnz = nbr_ptr[n];
  int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  for (int64_t s = 0; s < n; ++s) pos[order[s]] = (int32_t)s;
  int bad_pattern = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t mat = 0; mat < B; ++mat) {
    double *Cd = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *Co = (double *)malloc(sizeof(double) * (size_t)((nnz ? nnz : 1) * bb));
    double *Lo = (double *)malloc(sizeof(double) * (size_t)((nnz ? nnz : 1) * bb));
    double *Di = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *Rv = (double *)malloc(sizeof(double) * (size_t)(n * bb));
    double *T = (double *)malloc(sizeof(double) * bb);
    double *u = (double *)malloc(sizeof(double) * (size_t)(n * bk + 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(n * bk + 1));
    double *t1 = (double *)malloc(sizeof(double) * (size_t)(bk + 1));
    const double *y = in + mat * n * bk;
    double *x = out + mat * n * bk;
    int32_t fail = 0;
    double ld = 0.0;
    if (junction_ldl(n, b, order, nbr_ptr, nbr, pos, diag + mat * n * bb, Aoff + mat * nnz * bb,
                     Cd, Co, Lo, Di, Rv, T, &fail, &ld))
      bad_pattern = 1;
    info[mat] = fail;
    if (fail) {
      fill_nan(x, n * bk);
    } else {
      if (mode == 0) {
        memcpy(u, y, sizeof(double) * (size_t)(n * bk));
        for (int64_t s = 0; s < n; ++s) {          /* L u' = y, elimination order */
          const int32_t v = order[s];
          for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t) {
            const int32_t wl = nbr[t];
            for (int i = 0; i < b; ++i)
              for (int64_t c = 0; c < k; ++c) {
                double acc = 0.0;
                for (int j = 0; j < b; ++j) acc += Lo[t * bb + i * b + j] * u[v * bk + j * k + c];
                u[wl * bk + i * k + c] -= acc;
              }
          }
        }
        for (int64_t v = 0; v < n; ++v) {          /* D w = u' */
          trsv_L(b, k, Rv + v * bb, u + v * bk, t1);
          trsv_LT(b, k, Rv + v * bb, t1, w + v * bk);
        }
      } else {
        for (int64_t v = 0; v < n; ++v) trsv_LT(b, k, Rv + v * bb, y + v * bk, w + v * bk);
      }
      for (int64_t s = n - 1; s >= 0; --s) {       /* L^T x = w, reverse order */
        const int32_t v = order[s];
        for (int i = 0; i < b; ++i)
          for (int64_t c = 0; c < k; ++c) {
            double acc = 0.0;
            for (int64_t t = nbr_ptr[s]; t < nbr_ptr[s + 1]; ++t) {
              const int32_t wl = nbr[t];
              for (int j = 0; j < b; ++j) acc += Lo[t * bb + j * b + i] * x[wl * bk + j * k + c];
            }
            x[v * bk + i * k + c] = w[v * bk + i * k + c] - acc;
          }
      }
    }
    free(Cd); free(Co); free(Lo); free(Di); free(Rv); free(T); free(u); free(w); free(t1);
  }
  free(pos);
  return bad_pattern ? 4 : 0;
}

/* Depth of every node of a valid tree (host helper for the tests); returns 0,
 * or 2 for an invalid parent array. */
ORACLE_API int oracle_tree_depths(int64_t n, const int32_t *parent, int32_t *depth) {
  int64_t root;
  if (n < 1 || !parent || !depth) return 1;
  return tree_depths(n, parent, depth, &root);
}

/* Number of OpenMP threads the batch loops use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
#endif
ORACLE_API int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads of the batch loops started from the
 * calling thread (n >= 1); returns the previous number. */
ORACLE_API int oracle_set_num_threads(int n) {
#ifdef _OPENMP
  const int old = omp_get_max_threads();
  if (n >= 1) omp_set_num_threads(n);
  return old;
#else
  (void)n;
  return 1;
#endif
}
