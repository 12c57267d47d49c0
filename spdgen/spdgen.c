/*
 * spdgen.c -- seeded synthetic inputs for the block chain / star / tree SPD
 * workloads.  This file only MAKES input matrices; it holds none of the
 * selected-inverse arithmetic, and both the float64 oracle and the GPU path
 * consume what it writes.
 *
 * Random numbers: Philox4x32-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2,
 * 3", SC 2011), written here from that definition.  Every value is a pure
 * function of (seed, stream, matrix index, entry index), so any single matrix
 * of a batch (or any block of it) can be regenerated on its own.
 *
 * Normals: Box-Muller on two 53-bit uniforms, both outputs used.
 *
 * Workload recipe (the batched SPD generators of the gabp-sparse-inv 0.3.2
 * project page, Quickstart section, restated with an explicit diagonal rule):
 *   off-diagonal blocks  iid N(0, 1/b)  (variance 1/b)
 *   diagonal blocks      D = W W^T / b + (diag_load + r) I,  W iid N(0,1) b x b,
 *   r = Gershgorin radius of the block row's off-diagonal blocks, each block
 *       taken as it sits in that block row (row-abs maximum per block, summed
 *       over the blocks of the row for star centres and tree nodes).
 * Hence lambda_min(A) >= diag_load for every generated matrix.
 *
 * Streams (Philox key word 1): 0 = off-diagonal blocks, 1 = W of the
 * non-centre diagonal blocks, 2 = W of a star centre, 3 = tree parent draws.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SPDGEN_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------- Philox */

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t y0 = hi1 ^ c[1] ^ k[0];
  const uint32_t y2 = hi0 ^ c[3] ^ k[1];
  c[0] = y0;
  c[1] = lo1;
  c[2] = y2;
  c[3] = lo0;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants between
 * rounds. */
SPDGEN_API void spdgen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                     uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

static inline double u53(uint32_t a, uint32_t b) {
  /* 53-bit uniform in [0, 1) */
  const uint64_t m = ((uint64_t)(a >> 5) << 26) | (uint64_t)(b >> 6);
  return (double)m * (1.0 / 9007199254740992.0);
}

/* Normal number `e` (0-based) of stream `stream`, matrix `mat`. */
static inline double normal_at(uint64_t seed, uint32_t stream, uint64_t mat, uint64_t e) {
  const uint64_t pair = e >> 1;
  const uint32_t ctr[4] = {(uint32_t)pair, (uint32_t)(pair >> 32), (uint32_t)mat,
                           (uint32_t)(mat >> 32)};
  const uint32_t key[2] = {(uint32_t)seed, stream ^ ((uint32_t)(seed >> 32) << 8)};
  uint32_t o[4];
  spdgen_philox4x32_10(ctr, key, o);
  const double u1 = 1.0 - u53(o[0], o[1]); /* (0, 1] */
  const double u2 = u53(o[2], o[3]);
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 6.283185307179586476925286766559 * u2;
  return (e & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* Both normals of pair `pair`. */
static inline void normal_pair(uint64_t seed, uint32_t stream, uint64_t mat, uint64_t pair,
                               double *z0, double *z1) {
  const uint32_t ctr[4] = {(uint32_t)pair, (uint32_t)(pair >> 32), (uint32_t)mat,
                           (uint32_t)(mat >> 32)};
  const uint32_t key[2] = {(uint32_t)seed, stream ^ ((uint32_t)(seed >> 32) << 8)};
  uint32_t o[4];
  spdgen_philox4x32_10(ctr, key, o);
  const double u1 = 1.0 - u53(o[0], o[1]);
  const double u2 = u53(o[2], o[3]);
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 6.283185307179586476925286766559 * u2;
  *z0 = rad * cos(ang);
  *z1 = rad * sin(ang);
}

/* Fill n normals [e0, e0+n) of a stream, scaled; each pair is drawn once.
 * Element e always equals scale * normal_at(seed, stream, mat, e). */
static void normals(uint64_t seed, uint32_t stream, uint64_t mat, uint64_t e0, int64_t n,
                    double scale, double *out) {
  int64_t i = 0;
  if (n > 0 && (e0 & 1)) {
    out[0] = scale * normal_at(seed, stream, mat, e0);
    i = 1;
  }
  for (; i + 1 < n; i += 2) {
    double z0, z1;
    normal_pair(seed, stream, mat, (e0 + (uint64_t)i) >> 1, &z0, &z1);
    out[i] = scale * z0;
    out[i + 1] = scale * z1;
  }
  if (i < n) out[i] = scale * normal_at(seed, stream, mat, e0 + (uint64_t)i);
}

SPDGEN_API double spdgen_normal(uint64_t seed, uint32_t stream, uint64_t mat, uint64_t e) {
  return normal_at(seed, stream, mat, e);
}

/* D = W W^T / b + shift * I, lower triangle computed, then mirrored, so that
 * D is exactly symmetric. */
static void gram_block(int b, const double *W, double shift, double *D) {
  for (int r = 0; r < b; ++r)
    for (int c = 0; c <= r; ++c) {
      double s = 0.0;
      for (int k = 0; k < b; ++k) s += W[r * b + k] * W[c * b + k];
      s /= (double)b;
      if (r == c) s += shift;
      D[r * b + c] = s;
      D[c * b + r] = s;
    }
}

/* max over rows of the absolute row sum of block B (b x b, row-major) */
static double rowabs_max(int b, const double *B) {
  double m = 0.0;
  for (int r = 0; r < b; ++r) {
    double s = 0.0;
    for (int c = 0; c < b; ++c) s += fabs(B[r * b + c]);
    if (s > m) m = s;
  }
  return m;
}

/* max over columns of the absolute column sum = rowabs_max of B^T */
static double colabs_max(int b, const double *B) {
  double m = 0.0;
  for (int c = 0; c < b; ++c) {
    double s = 0.0;
    for (int r = 0; r < b; ++r) s += fabs(B[r * b + c]);
    if (s > m) m = s;
  }
  return m;
}

/* ----------------------------------------------------------------- chain */

/* Block-tridiagonal chain, matrices [m0, m0+count) of a batch.
 *   diag  [count][L][b][b]     D_i
 *   lower [count][L-1][b][b]   lower[i] = A_{i+1,i}
 * Row i of the block matrix holds lower[i-1] (as is) and lower[i]^T, so its
 * Gershgorin radius is max_r ( sum_s |lower[i-1][r][s]| + sum_s |lower[i][s][r]| ). */
SPDGEN_API void spdgen_chain(uint64_t seed, int64_t m0, int64_t count, int64_t L, int b,
                             double diag_load, double *diag, double *lower) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < count; ++m) {
    const uint64_t mat = (uint64_t)(m0 + m);
    double *Dm = diag + m * L * bb;
    double *Cm = lower + m * (L - 1) * bb;
    if (L > 1) normals(seed, 0, mat, 0, (L - 1) * bb, sd, Cm);
    double *W = (double *)malloc(sizeof(double) * bb);
    for (int64_t i = 0; i < L; ++i) {
      normals(seed, 1, mat, (uint64_t)(i * bb), bb, 1.0, W);
      double r = 0.0;
      for (int row = 0; row < b; ++row) {
        double s = 0.0;
        if (i >= 1)
          for (int c = 0; c < b; ++c) s += fabs(Cm[(i - 1) * bb + row * b + c]);
        if (i <= L - 2)
          for (int c = 0; c < b; ++c) s += fabs(Cm[i * bb + c * b + row]);
        if (s > r) r = s;
      }
      gram_block(b, W, diag_load + r, Dm + i * bb);
    }
    free(W);
  }
}

/* ------------------------------------------------------------------ star */

/* Block arrowhead, matrices [m0, m0+count):
 *   center   [count][b][b]     A_{0,0}
 *   leaves   [count][K][b][b]  A_{j,j} (leaf j is block j+1)
 *   coupling [count][K][b][b]  A_{j,0} (leaf row, centre column)
 * leaf radius   = rowabs_max(A_{j,0})
 * centre radius = sum_j rowabs_max(A_{0,j}) = sum_j colabs_max(coupling[j]) */
SPDGEN_API void spdgen_star(uint64_t seed, int64_t m0, int64_t count, int64_t K, int b,
                            double diag_load, double *center, double *leaves,
                            double *coupling) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < count; ++m) {
    const uint64_t mat = (uint64_t)(m0 + m);
    double *Fm = coupling + m * K * bb;
    double *Lm = leaves + m * K * bb;
    normals(seed, 0, mat, 0, K * bb, sd, Fm);
    double *W = (double *)malloc(sizeof(double) * bb);
    double rc = 0.0;
    for (int64_t j = 0; j < K; ++j) {
      normals(seed, 1, mat, (uint64_t)(j * bb), bb, 1.0, W);
      gram_block(b, W, diag_load + rowabs_max(b, Fm + j * bb), Lm + j * bb);
      rc += colabs_max(b, Fm + j * bb);
    }
    normals(seed, 2, mat, 0, bb, 1.0, W);
    gram_block(b, W, diag_load + rc, center + m * bb);
    free(W);
  }
}

/* ------------------------------------------------------------------ tree */

/* Random recursive tree: parent[0] = -1, parent[v] = floor(u_v * v) with u_v
 * uniform in [0,1), i.e. uniform over [0, v). */
SPDGEN_API void spdgen_random_recursive_tree(uint64_t seed, int64_t n, int32_t *parent) {
  if (n <= 0) return;
  parent[0] = -1;
#pragma omp parallel for schedule(static)
  for (int64_t v = 1; v < n; ++v) {
    const uint32_t ctr[4] = {(uint32_t)v, (uint32_t)((uint64_t)v >> 32), 0u, 0u};
    const uint32_t key[2] = {(uint32_t)seed, 3u ^ ((uint32_t)(seed >> 32) << 8)};
    uint32_t o[4];
    spdgen_philox4x32_10(ctr, key, o);
    int64_t p = (int64_t)floor(u53(o[0], o[1]) * (double)v);
    if (p >= v) p = v - 1;
    parent[v] = (int32_t)p;
  }
}

/* Tree-structured SPD values for a given parent array (one matrix, index 0).
 *   diag [n][b][b]  D_v
 *   edge [n][b][b]  edge[v] = A_{parent(v),v}; the root slot is zero.
 * radius(v) = rowabs_max(A_{v,parent(v)}) + sum_{children c} rowabs_max(A_{v,c})
 *           = colabs_max(edge[v]) + sum_c rowabs_max(edge[c]).
 * parent must be a valid rooted tree (checked by the caller). */
SPDGEN_API void spdgen_tree(uint64_t seed, int64_t n, int b, double diag_load,
                            const int32_t *parent, double *diag, double *edge) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
  double *rad = (double *)calloc((size_t)n, sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < n; ++v) {
    if (parent[v] < 0)
      memset(edge + v * bb, 0, sizeof(double) * bb);
    else
      normals(seed, 0, 0, (uint64_t)(v * bb), bb, sd, edge + v * bb);
  }
  /* radius contributions, serial (a parent collects from its children) */
  for (int64_t v = 0; v < n; ++v) {
    if (parent[v] < 0) continue;
    rad[v] += colabs_max(b, edge + v * bb);
    rad[parent[v]] += rowabs_max(b, edge + v * bb);
  }
#pragma omp parallel
  {
    double *W = (double *)malloc(sizeof(double) * bb);
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
      normals(seed, 1, 0, (uint64_t)(v * bb), bb, 1.0, W);
      gram_block(b, W, diag_load + rad[v], diag + v * bb);
    }
    free(W);
  }
  free(rad);
}

/* ------------------------------------------------------------ cotangents */

/* Standard normal arrays for matrices [m0, m0+count), `per` numbers per
 * matrix, from stream 16 + k (k selects one of several arrays; the streams
 * of the SPD inputs are below 16).  Used as the cotangents that seed a
 * vector-Jacobian product. */
SPDGEN_API void spdgen_cotangent(uint64_t seed, uint32_t k, int64_t m0, int64_t count, int64_t per,
                                 double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < count; ++m)
    normals(seed, 16u + k, (uint64_t)(m0 + m), 0, per, 1.0, out + m * per);
}

/* ------------------------------------------------------- non-symmetric */

/* D = R + shift I with R iid N(0, 1/b) and shift = load + max_r (sum_s
 * |R_rs| + extra[r]): every scalar row of the block row is strictly
 * diagonally dominant by at least `load` (extra[r] = the absolute row sum of
 * the row's other blocks; |R_rr| is counted so that a negative R_rr cannot
 * eat into the margin), so elimination without pivoting is safe. */
static void dominant_block(int b, const double *R, const double *extra, double load, double *D) {
  double shift = 0.0;
  for (int r = 0; r < b; ++r) {
    double s = extra ? extra[r] : 0.0;
    for (int c = 0; c < b; ++c) s += fabs(R[r * b + c]);
    if (s > shift) shift = s;
  }
  shift += load;
  for (int r = 0; r < b; ++r)
    for (int c = 0; c < b; ++c) D[r * b + c] = R[r * b + c] + (r == c ? shift : 0.0);
}

/* Block lower-bidiagonal M (the non-symmetric chain of "Implemented and
 * tested kernels"), matrices [m0, m0+count):
 *   diag  [count][L][b][b]   M_ii (general)
 *   lower [count][L-1][b][b] lower[i] = M_{i+1,i} */
SPDGEN_API void spdgen_nonsym_bidiag(uint64_t seed, int64_t m0, int64_t count, int64_t L, int b,
                                     double diag_load, double *diag, double *lower) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < count; ++m) {
    const uint64_t mat = (uint64_t)(m0 + m);
    double *Cm = lower + m * (L - 1) * bb;
    if (L > 1) normals(seed, 4, mat, 0, (L - 1) * bb, sd, Cm);
    double *R = (double *)malloc(sizeof(double) * bb);
    double *ex = (double *)malloc(sizeof(double) * b);
    for (int64_t i = 0; i < L; ++i) {
      normals(seed, 5, mat, (uint64_t)(i * bb), bb, sd, R);
      for (int r = 0; r < b; ++r) {
        ex[r] = 0.0;
        if (i >= 1)
          for (int c = 0; c < b; ++c) ex[r] += fabs(Cm[(i - 1) * bb + r * b + c]);
      }
      dominant_block(b, R, ex, diag_load, diag + m * L * bb + i * bb);
    }
    free(R);
    free(ex);
  }
}

/* Tree-structured non-symmetric matrix for a given parent array: two
 * independent directed edge blocks per non-root node.
 *   diag [n][b][b]  M_vv (general)
 *   up   [n][b][b]  up[v]   = M_{parent(v),v}
 *   down [n][b][b]  down[v] = M_{v,parent(v)}     (root slots zero)
 * Block row v holds down[v] and up[c] for every child c. */
SPDGEN_API void spdgen_nonsym_tree(uint64_t seed, int64_t n, int b, double diag_load,
                                   const int32_t *parent, double *diag, double *up,
                                   double *down) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
  double *ex = (double *)calloc((size_t)(n * b), sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < n; ++v) {
    if (parent[v] < 0) {
      memset(up + v * bb, 0, sizeof(double) * bb);
      memset(down + v * bb, 0, sizeof(double) * bb);
    } else {
      normals(seed, 6, 0, (uint64_t)(v * bb), bb, sd, up + v * bb);
      normals(seed, 7, 0, (uint64_t)(v * bb), bb, sd, down + v * bb);
    }
  }
  for (int64_t v = 0; v < n; ++v) { /* row sums: serial, a parent collects from children */
    const int64_t p = parent[v];
    if (p < 0) continue;
    for (int r = 0; r < b; ++r)
      for (int c = 0; c < b; ++c) {
        ex[v * b + r] += fabs(down[v * bb + r * b + c]);
        ex[p * b + r] += fabs(up[v * bb + r * b + c]);
      }
  }
#pragma omp parallel
  {
    double *R = (double *)malloc(sizeof(double) * bb);
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
      normals(seed, 8, 0, (uint64_t)(v * bb), bb, sd, R);
      dominant_block(b, R, ex + v * b, diag_load, diag + v * bb);
    }
    free(R);
  }
  free(ex);
}

/* --------------------------------------------------------- general graph */

/* SPD values on an arbitrary block pattern shared by a batch (matrices
 * [m0, m0+count)): the random_spd_graph(num_nodes, edges, block_size, seed)
 * helper of the gabp-sparse-inv page's junction-tree section, restated with
 * the same recipe as the tree.
 *   edge_i, edge_j [m]      the pattern edges, edge_i[e] > edge_j[e]
 *   diag     [count][n][b][b]   D_v
 *   edge_val [count][m][b][b]   edge_val[e] = A_{edge_i[e], edge_j[e]}
 * radius(v) = sum over edges at v of the row-abs maximum of the block as it
 * sits in row v (rowabs_max for the row edge_i, colabs_max for edge_j).
 * Streams 9 (edge blocks) and 10 (W of the diagonal blocks). */
SPDGEN_API void spdgen_graph(uint64_t seed, int64_t m0, int64_t count, int64_t n, int64_t m,
                             int b, double diag_load, const int32_t *edge_i,
                             const int32_t *edge_j, double *diag, double *edge_val) {
  const int64_t bb = (int64_t)b * b;
  const double sd = 1.0 / sqrt((double)b);
#pragma omp parallel for schedule(static)
  for (int64_t mat = 0; mat < count; ++mat) {
    double *E = edge_val + mat * m * bb, *D = diag + mat * n * bb;
    double *rad = (double *)calloc((size_t)n, sizeof(double));
    double *W = (double *)malloc(sizeof(double) * bb);
    for (int64_t e = 0; e < m; ++e) {
      normals(seed, 9, (uint64_t)(m0 + mat), (uint64_t)(e * bb), bb, sd, E + e * bb);
      rad[edge_i[e]] += rowabs_max(b, E + e * bb);
      rad[edge_j[e]] += colabs_max(b, E + e * bb);
    }
    for (int64_t v = 0; v < n; ++v) {
      normals(seed, 10, (uint64_t)(m0 + mat), (uint64_t)(v * bb), bb, 1.0, W);
      gram_block(b, W, diag_load + rad[v], D + v * bb);
    }
    free(W);
    free(rad);
  }
}
