// generic.hip -- selected inverse kernels for any block size 1 <= b <= 32.
// One workgroup per chain / per star leaf / per tree node, blocks in LDS.
// These are the fallback for block sizes without a specialised kernel; the
// recurrences are the collect / root / distribute steps of the
// gabp-sparse-inv 0.3.2 page ("Implemented and tested kernels"):
//   collect:    S_v = D_v - sum_c M_c,  Sinv_v = S_v^{-1},
//               X_v = E_v Sinv_v,  M_v = X_v E_v^T      (E_v = A_{p,v})
//   root:       G_rr = Sinv_r
//   distribute: V = G_pp X_v,  G_{p,v} = -V,  G_vv = Sinv_v + X_v^T V
// log det A = sum of ln(pivots) of every S_v.
#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {

namespace {

inline int threads_for(int b) { return b <= 8 ? 64 : 256; }

template <typename T>
__global__ void chain_generic(int64_t L, int b, const T *__restrict__ diag,
                              const T *__restrict__ lower, T *__restrict__ G_diag,
                              T *__restrict__ G_lower, double *__restrict__ logdet,
                              int32_t *__restrict__ info, T *__restrict__ state) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *C = S + bb, *X = C + bb, *M = X + bb, *G = M + bb, *V = G + bb, *col = V + bb;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * bb;
  const T *Cm = lower + m * (L - 1) * bb;
  T *Gd = G_diag + m * L * bb;
  T *Gl = G_lower + m * (L - 1) * bb;
  T *st = state + m * L * 2 * bb;  // per block i: Sinv_i, X_i

  double ld = 0.0;
  int32_t fail = 0;
  wg::load_sym_lower(S, D, b);
  for (int64_t i = 0; i < L; ++i) {
    double ldi;
    if (wg::spd_inverse(S, b, col, &ldi)) {
      fail = static_cast<int32_t>(i + 1);
      break;
    }
    ld += ldi;
    if (i == L - 1) break;
    wg::copy(st + 2 * i * bb, S, bb);
    wg::copy(C, Cm + i * bb, bb);
    wg::gemm<T, false, false>(X, C, S, b);              // X_i = C_i Sinv_i
    wg::copy(st + (2 * i + 1) * bb, X, bb);
    wg::load_sym_lower(S, D + (i + 1) * bb, b);
    wg::gemm_sym<T, false, true>(S, S, X, C, b, T(-1));  // S_{i+1} = D_{i+1} - X_i C_i^T
  }
  if (fail) {
    if (threadIdx.x == 0) {
      logdet[m] = wg::qnan<double>();
      if (info) info[m] = fail;
    }
    for (int64_t e = threadIdx.x; e < L * bb; e += blockDim.x) Gd[e] = wg::qnan<T>();
    for (int64_t e = threadIdx.x; e < (L - 1) * bb; e += blockDim.x) Gl[e] = wg::qnan<T>();
    return;
  }
  if (threadIdx.x == 0) {
    logdet[m] = ld;
    if (info) info[m] = 0;
  }
  // root closure: G_{L-1,L-1} = Sinv_{L-1} (still in S)
  wg::copy(G, S, bb);
  wg::copy(Gd + (L - 1) * bb, G, bb);
  for (int64_t i = L - 2; i >= 0; --i) {
    wg::copy(X, st + (2 * i + 1) * bb, bb);
    wg::copy(M, st + 2 * i * bb, bb);
    wg::gemm<T, false, false>(V, G, X, b);               // V = G_{i+1,i+1} X_i
    wg::copy_scaled(Gl + i * bb, V, bb, T(-1));          // G_{i+1,i} = -V
    wg::gemm_sym<T, true, false>(G, M, X, V, b, T(1));   // G_ii = Sinv_i + X_i^T V
    wg::copy(Gd + i * bb, G, bb);
  }
}

// ------------------------------------------------------------------ star

// Leaf collect: one workgroup per (matrix, leaf).  A leaf has no children,
// so S_j = D_j.  The centre is the parent: E_j = A_{0,j} = coupling[j]^T.
//   X_j = E_j Sinv_j = coupling[j]^T Sinv_j,  M_j = X_j coupling[j]
template <typename T>
__global__ void star_leaf_collect(int64_t K, int b, const T *__restrict__ leaves,
                                  const T *__restrict__ coupling, T *__restrict__ st_sinv,
                                  T *__restrict__ st_x, T *__restrict__ st_m,
                                  double *__restrict__ st_ld, int32_t *__restrict__ st_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *F = S + bb, *X = F + bb, *col = X + bb;
  const int64_t leaf = blockIdx.x;  // m * K + j
  wg::load_sym_lower(S, leaves + leaf * bb, b);
  double ld;
  if (wg::spd_inverse(S, b, col, &ld)) {
    if (threadIdx.x == 0) {
      st_fail[leaf] = 1;
      st_ld[leaf] = wg::qnan<double>();
    }
    return;
  }
  if (threadIdx.x == 0) {
    st_fail[leaf] = 0;
    st_ld[leaf] = ld;
  }
  wg::copy(st_sinv + leaf * bb, S, bb);
  wg::copy(F, coupling + leaf * bb, bb);
  wg::gemm<T, true, false>(X, F, S, b);                     // X_j = F^T Sinv_j
  wg::copy(st_x + leaf * bb, X, bb);
  wg::gemm_sym<T, false, false>(st_m + leaf * bb, nullptr, X, F, b, T(1));  // M_j = X_j F
}

// Centre: one workgroup per matrix.  S_0 = A_00 - sum_j M_j (index order),
// G_00 = S_0^{-1}; log det = sum of leaf terms (index order) + centre term.
template <typename T>
__global__ void star_center(int64_t K, int b, const T *__restrict__ center,
                            const T *__restrict__ st_m, const double *__restrict__ st_ld,
                            const int32_t *__restrict__ st_fail, T *__restrict__ G_center,
                            double *__restrict__ logdet, int32_t *__restrict__ info,
                            int32_t *__restrict__ mat_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t first_bad;
  const int bb = b * b;
  T *S = smem, *col = S + bb;
  const int64_t m = blockIdx.x;
  if (threadIdx.x == 0) first_bad = INT_MAX;
  __syncthreads();
  for (int64_t j = threadIdx.x; j < K; j += blockDim.x)
    if (st_fail[m * K + j]) atomicMin(&first_bad, static_cast<int32_t>(j));
  wg::load_sym_lower(S, center + m * bb, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    T s = S[e];
    for (int64_t j = 0; j < K; ++j) s -= st_m[(m * K + j) * bb + e];
    S[e] = s;
  }
  __syncthreads();
  int32_t fail = 0;
  double ldc = 0.0;
  if (first_bad != INT_MAX)
    fail = first_bad + 2;
  else if (wg::spd_inverse(S, b, col, &ldc))
    fail = 1;
  if (threadIdx.x == 0) {
    if (info) info[m] = fail;
    mat_fail[m] = fail;
    if (fail) {
      logdet[m] = wg::qnan<double>();
    } else {
      double ld = 0.0;
      for (int64_t j = 0; j < K; ++j) ld += st_ld[m * K + j];
      logdet[m] = ld + ldc;
    }
  }
  if (fail) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) G_center[m * bb + e] = wg::qnan<T>();
    return;
  }
  wg::copy(G_center + m * bb, S, bb);
}

// Leaf distribute: V = G_00 X_j (so G_{0,j} = -V), G_cross[j] = G_{j,0} = -V^T,
// G_leaf[j] = Sinv_j + X_j^T V.
template <typename T>
__global__ void star_leaf_distribute(int64_t K, int b, const T *__restrict__ G_center,
                                     const T *__restrict__ st_sinv, const T *__restrict__ st_x,
                                     const int32_t *__restrict__ mat_fail,
                                     T *__restrict__ G_leaf, T *__restrict__ G_cross) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *G = smem, *X = G + bb, *V = X + bb, *Si = V + bb;
  const int64_t leaf = blockIdx.x;
  const int64_t m = leaf / K;
  if (mat_fail[m]) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      G_leaf[leaf * bb + e] = wg::qnan<T>();
      G_cross[leaf * bb + e] = wg::qnan<T>();
    }
    return;
  }
  wg::copy(G, G_center + m * bb, bb);
  wg::copy(X, st_x + leaf * bb, bb);
  wg::copy(Si, st_sinv + leaf * bb, bb);
  wg::gemm<T, false, false>(V, G, X, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    const int r = e / b, c = e % b;
    G_cross[leaf * bb + e] = -V[c * b + r];
  }
  wg::gemm_sym<T, true, false>(G_leaf + leaf * bb, Si, X, V, b, T(1));
}

// ------------------------------------------------------------------ tree

// Collect for one depth level: positions [p0, p1) of the breadth-first order.
template <typename T>
__global__ void tree_collect_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                   const int32_t *__restrict__ child_beg,
                                   const int32_t *__restrict__ child_end,
                                   const int32_t *__restrict__ fail_rank, const T *__restrict__ diag,
                                   const T *__restrict__ edge, T *__restrict__ st_sinv,
                                   T *__restrict__ st_x, T *__restrict__ st_m,
                                   double *__restrict__ st_ld, int32_t *__restrict__ st_fail,
                                   int32_t *__restrict__ first_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t child_failed;
  const int bb = b * b;
  T *S = smem, *E = S + bb, *X = E + bb, *col = X + bb;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  const int32_t cb = child_beg[p], ce = child_end[p];
  if (threadIdx.x == 0) child_failed = 0;
  __syncthreads();
  for (int32_t c = cb + threadIdx.x; c < ce; c += blockDim.x)
    if (st_fail[c]) child_failed = 1;
  wg::load_sym_lower(S, diag + v * bb, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    T s = S[e];
    for (int32_t c = cb; c < ce; ++c) s -= st_m[static_cast<int64_t>(c) * bb + e];
    S[e] = s;
  }
  __syncthreads();
  double ld;
  if (child_failed || wg::spd_inverse(S, b, col, &ld)) {
    if (threadIdx.x == 0) {
      st_fail[p] = 1;
      st_ld[p] = wg::qnan<double>();
      if (!child_failed) atomicMin(first_fail, fail_rank[p]);
    }
    return;
  }
  if (threadIdx.x == 0) {
    st_fail[p] = 0;
    st_ld[p] = ld;
  }
  wg::copy(st_sinv + p * bb, S, bb);
  if (p == 0) return;  // the root has no parent edge
  wg::copy(E, edge + v * bb, bb);
  wg::gemm<T, false, false>(X, E, S, b);                              // X_v = E_v Sinv_v
  wg::copy(st_x + p * bb, X, bb);
  wg::gemm_sym<T, false, true>(st_m + p * bb, nullptr, X, E, b, T(1));  // M_v = X_v E_v^T
}

// Distribute for one depth level >= 1 (the root is closed by tree_root).
template <typename T>
__global__ void tree_distribute_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                      const int32_t *__restrict__ parent_pos,
                                      const T *__restrict__ st_sinv, const T *__restrict__ st_x,
                                      const int32_t *__restrict__ first_fail,
                                      T *__restrict__ G_diag, T *__restrict__ G_edge) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *G = smem, *X = G + bb, *V = X + bb, *Si = V + bb;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  if (*first_fail != INT_MAX) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      G_diag[v * bb + e] = wg::qnan<T>();
      G_edge[v * bb + e] = wg::qnan<T>();
    }
    return;
  }
  const int64_t u = node_at[parent_pos[p]];
  wg::copy(G, G_diag + u * bb, bb);
  wg::copy(X, st_x + p * bb, bb);
  wg::copy(Si, st_sinv + p * bb, bb);
  wg::gemm<T, false, false>(V, G, X, b);
  wg::copy_scaled(G_edge + v * bb, V, bb, T(-1));
  wg::gemm_sym<T, true, false>(G_diag + v * bb, Si, X, V, b, T(1));
}

// Root closure plus the deterministic log-det reduction and info.
template <typename T>
__global__ void tree_root(int64_t n, int b, const int32_t *__restrict__ node_at,
                          const int32_t *__restrict__ rank_node, const T *__restrict__ st_sinv,
                          const double *__restrict__ st_ld, const int32_t *__restrict__ first_fail,
                          T *__restrict__ G_diag, T *__restrict__ G_edge,
                          double *__restrict__ logdet, int32_t *__restrict__ info) {
  __shared__ double part[256];
  const int bb = b * b;
  const int64_t r = node_at[0];
  const bool failed = *first_fail != INT_MAX;
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    G_diag[r * bb + e] = failed ? wg::qnan<T>() : st_sinv[e];
    G_edge[r * bb + e] = T(0);
  }
  // fixed-order reduction: contiguous chunk per thread, then a fixed tree
  const int nt = blockDim.x;
  const int64_t chunk = (n + nt - 1) / nt;
  double s = 0.0;
  const int64_t a = threadIdx.x * chunk;
  for (int64_t k = a; k < a + chunk && k < n; ++k) s += st_ld[k];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = nt / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *logdet = failed ? wg::qnan<double>() : part[0];
    if (info) *info = failed ? rank_node[*first_fail] + 1 : 0;
  }
}

__global__ void init_int(int32_t *p, int32_t v) { *p = v; }

}  // namespace

// ------------------------------------------------------------ launchers

size_t chain_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  if (b <= 8) return chain_small_workspace_bytes(dtype_bytes, B, L);
  if (b == 16) return chain16_workspace_bytes(dtype_bytes, B, L);
  if (b == 32) {
    const int P = chain32_segments(B, L);
    return P ? chain32_seg_workspace_bytes(dtype_bytes, B, L, P)
             : chain32_workspace_bytes(dtype_bytes, B, L);
  }
  return align_up(static_cast<size_t>(B) * L * 2 * b * b * dtype_bytes);
}

template <typename T>
hipError_t chain_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *G_diag,
                        T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b <= 8)
    return chain_small_launch<T>(B, L, b, diag, lower, G_diag, G_lower, logdet, info, ws, s);
  if (b == 16) return chain16_launch<T>(B, L, diag, lower, G_diag, G_lower, logdet, info, ws, s);
  if (b == 32) {
    const int P = chain32_segments(B, L);
    return P ? chain32_seg_launch<T>(B, L, P, diag, lower, G_diag, G_lower, logdet, info, ws, s)
             : chain32_launch<T>(B, L, diag, lower, G_diag, G_lower, logdet, info, ws, s);
  }
  const int nt = threads_for(b);
  const size_t shm = (6 * b * b + b) * sizeof(T);
  hipLaunchKernelGGL(chain_generic<T>, dim3(static_cast<unsigned>(B)), dim3(nt), shm, s, L, b,
                     diag, lower, G_diag, G_lower, logdet, info, static_cast<T *>(ws));
  return hipGetLastError();
}

size_t star_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if (b == 32) return star32_workspace_bytes(dtype_bytes, B, K);
  const size_t nl = static_cast<size_t>(B) * K, bb = static_cast<size_t>(b) * b;
  return align_up(3 * nl * bb * dtype_bytes) + align_up(nl * sizeof(double)) +
         align_up(nl * sizeof(int32_t)) + align_up(B * sizeof(int32_t));
}

template <typename T>
hipError_t star_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                       const T *coupling, T *G_center, T *G_leaf, T *G_cross, double *logdet,
                       int32_t *info, void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b == 32)
    return star32_launch<T>(B, K, center, leaves, coupling, G_center, G_leaf, G_cross, logdet,
                            info, ws, s);
  const size_t nl = static_cast<size_t>(B) * K, bb = static_cast<size_t>(b) * b;
  Carve cv(ws);
  T *st = cv.take<T>(3 * nl * bb);
  double *st_ld = cv.take<double>(nl);
  int32_t *st_fail = cv.take<int32_t>(nl);
  int32_t *mat_fail = cv.take<int32_t>(B);
  T *st_sinv = st, *st_x = st + nl * bb, *st_m = st + 2 * nl * bb;
  const int nt = threads_for(b);
  if (nl)
    hipLaunchKernelGGL(star_leaf_collect<T>, dim3(static_cast<unsigned>(nl)), dim3(nt),
                       (3 * bb + b) * sizeof(T), s, K, b, leaves, coupling, st_sinv, st_x, st_m,
                       st_ld, st_fail);
  hipLaunchKernelGGL(star_center<T>, dim3(static_cast<unsigned>(B)), dim3(nt),
                     (bb + b) * sizeof(T), s, K, b, center, st_m, st_ld, st_fail, G_center,
                     logdet, info, mat_fail);
  if (nl)
    hipLaunchKernelGGL(star_leaf_distribute<T>, dim3(static_cast<unsigned>(nl)), dim3(nt),
                       4 * bb * sizeof(T), s, K, b, G_center, st_sinv, st_x, mat_fail, G_leaf,
                       G_cross);
  return hipGetLastError();
}

size_t tree_workspace_bytes(const selinv_tree_plan *plan) {
  if (plan->b <= 8) return tree8_workspace_bytes(plan);
  const size_t n = plan->n, bb = static_cast<size_t>(plan->b) * plan->b;
  return align_up(3 * n * bb * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         align_up(n * sizeof(int32_t)) + align_up(sizeof(int32_t));
}

template <typename T>
hipError_t tree_launch(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag,
                       T *G_edge, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  if (plan->b <= 8) return tree8_launch<T>(plan, diag, edge, G_diag, G_edge, logdet, info, ws, s);
  const size_t n = plan->n;
  const int b = plan->b;
  const size_t bb = static_cast<size_t>(b) * b;
  Carve cv(ws);
  T *st = cv.take<T>(3 * n * bb);
  double *st_ld = cv.take<double>(n);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  T *st_sinv = st, *st_x = st + n * bb, *st_m = st + 2 * n * bb;
  const TreePlanDev &d = plan->dev;
  const int nt = threads_for(b);
  hipLaunchKernelGGL(init_int, dim3(1), dim3(1), 0, s, first_fail, INT_MAX);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(tree_collect_level<T>, dim3(static_cast<unsigned>(p1 - p0)), dim3(nt),
                       (3 * bb + b) * sizeof(T), s, p0, b, d.node_at, d.child_beg, d.child_end,
                       d.fail_rank, diag, edge, st_sinv, st_x, st_m, st_ld, st_fail, first_fail);
  }
  hipLaunchKernelGGL(tree_root<T>, dim3(1), dim3(256), 0, s, static_cast<int64_t>(n), b,
                     d.node_at, d.rank_node, st_sinv, st_ld, first_fail, G_diag, G_edge, logdet,
                     info);
  for (int32_t lev = 1; lev < plan->levels; ++lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(tree_distribute_level<T>, dim3(static_cast<unsigned>(p1 - p0)), dim3(nt),
                       4 * bb * sizeof(T), s, p0, b, d.node_at, d.parent_pos, st_sinv, st_x,
                       first_fail, G_diag, G_edge);
  }
  return hipGetLastError();
}

#define SELINV_INSTANTIATE(T)                                                                  \
  template hipError_t chain_launch<T>(int64_t, int64_t, int32_t, const T *, const T *, T *, T *, \
                                      double *, int32_t *, void *, hipStream_t);              \
  template hipError_t star_launch<T>(int64_t, int64_t, int32_t, const T *, const T *, const T *, \
                                     T *, T *, T *, double *, int32_t *, void *, hipStream_t); \
  template hipError_t tree_launch<T>(const selinv_tree_plan *, const T *, const T *, T *, T *,  \
                                     double *, int32_t *, void *, hipStream_t);
SELINV_INSTANTIATE(float)
SELINV_INSTANTIATE(double)
#undef SELINV_INSTANTIATE

}  // namespace selinv
