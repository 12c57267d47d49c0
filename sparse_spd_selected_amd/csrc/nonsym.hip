// nonsym.hip -- the non-symmetric ladder of the gabp-sparse-inv 0.3.2 page
// ("Implemented and tested kernels", items Non-symmetric chain and
// Non-symmetric tree), for any block size 1 <= b <= 32, blocks in LDS
// (block_wg.h).  No pivoting anywhere: the page's kernels eliminate without
// it, which is safe while the matrix is block-diagonally dominant; a zero or
// non-finite pivot is reported through info.
//
// Block lower-bidiagonal M (fully local, two batched block operations):
//   G_ii = M_ii^{-1},  G_{i+1,i} = -G_{i+1,i+1} M_{i+1,i} G_ii
// Non-symmetric tree, up[v] = M_{p,v}, down[v] = M_{v,p} (two-sided
// elimination, children first, on the level schedule of tree_plan.cpp):
//   collect:    S_v = M_vv - sum_children up_c S_c^{-1} down_c
//   root:       G_rr = S_r^{-1}
//   distribute: G_{p,v} = -G_pp up_v S_v^{-1},  G_{v,p} = -S_v^{-1} down_v G_pp,
//               G_vv = S_v^{-1} + (S_v^{-1} down_v) G_pp (up_v S_v^{-1})
#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {

namespace {

inline int ns_threads(int b) { return b <= 8 ? 64 : 256; }

__global__ void ns_fill_int(int32_t *p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// one workgroup per diagonal block
template <typename T>
__global__ void bidiag_inverse(int64_t L, int b, const T *__restrict__ diag,
                               T *__restrict__ G_diag, int32_t *__restrict__ first_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *A = smem, *rk = A + bb, *ck = rk + b;
  const int64_t blk = blockIdx.x, m = blk / L, i = blk % L;
  wg::copy(A, diag + blk * bb, bb);
  if (wg::gen_inverse(A, b, rk, ck)) {
    if (threadIdx.x == 0) atomicMin(first_fail + m, static_cast<int32_t>(i));
    return;
  }
  wg::copy(G_diag + blk * bb, A, bb);
}

// one workgroup per block row: G_{i+1,i} (i < L - 1), NaN for failed matrices,
// info from the row-0 workgroup
template <typename T>
__global__ void bidiag_lower(int64_t L, int b, const T *__restrict__ lower,
                             const int32_t *__restrict__ first_fail, T *__restrict__ G_diag,
                             T *__restrict__ G_lower, int32_t *__restrict__ info) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *Gi = smem, *Gn = Gi + bb, *C = Gn + bb, *T1 = C + bb;
  const int64_t blk = blockIdx.x, m = blk / L, i = blk % L;
  const int32_t ff = first_fail[m];
  if (i == 0 && threadIdx.x == 0 && info) info[m] = ff == INT_MAX ? 0 : ff + 1;
  T *Gl = G_lower + (m * (L - 1) + i) * bb;
  if (ff != INT_MAX) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      G_diag[blk * bb + e] = wg::qnan<T>();
      if (i < L - 1) Gl[e] = wg::qnan<T>();
    }
    return;
  }
  if (i == L - 1) return;
  wg::copy(Gi, G_diag + blk * bb, bb);
  wg::copy(Gn, G_diag + (blk + 1) * bb, bb);
  wg::copy(C, lower + (m * (L - 1) + i) * bb, bb);
  wg::gemm<T, false, false>(T1, C, Gi, b);  // M_{i+1,i} G_ii
  wg::gemm<T, false, false>(C, Gn, T1, b);  // G_{i+1,i+1} M_{i+1,i} G_ii
  wg::copy_scaled(Gl, C, bb, T(-1));
}

// ------------------------------------------------------------------ tree
template <typename T>
__global__ void nstree_collect_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                     const int32_t *__restrict__ child_beg,
                                     const int32_t *__restrict__ child_end,
                                     const int32_t *__restrict__ fail_rank,
                                     const T *__restrict__ diag, const T *__restrict__ up,
                                     const T *__restrict__ down, T *__restrict__ st_sinv,
                                     T *__restrict__ st_m, int32_t *__restrict__ st_fail,
                                     int32_t *__restrict__ first_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t child_failed;
  const int bb = b * b;
  T *S = smem, *U = S + bb, *T1 = U + bb, *rk = T1 + bb, *ck = rk + b;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  const int32_t cb = child_beg[p], ce = child_end[p];
  if (threadIdx.x == 0) child_failed = 0;
  __syncthreads();
  for (int32_t c = cb + threadIdx.x; c < ce; c += blockDim.x)
    if (st_fail[c]) child_failed = 1;
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    T s = diag[v * bb + e];
    for (int32_t c = cb; c < ce; ++c) s -= st_m[static_cast<int64_t>(c) * bb + e];
    S[e] = s;
  }
  __syncthreads();
  if (child_failed || wg::gen_inverse(S, b, rk, ck)) {
    if (threadIdx.x == 0) {
      st_fail[p] = 1;
      if (!child_failed) atomicMin(first_fail, fail_rank[p]);
    }
    return;
  }
  if (threadIdx.x == 0) st_fail[p] = 0;
  wg::copy(st_sinv + p * bb, S, bb);
  if (p == 0) return;
  wg::copy(U, down + v * bb, bb);
  wg::gemm<T, false, false>(T1, S, U, b);  // S^{-1} down_v
  wg::copy(U, up + v * bb, bb);
  wg::gemm<T, false, false>(st_m + p * bb, U, T1, b);  // up_v S^{-1} down_v
}

template <typename T>
__global__ void nstree_root(int b, const int32_t *__restrict__ node_at,
                            const int32_t *__restrict__ rank_node, const T *__restrict__ st_sinv,
                            const int32_t *__restrict__ first_fail, T *__restrict__ G_diag,
                            T *__restrict__ G_up, T *__restrict__ G_down,
                            int32_t *__restrict__ info) {
  const int bb = b * b;
  const int64_t r = node_at[0];
  const bool failed = *first_fail != INT_MAX;
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    G_diag[r * bb + e] = failed ? wg::qnan<T>() : st_sinv[e];
    G_up[r * bb + e] = T(0);
    G_down[r * bb + e] = T(0);
  }
  if (threadIdx.x == 0 && info) *info = failed ? rank_node[*first_fail] + 1 : 0;
}

template <typename T>
__global__ void nstree_distribute_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                        const int32_t *__restrict__ parent_node,
                                        const T *__restrict__ up, const T *__restrict__ down,
                                        const T *__restrict__ st_sinv,
                                        const int32_t *__restrict__ first_fail,
                                        T *__restrict__ G_diag, T *__restrict__ G_up,
                                        T *__restrict__ G_down) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *G = smem, *Si = G + bb, *E = Si + bb, *A1 = E + bb, *A2 = A1 + bb, *A3 = A2 + bb;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  if (*first_fail != INT_MAX) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      G_diag[v * bb + e] = wg::qnan<T>();
      G_up[v * bb + e] = wg::qnan<T>();
      G_down[v * bb + e] = wg::qnan<T>();
    }
    return;
  }
  const int64_t u = parent_node[p];
  wg::copy(G, G_diag + u * bb, bb);
  wg::copy(Si, st_sinv + p * bb, bb);
  wg::copy(E, up + v * bb, bb);
  wg::gemm<T, false, false>(A1, E, Si, b);  // up_v S^{-1}
  wg::gemm<T, false, false>(A2, G, A1, b);  // G_pp up_v S^{-1} = -G_{p,v}
  wg::copy_scaled(G_up + v * bb, A2, bb, T(-1));
  wg::copy(E, down + v * bb, bb);
  wg::gemm<T, false, false>(A1, Si, E, b);  // S^{-1} down_v
  wg::gemm<T, false, false>(A3, A1, G, b);  // S^{-1} down_v G_pp = -G_{v,p}
  wg::copy_scaled(G_down + v * bb, A3, bb, T(-1));
  wg::gemm_axpby<T, false, false>(G_diag + v * bb, T(1), Si, T(1), A1, A2, b);
}

}  // namespace

size_t bidiag_workspace_bytes(int64_t B) { return align_up(static_cast<size_t>(B) * sizeof(int32_t)); }

template <typename T>
hipError_t bidiag_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                         T *G_diag, T *G_lower, int32_t *info, void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b == 16) return bidiag16_launch<T>(B, L, diag, lower, G_diag, G_lower, info, s);
  int32_t *first_fail = static_cast<int32_t *>(ws);
  const int nt = ns_threads(b);
  const size_t bb = static_cast<size_t>(b) * b;
  hipLaunchKernelGGL(ns_fill_int, dim3(static_cast<unsigned>((B + 255) / 256)), dim3(256), 0, s,
                     first_fail, B, INT_MAX);
  const dim3 grid(static_cast<unsigned>(B * L));
  hipLaunchKernelGGL(bidiag_inverse<T>, grid, dim3(nt), (bb + 2 * b) * sizeof(T), s, L, b, diag,
                     G_diag, first_fail);
  hipLaunchKernelGGL(bidiag_lower<T>, grid, dim3(nt), 4 * bb * sizeof(T), s, L, b, lower,
                     first_fail, G_diag, G_lower, info);
  return hipGetLastError();
}

size_t nonsym_tree_workspace_bytes(const selinv_tree_plan *plan) {
  if (plan->b <= 8) return nstree8_workspace_bytes(plan);
  const size_t n = plan->n, bb = static_cast<size_t>(plan->b) * plan->b;
  return 2 * align_up(n * bb * plan->dtype_bytes) + align_up(n * sizeof(int32_t)) +
         align_up(sizeof(int32_t));
}

template <typename T>
hipError_t nonsym_tree_launch(const selinv_tree_plan *plan, const T *diag, const T *up,
                              const T *down, T *G_diag, T *G_up, T *G_down, int32_t *info,
                              void *ws, hipStream_t s) {
  if (plan->b <= 8)
    return nstree8_launch<T>(plan, diag, up, down, G_diag, G_up, G_down, info, ws, s);
  const size_t n = plan->n;
  const int b = plan->b;
  const size_t bb = static_cast<size_t>(b) * b;
  Carve cv(ws);
  T *st_sinv = cv.take<T>(n * bb);
  T *st_m = cv.take<T>(n * bb);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int nt = ns_threads(b);
  hipLaunchKernelGGL(ns_fill_int, dim3(1), dim3(1), 0, s, first_fail, int64_t(1), INT_MAX);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(nstree_collect_level<T>, dim3(static_cast<unsigned>(p1 - p0)), dim3(nt),
                       (3 * bb + 2 * b) * sizeof(T), s, p0, b, d.node_at, d.child_beg,
                       d.child_end, d.fail_rank, diag, up, down, st_sinv, st_m, st_fail,
                       first_fail);
  }
  hipLaunchKernelGGL(nstree_root<T>, dim3(1), dim3(256), 0, s, b, d.node_at, d.rank_node, st_sinv,
                     first_fail, G_diag, G_up, G_down, info);
  for (int32_t lev = 1; lev < plan->levels; ++lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(nstree_distribute_level<T>, dim3(static_cast<unsigned>(p1 - p0)),
                       dim3(nt), 6 * bb * sizeof(T), s, p0, b, d.node_at, d.parent_node, up, down,
                       st_sinv, first_fail, G_diag, G_up, G_down);
  }
  return hipGetLastError();
}

#define SELINV_INSTANTIATE(T)                                                                    \
  template hipError_t bidiag_launch<T>(int64_t, int64_t, int32_t, const T *, const T *, T *, T *, \
                                       int32_t *, void *, hipStream_t);                           \
  template hipError_t nonsym_tree_launch<T>(const selinv_tree_plan *, const T *, const T *,       \
                                            const T *, T *, T *, T *, int32_t *, void *,          \
                                            hipStream_t);
SELINV_INSTANTIATE(float)
SELINV_INSTANTIATE(double)
#undef SELINV_INSTANTIATE

}  // namespace selinv
