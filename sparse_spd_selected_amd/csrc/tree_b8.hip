// tree_b8.hip -- tree selected inverse for block sizes b <= 8 on the
// breadth-first depth level-set schedule of tree_plan.cpp (gabp-sparse-inv
// 0.3.2 page, item Tree of "Implemented and tested kernels": collect
// leaves -> root, then distribute root -> leaves; the batched form loops over
// levels, each level a few batched block operations).
//
// Blocks are held one row per lane (rows8.h), eight tree nodes per
// wavefront.  Per node v (position p), with E_v = edge[v] = A_{parent,v}:
//   collect:    S_v = D_v - sum_children M_c (children contiguous, in order),
//               Sinv_v = S_v^{-1},  X_v = E_v Sinv_v,  M_v = X_v E_v^T
//   root:       G_rr = Sinv_r  (written by the level-0 collect)
//   distribute: X_v = E_v Sinv_v,  V = G_pp X_v,  G_edge[v] = -V,
//               G_diag[v] = Sinv_v + X_v^T V
// Sinv_v and M_v live in the workspace as padded 8 x 8 blocks indexed by
// position; X_v is recomputed from the re-read edge block.
#include <climits>

#include "internal.h"
#include "rows8.h"

namespace selinv {

namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup
constexpr int kSlots = 8;  // nodes per wavefront

// kFactor: the collect pass of the shared factor: the packed lower triangle
// of Sinv_v (wg-style layout, packed_entries(b) per position) goes to
// st_sinv, which may be null (log det only); G_diag, G_edge are unused.
template <typename T, bool kFactor>
__global__ __launch_bounds__(256) void tree8_collect(
    int64_t p0, int64_t p1, int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ child_beg, const int32_t *__restrict__ child_end,
    const int32_t *__restrict__ fail_rank, const T *__restrict__ diag, const T *__restrict__ edge,
    T *__restrict__ st_sinv, T *__restrict__ st_m, double *__restrict__ st_ld,
    int32_t *__restrict__ st_fail, int32_t *__restrict__ first_fail, T *__restrict__ G_diag,
    T *__restrict__ G_edge) {
  __shared__ __align__(32) T lds[kWaves][2][kSlots * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[wave][0]}, sb{lds[wave][1]};
  const int64_t p = p0 + (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * kSlots + s;
  const bool valid = p < p1;
  const int bb = b * b;
  int64_t v = 0;
  int32_t cb = 0, ce = 0;
  if (valid) {
    v = node_at[p];
    cb = child_beg[p];
    ce = child_end[p];
  }
  r8::Row<T> S = r8::load_sym(diag + v * bb, b, i);  // slots past the level re-read node 0
  bool child_failed = false;
  // children's messages, four loads in flight at a time, subtracted in child order
  for (int32_t c0 = cb; c0 < ce; c0 += 4) {
    r8::Row<T> mc[4];
    int32_t fc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t c = min(c0 + q, ce - 1);
      mc[q] = r8::load8(st_m + static_cast<int64_t>(c) * 64, i);
      fc[q] = st_fail[c];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (c0 + q < ce) {
#pragma unroll
        for (int k = 0; k < 8; ++k) S.v[k] -= mc[q].v[k];
        child_failed |= fc[q] != 0;
      }
    }
  }
  f16::PivotLog pl;
  const bool bad = r8::gj_inverse(S, sa, s, i, pl);
  if (valid && i == 0) {
    const bool failed = bad || child_failed;
    st_fail[p] = failed ? 1 : 0;
    st_ld[p] = failed ? static_cast<double>(__builtin_nan("")) : pl.log();
    if (bad && !child_failed) atomicMin(first_fail, fail_rank[p]);
  }
  if constexpr (kFactor) {
    if (valid && st_sinv && i < b) {  // row i of the packed lower triangle
      T *row = st_sinv + p * ((b * (b + 1) / 2 + 3) / 4 * 4) + i * (i + 1) / 2;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c <= i) row[c] = S.v[c];
    }
  } else {
    if (valid) r8::store8(st_sinv + p * 64, i, S);
    if (p == 0) {  // root closure: G_rr = Sinv_r, and the root's edge slot is zero
      r8::store(G_diag + v * bb, b, i, S);
      r8::store(G_edge + v * bb, b, i, r8::zero<T>());
    }
  }
  // message to the parent (all slots take part in the staging; only valid
  // non-root slots store)
  const r8::Row<T> E = (valid && p != 0) ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  f16::wave_sync();
  sa.put(s, i, S);
  sb.put(s, i, E);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(E, sa, s, r8::zero<T>());   // E_v Sinv_v
  const r8::Row<T> M = r8::mul_t(X, sb, s, r8::zero<T>());  // X_v E_v^T
  if (valid && p != 0) r8::store8(st_m + p * 64, i, M);
}

template <typename T>
__global__ __launch_bounds__(256) void tree8_distribute(
    int64_t p0, int64_t p1, int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ parent_node, const T *__restrict__ edge,
    const T *__restrict__ st_sinv, const int32_t *__restrict__ first_fail, T *__restrict__ G_diag,
    T *__restrict__ G_edge) {
  __shared__ __align__(32) T lds[kWaves][2][kSlots * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[wave][0]}, sb{lds[wave][1]};
  const int64_t p = p0 + (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * kSlots + s;
  const bool valid = p < p1;
  const int bb = b * b;
  const bool failed = *first_fail != INT_MAX;
  int64_t v = 0, u = 0;
  if (valid) {
    v = node_at[p];
    u = parent_node[p];
  }
  const r8::Row<T> Si = valid ? r8::load8(st_sinv + p * 64, i) : r8::zero<T>();
  const r8::Row<T> E = valid ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  const r8::Row<T> G = valid ? r8::load(G_diag + u * bb, b, i) : r8::zero<T>();
  sa.put(s, i, Si);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(E, sa, s, r8::zero<T>());  // E_v Sinv_v
  sb.put(s, i, X);
  f16::wave_sync();
  const r8::Row<T> V = r8::mul(G, sb, s, r8::zero<T>());  // G_pp X_v
  f16::wave_sync();
  sa.put(s, i, V);
  f16::wave_sync();
  const r8::Row<T> Gv = r8::mul_tn(sb, sa, s, i, Si);     // Sinv_v + X_v^T V
  if (!valid) return;
  if (failed) {
    r8::Row<T> nan;
#pragma unroll
    for (int k = 0; k < 8; ++k) nan.v[k] = static_cast<T>(__builtin_nan(""));
    r8::store(G_edge + v * bb, b, i, nan);
    r8::store(G_diag + v * bb, b, i, nan);
    return;
  }
  r8::store(G_edge + v * bb, b, i, r8::neg(V));
  r8::store(G_diag + v * bb, b, i, Gv);
}

// log det A = sum of the per-node terms in a fixed order, in two stages:
// workgroup w reduces the contiguous chunk [w * chunk, (w + 1) * chunk)
// (thread t takes entries t, t + 1024, ... of the chunk, then a fixed tree),
// and one workgroup adds the partials in index order and sets info.
constexpr int kFinishGroups = 128;

__global__ __launch_bounds__(1024) void tree8_ld_partial(int64_t n, int64_t chunk,
                                                         const double *__restrict__ st_ld,
                                                         double *__restrict__ partial) {
  __shared__ double part[1024];
  const int64_t a = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t e = min(a + chunk, n);
  double acc = 0.0;
  for (int64_t k = a + threadIdx.x; k < e; k += 1024) acc += st_ld[k];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(64) void tree8_finish(const double *__restrict__ partial,
                                                   const int32_t *__restrict__ rank_node,
                                                   const int32_t *__restrict__ first_fail,
                                                   double *__restrict__ logdet,
                                                   int32_t *__restrict__ info) {
  if (threadIdx.x != 0) return;
  double acc = 0.0;
  for (int w = 0; w < kFinishGroups; ++w) acc += partial[w];
  const bool failed = *first_fail != INT_MAX;
  *logdet = failed ? __builtin_nan("") : acc;
  if (info) *info = failed ? rank_node[*first_fail] + 1 : 0;
}

__global__ void tree8_init(int32_t *first_fail) { *first_fail = INT_MAX; }

}  // namespace

size_t tree8_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return 2 * align_up(n * 64 * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         align_up(n * sizeof(int32_t)) + align_up(sizeof(int32_t)) +
         align_up(kFinishGroups * sizeof(double));
}

template <typename T>
hipError_t tree8_launch(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag,
                        T *G_edge, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  const int64_t n = plan->n;
  const int b = plan->b;
  Carve cv(ws);
  T *st_sinv = cv.take<T>(n * 64);
  T *st_m = cv.take<T>(n * 64);
  double *st_ld = cv.take<double>(n);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  double *partial = cv.take<double>(kFinishGroups);
  const TreePlanDev &d = plan->dev;
  const int64_t per_block = kWaves * kSlots;
  hipLaunchKernelGGL(tree8_init, dim3(1), dim3(1), 0, s, first_fail);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    const unsigned grid = static_cast<unsigned>((p1 - p0 + per_block - 1) / per_block);
    hipLaunchKernelGGL((tree8_collect<T, false>), dim3(grid), dim3(256), 0, s, p0, p1, b, d.node_at,
                       d.child_beg, d.child_end, d.fail_rank, diag, edge, st_sinv, st_m, st_ld,
                       st_fail, first_fail, G_diag, G_edge);
  }
  for (int32_t lev = 1; lev < plan->levels; ++lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    const unsigned grid = static_cast<unsigned>((p1 - p0 + per_block - 1) / per_block);
    hipLaunchKernelGGL(tree8_distribute<T>, dim3(grid), dim3(256), 0, s, p0, p1, b, d.node_at,
                       d.parent_node, edge, st_sinv, first_fail, G_diag, G_edge);
  }
  const int64_t chunk = (n + kFinishGroups - 1) / kFinishGroups;
  hipLaunchKernelGGL(tree8_ld_partial, dim3(kFinishGroups), dim3(1024), 0, s, n, chunk, st_ld,
                     partial);
  hipLaunchKernelGGL(tree8_finish, dim3(1), dim3(64), 0, s, partial, d.rank_node, first_fail,
                     logdet, info);
  return hipGetLastError();
}

size_t tree8_factor_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return align_up(n * 64 * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         align_up(n * sizeof(int32_t)) + align_up(sizeof(int32_t)) +
         align_up(kFinishGroups * sizeof(double));
}

template <typename T>
hipError_t tree8_factor_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                               T *factor, double *logdet, int32_t *info, void *ws,
                               hipStream_t s) {
  const int64_t n = plan->n;
  const int b = plan->b;
  Carve cv(ws);
  T *st_m = cv.take<T>(n * 64);
  double *st_ld = cv.take<double>(n);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  double *partial = cv.take<double>(kFinishGroups);
  const TreePlanDev &d = plan->dev;
  const int64_t per_block = kWaves * kSlots;
  hipLaunchKernelGGL(tree8_init, dim3(1), dim3(1), 0, s, first_fail);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    const unsigned grid = static_cast<unsigned>((p1 - p0 + per_block - 1) / per_block);
    hipLaunchKernelGGL((tree8_collect<T, true>), dim3(grid), dim3(256), 0, s, p0, p1, b,
                       d.node_at, d.child_beg, d.child_end, d.fail_rank, diag, edge, factor, st_m,
                       st_ld, st_fail, first_fail, nullptr, nullptr);
  }
  const int64_t chunk = (n + kFinishGroups - 1) / kFinishGroups;
  hipLaunchKernelGGL(tree8_ld_partial, dim3(kFinishGroups), dim3(1024), 0, s, n, chunk, st_ld,
                     partial);
  hipLaunchKernelGGL(tree8_finish, dim3(1), dim3(64), 0, s, partial, d.rank_node, first_fail,
                     logdet, info);
  return hipGetLastError();
}

template hipError_t tree8_factor_launch<float>(const selinv_tree_plan *, const float *,
                                               const float *, float *, double *, int32_t *,
                                               void *, hipStream_t);
template hipError_t tree8_factor_launch<double>(const selinv_tree_plan *, const double *,
                                                const double *, double *, double *, int32_t *,
                                                void *, hipStream_t);
template hipError_t tree8_launch<float>(const selinv_tree_plan *, const float *, const float *,
                                        float *, float *, double *, int32_t *, void *,
                                        hipStream_t);
template hipError_t tree8_launch<double>(const selinv_tree_plan *, const double *, const double *,
                                         double *, double *, double *, int32_t *, void *,
                                         hipStream_t);

}  // namespace selinv
