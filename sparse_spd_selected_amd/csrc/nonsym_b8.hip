// nonsym_b8.hip -- non-symmetric tree selected inverse for block sizes
// b <= 8 on the depth level-set schedule of tree_plan.cpp (gabp-sparse-inv
// page, "Implemented and tested kernels", item Non-symmetric tree: two-sided
// elimination with independent directed edge blocks, no pivoting).
//
// Blocks are held one row per lane (rows8.h), eight tree nodes per
// wavefront.  Per node v (position p) with up_v = M_{parent,v} and
// down_v = M_{v,parent}:
//   collect:    S_v = M_vv - sum_children up_c S_c^{-1} down_c,
//               Sinv_v = S_v^{-1} (Gauss-Jordan, no pivoting),
//               message up_v Sinv_v down_v to the parent
//   distribute: A = up_v Sinv_v, G_{p,v} = -G_pp A,
//               B = Sinv_v down_v, G_{v,p} = -B G_pp,
//               G_vv = Sinv_v + B G_pp A
// Diagonal blocks smaller than 8 are padded with the identity, the others
// with zeros, so every operation is an 8 x 8 one.  Sinv_v and the messages
// live in the workspace as padded 8 x 8 blocks indexed by position; once the
// parent has consumed a message, the slot holds G_vv for the node's children.
// Each pass is one launch over the plan's tiles with per-position flags
// between producer and consumer tiles (dataflow.h); messages, failure flags
// and the G_vv copies are exchanged through device-coherent accesses in the
// interleaved layout.
#include <climits>

#include "dataflow.h"
#include "internal.h"
#include "rows8.h"

namespace selinv {

namespace {

constexpr int kSlots = kTreeTile;  // nodes per wavefront

// row i of a general b x b diagonal block, identity-padded beyond b
template <typename T>
__device__ __forceinline__ r8::Row<T> load_diag(const T *P, int b, int i) {
  r8::Row<T> r = r8::load(P, b, i);
  if (i >= b) r.v[i] = T(1);
  return r;
}

// In-place inverse of the general 8 x 8 block of each slot (row i per lane)
// by Gauss-Jordan without pivoting: pivot k (d = a_kk) maps a_ij -> a_ij -
// a_ik a_kj / d (i, j != k), a_kj -> a_kj / d, a_ik -> -a_ik / d, a_kk ->
// 1 / d.  Row k is broadcast through `st`; a lane's a_ik is its own.  Returns
// true if a pivot of this lane's slot is zero or not finite.
template <typename T>
__device__ __forceinline__ bool gen_inverse8(r8::Row<T> &a, const r8::Stage<T> &st, int s,
                                             int i) {
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (i == k) st.put(s, k, a);
    f16::wave_sync();
    const r8::Row<T> rk = st.row(s, k);
    f16::wave_sync();
    const T d = rk.v[k];
    bad |= !(d != T(0)) || !__builtin_isfinite(d);
    const T inv = f16::rcp<T>(d);
    if (i == k) {
#pragma unroll
      for (int c = 0; c < 8; ++c) a.v[c] = c == k ? inv : rk.v[c] * inv;
    } else {
      const T f = a.v[k] * inv;
#pragma unroll
      for (int c = 0; c < 8; ++c) a.v[c] = c == k ? -f : a.v[c] - f * rk.v[c];
    }
  }
  return bad;
}

// Collect of one tile; workgroup w takes tile tiles - 1 - w (deepest level
// first); flags[p] becomes 1.
template <typename T>
__global__ __launch_bounds__(64) void nstree8_collect(
    int32_t tiles, const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi,
    int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ child_beg, const int32_t *__restrict__ child_end,
    const int32_t *__restrict__ fail_rank, const T *__restrict__ diag, const T *__restrict__ up,
    const T *__restrict__ down, T *__restrict__ st_sinv, T *__restrict__ st_m,
    int32_t *__restrict__ st_fail, int32_t *__restrict__ first_fail,
    int32_t *__restrict__ flags, int32_t *__restrict__ timeout, uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int32_t t = tiles - 1 - static_cast<int32_t>(blockIdx.x);
  const int64_t p = tile_lo[t] + s;
  const bool valid = p < tile_hi[t];
  const int bb = b * b;
  int64_t v = 0;
  int32_t cb = 0, ce = 0;
  if (valid) {
    v = node_at[p];
    cb = child_beg[p];
    ce = child_end[p];
  }
  r8::Row<T> S = load_diag(diag + v * bb, b, i);  // slots past the tile re-read node 0
  const bool edge = valid && p != 0;
  const r8::Row<T> Dn = edge ? r8::load(down + v * bb, b, i) : r8::zero<T>();
  const r8::Row<T> U = edge ? r8::load(up + v * bb, b, i) : r8::zero<T>();
  df::wait_flags(flags, cb, ce, 1, i, 8, timeout, deadline);
  df::acquire();
  bool child_failed = false;
  // children's messages, four loads in flight at a time, subtracted in child order
  for (int32_t c0 = cb; c0 < ce; c0 += 4) {
    r8::Row<T> mc[4];
    int32_t fc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t c = min(c0 + q, ce - 1);
      mc[q] = df::load_interleaved(st_m + static_cast<int64_t>(c) * 64, i);
      fc[q] = df::load_coherent(st_fail + c);
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
  const bool bad = gen_inverse8(S, sa, s, i);
  if (valid && i == 0) {
    df::store_coherent(st_fail + p, (bad || child_failed) ? int32_t(1) : int32_t(0));
    if (bad && !child_failed) atomicMin(first_fail, fail_rank[p]);
  }
  // message up_v Sinv_v down_v (all slots stage; valid non-root slots store)
  f16::wave_sync();
  sb.put(s, i, Dn);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(S, sb, s, r8::zero<T>());  // Sinv_v down_v
  f16::wave_sync();
  sa.put(s, i, X);
  f16::wave_sync();
  const r8::Row<T> M = r8::mul(U, sa, s, r8::zero<T>());  // up_v X
  if (edge) df::store_interleaved(st_m + p * 64, i, M);
  // the flag waits for every store issued so far: Sinv_v, read only by later
  // launches, goes after it
  df::publish(flags, p, valid && i == 0, 1);
  if (valid) r8::store8(st_sinv + p * 64, i, S);
}

// Distribute of one tile; workgroup w takes tile w + 1 (root level first).
// Waits for flags[parent] == 2, reads the parent's G (its message slot),
// stores its own G there and sets flags[p] = 2.
template <typename T>
__global__ __launch_bounds__(64) void nstree8_distribute(
    const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi, int b,
    const int32_t *__restrict__ node_at, const int32_t *__restrict__ parent_pos,
    const T *__restrict__ up, const T *__restrict__ down, const T *__restrict__ st_sinv,
    T *__restrict__ st_m, const int32_t *__restrict__ first_fail, T *__restrict__ G_diag,
    T *__restrict__ G_up, T *__restrict__ G_down, int32_t *__restrict__ flags,
    int32_t *__restrict__ timeout, uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int32_t t = static_cast<int32_t>(blockIdx.x) + 1;
  const int64_t p = tile_lo[t] + s;
  const bool valid = p < tile_hi[t];
  const int bb = b * b;
  int64_t v = 0, q = 0;
  if (valid) {
    v = node_at[p];
    q = parent_pos[p];
  }
  const r8::Row<T> Si = valid ? r8::load8(st_sinv + p * 64, i) : r8::zero<T>();
  const r8::Row<T> U = valid ? r8::load(up + v * bb, b, i) : r8::zero<T>();
  const r8::Row<T> Dn = valid ? r8::load(down + v * bb, b, i) : r8::zero<T>();
  // the products that do not involve the parent are formed before the wait
  sa.put(s, i, Si);
  sb.put(s, i, Dn);
  f16::wave_sync();
  const r8::Row<T> A = r8::mul(U, sa, s, r8::zero<T>());   // up_v Sinv_v
  const r8::Row<T> Bm = r8::mul(Si, sb, s, r8::zero<T>());  // Sinv_v down_v
  f16::wave_sync();
  sa.put(s, i, A);
  if (valid && i == 0) df::wait_flags(flags, q, q + 1, 2, 0, 1, timeout, deadline);
  df::acquire();
  const bool failed = *first_fail != INT_MAX || df::timed_out(timeout);
  const r8::Row<T> G = valid ? df::load_interleaved(st_m + q * 64, i) : r8::zero<T>();
  sb.put(s, i, G);
  f16::wave_sync();
  const r8::Row<T> V = r8::mul(G, sa, s, r8::zero<T>());    // G_pp A = -G_{p,v}
  const r8::Row<T> W = r8::mul(Bm, sb, s, r8::zero<T>());   // B G_pp = -G_{v,p}
  f16::wave_sync();
  sa.put(s, i, V);
  f16::wave_sync();
  const r8::Row<T> Gv = r8::mul(Bm, sa, s, Si);              // Sinv_v + B G_pp A
  r8::Row<T> nan;
#pragma unroll
  for (int k = 0; k < 8; ++k) nan.v[k] = static_cast<T>(__builtin_nan(""));
  if (valid && !failed) df::store_interleaved(st_m + p * 64, i, Gv);  // for the children
  df::publish(flags, p, valid && i == 0, 2);
  if (valid) {  // the outputs, read only after this launch
    r8::store(G_up + v * bb, b, i, failed ? nan : r8::neg(V));
    r8::store(G_down + v * bb, b, i, failed ? nan : r8::neg(W));
    r8::store(G_diag + v * bb, b, i, failed ? nan : Gv);
  }
}

// the root (a launch between the passes): G_rr = Sinv_r (NaN after a
// failure), zero edge slots; G_rr also goes to the root's message slot
// (interleaved, element (i, c) at c * 8 + i) for its children, and
// flags[0] = 2
template <typename T>
__global__ __launch_bounds__(64) void nstree8_root(int b, const int32_t *__restrict__ node_at,
                                                   const T *__restrict__ st_sinv,
                                                   T *__restrict__ st_m,
                                                   const int32_t *__restrict__ first_fail,
                                                   T *__restrict__ G_diag, T *__restrict__ G_up,
                                                   T *__restrict__ G_down,
                                                   int32_t *__restrict__ flags) {
  const int bb = b * b;
  const int64_t r = node_at[0];
  const bool failed = *first_fail != INT_MAX;
  for (int e = threadIdx.x; e < bb; e += 64) {
    const int row = e / b, c = e - row * b;
    G_diag[r * bb + e] = failed ? static_cast<T>(__builtin_nan("")) : st_sinv[row * 8 + c];
    G_up[r * bb + e] = T(0);
    G_down[r * bb + e] = T(0);
  }
  const int row = threadIdx.x >> 3, c = threadIdx.x & 7;  // the padded 8 x 8 block
  st_m[c * 8 + row] = st_sinv[row * 8 + c];
  if (threadIdx.x == 0) flags[0] = 2;
}

// info = -1 if a dataflow wait gave up
__global__ void nstree8_finish(const int32_t *__restrict__ rank_node,
                               const int32_t *__restrict__ first_fail,
                               const int32_t *__restrict__ timeout, int32_t *__restrict__ info) {
  if (info)
    *info = *timeout != 0 ? -1 : *first_fail != INT_MAX ? rank_node[*first_fail] + 1 : 0;
}

}  // namespace

size_t nstree8_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return 2 * align_up(n * 64 * plan->dtype_bytes) + 2 * align_up(n * sizeof(int32_t)) +
         2 * align_up(sizeof(int32_t));
}

template <typename T>
hipError_t nstree8_launch(const selinv_tree_plan *plan, const T *diag, const T *up, const T *down,
                          T *G_diag, T *G_up, T *G_down, int32_t *info, void *ws, hipStream_t s) {
  const int64_t n = plan->n;
  const int b = plan->b;
  Carve cv(ws);
  T *st_sinv = cv.take<T>(n * 64);
  T *st_m = cv.take<T>(n * 64);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  int32_t *flags = cv.take<int32_t>(n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  const uint64_t wt = wait_limit_ticks();
  hipError_t e = df::launch_init(n, flags, first_fail, timeout, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nstree8_collect<T>, dim3(tiles), dim3(64), 0, s, tiles, d.tile_lo,
                     d.tile_hi, b, d.node_at, d.child_beg, d.child_end, d.fail_rank, diag, up,
                     down, st_sinv, st_m, st_fail, first_fail, flags, timeout, wt);
  hipLaunchKernelGGL(nstree8_root<T>, dim3(1), dim3(64), 0, s, b, d.node_at, st_sinv, st_m,
                     first_fail, G_diag, G_up, G_down, flags);
  if (tiles > 1)
    hipLaunchKernelGGL(nstree8_distribute<T>, dim3(tiles - 1), dim3(64), 0, s, d.tile_lo,
                       d.tile_hi, b, d.node_at, d.parent_pos, up, down, st_sinv, st_m,
                       first_fail, G_diag, G_up, G_down, flags, timeout, wt);
  hipLaunchKernelGGL(nstree8_finish, dim3(1), dim3(1), 0, s, d.rank_node, first_fail, timeout,
                     info);
  return hipGetLastError();
}

template hipError_t nstree8_launch<float>(const selinv_tree_plan *, const float *, const float *,
                                          const float *, float *, float *, float *, int32_t *,
                                          void *, hipStream_t);
template hipError_t nstree8_launch<double>(const selinv_tree_plan *, const double *,
                                           const double *, const double *, double *, double *,
                                           double *, int32_t *, void *, hipStream_t);

}  // namespace selinv
