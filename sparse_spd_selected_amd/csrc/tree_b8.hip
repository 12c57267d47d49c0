// tree_b8.hip -- tree selected inverse for block sizes b <= 8 on the
// breadth-first depth level-set schedule of tree_plan.cpp (gabp-sparse-inv
// 0.3.2 page, item Tree of "Implemented and tested kernels": collect
// leaves -> root, then distribute root -> leaves; the batched form loops over
// levels, each level a few batched block operations).
//
// Blocks are held one row per lane (rows8.h), eight tree nodes (one tile of
// the plan) per wavefront.  Per node v (position p), with E_v = edge[v] =
// A_{parent,v}:
//   collect:    S_v = D_v - sum_children M_c (children contiguous, in order),
//               Sinv_v = S_v^{-1},  X_v = E_v Sinv_v,  M_v = X_v E_v^T
//   root:       G_rr = Sinv_r  (written by the collect)
//   distribute: X_v = E_v Sinv_v,  V = G_pp X_v,  G_edge[v] = -V,
//               G_diag[v] = Sinv_v + X_v^T V
// Each pass is ONE launch over all tiles, ordered by level, with per-position
// flags between producer and consumer tiles (dataflow.h) in place of a
// launch per level: a tile starts its loads as soon as it is resident and
// waits only for its own children (collect) or parents (distribute), so
// consecutive levels overlap.  Sinv_v lives in the workspace as a padded
// 8 x 8 block indexed by position, M_v as an interleaved 8 x 8 block; X_v is
// recomputed from the re-read edge block.
#include <algorithm>
#include <climits>

#include "dataflow.h"
#include "internal.h"
#include "rows8.h"

namespace selinv {

namespace {

constexpr int kSlots = kTreeTile;  // nodes per wavefront

using df::load_coherent;
using df::store_coherent;

// Collect of one tile; grid = number of tiles, workgroup w takes tile
// tiles - 1 - w (deepest level first).  The diagonal and edge blocks are
// loaded before the wait for the children.  flags[p] becomes 1 (2 for the
// root, whose G block the collect writes).
// kFactor: the collect pass of the shared factor: the packed lower triangle
// of Sinv_v (wg-style layout, packed_entries(b) per position) goes to
// st_sinv, which may be null (log det only); G_diag, G_edge are unused.
template <typename T, bool kFactor, bool kFull>
__global__ __launch_bounds__(64) void tree8_collect(
    int32_t tiles, int b_arg, const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi,
    const int32_t *__restrict__ node_at, const int32_t *__restrict__ child_beg,
    const int32_t *__restrict__ child_end, const int32_t *__restrict__ fail_rank,
    const T *__restrict__ diag, const T *__restrict__ edge, T *__restrict__ st_sinv,
    T *__restrict__ st_m, double *__restrict__ st_ld, int32_t *__restrict__ st_fail,
    int32_t *__restrict__ first_fail, T *__restrict__ G_diag, T *__restrict__ G_edge,
    int32_t *__restrict__ flags, int32_t *__restrict__ timeout, uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int b = kFull ? 8 : b_arg;  // compiled for b = 8 on its own
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
  r8::Row<T> S = r8::load_sym(diag + v * bb, b, i);  // slots past the tile re-read node 0
  const r8::Row<T> E = (valid && p != 0) ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  df::wait_flags(flags, cb, ce, 1, i, 8, timeout, deadline);
  df::acquire();
  bool child_failed = false;
  for (int32_t c0 = cb; c0 < ce; c0 += 4) {
    r8::Row<T> mc[4];
    int32_t fc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t c = min(c0 + q, ce - 1);
      mc[q] = df::load_interleaved(st_m + static_cast<int64_t>(c) * 64, i);
      fc[q] = load_coherent(st_fail + c);
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
  // What the parent reads in this launch is stored before the flag (which
  // waits for every store issued so far); the rest only after it.
  const bool failed = bad || child_failed;
  if (valid && i == 0) store_coherent(st_fail + p, failed ? int32_t(1) : int32_t(0));
  f16::wave_sync();
  sa.put(s, i, S);
  sb.put(s, i, E);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(E, sa, s, r8::zero<T>());   // E_v Sinv_v
  const r8::Row<T> M = r8::mul_t(X, sb, s, r8::zero<T>());  // X_v E_v^T
  if (valid && p != 0) df::store_interleaved(st_m + p * 64, i, M);
  df::publish(flags, p, valid && i == 0, (!kFactor && p == 0) ? 2 : 1);
  if (valid && i == 0) {
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
      df::store_transposed(G_diag + v * bb, b, i, S);
      r8::store(G_edge + v * bb, b, i, r8::zero<T>());
    }
  }
}

// Distribute of one tile; grid = tiles - 1, workgroup w takes tile w + 1
// (root level first; the root's tile is finished by the collect).  Waits for
// flags[parent] == 2, reads the parent's G_diag block, sets flags[p] = 2.
template <typename T, bool kFull>
__global__ __launch_bounds__(64) void tree8_distribute(
    int b_arg, const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi,
    const int32_t *__restrict__ node_at, const int32_t *__restrict__ parent_pos,
    const int32_t *__restrict__ parent_node, const T *__restrict__ edge,
    const T *__restrict__ st_sinv, const int32_t *__restrict__ first_fail,
    T *__restrict__ G_diag, T *__restrict__ G_edge, int32_t *__restrict__ flags,
    int32_t *__restrict__ timeout, uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int b = kFull ? 8 : b_arg;  // compiled for b = 8 on its own
  const int32_t t = static_cast<int32_t>(blockIdx.x) + 1;
  const int64_t p = tile_lo[t] + s;
  const bool valid = p < tile_hi[t];
  const int bb = b * b;
  int64_t v = 0, u = 0;
  int32_t pp = 0;
  if (valid) {
    v = node_at[p];
    u = parent_node[p];
    pp = parent_pos[p];
  }
  const r8::Row<T> Si = valid ? r8::load8(st_sinv + p * 64, i) : r8::zero<T>();
  const r8::Row<T> E = valid ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  // X_v does not depend on the parent: formed before the wait
  sa.put(s, i, Si);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(E, sa, s, r8::zero<T>());  // E_v Sinv_v
  sb.put(s, i, X);
  if (valid && i == 0) df::wait_flags(flags, pp, pp + 1, 2, 0, 1, timeout, deadline);
  df::acquire();
  const bool failed = *first_fail != INT_MAX || df::timed_out(timeout);
  const r8::Row<T> G = valid ? df::load_transposed(G_diag + u * bb, b, i) : r8::zero<T>();
  const r8::Row<T> V = r8::mul(G, sb, s, r8::zero<T>());  // G_pp X_v
  f16::wave_sync();
  sa.put(s, i, V);
  f16::wave_sync();
  const r8::Row<T> Gv = r8::mul_tn(sb, sa, s, i, Si);     // Sinv_v + X_v^T V
  r8::Row<T> nan;
#pragma unroll
  for (int k = 0; k < 8; ++k) nan.v[k] = static_cast<T>(__builtin_nan(""));
  // G_vv is read by the children in this launch: stored before the flag;
  // G_edge only after it
  if (valid) df::store_transposed(G_diag + v * bb, b, i, failed ? nan : Gv);
  df::publish(flags, p, valid && i == 0, 2);
  if (valid) r8::store(G_edge + v * bb, b, i, failed ? nan : r8::neg(V));
}

// ------------------------------------------------------------------ solve
// x = A^-1 y from the shared factor (packed lower triangle of Sinv_v per
// position, r (r + 1) / 2 + c, padded to a multiple of 4 entries):
//   forward, children first:  u_v = y_v - sum_children E_c w_c,  w_v = Sinv_v u_v
//   backward, parents first:  x_v = w_v - Sinv_v E_v^T x_parent  (x_root = w_root)
// Right-hand sides go in chunks of kw = min(k, 8) columns; lane (s, i) holds
// row i of its node's b x kw chunk, zero-padded to 8 x 8, so every step is an
// 8 x 8 product.  Both passes are single launches over (tile, chunk) pairs on
// the dataflow schedule; flags and messages are chunk-major, the message
// E_v w_v at [chunk][position][c * 8 + i].  x is written by the forward pass
// (w_v) and overwritten by the backward pass (coherently: children read it).
// A call whose dataflow wait gives up leaves NaN in x (at least in the
// blocks of the workgroups that saw it, all of them if it was the forward).
constexpr int kSolveCols = 8;

template <typename T>
__device__ __forceinline__ r8::Row<T> packed_row(const T *P, int b, int i) {
  r8::Row<T> r;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    r.v[c] = (i < b && c < b) ? P[c <= i ? i * (i + 1) / 2 + c : c * (c + 1) / 2 + i] : T(0);
  return r;
}

// row i of the b x kc chunk of node v's k columns, starting at column c0
template <typename T, bool kCoherent>
__device__ __forceinline__ r8::Row<T> load_cols(const T *X, int64_t v, int b, int64_t k,
                                                int64_t c0, int kc, int i) {
  r8::Row<T> r;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const T *a = X + (v * b + i) * k + c0 + c;
    r.v[c] = (i < b && c < kc) ? (kCoherent ? df::load_coherent(a) : *a) : T(0);
  }
  return r;
}

template <typename T, bool kCoherent>
__device__ __forceinline__ void store_cols(T *X, int64_t v, int b, int64_t k, int64_t c0, int kc,
                                           int i, const r8::Row<T> &r) {
  if (i >= b) return;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    T *a = X + (v * b + i) * k + c0 + c;
    if (c < kc) {
      if (kCoherent)
        df::store_coherent(a, r.v[c]);
      else
        *a = r.v[c];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(64) void tree8_solve_fwd(
    int32_t tiles, int nch, int64_t n, int64_t k, int kw, const int32_t *__restrict__ tile_lo,
    const int32_t *__restrict__ tile_hi, int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ child_beg, const int32_t *__restrict__ child_end,
    const T *__restrict__ edge, const T *__restrict__ factor, const T *__restrict__ y,
    T *__restrict__ x, T *__restrict__ msg, int32_t *__restrict__ flags,
    int32_t *__restrict__ timeout, uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int chunk = static_cast<int>(blockIdx.x % nch);
  const int32_t t = tiles - 1 - static_cast<int32_t>(blockIdx.x / nch);
  const int64_t c0 = int64_t(chunk) * kSolveCols;
  const int kc = static_cast<int>(min<int64_t>(kw, k - c0));
  const int64_t p = tile_lo[t] + s;
  const bool valid = p < tile_hi[t];
  const int bb = b * b, pk = (b * (b + 1) / 2 + 3) / 4 * 4;
  int64_t v = 0;
  int32_t cb = 0, ce = 0;
  if (valid) {
    v = node_at[p];
    cb = child_beg[p];
    ce = child_end[p];
  }
  const r8::Row<T> Si = valid ? packed_row(factor + p * pk, b, i) : r8::zero<T>();
  r8::Row<T> U = valid ? load_cols<T, false>(y, v, b, k, c0, kc, i) : r8::zero<T>();
  const r8::Row<T> E = (valid && p != 0) ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  int32_t *fl = flags + chunk * n;
  T *mg = msg + chunk * n * (8 * kw);
  df::wait_flags(fl, cb, ce, 1, i, 8, timeout, deadline);
  df::acquire();
  for (int32_t c = cb; c < ce; ++c) {  // children in order
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (cc < kc) U.v[cc] -= df::load_coherent(mg + int64_t(c) * (8 * kw) + cc * 8 + i);
  }
  sa.put(s, i, U);
  f16::wave_sync();
  const r8::Row<T> W = r8::mul(Si, sa, s, r8::zero<T>());  // Sinv_v u_v
  if (valid) store_cols<T, false>(x, v, b, k, c0, kc, i, W);
  sb.put(s, i, W);
  f16::wave_sync();
  const r8::Row<T> M = r8::mul(E, sb, s, r8::zero<T>());  // E_v w_v
  if (valid && p != 0) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (cc < kc) df::store_coherent(mg + p * (8 * kw) + cc * 8 + i, M.v[cc]);
  }
  df::publish(fl, p, valid && i == 0, 1);
}

// kSample: x = L^-T D^-1/2 z instead, w_v = U_v z_v (U_v U_v^T = Sinv_v, U_v
// upper triangular) formed from z before the wait; no forward pass.  Held to
// two wavefronts per SIMD: the f64 sampler would otherwise take one (its
// unrolled reversed Cholesky needs ~300 registers; two with some spilled are
// faster).
template <typename T, bool kSample>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void tree8_solve_bwd(
    int nch, int64_t n, int64_t k, int kw, const int32_t *__restrict__ tile_lo,
    const int32_t *__restrict__ tile_hi, int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ parent_pos, const int32_t *__restrict__ parent_node,
    const T *__restrict__ edge, const T *__restrict__ factor, const T *__restrict__ z,
    T *__restrict__ x, int32_t *__restrict__ flags, int32_t *__restrict__ timeout,
    uint64_t wait_ticks) {
  __shared__ __align__(32) T lds[2][kSlots * 64];
  const uint64_t deadline = df::deadline_after(wait_ticks);
  const int lane = threadIdx.x;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[0]}, sb{lds[1]};
  const int chunk = static_cast<int>(blockIdx.x % nch);
  const int32_t t = static_cast<int32_t>(blockIdx.x / nch);
  const int64_t c0 = int64_t(chunk) * kSolveCols;
  const int kc = static_cast<int>(min<int64_t>(kw, k - c0));
  const int64_t p = tile_lo[t] + s;
  const bool valid = p < tile_hi[t];
  const bool has_parent = valid && p != 0;
  const int bb = b * b, pk = (b * (b + 1) / 2 + 3) / 4 * 4;
  int64_t v = 0, u = 0, q = 0;
  if (valid) v = node_at[p];
  if (has_parent) {
    u = parent_node[p];
    q = parent_pos[p];
  }
  const r8::Row<T> Si = valid ? packed_row(factor + p * pk, b, i) : r8::zero<T>();
  r8::Row<T> W;
  if constexpr (kSample) {  // w_v = U_v z_v
    const r8::Row<T> Zr = valid ? load_cols<T, false>(z, v, b, k, c0, kc, i) : r8::zero<T>();
    const r8::Row<T> U = r8::rev_cholesky(Si, sa, s, i, b);
    sb.put(s, i, Zr);
    f16::wave_sync();
    W = r8::mul(U, sb, s, r8::zero<T>());
    f16::wave_sync();
  } else {
    W = valid ? load_cols<T, false>(x, v, b, k, c0, kc, i) : r8::zero<T>();
  }
  const r8::Row<T> E = has_parent ? r8::load(edge + v * bb, b, i) : r8::zero<T>();
  sa.put(s, i, E);  // staged before the wait (the acquire orders it)
  int32_t *fl = flags + chunk * n;
  if (has_parent && i == 0) df::wait_flags(fl, q, q + 1, 2, 0, 1, timeout, deadline);
  df::acquire();
  const r8::Row<T> Xp = has_parent ? load_cols<T, true>(x, u, b, k, c0, kc, i) : r8::zero<T>();
  sb.put(s, i, Xp);
  f16::wave_sync();
  const r8::Row<T> Tt = r8::mul_tn(sa, sb, s, i, r8::zero<T>());  // E_v^T x_parent
  f16::wave_sync();
  sa.put(s, i, Tt);
  f16::wave_sync();
  const r8::Row<T> V = r8::mul(Si, sa, s, r8::zero<T>());  // Sinv_v E_v^T x_parent
  const bool gave_up = df::timed_out(timeout);  // then x is NaN, not silently wrong
  r8::Row<T> X;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    X.v[c] = gave_up ? static_cast<T>(__builtin_nan("")) : W.v[c] - V.v[c];
  if (valid) store_cols<T, true>(x, v, b, k, c0, kc, i, X);
  df::publish(fl, p, valid && i == 0, 2);
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

// info = -1 (and a NaN log det) if a dataflow wait gave up (timeout != 0).
__global__ __launch_bounds__(64) void tree8_finish(const double *__restrict__ partial,
                                                   const int32_t *__restrict__ rank_node,
                                                   const int32_t *__restrict__ first_fail,
                                                   const int32_t *__restrict__ timeout,
                                                   double *__restrict__ logdet,
                                                   int32_t *__restrict__ info) {
  if (threadIdx.x != 0) return;
  double acc = 0.0;
  for (int w = 0; w < kFinishGroups; ++w) acc += partial[w];
  const bool failed = *first_fail != INT_MAX;
  const bool gave_up = timeout && *timeout != 0;
  *logdet = (failed || gave_up) ? __builtin_nan("") : acc;
  if (info) *info = gave_up ? -1 : failed ? rank_node[*first_fail] + 1 : 0;
}

}  // namespace

size_t tree8_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return 2 * align_up(n * 64 * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         2 * align_up(n * sizeof(int32_t)) + 2 * align_up(sizeof(int32_t)) +
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
  int32_t *flags = cv.take<int32_t>(n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  const uint64_t wt = wait_limit_ticks();
  hipError_t e = df::launch_init(n, flags, first_fail, timeout, s);
  if (e != hipSuccess) return e;
  auto collect = b == 8 ? tree8_collect<T, false, true> : tree8_collect<T, false, false>;
  auto distribute = b == 8 ? tree8_distribute<T, true> : tree8_distribute<T, false>;
  hipLaunchKernelGGL(collect, dim3(tiles), dim3(64), 0, s, tiles, b, d.tile_lo, d.tile_hi,
                     d.node_at, d.child_beg, d.child_end, d.fail_rank, diag, edge, st_sinv, st_m,
                     st_ld, st_fail, first_fail, G_diag, G_edge, flags, timeout, wt);
  if (tiles > 1)
    hipLaunchKernelGGL(distribute, dim3(tiles - 1), dim3(64), 0, s, b, d.tile_lo, d.tile_hi,
                       d.node_at, d.parent_pos, d.parent_node, edge, st_sinv, first_fail, G_diag,
                       G_edge, flags, timeout, wt);
  const int64_t chunk = (n + kFinishGroups - 1) / kFinishGroups;
  hipLaunchKernelGGL(tree8_ld_partial, dim3(kFinishGroups), dim3(1024), 0, s, n, chunk, st_ld,
                     partial);
  hipLaunchKernelGGL(tree8_finish, dim3(1), dim3(64), 0, s, partial, d.rank_node, first_fail,
                     timeout, logdet, info);
  return hipGetLastError();
}

size_t tree8_factor_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return align_up(n * 64 * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         2 * align_up(n * sizeof(int32_t)) + 2 * align_up(sizeof(int32_t)) +
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
  int32_t *flags = cv.take<int32_t>(n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  hipError_t e = df::launch_init(n, flags, first_fail, timeout, s);
  if (e != hipSuccess) return e;
  auto collect = b == 8 ? tree8_collect<T, true, true> : tree8_collect<T, true, false>;
  hipLaunchKernelGGL(collect, dim3(tiles), dim3(64), 0, s, tiles, b, d.tile_lo,
                     d.tile_hi, d.node_at, d.child_beg, d.child_end, d.fail_rank, diag, edge,
                     factor, st_m, st_ld, st_fail, first_fail, nullptr, nullptr, flags, timeout,
                     wait_limit_ticks());
  const int64_t chunk = (n + kFinishGroups - 1) / kFinishGroups;
  hipLaunchKernelGGL(tree8_ld_partial, dim3(kFinishGroups), dim3(1024), 0, s, n, chunk, st_ld,
                     partial);
  hipLaunchKernelGGL(tree8_finish, dim3(1), dim3(64), 0, s, partial, d.rank_node, first_fail,
                     timeout, logdet, info);
  return hipGetLastError();
}

size_t tree8_solve_workspace_bytes(const selinv_tree_plan *plan, int64_t k) {
  if (k <= 0) return 0;
  const size_t n = plan->n, nch = (k + kSolveCols - 1) / kSolveCols;
  const size_t kw = std::min<int64_t>(k, kSolveCols);
  return align_up(nch * n * 8 * kw * plan->dtype_bytes) + align_up(nch * n * sizeof(int32_t)) +
         align_up(sizeof(int32_t));
}

template <typename T>
hipError_t tree8_solve_launch(const selinv_tree_plan *plan, int64_t k, const T *edge,
                              const T *factor, const T *y, T *x, void *ws, hipStream_t s) {
  if (k <= 0) return hipSuccess;
  const int64_t n = plan->n;
  const int b = plan->b;
  const int nch = static_cast<int>((k + kSolveCols - 1) / kSolveCols);
  const int kw = static_cast<int>(std::min<int64_t>(k, kSolveCols));
  Carve cv(ws);
  T *msg = cv.take<T>(int64_t(nch) * n * 8 * kw);
  int32_t *flags = cv.take<int32_t>(int64_t(nch) * n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  const uint64_t wt = wait_limit_ticks();
  hipError_t e = df::launch_init(int64_t(nch) * n, flags, nullptr, timeout, s);
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>(int64_t(tiles) * nch);
  hipLaunchKernelGGL(tree8_solve_fwd<T>, dim3(grid), dim3(64), 0, s, tiles, nch, n, k, kw,
                     d.tile_lo, d.tile_hi, b, d.node_at, d.child_beg, d.child_end, edge, factor,
                     y, x, msg, flags, timeout, wt);
  hipLaunchKernelGGL((tree8_solve_bwd<T, false>), dim3(grid), dim3(64), 0, s, nch, n, k, kw,
                     d.tile_lo, d.tile_hi, b, d.node_at, d.parent_pos, d.parent_node, edge, factor,
                     static_cast<const T *>(nullptr), x, flags, timeout, wt);
  return hipGetLastError();
}

// Sampling on the same single-launch parents-first schedule (no forward
// pass); the workspace is the solve's.
template <typename T>
hipError_t tree8_sample_launch(const selinv_tree_plan *plan, int64_t k, const T *edge,
                               const T *factor, const T *z, T *x, void *ws, hipStream_t s) {
  if (k <= 0) return hipSuccess;
  if (!ws) return hipErrorInvalidValue;  // the flags live in the workspace
  const int64_t n = plan->n;
  const int b = plan->b;
  const int nch = static_cast<int>((k + kSolveCols - 1) / kSolveCols);
  const int kw = static_cast<int>(std::min<int64_t>(k, kSolveCols));
  Carve cv(ws);
  (void)cv.take<T>(int64_t(nch) * n * 8 * kw);  // the solve's messages: unused
  int32_t *flags = cv.take<int32_t>(int64_t(nch) * n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  hipError_t e = df::launch_init(int64_t(nch) * n, flags, nullptr, timeout, s);
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>(int64_t(tiles) * nch);
  hipLaunchKernelGGL((tree8_solve_bwd<T, true>), dim3(grid), dim3(64), 0, s, nch, n, k, kw,
                     d.tile_lo, d.tile_hi, b, d.node_at, d.parent_pos, d.parent_node, edge, factor,
                     z, x, flags, timeout, wait_limit_ticks());
  return hipGetLastError();
}

template hipError_t tree8_sample_launch<float>(const selinv_tree_plan *, int64_t, const float *,
                                               const float *, const float *, float *, void *,
                                               hipStream_t);
template hipError_t tree8_sample_launch<double>(const selinv_tree_plan *, int64_t,
                                                const double *, const double *, const double *,
                                                double *, void *, hipStream_t);

template hipError_t tree8_solve_launch<float>(const selinv_tree_plan *, int64_t, const float *,
                                              const float *, const float *, float *, void *,
                                              hipStream_t);
template hipError_t tree8_solve_launch<double>(const selinv_tree_plan *, int64_t,
                                               const double *, const double *, const double *,
                                               double *, void *, hipStream_t);

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
