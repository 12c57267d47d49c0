// vjp_tree_b8.hip -- reverse mode of the tree selected inverse for block
// sizes b <= 8 on the breadth-first level-set schedule (the backward of
// gabp-sparse-inv 0.3.2, "Implemented and tested kernels", item
// Differentiable tree: a second collect / distribute pair on the same tree,
// with a level-set batched path mirroring the forward one).
//
// Blocks are held one row per lane, eight nodes per wavefront (rows8.h),
// padded to 8 x 8 (identity on diagonal blocks, zero elsewhere; the padding
// stays decoupled through every product below).  Per node v at position p,
// with E_v = edge[v], cotangents Gd_v (on G_vv), Ge_v (on G_{parent,v}) and
// lb (on log det):
//   collect (deepest level first):
//     S_v   = D_v - sum_children M_c,   GG_v = sym(Gd_v) + sum_children N_c
//     Sinv_v = S_v^{-1},  P_v = sym(lb Sinv_v - Sinv_v GG_v Sinv_v)
//     X_v = E_v Sinv_v,  M_v = X_v E_v^T,  W = X_v GG_v,
//     Z_v = (2 W - Ge_v) Sinv_v,  N_v = sym((W - Ge_v) X_v^T)
//   root: diag_bar[r] = P_r, G_rr = Sinv_r
//   distribute (level 1 down), u = parent(v):
//     A1 = G_uu Z_v,  T2 = diag_bar[u] X_v,  Q = A1 - T2,
//     edge_bar[v] = Q - T2,  diag_bar[v] = P_v - sym(X_v^T Q),
//     G_vv = Sinv_v + X_v^T G_uu X_v
// Workspace per position (8 x 8 each): Sinv, P, X, Z, M, N; the M slot holds
// G_vv in the distribute pass (the parent has consumed M by then).
// Each pass is one launch over the plan's tiles with per-position flags
// between producer and consumer tiles (dataflow.h): M, N and the failure
// flags (collect) and the M slot and diag_bar (distribute) are exchanged
// through device-coherent accesses, M / N / G in the interleaved layout,
// diag_bar (exactly symmetric) transposed.
#include <climits>

#include "dataflow.h"
#include "internal.h"
#include "rows8.h"

namespace selinv {

namespace {

constexpr int kSlots = kTreeTile;  // nodes per wavefront
enum { kSinv = 0, kP, kX, kZ, kM, kN, kArrays };
constexpr int kChildBatch = 2;  // children's (M, N) pairs loaded together

template <typename T>
__device__ __forceinline__ r8::Row<T> column(const r8::Stage<T> &st, int s, int i) {
  r8::Row<T> r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = st.at(s, k, i);
  return r;
}

template <typename T>
__device__ __forceinline__ r8::Row<T> axpby(T a, const r8::Row<T> &x, T b, const r8::Row<T> &y) {
  r8::Row<T> r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = a * x.v[k] + b * y.v[k];
  return r;
}

template <typename T>
__device__ __forceinline__ r8::Row<T> nan_row() {
  r8::Row<T> r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = static_cast<T>(__builtin_nan(""));
  return r;
}

// Symmetric part of a block given row-wise (row i of this lane), through the
// stage: (R + R^T) / 2.  Leaves the block in the stage.
template <typename T>
__device__ __forceinline__ r8::Row<T> sym_rows(const r8::Row<T> &r, const r8::Stage<T> &st, int s,
                                               int i) {
  f16::wave_sync();
  st.put(s, i, r);
  f16::wave_sync();
  return axpby(T(0.5), r, T(0.5), column(st, s, i));
}

// Collect of one tile; workgroup w takes tile tiles - 1 - w (deepest level
// first); flags[p] becomes 1 (2 for the root).  The messages M, N are formed
// and published first; P and Z, read only by the distribute launch, after the
// flag.  Two wavefronts per SIMD (f64: 256 VGPRs, a few spilled) beat one.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void tree8_vjp_collect(
    int32_t tiles, const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi,
    int b, const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ child_beg, const int32_t *__restrict__ child_end,
    const int32_t *__restrict__ fail_rank, const T *__restrict__ diag, const T *__restrict__ edge,
    const T *__restrict__ gd, const T *__restrict__ ge, const double *__restrict__ ld_bar,
    T *__restrict__ st, int64_t n, int32_t *__restrict__ st_fail,
    int32_t *__restrict__ first_fail, T *__restrict__ d_bar, T *__restrict__ e_bar,
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
  const T lb = ld_bar ? static_cast<T>(*ld_bar) : T(0);
  auto arr = [&](int k) { return st + k * n * 64; };
  int64_t v = 0;
  int32_t cb = 0, ce = 0;
  if (valid) {
    v = node_at[p];
    cb = child_beg[p];
    ce = child_end[p];
  }
  // slots past the level work on node 0 and store nothing
  r8::Row<T> S = r8::load_sym(diag + v * bb, b, i);
  const r8::Row<T> E = r8::load(edge + v * bb, b, i);
  const r8::Row<T> Ge = r8::load(ge + v * bb, b, i);
  r8::Row<T> GG = sym_rows(r8::load(gd + v * bb, b, i), sb, s, i);
  df::wait_flags(flags, cb, ce, 1, i, 8, timeout, deadline);
  df::acquire();
  bool child_failed = false;
  for (int32_t c0 = cb; c0 < ce; c0 += kChildBatch) {  // children in flight, summed in order
    r8::Row<T> mc[kChildBatch], nc[kChildBatch];
    int32_t fc[kChildBatch];
#pragma unroll
    for (int q = 0; q < kChildBatch; ++q) {
      const int64_t c = min(c0 + q, ce - 1);
      mc[q] = df::load_interleaved(arr(kM) + c * 64, i);
      nc[q] = df::load_interleaved(arr(kN) + c * 64, i);
      fc[q] = df::load_coherent(st_fail + c);
    }
#pragma unroll
    for (int q = 0; q < kChildBatch; ++q) {
      if (c0 + q < ce) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          S.v[k] -= mc[q].v[k];
          GG.v[k] += nc[q].v[k];
        }
        child_failed |= fc[q] != 0;
      }
    }
  }
  f16::PivotLog pl;
  const bool bad = r8::gj_inverse(S, sa, s, i, pl);  // S <- Sinv
  if (valid && i == 0) {
    df::store_coherent(st_fail + p, (bad || child_failed) ? int32_t(1) : int32_t(0));
    if (bad && !child_failed) atomicMin(first_fail, fail_rank[p]);
  }
  // messages to the parent first (they are on the chain of every level)
  f16::wave_sync();
  sa.put(s, i, S);
  f16::wave_sync();
  const r8::Row<T> X = r8::mul(E, sa, s, r8::zero<T>());  // E Sinv
  sb.put(s, i, E);
  f16::wave_sync();
  const r8::Row<T> M = r8::mul_t(X, sb, s, r8::zero<T>());  // X E^T
  f16::wave_sync();
  sb.put(s, i, GG);
  f16::wave_sync();
  const r8::Row<T> W = r8::mul(X, sb, s, r8::zero<T>());  // X GG
  const r8::Row<T> Y1 = axpby(T(1), W, T(-1), Ge);
  f16::wave_sync();
  sb.put(s, i, X);
  f16::wave_sync();
  const r8::Row<T> N = sym_rows(r8::mul_t(Y1, sb, s, r8::zero<T>()), sb, s, i);  // sym(Y1 X^T)
  // what the parent reads in this launch goes before the flag (which waits
  // for every store issued so far), what only later launches read after it
  if (valid && p != 0) {
    df::store_interleaved(arr(kM) + p * 64, i, M);
    df::store_interleaved(arr(kN) + p * 64, i, N);
  }
  df::publish(flags, p, valid && i == 0, p == 0 ? 2 : 1);
  // for the distribute (sa still holds Sinv): Z = (2 W - Ge) Sinv and
  // P = sym(lb Sinv - Sinv (GG Sinv))
  const r8::Row<T> Z = r8::mul(axpby(T(1), W, T(1), Y1), sa, s, r8::zero<T>());
  const r8::Row<T> U = r8::mul(GG, sa, s, r8::zero<T>());  // row i of GG Sinv
  f16::wave_sync();
  sb.put(s, i, U);
  f16::wave_sync();
  const r8::Row<T> P =
      sym_rows(axpby(lb, S, T(-1), r8::mul(S, sb, s, r8::zero<T>())), sb, s, i);
  if (valid) {
    r8::store8(arr(kSinv) + p * 64, i, S);
    r8::store8(arr(kP) + p * 64, i, P);
  }
  if (valid && p != 0) {
    r8::store8(arr(kX) + p * 64, i, X);
    r8::store8(arr(kZ) + p * 64, i, Z);
  }
  if (valid && p == 0) {  // the root: diag_bar = P, G_rr = Sinv (in its M slot)
    // every other collect has published before the root runs; first_fail is
    // read coherently (another XCD may have lowered it)
    const bool failed = bad || child_failed || df::load_coherent(first_fail) != INT_MAX;
    r8::store(d_bar + v * bb, b, i, failed ? nan_row<T>() : P);
    r8::store(e_bar + v * bb, b, i, r8::zero<T>());
    df::store_interleaved(arr(kM) + p * 64, i, S);
  }
}

// Distribute of one tile; workgroup w takes tile w + 1 (root level first).
// Waits for flags[parent] == 2, then reads the parent's G (M slot) and
// diag_bar; sets flags[p] = 2.
template <typename T>
__global__ __launch_bounds__(64) void tree8_vjp_distribute(
    const int32_t *__restrict__ tile_lo, const int32_t *__restrict__ tile_hi, int b,
    const int32_t *__restrict__ node_at,
    const int32_t *__restrict__ parent_pos, const int32_t *__restrict__ parent_node,
    T *__restrict__ st, int64_t n, const int32_t *__restrict__ first_fail,
    T *__restrict__ d_bar, T *__restrict__ e_bar, int32_t *__restrict__ flags,
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
  auto arr = [&](int k) { return st + k * n * 64; };
  int64_t v = 0, u = 0, q = 0, pp = 0;
  if (valid) {
    v = node_at[p];
    u = parent_node[p];
    q = parent_pos[p];
    pp = p;
  }
  const r8::Row<T> X = r8::load8(arr(kX) + pp * 64, i);
  const r8::Row<T> Z = r8::load8(arr(kZ) + pp * 64, i);
  const r8::Row<T> P = r8::load8(arr(kP) + pp * 64, i);
  const r8::Row<T> Si = r8::load8(arr(kSinv) + pp * 64, i);
  sa.put(s, i, X);  // staged before the wait (the acquire orders them)
  sb.put(s, i, Z);
  if (valid && i == 0) df::wait_flags(flags, q, q + 1, 2, 0, 1, timeout, deadline);
  df::acquire();
  const r8::Row<T> G = df::load_interleaved(arr(kM) + q * 64, i);  // G of the parent
  const r8::Row<T> Db = df::load_transposed(d_bar + u * bb, b, i);
  const r8::Row<T> T2 = r8::mul(Db, sa, s, r8::zero<T>());  // Dbar_u X
  const r8::Row<T> V = r8::mul(G, sa, s, r8::zero<T>());    // G_uu X
  const r8::Row<T> Q = axpby(T(1), r8::mul(G, sb, s, r8::zero<T>()), T(-1), T2);
  const r8::Row<T> Eb = axpby(T(1), Q, T(-1), T2);
  f16::wave_sync();
  sb.put(s, i, Q);
  f16::wave_sync();
  const r8::Row<T> R = r8::mul_tn(sa, sb, s, i, r8::zero<T>());  // row i of X^T Q
  f16::wave_sync();
  sb.put(s, i, V);
  f16::wave_sync();
  const r8::Row<T> Gv = r8::mul_tn(sa, sb, s, i, Si);  // Sinv + X^T V
  const r8::Row<T> Dn = axpby(T(1), P, T(-1), sym_rows(R, sb, s, i));
  const bool failed = *first_fail != INT_MAX || df::timed_out(timeout);
  if (valid) {  // read by the children in this launch
    if (failed) {
      df::store_transposed(d_bar + v * bb, b, i, nan_row<T>());
    } else {
      df::store_transposed(d_bar + v * bb, b, i, Dn);
      df::store_interleaved(arr(kM) + p * 64, i, Gv);
    }
  }
  df::publish(flags, p, valid && i == 0, 2);
  if (valid) r8::store(e_bar + v * bb, b, i, failed ? nan_row<T>() : Eb);
}

// info = -1 if a dataflow wait gave up
__global__ void tree8_vjp_finish(const int32_t *__restrict__ rank_node,
                                 const int32_t *__restrict__ first_fail,
                                 const int32_t *__restrict__ timeout,
                                 int32_t *__restrict__ info) {
  if (info)
    *info = *timeout != 0 ? -1 : *first_fail != INT_MAX ? rank_node[*first_fail] + 1 : 0;
}

}  // namespace

size_t tree8_vjp_workspace_bytes(const selinv_tree_plan *plan) {
  const size_t n = plan->n;
  return align_up(kArrays * n * 64 * plan->dtype_bytes) + 2 * align_up(n * sizeof(int32_t)) +
         2 * align_up(sizeof(int32_t));
}

template <typename T>
hipError_t tree8_vjp_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                            const T *gd, const T *ge, const double *ld_bar, T *d_bar, T *e_bar,
                            int32_t *info, void *ws, hipStream_t s) {
  const int64_t n = plan->n;
  const int b = plan->b;
  Carve cv(ws);
  T *st = cv.take<T>(kArrays * n * 64);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  int32_t *flags = cv.take<int32_t>(n);
  int32_t *timeout = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int32_t tiles = static_cast<int32_t>(plan->tiles);
  const uint64_t wt = wait_limit_ticks();
  hipError_t e = df::launch_init(n, flags, first_fail, timeout, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree8_vjp_collect<T>, dim3(tiles), dim3(64), 0, s, tiles, d.tile_lo,
                     d.tile_hi, b, d.node_at, d.child_beg, d.child_end, d.fail_rank, diag, edge,
                     gd, ge, ld_bar, st, n, st_fail, first_fail, d_bar, e_bar, flags, timeout, wt);
  if (tiles > 1)
    hipLaunchKernelGGL(tree8_vjp_distribute<T>, dim3(tiles - 1), dim3(64), 0, s, d.tile_lo,
                       d.tile_hi, b, d.node_at, d.parent_pos, d.parent_node, st, n, first_fail,
                       d_bar, e_bar, flags, timeout, wt);
  hipLaunchKernelGGL(tree8_vjp_finish, dim3(1), dim3(1), 0, s, d.rank_node, first_fail, timeout,
                     info);
  return hipGetLastError();
}

template hipError_t tree8_vjp_launch<float>(const selinv_tree_plan *, const float *,
                                            const float *, const float *, const float *,
                                            const double *, float *, float *, int32_t *, void *,
                                            hipStream_t);
template hipError_t tree8_vjp_launch<double>(const selinv_tree_plan *, const double *,
                                             const double *, const double *, const double *,
                                             const double *, double *, double *, int32_t *,
                                             void *, hipStream_t);

}  // namespace selinv
