// junction.hip -- selected inverse of general sparse SPD matrices on their
// filled (chordal) pattern, batched over matrices that share the pattern
// (gabp-sparse-inv page, junction-tree section: sparse block Cholesky, then
// the multi-neighbour Takahashi recurrence, level by level over the
// elimination tree).
//
// Cholesky form.  With A = L~ L~^T, L~_vv = R_v (lower) and the off-diagonal
// factor blocks W_{w,v} = C_{w,v} R_v^-T for the later neighbours w of v:
//   factor (levels upward, children first), for every target t of node v
//   (t = v or t in N(v)):
//       C_{t,v} = A_{t,v} - sum_u W_{t,u} W_{v,u}^T
//   over the earlier nodes u whose clique holds both v and t; then
//       R_v = chol(C_vv),  W_{t,v} = C_{t,v} R_v^-T,  log det += 2 sum ln R_kk
//   Takahashi (levels downward, root first), N = N(v):
//       G_{w,v} = -(sum_{x in N} G_{w,x} W_{x,v}) R_v^-1          (w in N)
//       G_vv    = R_v^-T (R_v^-1 - sum_{w in N} W_{w,v}^T G_{w,v})
// (the LDL^T recurrences of the page with L_{w,v} = W_{w,v} R_v^-1 and
// D_v = R_v R_v^T).  Every block read lies in S because N(v) is a clique.
//
// Work decomposition.  One workgroup per (target or slot, matrix), four
// launches per level: the Schur sums of all targets of the level, their
// scaling by R_v^-T (each workgroup refactors its node's b x b pivot; the
// diagonal target also stores R_v^-1 and the log det term), the rows
// G_{w,v} of the level, and its diagonal blocks.  Every workgroup owns what
// it writes, sums run in a fixed order (pairs in elimination order, then a
// fixed reduction tree), so results are deterministic and need no atomics
// except the first-failure index.  Sums of b x b products are staged
// through LDS in rounds of several pairs; each group of b*b threads takes
// every G-th pair of a round (G = 256 / b^2 groups for b <= 16).
#include <hip/hip_runtime.h>

#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {
namespace {

constexpr int kJT = 256;  // threads per workgroup

// Pairs per staging round: buffers of 2048 elements (1024 for b > 16), so
// that with the four extra blocks a workgroup stays under 64 KB of LDS.
__host__ __device__ inline int stage_pairs(int bb) {
  const int c = (bb <= 256 ? 2048 : 1024) / bb;
  return c < 1 ? 1 : (c > 64 ? 64 : c);
}

// LDS: two staging buffers, a reduction buffer of kJT, and four blocks
template <typename T>
size_t lds_bytes(int b) {
  const int bb = b * b;
  return sizeof(T) * (2 * size_t(stage_pairs(bb)) * bb + kJT + 4 * size_t(bb));
}

enum Mode { kABt = 0, kAB = 1, kAtB = 2 };

template <int MODE, typename T>
__device__ inline T dot_block(const T *A, const T *Bm, int b, int r, int c) {
  T s = T(0);
  for (int k = 0; k < b; ++k) {
    const T a = MODE == kAtB ? A[k * b + r] : A[r * b + k];
    const T x = MODE == kABt ? Bm[c * b + k] : Bm[k * b + c];
    s += a * x;
  }
  return s;
}

// Sum over q < count of op(A_q) op(B_q) into `out` (LDS, bb entries).
// stage(q, el, a_val, b_val) returns entry el of A_q and of B_q (already in
// the orientation MODE expects).  Deterministic: fixed pair-to-group map and
// fixed reduction order.
template <int MODE, typename T, typename Stage>
__device__ inline void staged_sum(T *out, int count, int b, T *sa, T *sb, T *red, Stage stage) {
  const int bb = b * b, t = threadIdx.x;
  const int CH = stage_pairs(bb);
  const bool small = bb <= kJT;
  const int G = small ? kJT / bb : 1;
  const int g = small ? t / bb : 0;
  T acc[4] = {T(0), T(0), T(0), T(0)};
  for (int q0 = 0; q0 < count; q0 += CH) {
    const int cnt = count - q0 < CH ? count - q0 : CH;
    for (int idx = t; idx < cnt * bb; idx += kJT) {
      const int q = idx / bb, el = idx - q * bb;
      T av, bv;
      stage(q0 + q, el, av, bv);
      sa[idx] = av;
      sb[idx] = bv;
    }
    __syncthreads();
    if (small) {
      if (g < G) {
        const int e = t - g * bb, r = e / b, c = e - r * b;
        for (int q = g; q < cnt; q += G) acc[0] += dot_block<MODE>(sa + q * bb, sb + q * bb, b, r, c);
      }
    } else {
      for (int i = 0; i < 4; ++i) {
        const int e = t + i * kJT;
        if (e >= bb) break;
        const int r = e / b, c = e - r * b;
        for (int q = 0; q < cnt; ++q) acc[i] += dot_block<MODE>(sa + q * bb, sb + q * bb, b, r, c);
      }
    }
    __syncthreads();
  }
  if (small) {
    red[t] = acc[0];
    __syncthreads();
    if (t < bb) {
      T s = T(0);
      for (int gg = 0; gg < G; ++gg) s += red[gg * bb + t];
      out[t] = s;
    }
  } else {
    for (int i = 0; i < 4; ++i) {
      const int e = t + i * kJT;
      if (e < bb) out[e] = acc[i];
    }
  }
  __syncthreads();
}

// S (LDS; lower triangle read) = R R^T: R overwrites the lower triangle of S
// and Rinv (LDS) receives R^-1 (lower, zero above).  Returns 1, uniformly,
// if a pivot is not > 0 (NaN included); *logdet = ln det S.
template <typename T>
__device__ inline int chol_inverse(T *S, T *Rinv, int b, double *logdet) {
  const int t = threadIdx.x;
  double ld = 0.0;
  for (int j = 0; j < b; ++j) {
    const T d = S[j * b + j];
    if (!(d > T(0))) return 1;
    ld += log(static_cast<double>(d));
    const T r = sqrt(d);
    for (int i = j + 1 + t; i < b; i += kJT) S[i * b + j] /= r;
    __syncthreads();
    const int rem = b - j - 1;
    for (int e = t; e < rem * rem; e += kJT) {
      const int i = j + 1 + e / rem, l = j + 1 + e % rem;
      if (l <= i) S[i * b + l] -= S[i * b + j] * S[l * b + j];
    }
    __syncthreads();
  }
  for (int j = t; j < b; j += kJT) S[j * b + j] = sqrt(S[j * b + j]);
  __syncthreads();
  // R X = I, one column of X per thread
  for (int c = t; c < b; c += kJT) {
    for (int i = 0; i < b; ++i) {
      T s = i == c ? T(1) : T(0);
      for (int k = c; k < i; ++k) s -= S[i * b + k] * Rinv[k * b + c];
      Rinv[i * b + c] = i < c ? T(0) : s / S[i * b + i];
    }
  }
  __syncthreads();
  *logdet = ld;
  return 0;
}

template <typename T>
__global__ void __launch_bounds__(kJT) jt_init(int32_t *info_ws, int64_t B) {
  const int64_t m = blockIdx.x * int64_t(kJT) + threadIdx.x;
  if (m < B) info_ws[m] = INT_MAX;
}

// Schur sums of the targets [tbase, tbase + gridDim.x) for matrix blockIdx.y
template <typename T>
__global__ void __launch_bounds__(kJT) jt_fwd_update(JunctionPlanDev P, int64_t tbase, int64_t n,
                                                     int64_t m_edges, int64_t nnz, int b,
                                                     const T *__restrict__ diag,
                                                     const T *__restrict__ edge_val, T *W, T *Cd) {
  extern __shared__ char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, CH = stage_pairs(bb);
  T *sa = smem, *sb = sa + CH * bb, *red = sb + CH * bb, *acc = red + kJT;
  const int64_t tg = tbase + blockIdx.x, mat = blockIdx.y;
  const int v = P.tgt_node[tg];
  const int64_t a = tg - (int64_t(P.colptr[v]) + v);  // 0 = the diagonal
  const int32_t f0 = P.fptr[tg], f1 = P.fptr[tg + 1];
  const T *Wm = W + mat * nnz * bb;
  const int32_t *fp = P.fpair;
  staged_sum<kABt>(acc, f1 - f0, b, sa, sb, red, [&](int q, int el, T &av, T &bv) {
    av = Wm[int64_t(fp[2 * (f0 + q)]) * bb + el];
    bv = Wm[int64_t(fp[2 * (f0 + q) + 1]) * bb + el];
  });
  const int32_t enc = P.ain[tg];
  if (a == 0) {
    const T *D = diag + (mat * n + enc) * bb;
    T *dst = Cd + (mat * n + v) * bb;
    for (int e = threadIdx.x; e < bb; e += kJT) {
      const int r = e / b, c = e - r * b;
      dst[e] = (r >= c ? D[r * b + c] : D[c * b + r]) - acc[e];
    }
  } else {
    T *dst = W + (mat * nnz + P.colptr[v] + (a - 1)) * bb;
    const T *E = enc < 0 ? nullptr : edge_val + (mat * m_edges + (enc >> 1)) * bb;
    const bool tr = enc >= 0 && (enc & 1);
    for (int e = threadIdx.x; e < bb; e += kJT) {
      const int r = e / b, c = e - r * b;
      const T base = E ? (tr ? E[c * b + r] : E[e]) : T(0);
      dst[e] = base - acc[e];
    }
  }
}

// R_v from C_vv; diagonal targets store R_v^-1, the log det term and a
// failure; slot targets scale W_{t,v} = C_{t,v} R_v^-T in place
template <typename T>
__global__ void __launch_bounds__(kJT) jt_fwd_scale(JunctionPlanDev P, int64_t tbase, int64_t n,
                                                    int64_t nnz, int b, T *W, const T *Cd, T *Rinv,
                                                    double *ld_ws, int32_t *info_ws) {
  extern __shared__ char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *Ri = S + bb, *X = Ri + bb;
  const int64_t tg = tbase + blockIdx.x, mat = blockIdx.y;
  const int v = P.tgt_node[tg];
  const int64_t a = tg - (int64_t(P.colptr[v]) + v);
  wg::copy(S, Cd + (mat * n + v) * bb, bb);
  double ld = 0.0;
  const int fail = chol_inverse(S, Ri, b, &ld);
  if (fail) wg::fill(Ri, bb, wg::qnan<T>());
  if (a == 0) {
    wg::copy(Rinv + (mat * n + v) * bb, Ri, bb);
    if (threadIdx.x == 0) {
      ld_ws[mat * n + v] = fail ? static_cast<double>(wg::qnan<T>()) : ld;
      if (fail) atomicMin(info_ws + mat, P.node_pos[v]);
    }
  } else {
    T *Wt = W + (mat * nnz + P.colptr[v] + (a - 1)) * bb;
    wg::copy(X, Wt, bb);
    wg::gemm<T, false, true>(S, X, Ri, b);  // C R^-T (S is free now)
    wg::copy(Wt, S, bb);
  }
}

// G_{w,v} for the slots [sbase, sbase + gridDim.x) of matrix blockIdx.y
template <typename T>
__global__ void __launch_bounds__(kJT) jt_bwd_rows(JunctionPlanDev P, int64_t sbase, int64_t n,
                                                   int64_t nnz, int b, const T *__restrict__ W,
                                                   const T *__restrict__ Rinv, const T *G_diag,
                                                   T *G_lower) {
  extern __shared__ char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, CH = stage_pairs(bb);
  T *sa = smem, *sb = sa + CH * bb, *red = sb + CH * bb, *acc = red + kJT, *Ri = acc + bb,
    *X = Ri + bb;
  const int64_t s = sbase + blockIdx.x, mat = blockIdx.y;
  const int v = P.slot_node[s];
  const int32_t c0 = P.colptr[v];
  const int k = P.colptr[v + 1] - c0, a = static_cast<int>(s - c0);
  const int32_t *gt = P.gtab + P.gptr[v] + int64_t(a) * k;
  const T *Wm = W + mat * nnz * bb;
  const T *Gd = G_diag + mat * n * bb, *Gl = G_lower + mat * nnz * bb;
  staged_sum<kAB>(acc, k, b, sa, sb, red, [&](int q, int el, T &av, T &bv) {
    const int32_t enc = gt[q];
    if (enc < 0) {
      av = Gd[int64_t(-enc - 1) * bb + el];
    } else {
      const int r = el / b, c = el - r * b;
      av = Gl[int64_t(enc >> 1) * bb + ((enc & 1) ? c * b + r : el)];
    }
    bv = Wm[int64_t(c0 + q) * bb + el];
  });
  wg::copy(Ri, Rinv + (mat * n + v) * bb, bb);
  wg::gemm<T, false, false>(X, acc, Ri, b);   // T_w R_v^-1
  const int32_t o = P.outenc[s];
  T *dst = G_lower + (mat * nnz + (o >> 1)) * bb;
  for (int e = threadIdx.x; e < bb; e += kJT) {
    const int r = e / b, c = e - r * b;
    dst[e] = -((o & 1) ? X[c * b + r] : X[e]);
  }
}

// G_vv for the nodes [nbase, nbase + gridDim.x) of matrix blockIdx.y
template <typename T>
__global__ void __launch_bounds__(kJT) jt_bwd_diag(JunctionPlanDev P, int64_t nbase, int64_t n,
                                                   int64_t nnz, int b, const T *__restrict__ W,
                                                   const T *__restrict__ Rinv, T *G_diag,
                                                   const T *G_lower) {
  extern __shared__ char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, CH = stage_pairs(bb);
  T *sa = smem, *sb = sa + CH * bb, *red = sb + CH * bb, *acc = red + kJT, *Ri = acc + bb,
    *X = Ri + bb, *Y = X + bb;
  const int64_t v = nbase + blockIdx.x, mat = blockIdx.y;
  const int32_t c0 = P.colptr[v];
  const int k = P.colptr[v + 1] - c0;
  const T *Wm = W + mat * nnz * bb, *Gl = G_lower + mat * nnz * bb;
  staged_sum<kAtB>(acc, k, b, sa, sb, red, [&](int q, int el, T &av, T &bv) {
    av = Wm[int64_t(c0 + q) * bb + el];
    const int32_t o = P.outenc[c0 + q];
    const int r = el / b, c = el - r * b;
    bv = Gl[int64_t(o >> 1) * bb + ((o & 1) ? c * b + r : el)];
  });
  wg::copy(Ri, Rinv + (mat * n + v) * bb, bb);
  for (int e = threadIdx.x; e < bb; e += kJT) X[e] = Ri[e] - acc[e];
  __syncthreads();
  wg::gemm<T, true, false>(Y, Ri, X, b);      // R^-T (R^-1 - W^T G)
  wg::sym_part(X, Y, b);
  wg::copy(G_diag + (mat * n + P.node_label[v]) * bb, X, bb);
}

// log det = sum of the per-node terms in a fixed order; info from the
// earliest failing elimination position
template <typename T>
__global__ void __launch_bounds__(kJT) jt_finish(JunctionPlanDev P, int64_t n,
                                                 const double *ld_ws, const int32_t *info_ws,
                                                 double *logdet, int32_t *info) {
  __shared__ double red[kJT];
  const int64_t mat = blockIdx.x;
  double s = 0.0;
  for (int64_t v = threadIdx.x; v < n; v += kJT) s += ld_ws[mat * n + v];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kJT / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t f = info_ws[mat];
    logdet[mat] = f == INT_MAX ? red[0] : __builtin_nan("");
    if (info) info[mat] = f == INT_MAX ? 0 : 1 + P.order[f];
  }
}

struct JtWs {
  void *W, *Cd, *Rinv;
  double *ld;
  int32_t *info;
};

JtWs carve(const selinv_junction_plan *plan, int64_t B, void *ws) {
  const size_t bb = size_t(plan->b) * plan->b, es = plan->dtype_bytes;
  Carve cv(ws);
  JtWs w;
  w.W = cv.take<char>(B * plan->nnz * bb * es);
  w.Cd = cv.take<char>(B * plan->n * bb * es);
  w.Rinv = cv.take<char>(B * plan->n * bb * es);
  w.ld = cv.take<double>(B * plan->n);
  w.info = cv.take<int32_t>(B);
  return w;
}

}  // namespace

size_t junction_workspace_bytes(const selinv_junction_plan *plan, int64_t B) {
  const size_t bb = size_t(plan->b) * plan->b, es = plan->dtype_bytes;
  Carve cv(nullptr);
  cv.take<char>(B * plan->nnz * bb * es);
  cv.take<char>(B * plan->n * bb * es);
  cv.take<char>(B * plan->n * bb * es);
  cv.take<double>(B * plan->n);
  cv.take<int32_t>(B);
  return cv.off;
}

template <typename T>
hipError_t junction_launch(const selinv_junction_plan *plan, int64_t B, const T *diag,
                           const T *edge_val, T *G_diag, T *G_lower, double *logdet,
                           int32_t *info, void *ws, hipStream_t s) {
  const int b = plan->b;
  const int64_t n = plan->n, nnz = plan->nnz, m = plan->m;
  const JunctionPlanDev &P = plan->dev;
  const JtWs w = carve(plan, B, ws);
  T *W = static_cast<T *>(w.W), *Cd = static_cast<T *>(w.Cd), *Rinv = static_cast<T *>(w.Rinv);
  const size_t lds = lds_bytes<T>(b);
  const auto &lo = plan->level_off;
  const auto &cp = plan->colptr_host;
  const unsigned By = static_cast<unsigned>(B);
  jt_init<T><<<dim3(static_cast<unsigned>((B + kJT - 1) / kJT)), dim3(kJT), 0, s>>>(w.info, B);
  for (int32_t l = 0; l < plan->levels; ++l) {
    const int64_t t0 = cp[lo[l]] + lo[l], t1 = cp[lo[l + 1]] + lo[l + 1];
    const dim3 grid(static_cast<unsigned>(t1 - t0), By);
    jt_fwd_update<T><<<grid, dim3(kJT), lds, s>>>(P, t0, n, m, nnz, b, diag, edge_val, W, Cd);
    jt_fwd_scale<T><<<grid, dim3(kJT), lds, s>>>(P, t0, n, nnz, b, W, Cd, Rinv, w.ld, w.info);
  }
  for (int32_t l = plan->levels - 1; l >= 0; --l) {
    const int64_t s0 = cp[lo[l]], s1 = cp[lo[l + 1]];
    if (s1 > s0)
      jt_bwd_rows<T><<<dim3(static_cast<unsigned>(s1 - s0), By), dim3(kJT), lds, s>>>(
          P, s0, n, nnz, b, W, Rinv, G_diag, G_lower);
    jt_bwd_diag<T><<<dim3(static_cast<unsigned>(lo[l + 1] - lo[l]), By), dim3(kJT), lds, s>>>(
        P, lo[l], n, nnz, b, W, Rinv, G_diag, G_lower);
  }
  jt_finish<T><<<dim3(By), dim3(kJT), 0, s>>>(P, n, w.ld, w.info, logdet, info);
  return hipGetLastError();
}

template hipError_t junction_launch<double>(const selinv_junction_plan *, int64_t, const double *,
                                            const double *, double *, double *, double *,
                                            int32_t *, void *, hipStream_t);
template hipError_t junction_launch<float>(const selinv_junction_plan *, int64_t, const float *,
                                           const float *, float *, float *, double *, int32_t *,
                                           void *, hipStream_t);

}  // namespace selinv
