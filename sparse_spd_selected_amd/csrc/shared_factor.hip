// shared_factor.hip -- the siblings that reuse the collect's factor (the
// gabp-sparse-inv 0.3.2 page: log det "straight from the same LDL^T
// factorization", the SPD solve x = A^{-1} b sharing one factorization, and
// Gaussian samples x ~ N(0, A^{-1}) "reusing the same factorization").
//
// The collect is a block LDL^T factorisation A = L D L^T with
// D = blockdiag(S_v) and L_{p,v} = X_v = E_v S_v^{-1} (E_v = A_{p,v}).  The
// factor kept here is S_v^{-1} as a packed lower triangle per block
// (wg::packed_entries(b) entries); X_v is never stored, since every use of it
// is a product with a vector: X_v u = E_v (S_v^{-1} u), X_v^T x = S_v^{-1}
// (E_v^T x).
//   factor:  the collect pass (S_v, S_v^{-1}, log det, pivot test)
//   solve:   u = y; children first: w_v = S_v^{-1} u_v, u_p -= E_v w_v;
//            parents first: x_root = w_root, x_v = w_v - S_v^{-1} E_v^T x_p
//   sample:  x = L^{-T} D^{-1/2} z with D^{-1/2}_v = U_v, the upper
//            triangular factor of S_v^{-1} (U_v U_v^T = S_v^{-1}; with
//            S_v = R_v R_v^T, U_v = R_v^{-T}):
//            parents first: x_v = U_v z_v - S_v^{-1} E_v^T x_p
// Vectors are [..., n, b, k] (k right-hand sides, k fastest).  Solve and
// sample split the k columns into chunks of at most kChunk, one workgroup per
// (matrix or node, chunk).  One workgroup per chain / leaf / node, blocks in
// LDS (block_wg.h); the b = 16 chain factor runs on the matrix cores
// (chain_b16.hip).
#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {

namespace {

constexpr int kChunk = 16;  // right-hand-side columns per workgroup

inline int sf_threads(int b) { return b <= 8 ? 64 : 256; }
inline int nchunks(int64_t k) { return static_cast<int>((k + kChunk - 1) / kChunk); }

// ----------------------------------------------------------------- chain
template <typename T>
__global__ void chain_factor_generic(int64_t L, int b, const T *__restrict__ diag,
                                     const T *__restrict__ lower, T *__restrict__ factor,
                                     double *__restrict__ logdet, int32_t *__restrict__ info) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *S = smem, *X = S + bb, *col = X + bb;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * bb;
  const T *C = lower + m * (L - 1) * bb;
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
    if (factor) wg::pack_lower(factor + (m * L + i) * pk, S, b);
    if (i == L - 1) break;
    wg::gemm<T, false, false>(X, C + i * bb, S, b);  // X_i = C_i Sinv_i
    wg::load_sym_lower(S, D + (i + 1) * bb, b);
    wg::gemm_sym<T, false, true>(S, S, X, C + i * bb, b, T(-1));
  }
  if (threadIdx.x == 0) {
    logdet[m] = fail ? wg::qnan<double>() : ld;
    if (info) info[m] = fail;
  }
}

// Solve (kSample = false) or sample (true) for one chain and one chunk of
// columns; the chain is the path rooted at its last block (the child of
// block i is i - 1, E_i = lower[i]).
template <typename T, bool kSample>
__global__ void chain_apply_generic(int64_t L, int b, int64_t k, int nch,
                                    const T *__restrict__ lower, const T *__restrict__ factor,
                                    const T *__restrict__ in, T *__restrict__ out) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *U = Si + bb, *u = U + bb, *w = u + b * kChunk, *t = w + b * kChunk;
  const int64_t m = blockIdx.x / nch;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  const T *C = lower + m * (L - 1) * bb;
  const T *F = factor + m * L * pk;
  auto vec = [&](const T *base, int64_t i) { return base + ((m * L + i) * b) * k + c0; };
  auto vec_w = [&](T *base, int64_t i) { return base + ((m * L + i) * b) * k + c0; };
  // load / store a b x kc block of a vector array (row stride k) to LDS (row stride kc)
  auto load = [&](T *dst, const T *src) {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x) dst[e] = src[(e / kc) * k + e % kc];
    __syncthreads();
  };
  auto store = [&](T *dst, const T *src) {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x) dst[(e / kc) * k + e % kc] = src[e];
    __syncthreads();
  };
  if (!kSample) {
    // L u = y and D w = u, children first: w_i = Sinv_i u_i, u_{i+1} -= E_i w_i
    for (int64_t i = 0; i < L; ++i) {
      load(u, vec(in, i));
      if (i > 0) wg::bmv<T, false>(u, kc, T(1), u, T(-1), C + (i - 1) * bb, w, kc, b, kc);
      wg::unpack_sym(Si, F + i * pk, b);
      wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), Si, u, kc, b, kc);
      store(vec_w(out, i), w);
    }
  }
  // L^T x = w, parents first; the sampler's w_i = U_i z_i
  for (int64_t i = L - 1; i >= 0; --i) {
    wg::unpack_sym(Si, F + i * pk, b);
    if (kSample) {
      load(u, vec(in, i));
      wg::rev_cholesky(U, Si, b);
      wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), U, u, kc, b, kc);
    } else {
      load(w, vec(out, i));
    }
    if (i < L - 1) {  // x_i = w_i - Sinv_i (E_i^T x_{i+1}), x_{i+1} in t
      wg::bmv<T, true>(u, kc, T(0), nullptr, T(1), C + i * bb, t, kc, b, kc);
      wg::bmv<T, false>(w, kc, T(1), w, T(-1), Si, u, kc, b, kc);
    }
    store(vec_w(out, i), w);
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x) t[e] = w[e];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ star
// Factor layout: leaves [B][K][pk], then centres [B][pk].  The centre is the
// parent of every leaf, E_j = A_{0,j} = coupling[j]^T.
template <typename T>
__global__ void star_factor_leaf(int64_t K, int b, const T *__restrict__ leaves,
                                 const T *__restrict__ coupling, T *__restrict__ factor,
                                 T *__restrict__ st_m, double *__restrict__ st_ld,
                                 int32_t *__restrict__ st_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *S = smem, *X = S + bb, *col = X + bb;
  const int64_t leaf = blockIdx.x;
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
  if (factor) wg::pack_lower(factor + leaf * pk, S, b);
  const T *F = coupling + leaf * bb;
  wg::gemm<T, true, false>(X, F, S, b);                                   // F^T Sinv
  wg::gemm_sym<T, false, false>(st_m + leaf * bb, nullptr, X, F, b, T(1));  // F^T Sinv F
}

template <typename T>
__global__ void star_factor_center(int64_t B, int64_t K, int b, const T *__restrict__ center,
                                   const T *__restrict__ st_m, const double *__restrict__ st_ld,
                                   const int32_t *__restrict__ st_fail, T *__restrict__ factor,
                                   double *__restrict__ logdet, int32_t *__restrict__ info) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t first_bad;
  const int bb = b * b, pk = wg::packed_entries(b);
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
    if (fail) {
      logdet[m] = wg::qnan<double>();
    } else {
      double ld = 0.0;
      for (int64_t j = 0; j < K; ++j) ld += st_ld[m * K + j];
      logdet[m] = ld + ldc;
    }
  }
  if (!fail && factor) wg::pack_lower(factor + (B * K + m) * pk, S, b);
}

// Solve, leaves first: w_j = Sinv_j y_j (to out), message E_j w_j = F_j^T w_j
template <typename T>
__global__ void star_solve_leaf_fwd(int64_t K, int b, int64_t k, int nch,
                                    const T *__restrict__ coupling, const T *__restrict__ factor,
                                    const T *__restrict__ y_leaves, T *__restrict__ x_leaves,
                                    T *__restrict__ msg) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *u = Si + bb, *w = u + b * kChunk;
  const int64_t leaf = blockIdx.x / nch;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  const T *yv = y_leaves + leaf * b * k + c0;
  T *xv = x_leaves + leaf * b * k + c0;
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) u[e] = yv[(e / kc) * k + e % kc];
  wg::unpack_sym(Si, factor + leaf * pk, b);
  wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), Si, u, kc, b, kc);
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) xv[(e / kc) * k + e % kc] = w[e];
  wg::bmv<T, true>(msg + leaf * b * k + c0, static_cast<int>(k), T(0), nullptr, T(1),
                   coupling + leaf * bb, w, kc, b, kc);
}

// Centre: u_0 = y_0 - sum_j messages (solve, index order), x_0 = Sinv_0 u_0;
// or x_0 = U_0 z_0 (sample)
template <typename T, bool kSample>
__global__ void star_apply_center(int64_t B, int64_t K, int b, int64_t k, int nch,
                                  const T *__restrict__ factor, const T *__restrict__ in_center,
                                  const T *__restrict__ msg, T *__restrict__ x_center) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *U = Si + bb, *u = U + bb, *w = u + b * kChunk;
  const int64_t m = blockIdx.x / nch;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) {
    const int r = e / kc, c = e % kc;
    T s = in_center[(m * b + r) * k + c0 + c];
    if (!kSample)
      for (int64_t j = 0; j < K; ++j) s -= msg[((m * K + j) * b + r) * k + c0 + c];
    u[e] = s;
  }
  wg::unpack_sym(Si, factor + (B * K + m) * pk, b);
  if (kSample) {
    wg::rev_cholesky(U, Si, b);
    wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), U, u, kc, b, kc);
  } else {
    wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), Si, u, kc, b, kc);
  }
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
    x_center[(m * b + e / kc) * k + c0 + e % kc] = w[e];
}

// Leaves, parents first: x_j = w_j - Sinv_j (F_j x_0), w_j = out (solve) or
// U_j z_j (sample)
template <typename T, bool kSample>
__global__ void star_apply_leaf_bwd(int64_t K, int b, int64_t k, int nch,
                                    const T *__restrict__ coupling, const T *__restrict__ factor,
                                    const T *__restrict__ z_leaves,
                                    const T *__restrict__ x_center, T *__restrict__ x_leaves) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *U = Si + bb, *u = U + bb, *w = u + b * kChunk, *t = w + b * kChunk;
  const int64_t leaf = blockIdx.x / nch;
  const int64_t m = leaf / K;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  T *xv = x_leaves + leaf * b * k + c0;
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
    t[e] = x_center[(m * b + e / kc) * k + c0 + e % kc];
  wg::unpack_sym(Si, factor + leaf * pk, b);
  if (kSample) {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
      u[e] = z_leaves[leaf * b * k + (e / kc) * k + c0 + e % kc];
    wg::rev_cholesky(U, Si, b);
    wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), U, u, kc, b, kc);
  } else {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x) w[e] = xv[(e / kc) * k + e % kc];
    __syncthreads();
  }
  wg::bmv<T, false>(u, kc, T(0), nullptr, T(1), coupling + leaf * bb, t, kc, b, kc);  // F x_0
  wg::bmv<T, false>(w, kc, T(1), w, T(-1), Si, u, kc, b, kc);
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) xv[(e / kc) * k + e % kc] = w[e];
}

// ------------------------------------------------------------------ tree
// Factor layout: [n][pk] by breadth-first position.
template <typename T>
__global__ void tree_factor_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                  const int32_t *__restrict__ child_beg,
                                  const int32_t *__restrict__ child_end,
                                  const int32_t *__restrict__ fail_rank,
                                  const T *__restrict__ diag, const T *__restrict__ edge,
                                  T *__restrict__ factor, T *__restrict__ st_m,
                                  double *__restrict__ st_ld, int32_t *__restrict__ st_fail,
                                  int32_t *__restrict__ first_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t child_failed;
  const int bb = b * b, pk = wg::packed_entries(b);
  T *S = smem, *X = S + bb, *col = X + bb;
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
  if (factor) wg::pack_lower(factor + p * pk, S, b);
  if (p == 0) return;
  const T *E = edge + v * bb;
  wg::gemm<T, false, false>(X, E, S, b);
  wg::gemm_sym<T, false, true>(st_m + p * bb, nullptr, X, E, b, T(1));
}

// log det = fixed-order sum of the per-node terms; info
__global__ void tree_factor_finish(int64_t n, const int32_t *__restrict__ rank_node,
                                   const double *__restrict__ st_ld,
                                   const int32_t *__restrict__ first_fail,
                                   double *__restrict__ logdet, int32_t *__restrict__ info) {
  __shared__ double part[256];
  const int nt = blockDim.x;
  const int64_t chunk = (n + nt - 1) / nt;
  double s = 0.0;
  const int64_t a = threadIdx.x * chunk;
  for (int64_t q = a; q < a + chunk && q < n; ++q) s += st_ld[q];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = nt / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const bool failed = *first_fail != INT_MAX;
    *logdet = failed ? wg::qnan<double>() : part[0];
    if (info) *info = failed ? rank_node[*first_fail] + 1 : 0;
  }
}

// Solve, children first, one level: u_v = y_v - sum_children msg_c,
// w_v = Sinv_v u_v (to out), msg_v = E_v w_v (by position)
template <typename T>
__global__ void tree_solve_fwd_level(int64_t p0, int b, int64_t k, int nch,
                                     const int32_t *__restrict__ node_at,
                                     const int32_t *__restrict__ child_beg,
                                     const int32_t *__restrict__ child_end,
                                     const T *__restrict__ edge, const T *__restrict__ factor,
                                     const T *__restrict__ y, T *__restrict__ x,
                                     T *__restrict__ msg) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *u = Si + bb, *w = u + b * kChunk;
  const int64_t p = p0 + blockIdx.x / nch;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  const int64_t v = node_at[p];
  const int32_t cb = child_beg[p], ce = child_end[p];
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) {
    const int r = e / kc, c = e % kc;
    T s = y[(v * b + r) * k + c0 + c];
    for (int32_t q = cb; q < ce; ++q) s -= msg[(static_cast<int64_t>(q) * b + r) * k + c0 + c];
    u[e] = s;
  }
  wg::unpack_sym(Si, factor + p * pk, b);
  wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), Si, u, kc, b, kc);
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
    x[(v * b + e / kc) * k + c0 + e % kc] = w[e];
  if (p != 0)
    wg::bmv<T, false>(msg + p * b * k + c0, static_cast<int>(k), T(0), nullptr, T(1),
                      edge + v * bb, w, kc, b, kc);
}

// Parents first, one level: x_v = w_v - Sinv_v E_v^T x_p, w_v = out (solve)
// or U_v z_v (sample); at the root (p = 0) only w
template <typename T, bool kSample>
__global__ void tree_apply_bwd_level(int64_t p0, int b, int64_t k, int nch,
                                     const int32_t *__restrict__ node_at,
                                     const int32_t *__restrict__ parent_node,
                                     const T *__restrict__ edge, const T *__restrict__ factor,
                                     const T *__restrict__ z, T *__restrict__ x) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b, pk = wg::packed_entries(b);
  T *Si = smem, *U = Si + bb, *u = U + bb, *w = u + b * kChunk, *t = w + b * kChunk;
  const int64_t p = p0 + blockIdx.x / nch;
  const int c0 = (blockIdx.x % nch) * kChunk;
  const int kc = static_cast<int>(min<int64_t>(kChunk, k - c0));
  const int64_t v = node_at[p];
  T *xv = x + v * b * k + c0;
  wg::unpack_sym(Si, factor + p * pk, b);
  if (kSample) {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
      u[e] = z[(v * b + e / kc) * k + c0 + e % kc];
    wg::rev_cholesky(U, Si, b);
    wg::bmv<T, false>(w, kc, T(0), nullptr, T(1), U, u, kc, b, kc);
  } else {
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x) w[e] = xv[(e / kc) * k + e % kc];
    __syncthreads();
  }
  if (p != 0) {
    const int64_t up = parent_node[p];
    for (int e = threadIdx.x; e < b * kc; e += blockDim.x)
      t[e] = x[(up * b + e / kc) * k + c0 + e % kc];
    __syncthreads();
    wg::bmv<T, true>(u, kc, T(0), nullptr, T(1), edge + v * bb, t, kc, b, kc);  // E^T x_p
    wg::bmv<T, false>(w, kc, T(1), w, T(-1), Si, u, kc, b, kc);
  }
  for (int e = threadIdx.x; e < b * kc; e += blockDim.x) xv[(e / kc) * k + e % kc] = w[e];
}

__global__ void sf_init_int(int32_t *p, int32_t v) { *p = v; }

inline size_t apply_smem(int b, int elems_per_block = 2) {
  return static_cast<size_t>(elems_per_block) * b * b + 3 * b * kChunk;
}

}  // namespace

// ------------------------------------------------------------ launchers

size_t chain_factor_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  return align_up(static_cast<size_t>(B) * L * wg::packed_entries(b) * dtype_bytes);
}

template <typename T>
hipError_t chain_factor_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                               T *factor, double *logdet, int32_t *info, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b == 16) return chain16_factor_launch<T>(B, L, diag, lower, factor, logdet, info, s);
  hipLaunchKernelGGL(chain_factor_generic<T>, dim3(static_cast<unsigned>(B)),
                     dim3(sf_threads(b)), (2 * b * b + b) * sizeof(T), s, L, b, diag, lower,
                     factor, logdet, info);
  return hipGetLastError();
}

template <typename T>
hipError_t chain_apply_launch(int64_t B, int64_t L, int32_t b, int64_t k, bool sample,
                              const T *lower, const T *factor, const T *in, T *out,
                              hipStream_t s) {
  if (B == 0 || k == 0) return hipSuccess;
  if (!sample && b == 16) return chain16_solve_launch<T>(B, L, k, lower, factor, in, out, s);
  if (sample && b == 16) return chain16_sample_launch<T>(B, L, k, lower, factor, in, out, s);
  const int nch = nchunks(k);
  const dim3 grid(static_cast<unsigned>(B * nch));
  const size_t shm = apply_smem(b) * sizeof(T);
  if (sample)
    hipLaunchKernelGGL((chain_apply_generic<T, true>), grid, dim3(sf_threads(b)), shm, s, L, b, k,
                       nch, lower, factor, in, out);
  else
    hipLaunchKernelGGL((chain_apply_generic<T, false>), grid, dim3(sf_threads(b)), shm, s, L, b,
                       k, nch, lower, factor, in, out);
  return hipGetLastError();
}

size_t star_factor_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  return align_up(static_cast<size_t>(B) * (K + 1) * wg::packed_entries(b) * dtype_bytes);
}

size_t star_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if (b == 32) return star32_factor_workspace_bytes(dtype_bytes, B, K);
  const size_t nl = static_cast<size_t>(B) * K;
  return align_up(nl * b * b * dtype_bytes) + align_up(nl * sizeof(double)) +
         align_up(nl * sizeof(int32_t));
}

template <typename T>
hipError_t star_factor_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                              const T *coupling, T *factor, double *logdet, int32_t *info,
                              void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b == 32)
    return star32_factor_launch<T>(B, K, center, leaves, coupling, factor, logdet, info, ws, s);
  const size_t nl = static_cast<size_t>(B) * K;
  Carve cv(ws);
  T *st_m = cv.take<T>(nl * b * b);
  double *st_ld = cv.take<double>(nl);
  int32_t *st_fail = cv.take<int32_t>(nl);
  const int nt = sf_threads(b);
  if (nl)
    hipLaunchKernelGGL(star_factor_leaf<T>, dim3(static_cast<unsigned>(nl)), dim3(nt),
                       (2 * b * b + b) * sizeof(T), s, K, b, leaves, coupling, factor, st_m,
                       st_ld, st_fail);
  hipLaunchKernelGGL(star_factor_center<T>, dim3(static_cast<unsigned>(B)), dim3(nt),
                     (b * b + b) * sizeof(T), s, B, K, b, center, st_m, st_ld, st_fail, factor,
                     logdet, info);
  return hipGetLastError();
}

size_t star_apply_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b, int64_t k) {
  return align_up(static_cast<size_t>(B) * K * b * k * dtype_bytes);
}

template <typename T>
hipError_t star_apply_launch(int64_t B, int64_t K, int32_t b, int64_t k, bool sample,
                             const T *coupling, const T *factor, const T *in_center,
                             const T *in_leaves, T *x_center, T *x_leaves, void *ws,
                             hipStream_t s) {
  if (B == 0 || k == 0) return hipSuccess;
  if (b == 32 && k <= 4)
    return star32_apply_launch<T>(B, K, k, sample, coupling, factor, in_center, in_leaves,
                                  x_center, x_leaves, ws, s);
  const int nch = nchunks(k);
  const size_t nl = static_cast<size_t>(B) * K;
  const int nt = sf_threads(b);
  const size_t shm = apply_smem(b) * sizeof(T);
  T *msg = static_cast<T *>(ws);
  if (!sample && nl)
    hipLaunchKernelGGL(star_solve_leaf_fwd<T>, dim3(static_cast<unsigned>(nl * nch)), dim3(nt),
                       shm, s, K, b, k, nch, coupling, factor, in_leaves, x_leaves, msg);
  if (sample)
    hipLaunchKernelGGL((star_apply_center<T, true>), dim3(static_cast<unsigned>(B * nch)),
                       dim3(nt), shm, s, B, K, b, k, nch, factor, in_center, msg, x_center);
  else
    hipLaunchKernelGGL((star_apply_center<T, false>), dim3(static_cast<unsigned>(B * nch)),
                       dim3(nt), shm, s, B, K, b, k, nch, factor, in_center, msg, x_center);
  if (nl) {
    if (sample)
      hipLaunchKernelGGL((star_apply_leaf_bwd<T, true>), dim3(static_cast<unsigned>(nl * nch)),
                         dim3(nt), shm, s, K, b, k, nch, coupling, factor, in_leaves, x_center,
                         x_leaves);
    else
      hipLaunchKernelGGL((star_apply_leaf_bwd<T, false>), dim3(static_cast<unsigned>(nl * nch)),
                         dim3(nt), shm, s, K, b, k, nch, coupling, factor, in_leaves, x_center,
                         x_leaves);
  }
  return hipGetLastError();
}

size_t tree_factor_bytes(const selinv_tree_plan *plan) {
  return align_up(static_cast<size_t>(plan->n) * wg::packed_entries(plan->b) * plan->dtype_bytes);
}

size_t tree_factor_workspace_bytes(const selinv_tree_plan *plan) {
  if (plan->b <= 8) return tree8_factor_workspace_bytes(plan);
  const size_t n = plan->n, bb = static_cast<size_t>(plan->b) * plan->b;
  return align_up(n * bb * plan->dtype_bytes) + align_up(n * sizeof(double)) +
         align_up(n * sizeof(int32_t)) + align_up(sizeof(int32_t));
}

template <typename T>
hipError_t tree_factor_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                              T *factor, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  if (plan->b <= 8)
    return tree8_factor_launch<T>(plan, diag, edge, factor, logdet, info, ws, s);
  const size_t n = plan->n;
  const int b = plan->b;
  Carve cv(ws);
  T *st_m = cv.take<T>(n * b * b);
  double *st_ld = cv.take<double>(n);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  hipLaunchKernelGGL(sf_init_int, dim3(1), dim3(1), 0, s, first_fail, INT_MAX);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(tree_factor_level<T>, dim3(static_cast<unsigned>(p1 - p0)),
                       dim3(sf_threads(b)), (2 * b * b + b) * sizeof(T), s, p0, b, d.node_at,
                       d.child_beg, d.child_end, d.fail_rank, diag, edge, factor, st_m, st_ld,
                       st_fail, first_fail);
  }
  hipLaunchKernelGGL(tree_factor_finish, dim3(1), dim3(256), 0, s, static_cast<int64_t>(n),
                     d.rank_node, st_ld, first_fail, logdet, info);
  return hipGetLastError();
}

size_t tree_apply_workspace_bytes(const selinv_tree_plan *plan, int64_t k) {
  if (plan->b <= 8) return tree8_solve_workspace_bytes(plan, k);
  return align_up(static_cast<size_t>(plan->n) * plan->b * k * plan->dtype_bytes);
}

template <typename T>
hipError_t tree_apply_launch(const selinv_tree_plan *plan, int64_t k, bool sample, const T *edge,
                             const T *factor, const T *in, T *out, void *ws, hipStream_t s) {
  if (k == 0) return hipSuccess;
  if (!sample && plan->b <= 8) return tree8_solve_launch<T>(plan, k, edge, factor, in, out, ws, s);
  if (sample && plan->b <= 8) return tree8_sample_launch<T>(plan, k, edge, factor, in, out, ws, s);
  const int b = plan->b;
  const int nch = nchunks(k);
  const int nt = sf_threads(b);
  const size_t shm = apply_smem(b) * sizeof(T);
  const TreePlanDev &d = plan->dev;
  T *msg = static_cast<T *>(ws);
  if (!sample)
    for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
      const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
      hipLaunchKernelGGL(tree_solve_fwd_level<T>, dim3(static_cast<unsigned>((p1 - p0) * nch)),
                         dim3(nt), shm, s, p0, b, k, nch, d.node_at, d.child_beg, d.child_end,
                         edge, factor, in, out, msg);
    }
  for (int32_t lev = 0; lev < plan->levels; ++lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    const dim3 grid(static_cast<unsigned>((p1 - p0) * nch));
    if (sample)
      hipLaunchKernelGGL((tree_apply_bwd_level<T, true>), grid, dim3(nt), shm, s, p0, b, k, nch,
                         d.node_at, d.parent_node, edge, factor, in, out);
    else
      hipLaunchKernelGGL((tree_apply_bwd_level<T, false>), grid, dim3(nt), shm, s, p0, b, k, nch,
                         d.node_at, d.parent_node, edge, factor, in, out);
  }
  return hipGetLastError();
}

#define SELINV_INSTANTIATE(T)                                                                    \
  template hipError_t chain_factor_launch<T>(int64_t, int64_t, int32_t, const T *, const T *,     \
                                             T *, double *, int32_t *, hipStream_t);              \
  template hipError_t chain_apply_launch<T>(int64_t, int64_t, int32_t, int64_t, bool, const T *,  \
                                            const T *, const T *, T *, hipStream_t);              \
  template hipError_t star_factor_launch<T>(int64_t, int64_t, int32_t, const T *, const T *,      \
                                            const T *, T *, double *, int32_t *, void *,          \
                                            hipStream_t);                                         \
  template hipError_t star_apply_launch<T>(int64_t, int64_t, int32_t, int64_t, bool, const T *,   \
                                           const T *, const T *, const T *, T *, T *, void *,     \
                                           hipStream_t);                                          \
  template hipError_t tree_factor_launch<T>(const selinv_tree_plan *, const T *, const T *, T *,  \
                                            double *, int32_t *, void *, hipStream_t);            \
  template hipError_t tree_apply_launch<T>(const selinv_tree_plan *, int64_t, bool, const T *,    \
                                           const T *, const T *, T *, void *, hipStream_t);
SELINV_INSTANTIATE(float)
SELINV_INSTANTIATE(double)
#undef SELINV_INSTANTIATE

}  // namespace selinv
