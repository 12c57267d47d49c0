// vjp_generic.hip -- reverse mode (vector-Jacobian product) of the selected
// inverse for any block size 1 <= b <= 32: one workgroup per chain / star
// leaf / tree node, blocks in LDS (block_wg.h).
//
// The gabp-sparse-inv 0.3.2 page ("Implemented and tested kernels", item
// Differentiable tree) describes the backward as a second collect / distribute
// pair on the same elimination tree.  Written out for a node v with parent p
// and edge block E_v = A_{p,v}, with the forward quantities
//   S_v = D_v - sum_children M_c,  Sinv_v = S_v^{-1},  X_v = E_v Sinv_v,
//   M_v = X_v E_v^T,  G_vv = Sinv_v + X_v^T G_pp X_v,  G_{p,v} = -G_pp X_v,
// and cotangents Gd_v on G_vv (only its symmetric part counts, G_vv being
// symmetric), Ge_v on G_{p,v} and lb on log det A, reverse mode gives
//   collect (leaves -> root):
//     GG_v  = sym(Gd_v) + sum_children sym((W_c - Ge_c) X_c^T),  W_v = X_v GG_v
//     P_v   = lb Sinv_v - Sinv_v GG_v Sinv_v
//     Z_v   = (2 W_v - Ge_v) Sinv_v
//   distribute (root -> leaves), Dbar_root = P_root:
//     Q_v    = G_pp Z_v - Dbar_p X_v
//     Ebar_v = Q_v - Dbar_p X_v
//     Dbar_v = P_v - sym(X_v^T Q_v)
// where Dbar_v is the cotangent of the symmetric diagonal input block and
// Ebar_v that of the edge block, which enters A twice (E_v at (p, v), E_v^T
// at (v, p)).  GG_v is the total cotangent of G_vv: the recursion
// GG_p += V_bar X^T with V_bar = X_v GG_v - Ge_v of the reverse distribute
// step depends only on collect quantities, so it runs inside the collect
// pass, and the reverse collect step folds into the distribute pass.  Both
// passes have the shape of the forward ones; G_vv is recomputed on the way
// down and never stored.
#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {

namespace {

inline int vjp_threads(int b) { return b <= 8 ? 64 : 256; }

// lb * Sinv - Sinv (GG Sinv): T1 is LDS scratch, Out may be global
template <typename T>
__device__ inline void p_block(T *Out, const T *Sinv, const T *GG, T *T1, T lb, int b) {
  const int bb = b * b;
  wg::gemm<T, false, false>(T1, GG, Sinv, b);                // GG Sinv
  wg::copy_scaled(Out, Sinv, bb, lb);
  wg::gemm_sym<T, false, false>(Out, Out, Sinv, T1, b, T(-1));  // symmetric in exact arithmetic
}

// W -> W - Ge (Y1) and Y -> 2 W - Ge (Y2); Ge read transposed when GE_T
template <typename T, bool GE_T>
__device__ inline void y_blocks(T *W, T *Y, const T *Ge, int b) {
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    const int r = e / b, c = e % b;
    const T w = W[e], ge = GE_T ? Ge[c * b + r] : Ge[e];
    W[e] = w - ge;
    Y[e] = (w + w) - ge;
  }
  __syncthreads();
}

// ----------------------------------------------------------------- chain
// One workgroup per chain; the chain is the path rooted at its last block
// (parent of block i is i + 1, E_i = lower[i]).  Workspace per block:
// Sinv_i, P_i, X_i, Z_i.
template <typename T>
__global__ void chain_vjp_generic(int64_t L, int b, const T *__restrict__ diag,
                                  const T *__restrict__ lower, const T *__restrict__ gd,
                                  const T *__restrict__ gl, const double *__restrict__ ld_bar,
                                  T *__restrict__ d_bar, T *__restrict__ l_bar,
                                  int32_t *__restrict__ info, T *__restrict__ state) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *GG = S + bb, *X = GG + bb, *W = X + bb, *Y = W + bb, *T1 = Y + bb,
    *col = T1 + bb;
  const int64_t m = blockIdx.x;
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const T *D = diag + m * L * bb;
  const T *C = lower + m * (L - 1) * bb;
  const T *Gd = gd + m * L * bb;
  const T *Gl = gl + m * (L - 1) * bb;
  T *Db = d_bar + m * L * bb;
  T *Cb = l_bar + m * (L - 1) * bb;
  T *st = state + m * L * 4 * bb;  // block i: Sinv, P, X, Z
  auto slot = [&](int64_t i, int k) { return st + (4 * i + k) * bb; };

  int32_t fail = 0;
  wg::load_sym_lower(S, D, b);
  wg::sym_part(GG, Gd, b);
  for (int64_t i = 0; i < L; ++i) {
    double ldi;
    if (wg::spd_inverse(S, b, col, &ldi)) {
      fail = static_cast<int32_t>(i + 1);
      break;
    }
    p_block(slot(i, 1), S, GG, T1, lb, b);
    wg::copy(slot(i, 0), S, bb);
    if (i == L - 1) break;
    const T *Ci = C + i * bb;
    wg::gemm<T, false, false>(X, Ci, S, b);   // X_i = C_i Sinv_i
    wg::copy(slot(i, 2), X, bb);
    wg::gemm<T, false, false>(W, X, GG, b);   // W_i = X_i GG_i
    y_blocks<T, false>(W, Y, Gl + i * bb, b);  // W <- W - Ge, Y <- 2 W - Ge
    wg::gemm<T, false, false>(slot(i, 3), Y, S, b);  // Z_i
    wg::load_sym_lower(S, D + (i + 1) * bb, b);
    wg::gemm_sym<T, false, true>(S, S, X, Ci, b, T(-1));  // S_{i+1} = D_{i+1} - X_i C_i^T
    wg::sym_part(GG, Gd + (i + 1) * bb, b);
    wg::gemm_symmetrized<T, false, true>(GG, GG, W, X, b, T(1));  // + sym((W - Ge) X^T)
  }
  if (fail) {
    if (threadIdx.x == 0 && info) info[m] = fail;
    for (int64_t e = threadIdx.x; e < L * bb; e += blockDim.x) Db[e] = wg::qnan<T>();
    for (int64_t e = threadIdx.x; e < (L - 1) * bb; e += blockDim.x) Cb[e] = wg::qnan<T>();
    return;
  }
  if (threadIdx.x == 0 && info) info[m] = 0;
  // distribute: G (in S) = Sinv_{L-1}, Dbar (in GG) = P_{L-1}
  T *G = S, *Dbar = GG, *T2 = X, *Q = W, *Dn = Y, *V = T1;
  wg::copy(Dbar, slot(L - 1, 1), bb);
  wg::copy(Db + (L - 1) * bb, Dbar, bb);
  for (int64_t i = L - 2; i >= 0; --i) {
    const T *Si = slot(i, 0), *Pi = slot(i, 1), *Xi = slot(i, 2), *Zi = slot(i, 3);
    wg::gemm<T, false, false>(T2, Dbar, Xi, b);                      // Dbar_{i+1} X_i
    wg::gemm_axpby<T, false, false>(Q, T(-1), T2, T(1), G, Zi, b);  // G Z - Dbar X
    for (int e = threadIdx.x; e < bb; e += blockDim.x) Cb[i * bb + e] = Q[e] - T2[e];
    wg::gemm_symmetrized<T, true, false>(Dn, Pi, Xi, Q, b, T(-1));  // P - sym(X^T Q)
    wg::gemm<T, false, false>(V, G, Xi, b);                          // V = G X
    wg::gemm_sym<T, true, false>(G, Si, Xi, V, b, T(1));             // G_ii = Sinv + X^T V
    wg::copy(Dbar, Dn, bb);
    wg::copy(Db + i * bb, Dn, bb);
  }
}

// ------------------------------------------------------------------ star
// Block 0 is the centre (the root); leaf j is a child with no children, so
// S_j = leaves[j] and GG_j = sym(Gleaf_bar[j]).  Its edge block is
// E_j = A_{0,j} = coupling[j]^T and the cotangent on G_{0,j} is
// Gcross_bar[j]^T; the cotangent of coupling[j] is Ebar_j^T.
// Workspace per leaf: P, X, Z, M, N (N = sym((W - Ge) X^T), the leaf's term
// of GG_0).
template <typename T>
__global__ void star_vjp_leaf_collect(int64_t K, int b, const T *__restrict__ leaves,
                                      const T *__restrict__ coupling, const T *__restrict__ gleaf,
                                      const T *__restrict__ gcross,
                                      const double *__restrict__ ld_bar, T *__restrict__ st,
                                      int32_t *__restrict__ st_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *GG = S + bb, *X = GG + bb, *W = X + bb, *Y = W + bb, *T1 = Y + bb,
    *col = T1 + bb;
  const int64_t leaf = blockIdx.x;  // m * K + j
  const int64_t m = leaf / K;
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  T *sP = st + (5 * leaf + 0) * bb, *sX = sP + bb, *sZ = sX + bb, *sM = sZ + bb, *sN = sM + bb;
  const T *F = coupling + leaf * bb;
  wg::load_sym_lower(S, leaves + leaf * bb, b);
  double ld;
  if (wg::spd_inverse(S, b, col, &ld)) {
    if (threadIdx.x == 0) st_fail[leaf] = 1;
    return;
  }
  if (threadIdx.x == 0) st_fail[leaf] = 0;
  wg::sym_part(GG, gleaf + leaf * bb, b);
  p_block(sP, S, GG, T1, lb, b);
  wg::gemm<T, true, false>(X, F, S, b);  // X_j = F^T Sinv_j
  wg::copy(sX, X, bb);
  wg::gemm_sym<T, false, false>(sM, nullptr, X, F, b, T(1));  // M_j = X_j F
  wg::gemm<T, false, false>(W, X, GG, b);
  y_blocks<T, true>(W, Y, gcross + leaf * bb, b);
  wg::gemm<T, false, false>(sZ, Y, S, b);
  wg::gemm_symmetrized<T, false, true>(sN, nullptr, W, X, b, T(1));
}

// Centre: S_0 = A_00 - sum_j M_j, GG_0 = sym(Gc_bar) + sum_j N_j (index
// order); G_00 = S_0^{-1} goes to the workspace, Dbar_0 = P_0 to center_bar.
template <typename T>
__global__ void star_vjp_center(int64_t K, int b, const T *__restrict__ center,
                                const T *__restrict__ gcenter, const double *__restrict__ ld_bar,
                                const T *__restrict__ st, const int32_t *__restrict__ st_fail,
                                T *__restrict__ G00, T *__restrict__ center_bar,
                                int32_t *__restrict__ info, int32_t *__restrict__ mat_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t first_bad;
  const int bb = b * b;
  T *S = smem, *GG = S + bb, *T1 = GG + bb, *col = T1 + bb;
  const int64_t m = blockIdx.x;
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  if (threadIdx.x == 0) first_bad = INT_MAX;
  __syncthreads();
  for (int64_t j = threadIdx.x; j < K; j += blockDim.x)
    if (st_fail[m * K + j]) atomicMin(&first_bad, static_cast<int32_t>(j));
  wg::load_sym_lower(S, center + m * bb, b);
  wg::sym_part(GG, gcenter + m * bb, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    T s = S[e], gg = GG[e];
    for (int64_t j = 0; j < K; ++j) {
      const T *sl = st + 5 * (m * K + j) * bb;
      s -= sl[3 * bb + e];
      gg += sl[4 * bb + e];
    }
    S[e] = s;
    GG[e] = gg;
  }
  __syncthreads();
  int32_t fail = 0;
  double ld;
  if (first_bad != INT_MAX)
    fail = first_bad + 2;
  else if (wg::spd_inverse(S, b, col, &ld))
    fail = 1;
  if (threadIdx.x == 0) {
    if (info) info[m] = fail;
    mat_fail[m] = fail;
  }
  if (fail) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) center_bar[m * bb + e] = wg::qnan<T>();
    return;
  }
  wg::copy(G00 + m * bb, S, bb);
  p_block(center_bar + m * bb, S, GG, T1, lb, b);
}

template <typename T>
__global__ void star_vjp_leaf_distribute(int64_t K, int b, const T *__restrict__ G00,
                                         const T *__restrict__ center_bar,
                                         const T *__restrict__ st,
                                         const int32_t *__restrict__ mat_fail,
                                         T *__restrict__ leaves_bar, T *__restrict__ coupling_bar) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *G = smem, *Dbar = G + bb, *T2 = Dbar + bb, *Q = T2 + bb;
  const int64_t leaf = blockIdx.x;
  const int64_t m = leaf / K;
  if (mat_fail[m]) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      leaves_bar[leaf * bb + e] = wg::qnan<T>();
      coupling_bar[leaf * bb + e] = wg::qnan<T>();
    }
    return;
  }
  const T *sP = st + 5 * leaf * bb, *sX = sP + bb, *sZ = sX + bb;
  wg::copy(G, G00 + m * bb, bb);
  wg::copy(Dbar, center_bar + m * bb, bb);
  wg::gemm<T, false, false>(T2, Dbar, sX, b);
  wg::gemm_axpby<T, false, false>(Q, T(-1), T2, T(1), G, sZ, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    const int r = e / b, c = e % b;
    coupling_bar[leaf * bb + e] = Q[c * b + r] - T2[c * b + r];  // Ebar_j^T
  }
  wg::gemm_symmetrized<T, true, false>(leaves_bar + leaf * bb, sP, sX, Q, b, T(-1));
}

// ------------------------------------------------------------------ tree
// Positions p of the plan's breadth-first order.  Workspace per position:
// Sinv, P, X, Z, M, N; the M slot of a position holds G_vv in the
// distribute pass (its M has been consumed by the parent by then).
template <typename T>
__global__ void tree_vjp_collect_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                       const int32_t *__restrict__ child_beg,
                                       const int32_t *__restrict__ child_end,
                                       const int32_t *__restrict__ fail_rank,
                                       const T *__restrict__ diag, const T *__restrict__ edge,
                                       const T *__restrict__ gd, const T *__restrict__ ge,
                                       const double *__restrict__ ld_bar, T *__restrict__ st,
                                       int32_t *__restrict__ st_fail,
                                       int32_t *__restrict__ first_fail) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  __shared__ int32_t child_failed;
  const int bb = b * b;
  T *S = smem, *GG = S + bb, *X = GG + bb, *W = X + bb, *Y = W + bb, *T1 = Y + bb,
    *col = T1 + bb;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  const int32_t cb = child_beg[p], ce = child_end[p];
  const T lb = ld_bar ? static_cast<T>(*ld_bar) : T(0);
  T *sS = st + 6 * p * bb, *sP = sS + bb, *sX = sP + bb, *sZ = sX + bb, *sM = sZ + bb,
    *sN = sM + bb;
  if (threadIdx.x == 0) child_failed = 0;
  __syncthreads();
  for (int32_t c = cb + threadIdx.x; c < ce; c += blockDim.x)
    if (st_fail[c]) child_failed = 1;
  wg::load_sym_lower(S, diag + v * bb, b);
  wg::sym_part(GG, gd + v * bb, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    T s = S[e], gg = GG[e];
    for (int32_t c = cb; c < ce; ++c) {
      const T *sc = st + 6 * static_cast<int64_t>(c) * bb;
      s -= sc[4 * bb + e];
      gg += sc[5 * bb + e];
    }
    S[e] = s;
    GG[e] = gg;
  }
  __syncthreads();
  double ld;
  if (child_failed || wg::spd_inverse(S, b, col, &ld)) {
    if (threadIdx.x == 0) {
      st_fail[p] = 1;
      if (!child_failed) atomicMin(first_fail, fail_rank[p]);
    }
    return;
  }
  if (threadIdx.x == 0) st_fail[p] = 0;
  wg::copy(sS, S, bb);
  p_block(sP, S, GG, T1, lb, b);
  if (p == 0) return;  // the root has no parent edge
  const T *E = edge + v * bb;
  wg::gemm<T, false, false>(X, E, S, b);  // X_v = E_v Sinv_v
  wg::copy(sX, X, bb);
  wg::gemm_sym<T, false, true>(sM, nullptr, X, E, b, T(1));  // M_v = X_v E_v^T
  wg::gemm<T, false, false>(W, X, GG, b);
  y_blocks<T, false>(W, Y, ge + v * bb, b);
  wg::gemm<T, false, false>(sZ, Y, S, b);
  wg::gemm_symmetrized<T, false, true>(sN, nullptr, W, X, b, T(1));
}

// Root: G_rr = Sinv_r into its G slot, Dbar_r = P_r, zero root edge slot,
// info.
template <typename T>
__global__ void tree_vjp_root(int b, const int32_t *__restrict__ node_at,
                              const int32_t *__restrict__ rank_node, T *__restrict__ st,
                              const int32_t *__restrict__ first_fail, T *__restrict__ d_bar,
                              T *__restrict__ e_bar, int32_t *__restrict__ info) {
  const int bb = b * b;
  const int64_t r = node_at[0];
  const bool failed = *first_fail != INT_MAX;
  for (int e = threadIdx.x; e < bb; e += blockDim.x) {
    st[4 * bb + e] = st[e];
    d_bar[r * bb + e] = failed ? wg::qnan<T>() : st[bb + e];
    e_bar[r * bb + e] = T(0);
  }
  if (threadIdx.x == 0 && info) *info = failed ? rank_node[*first_fail] + 1 : 0;
}

template <typename T>
__global__ void tree_vjp_distribute_level(int64_t p0, int b, const int32_t *__restrict__ node_at,
                                          const int32_t *__restrict__ parent_pos,
                                          const int32_t *__restrict__ parent_node,
                                          T *__restrict__ st,
                                          const int32_t *__restrict__ first_fail,
                                          T *__restrict__ d_bar, T *__restrict__ e_bar) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *G = smem, *Dbar = G + bb, *T2 = Dbar + bb, *Q = T2 + bb, *V = Q + bb;
  const int64_t p = p0 + blockIdx.x;
  const int64_t v = node_at[p];
  if (*first_fail != INT_MAX) {
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      d_bar[v * bb + e] = wg::qnan<T>();
      e_bar[v * bb + e] = wg::qnan<T>();
    }
    return;
  }
  const int64_t q = parent_pos[p], u = parent_node[p];
  const T *sS = st + 6 * p * bb, *sP = sS + bb, *sX = sP + bb, *sZ = sX + bb;
  T *sG = st + (6 * p + 4) * bb;
  wg::copy(G, st + (6 * q + 4) * bb, bb);
  wg::copy(Dbar, d_bar + u * bb, bb);
  wg::gemm<T, false, false>(T2, Dbar, sX, b);
  wg::gemm_axpby<T, false, false>(Q, T(-1), T2, T(1), G, sZ, b);
  for (int e = threadIdx.x; e < bb; e += blockDim.x) e_bar[v * bb + e] = Q[e] - T2[e];
  wg::gemm_symmetrized<T, true, false>(d_bar + v * bb, sP, sX, Q, b, T(-1));
  wg::gemm<T, false, false>(V, G, sX, b);
  wg::gemm_sym<T, true, false>(sG, sS, sX, V, b, T(1));
}

__global__ void vjp_init_int(int32_t *p, int32_t v) { *p = v; }

}  // namespace

// ------------------------------------------------------------ launchers

size_t chain_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  const int Pv = chain_vjp_segments(B, L, b);
  if (Pv > 0) return chain_vjp_seg_workspace_bytes(dtype_bytes, B, L, b, Pv);
  if (b == 16) return chain16_vjp_workspace_bytes(dtype_bytes, B, L);
  return align_up(static_cast<size_t>(B) * L * 4 * b * b * dtype_bytes);
}

template <typename T>
hipError_t chain_vjp_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                            const T *gd, const T *gl, const double *ld_bar, T *d_bar, T *l_bar,
                            int32_t *info, void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int Pv = chain_vjp_segments(B, L, b);
  if (Pv > 0)
    return chain_vjp_seg_launch<T>(B, L, b, Pv, diag, lower, gd, gl, ld_bar, d_bar, l_bar, info,
                                   ws, s);
  if (b == 16)
    return chain16_vjp_launch<T>(B, L, diag, lower, gd, gl, ld_bar, d_bar, l_bar, info, ws, s);
  const size_t shm = (6 * b * b + b) * sizeof(T);
  hipLaunchKernelGGL(chain_vjp_generic<T>, dim3(static_cast<unsigned>(B)), dim3(vjp_threads(b)),
                     shm, s, L, b, diag, lower, gd, gl, ld_bar, d_bar, l_bar, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

size_t star_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if (b == 32) return star32_vjp_workspace_bytes(dtype_bytes, B, K);
  const size_t nl = static_cast<size_t>(B) * K, bb = static_cast<size_t>(b) * b;
  return align_up(5 * nl * bb * dtype_bytes) + align_up(B * bb * dtype_bytes) +
         align_up(nl * sizeof(int32_t)) + align_up(B * sizeof(int32_t));
}

template <typename T>
hipError_t star_vjp_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                           const T *coupling, const T *gc, const T *gleaf, const T *gcross,
                           const double *ld_bar, T *center_bar, T *leaves_bar, T *coupling_bar,
                           int32_t *info, void *ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (b == 32)
    return star32_vjp_launch<T>(B, K, center, leaves, coupling, gc, gleaf, gcross, ld_bar,
                                center_bar, leaves_bar, coupling_bar, info, ws, s);
  const size_t nl = static_cast<size_t>(B) * K, bb = static_cast<size_t>(b) * b;
  Carve cv(ws);
  T *st = cv.take<T>(5 * nl * bb);
  T *G00 = cv.take<T>(B * bb);
  int32_t *st_fail = cv.take<int32_t>(nl);
  int32_t *mat_fail = cv.take<int32_t>(B);
  const int nt = vjp_threads(b);
  if (nl)
    hipLaunchKernelGGL(star_vjp_leaf_collect<T>, dim3(static_cast<unsigned>(nl)), dim3(nt),
                       (6 * bb + b) * sizeof(T), s, K, b, leaves, coupling, gleaf, gcross, ld_bar,
                       st, st_fail);
  hipLaunchKernelGGL(star_vjp_center<T>, dim3(static_cast<unsigned>(B)), dim3(nt),
                     (3 * bb + b) * sizeof(T), s, K, b, center, gc, ld_bar, st, st_fail, G00,
                     center_bar, info, mat_fail);
  if (nl)
    hipLaunchKernelGGL(star_vjp_leaf_distribute<T>, dim3(static_cast<unsigned>(nl)), dim3(nt),
                       4 * bb * sizeof(T), s, K, b, G00, center_bar, st, mat_fail, leaves_bar,
                       coupling_bar);
  return hipGetLastError();
}

size_t tree_vjp_workspace_bytes(const selinv_tree_plan *plan) {
  if (plan->b <= 8) return tree8_vjp_workspace_bytes(plan);
  const size_t n = plan->n, bb = static_cast<size_t>(plan->b) * plan->b;
  return align_up(6 * n * bb * plan->dtype_bytes) + align_up(n * sizeof(int32_t)) +
         align_up(sizeof(int32_t));
}

template <typename T>
hipError_t tree_vjp_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                           const T *gd, const T *ge, const double *ld_bar, T *d_bar, T *e_bar,
                           int32_t *info, void *ws, hipStream_t s) {
  if (plan->b <= 8)
    return tree8_vjp_launch<T>(plan, diag, edge, gd, ge, ld_bar, d_bar, e_bar, info, ws, s);
  const size_t n = plan->n;
  const int b = plan->b;
  const size_t bb = static_cast<size_t>(b) * b;
  Carve cv(ws);
  T *st = cv.take<T>(6 * n * bb);
  int32_t *st_fail = cv.take<int32_t>(n);
  int32_t *first_fail = cv.take<int32_t>(1);
  const TreePlanDev &d = plan->dev;
  const int nt = vjp_threads(b);
  hipLaunchKernelGGL(vjp_init_int, dim3(1), dim3(1), 0, s, first_fail, INT_MAX);
  for (int32_t lev = plan->levels - 1; lev >= 0; --lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(tree_vjp_collect_level<T>, dim3(static_cast<unsigned>(p1 - p0)), dim3(nt),
                       (6 * bb + b) * sizeof(T), s, p0, b, d.node_at, d.child_beg, d.child_end,
                       d.fail_rank, diag, edge, gd, ge, ld_bar, st, st_fail, first_fail);
  }
  hipLaunchKernelGGL(tree_vjp_root<T>, dim3(1), dim3(256), 0, s, b, d.node_at, d.rank_node, st,
                     first_fail, d_bar, e_bar, info);
  for (int32_t lev = 1; lev < plan->levels; ++lev) {
    const int64_t p0 = plan->level_off[lev], p1 = plan->level_off[lev + 1];
    hipLaunchKernelGGL(tree_vjp_distribute_level<T>, dim3(static_cast<unsigned>(p1 - p0)),
                       dim3(nt), 5 * bb * sizeof(T), s, p0, b, d.node_at, d.parent_pos,
                       d.parent_node, st, first_fail, d_bar, e_bar);
  }
  return hipGetLastError();
}

#define SELINV_INSTANTIATE(T)                                                                   \
  template hipError_t chain_vjp_launch<T>(int64_t, int64_t, int32_t, const T *, const T *,       \
                                          const T *, const T *, const double *, T *, T *,        \
                                          int32_t *, void *, hipStream_t);                       \
  template hipError_t star_vjp_launch<T>(int64_t, int64_t, int32_t, const T *, const T *,        \
                                         const T *, const T *, const T *, const T *,             \
                                         const double *, T *, T *, T *, int32_t *, void *,       \
                                         hipStream_t);                                           \
  template hipError_t tree_vjp_launch<T>(const selinv_tree_plan *, const T *, const T *,         \
                                         const T *, const T *, const double *, T *, T *,         \
                                         int32_t *, void *, hipStream_t);
SELINV_INSTANTIATE(float)
SELINV_INSTANTIATE(double)
#undef SELINV_INSTANTIATE

}  // namespace selinv
