// vjp_chain_seg.hip -- reverse mode of the chain selected inverse for a few
// long chains, parallel over segments of each chain.
//
// The two-pass reverse mode (vjp_generic.hip; the analytic backward of the
// gabp-sparse-inv 0.3.2 page's differentiable tree) is sequential along a
// chain.  With C_i = lower[i], X_i = C_i Sinv_i and the forward selected
// inverse G already computed (here by the segment-parallel forward), every
// recurrence it needs can be cut into segments:
//   * Sinv at a segment start a comes from G alone:  X_a = -G_{a+1,a+1}^{-1}
//     G_{a+1,a} and Sinv_a = G_aa - G_{a+1,a}^T G_{a+1,a+1}^{-1} G_{a+1,a}
//     (from G_{a+1,a} = -G_{a+1,a+1} X_a and G_aa = Sinv_a + X_a^T G_{a+1,a+1}
//     X_a); inside the segment the ordinary collect recurrence continues;
//   * the cotangent of G_ii obeys GG_{i+1} = X_i GG_i X_i^T + c_i with
//     c_i = sym(Gd_{i+1}) - sym(Gl_i X_i^T), an affine congruence: a segment
//     maps GG_a to GG_e = Phi GG_a Phi^T + Cm (Phi = X_{e-1} ... X_a);
//   * the input cotangent obeys Dbar_i = X_i^T Dbar_{i+1} X_i + r_i with
//     r_i = P_i - sym(X_i^T G_{i+1,i+1} Z_i), the same congruence run
//     backwards: Dbar_a = Phi^T Dbar_e Phi + R, R = sum_i Pi_i^T r_i Pi_i,
//     Pi_i = X_{i-1} ... X_a.
// Passes (one workgroup per segment unless noted, blocks in LDS):
//   forward selected inverse (any forward path) -> G, info
//   prep:  Sinv_i, X_i per block; the GG map (Phi, Cm) per segment
//   scan:  one workgroup per chain, GG at every segment start
//   mid:   P_i = lb Sinv_i - Sinv_i GG_i Sinv_i, Z_i = (2 X_i GG_i - Gl_i) Sinv_i,
//          the Dbar map's R per segment
//   scan:  one workgroup per chain, Dbar at every segment end (from P_{L-1})
//   out:   Dbar_i and lower_bar_i = G_{i+1,i+1} Z_i - 2 Dbar_{i+1} X_i, descending
#include <algorithm>
#include <climits>

#include "block_wg.h"
#include "internal.h"

namespace selinv {

namespace {

inline int cvs_threads(int b) { return b <= 8 ? 64 : 256; }

template <typename T>
__device__ inline void set_identity(T *A, int b) {
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) A[e] = (e / b == e % b) ? T(1) : T(0);
  __syncthreads();
}

struct SegRange {
  int64_t a0, a1;
};
__device__ inline SegRange seg_range(int64_t L, int P, int s) {
  return {static_cast<int64_t>(s) * L / P, static_cast<int64_t>(s + 1) * L / P};
}

template <typename T>
__global__ void cvs_prep(int64_t L, int b, int P, const T *__restrict__ diag,
                         const T *__restrict__ lower, const T *__restrict__ gd,
                         const T *__restrict__ gl, const T *__restrict__ Gd,
                         const T *__restrict__ Gl, T *__restrict__ sinv_ws, T *__restrict__ x_ws,
                         T *__restrict__ phi, T *__restrict__ cmap) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *S = smem, *X = S + bb, *Ph = X + bb, *Cm = Ph + bb, *T1 = Cm + bb, *T2 = T1 + bb,
    *Cs = T2 + bb, *col = Cs + bb;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange r = seg_range(L, P, s);
  const T *D = diag + m * L * bb, *C = lower + m * (L - 1) * bb;
  const T *GDm = Gd + m * L * bb, *GLm = Gl + m * (L - 1) * bb;
  const T *gdm = gd + m * L * bb, *glm = gl + m * (L - 1) * bb;
  double ld;
  if (s == 0) {
    wg::load_sym_lower(S, D, b);
    wg::spd_inverse(S, b, col, &ld);
  } else {  // Sinv_a = G_aa - G_{a+1,a}^T G_{a+1,a+1}^{-1} G_{a+1,a}
    wg::load_sym_lower(T1, GDm + (r.a0 + 1) * bb, b);
    wg::spd_inverse(T1, b, col, &ld);
    wg::copy(Cs, GLm + r.a0 * bb, bb);
    wg::gemm<T, false, false>(T2, T1, Cs, b);
    wg::gemm_sym<T, true, false>(S, GDm + r.a0 * bb, Cs, T2, b, T(-1));
  }
  set_identity(Ph, b);
  wg::fill(Cm, bb, T(0));
  for (int64_t i = r.a0; i < r.a1; ++i) {
    if (i > r.a0) {  // S_i = D_i - X_{i-1} C_{i-1}^T (X, Cs of the previous step)
      wg::load_sym_lower(S, D + i * bb, b);
      wg::gemm_sym<T, false, true>(S, S, X, Cs, b, T(-1));
      wg::spd_inverse(S, b, col, &ld);
    }
    wg::copy(sinv_ws + (m * L + i) * bb, S, bb);
    if (i == L - 1) break;
    wg::copy(Cs, C + i * bb, bb);
    wg::gemm<T, false, false>(X, Cs, S, b);  // X_i = C_i Sinv_i
    wg::copy(x_ws + (m * L + i) * bb, X, bb);
    wg::sym_part(T1, gdm + (i + 1) * bb, b);  // c_i = sym(Gd_{i+1}) - sym(Gl_i X_i^T)
    wg::copy(T2, glm + i * bb, bb);
    wg::gemm_symmetrized<T, false, true>(T1, T1, T2, X, b, T(-1));
    wg::gemm<T, false, false>(T2, X, Ph, b);  // Phi <- X_i Phi
    wg::copy(Ph, T2, bb);
    wg::gemm<T, false, false>(T2, X, Cm, b);  // Cm <- X_i Cm X_i^T + c_i
    wg::gemm_sym<T, false, true>(Cm, T1, T2, X, b, T(1));
  }
  wg::copy(phi + (m * P + s) * bb, Ph, bb);
  wg::copy(cmap + (m * P + s) * bb, Cm, bb);
}

// GG at every segment start, one workgroup per chain
template <typename T>
__global__ void cvs_gg_scan(int b, int P, int64_t L, const T *__restrict__ gd,
                            const T *__restrict__ phi, const T *__restrict__ cmap,
                            T *__restrict__ gg_start) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *GG = smem, *T2 = GG + bb, *Ph = T2 + bb;
  const int64_t m = blockIdx.x;
  wg::sym_part(GG, gd + m * L * bb, b);
  for (int s = 0; s < P; ++s) {
    const int64_t q = m * P + s;
    wg::copy(gg_start + q * bb, GG, bb);
    wg::copy(Ph, phi + q * bb, bb);
    wg::gemm<T, false, false>(T2, Ph, GG, b);
    wg::gemm_sym<T, false, true>(GG, cmap + q * bb, T2, Ph, b, T(1));  // base read once
  }
}

template <typename T>
__global__ void cvs_mid(int64_t L, int b, int P, const T *__restrict__ gd,
                        const T *__restrict__ gl, const double *__restrict__ ld_bar,
                        const T *__restrict__ Gd, const T *__restrict__ sinv_ws,
                        const T *__restrict__ x_ws, const T *__restrict__ gg_start,
                        T *__restrict__ p_ws, T *__restrict__ z_ws, T *__restrict__ rmap) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  // every operand of a product is staged in LDS first (one coalesced copy)
  T *GG = smem, *Pi = GG + bb, *R = Pi + bb, *Si = R + bb, *Xi = Si + bb, *A = Xi + bb,
    *Bq = A + bb, *Cq = Bq + bb;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange rg = seg_range(L, P, s);
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const T *gdm = gd + m * L * bb, *glm = gl + m * (L - 1) * bb, *GDm = Gd + m * L * bb;
  wg::copy(GG, gg_start + (m * P + s) * bb, bb);
  set_identity(Pi, b);
  wg::fill(R, bb, T(0));
  for (int64_t i = rg.a0; i < rg.a1; ++i) {
    T *Pw = p_ws + (m * L + i) * bb, *Zw = z_ws + (m * L + i) * bb;
    wg::copy(Si, sinv_ws + (m * L + i) * bb, bb);
    wg::gemm<T, false, false>(A, GG, Si, b);  // P_i = lb Sinv - Sinv (GG Sinv), in Cq
    wg::copy_scaled(Cq, Si, bb, lb);
    wg::gemm_sym<T, false, false>(Cq, Cq, Si, A, b, T(-1));
    wg::copy(Pw, Cq, bb);
    if (i == L - 1) break;
    wg::copy(Xi, x_ws + (m * L + i) * bb, bb);
    wg::gemm<T, false, false>(A, Xi, GG, b);  // W = X GG
    for (int e = threadIdx.x; e < bb; e += blockDim.x) {
      const T w = A[e], g = glm[i * bb + e];
      A[e] = w - g;          // Y1 = W - Gl
      Bq[e] = (w + w) - g;   // Y2 = 2 W - Gl
    }
    __syncthreads();
    wg::sym_part(GG, gdm + (i + 1) * bb, b);  // GG <- sym(Gd_{i+1}) + sym(Y1 X^T)
    wg::gemm_symmetrized<T, false, true>(GG, GG, A, Xi, b, T(1));
    wg::gemm<T, false, false>(A, Bq, Si, b);  // Z_i = Y2 Sinv
    wg::copy(Zw, A, bb);
    wg::copy(Bq, GDm + (i + 1) * bb, bb);
    wg::gemm<T, false, false>(Si, Bq, A, b);                          // G_{i+1} Z_i
    wg::gemm_symmetrized<T, true, false>(Bq, Cq, Xi, Si, b, T(-1));  // r_i = P - sym(X^T G Z)
    wg::gemm<T, false, false>(A, Bq, Pi, b);                          // R += Pi^T r Pi
    wg::gemm_sym<T, true, false>(R, R, Pi, A, b, T(1));
    wg::gemm<T, false, false>(A, Xi, Pi, b);  // Pi <- X_i Pi
    wg::copy(Pi, A, bb);
  }
  wg::copy(rmap + (m * P + s) * bb, R, bb);
}

// Dbar at every segment end (the first block after the segment; the root for
// the last one), one workgroup per chain
template <typename T>
__global__ void cvs_db_scan(int b, int P, int64_t L, const T *__restrict__ p_ws,
                            const T *__restrict__ phi, const T *__restrict__ rmap,
                            T *__restrict__ db_end) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *Db = smem, *T2 = Db + bb, *Ph = T2 + bb;
  const int64_t m = blockIdx.x;
  wg::copy(Db, p_ws + (m * L + L - 1) * bb, bb);
  for (int s = P - 1; s >= 0; --s) {
    const int64_t q = m * P + s;
    wg::copy(db_end + q * bb, Db, bb);
    wg::copy(Ph, phi + q * bb, bb);
    wg::gemm<T, false, false>(T2, Db, Ph, b);
    wg::gemm_sym<T, true, false>(Db, rmap + q * bb, Ph, T2, b, T(1));
  }
}

template <typename T>
__global__ void cvs_out(int64_t L, int b, int P, const T *__restrict__ Gd,
                        const T *__restrict__ x_ws, const T *__restrict__ z_ws,
                        const T *__restrict__ p_ws, const T *__restrict__ db_end,
                        const int32_t *__restrict__ info_ws, T *__restrict__ d_bar,
                        T *__restrict__ l_bar, int32_t *__restrict__ info) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *Db = smem, *T2 = Db + bb, *Q = T2 + bb, *Dn = Q + bb, *Xs = Dn + bb, *Zs = Xs + bb,
    *Gs = Zs + bb;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange rg = seg_range(L, P, s);
  const int64_t e = s == P - 1 ? L - 1 : rg.a1;
  T *Dbm = d_bar + m * L * bb, *Lbm = l_bar + m * (L - 1) * bb;
  if (s == 0 && threadIdx.x == 0 && info) info[m] = info_ws[m];
  if (info_ws[m]) {
    for (int64_t q = rg.a0 * bb + threadIdx.x; q < rg.a1 * bb; q += blockDim.x)
      Dbm[q] = wg::qnan<T>();
    for (int64_t q = rg.a0 * bb + threadIdx.x; q < min(rg.a1, L - 1) * bb; q += blockDim.x)
      Lbm[q] = wg::qnan<T>();
    return;
  }
  wg::copy(Db, db_end + (m * P + s) * bb, bb);
  if (s == P - 1) wg::copy(Dbm + (L - 1) * bb, Db, bb);  // Dbar_{L-1} = P_{L-1}
  for (int64_t i = e - 1; i >= rg.a0; --i) {
    wg::copy(Xs, x_ws + (m * L + i) * bb, bb);
    wg::copy(Zs, z_ws + (m * L + i) * bb, bb);
    wg::copy(Gs, Gd + (m * L + i + 1) * bb, bb);
    const T *Pi = p_ws + (m * L + i) * bb;
    wg::gemm<T, false, false>(T2, Db, Xs, b);                       // Dbar_{i+1} X_i
    wg::gemm_axpby<T, false, false>(Q, T(-1), T2, T(1), Gs, Zs, b);  // G Z - Dbar X
    for (int q = threadIdx.x; q < bb; q += blockDim.x) Lbm[i * bb + q] = Q[q] - T2[q];
    wg::gemm_symmetrized<T, true, false>(Dn, Pi, Xs, Q, b, T(-1));  // P - sym(X^T Q)
    wg::copy(Db, Dn, bb);
    wg::copy(Dbm + i * bb, Dn, bb);
  }
}

struct CvsLayout {
  size_t gd, gl, ld, info, fwd, sinv, x, p, z, phi, cmap, rmap, ggs, dbe, total;
};

CvsLayout cvs_layout(int dtype_bytes, int64_t B, int64_t L, int32_t b, int P) {
  CvsLayout o{};
  const size_t bb = static_cast<size_t>(b) * b, w = dtype_bytes;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  o.gd = take(B * L * bb * w);
  o.gl = take(B * (L - 1) * bb * w);
  o.ld = take(B * sizeof(double));
  o.info = take(B * sizeof(int32_t));
  o.fwd = take(chain_workspace_bytes(dtype_bytes, B, L, b));
  o.sinv = take(B * L * bb * w);
  o.x = take(B * L * bb * w);
  o.p = take(B * L * bb * w);
  o.z = take(B * L * bb * w);
  o.phi = take(B * P * bb * w);
  o.cmap = take(B * P * bb * w);
  o.rmap = take(B * P * bb * w);
  o.ggs = take(B * P * bb * w);
  o.dbe = take(B * P * bb * w);
  o.total = off;
  return o;
}

}  // namespace

int chain_vjp_segments(int64_t B, int64_t L, int32_t b) {
  if (b != 32 || B >= 512 || L < 512) return 0;
  return static_cast<int>(std::min<int64_t>(L / 128, 16384 / B));
}

size_t chain_vjp_seg_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b, int P) {
  return cvs_layout(dtype_bytes, B, L, b, P).total;
}

template <typename T>
hipError_t chain_vjp_seg_launch(int64_t B, int64_t L, int32_t b, int P, const T *diag,
                                const T *lower, const T *gd, const T *gl, const double *ld_bar,
                                T *d_bar, T *l_bar, int32_t *info, void *ws, hipStream_t s) {
  const CvsLayout o = cvs_layout(sizeof(T), B, L, b, P);
  char *base = static_cast<char *>(ws);
  T *Gd = reinterpret_cast<T *>(base + o.gd), *Gl = reinterpret_cast<T *>(base + o.gl);
  double *ld = reinterpret_cast<double *>(base + o.ld);
  int32_t *info_ws = reinterpret_cast<int32_t *>(base + o.info);
  T *sinv = reinterpret_cast<T *>(base + o.sinv), *x = reinterpret_cast<T *>(base + o.x);
  T *p = reinterpret_cast<T *>(base + o.p), *z = reinterpret_cast<T *>(base + o.z);
  T *phi = reinterpret_cast<T *>(base + o.phi), *cmap = reinterpret_cast<T *>(base + o.cmap);
  T *rmap = reinterpret_cast<T *>(base + o.rmap), *ggs = reinterpret_cast<T *>(base + o.ggs);
  T *dbe = reinterpret_cast<T *>(base + o.dbe);
  hipError_t e = chain_launch<T>(B, L, b, diag, lower, Gd, Gl, ld, info_ws, base + o.fwd, s);
  if (e != hipSuccess) return e;
  const int nt = cvs_threads(b);
  const size_t bb = static_cast<size_t>(b) * b;
  const dim3 segs(static_cast<unsigned>(B * P)), chains(static_cast<unsigned>(B));
  hipLaunchKernelGGL(cvs_prep<T>, segs, dim3(nt), (7 * bb + b) * sizeof(T), s, L, b, P, diag,
                     lower, gd, gl, Gd, Gl, sinv, x, phi, cmap);
  hipLaunchKernelGGL(cvs_gg_scan<T>, chains, dim3(nt), 3 * bb * sizeof(T), s, b, P, L, gd, phi,
                     cmap, ggs);
  hipLaunchKernelGGL(cvs_mid<T>, segs, dim3(nt), 8 * bb * sizeof(T), s, L, b, P, gd, gl, ld_bar,
                     Gd, sinv, x, ggs, p, z, rmap);
  hipLaunchKernelGGL(cvs_db_scan<T>, chains, dim3(nt), 3 * bb * sizeof(T), s, b, P, L, p, phi,
                     rmap, dbe);
  hipLaunchKernelGGL(cvs_out<T>, segs, dim3(nt), 7 * bb * sizeof(T), s, L, b, P, Gd, x, z, p, dbe,
                     info_ws, d_bar, l_bar, info);
  return hipGetLastError();
}

template hipError_t chain_vjp_seg_launch<float>(int64_t, int64_t, int32_t, int, const float *,
                                                const float *, const float *, const float *,
                                                const double *, float *, float *, int32_t *,
                                                void *, hipStream_t);
template hipError_t chain_vjp_seg_launch<double>(int64_t, int64_t, int32_t, int, const double *,
                                                 const double *, const double *, const double *,
                                                 const double *, double *, double *, int32_t *,
                                                 void *, hipStream_t);

}  // namespace selinv
