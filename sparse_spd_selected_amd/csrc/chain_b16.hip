// chain_b16.hip -- block-tridiagonal selected inverse for 16x16 blocks: one
// wavefront per chain, every block held in registers in the MFMA 16x16
// accumulator layout (frag16.h), block products on the matrix cores.
//
// Per chain (gabp-sparse-inv 0.3.2 page, "Implemented and tested kernels",
// item Chain: block LDL^T sweep then Takahashi back-recursion; the chain is
// the path rooted at its last block):
//   collect  i = 0 .. L-2:   Sinv_i = S_i^{-1} (Gauss-Jordan sweep),
//                            Y = Sinv_i C_i^T,  S_{i+1} = D_{i+1} - C_i Y
//   root:                    G_{L-1} = Sinv_{L-1}
//   distribute i = L-2 .. 0: X = C_i Sinv_i,  V = G_{i+1} X,
//                            G_lower[i] = -V,  G_i = Sinv_i + X^T V
// with C_i = lower[i] = A_{i+1,i}.  Only Sinv_i crosses from the collect to
// the distribute pass (workspace, 16x16 per block); C_i is re-read.
// Every product has its left factor available as O(A^T): C_i is loaded
// transposed (one 16/32-byte vector per lane), and Sinv_i, G are symmetric.
#include "frag16.h"
#include "internal.h"

namespace selinv {

namespace {

using f16::Frag;

template <typename T>
__global__ __launch_bounds__(64) void chain16_kernel(int64_t L, const T *__restrict__ diag,
                                                     const T *__restrict__ lower,
                                                     T *__restrict__ G_diag,
                                                     T *__restrict__ G_lower,
                                                     double *__restrict__ logdet,
                                                     int32_t *__restrict__ info,
                                                     T *__restrict__ state) {
  constexpr int BB = 256;
  __shared__ __align__(32) T col[16];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * BB;
  const T *C = lower + m * (L - 1) * BB;
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
  T *st = state + m * L * BB;

  double ld = 0.0;
  int32_t fail = 0;
  Frag<T> S = f16::load_sym(D, 16, g, j);
  Frag<T> Ct = f16::zero<T>(), Dn = f16::zero<T>();
  if (L > 1) {
    Ct = f16::load_t(C, 16, g, j);
    Dn = f16::load_sym(D + BB, 16, g, j);
  }
  for (int64_t i = 0; i < L; ++i) {
    f16::PivotLog pl;
    if (f16::gj_inverse(S, col, g, j, pl)) {
      fail = static_cast<int32_t>(i + 1);
      break;
    }
    ld += pl.log();
    if (i == L - 1) break;
    f16::store_t(st + i * BB, 16, S, g, j);
    const Frag<T> Ci = Ct, Di = Dn;
    if (i + 2 < L) {  // prefetch the next block's inputs
      Ct = f16::load_t(C + (i + 1) * BB, 16, g, j);
      Dn = f16::load_sym(D + (i + 2) * BB, 16, g, j);
    }
    const Frag<T> Y = f16::mm<T>(S, Ci, f16::zero<T>());   // Sinv_i C_i^T
    const Frag<T> M = f16::mm<T>(Ci, Y, f16::zero<T>());   // C_i Sinv_i C_i^T
    S = Di - M;
  }
  if (fail) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = lane; e < L * BB; e += 64) Gd[e] = nan;
    for (int64_t e = lane; e < (L - 1) * BB; e += 64) Gl[e] = nan;
    if (lane == 0) {
      logdet[m] = __builtin_nan("");
      if (info) info[m] = fail;
    }
    return;
  }
  Frag<T> G = S;  // G_{L-1,L-1} = Sinv_{L-1}
  f16::store_t(Gd + (L - 1) * BB, 16, G, g, j);
  Frag<T> Sn = f16::zero<T>(), Cn = f16::zero<T>();
  if (L > 1) {
    Sn = f16::load_t(st + (L - 2) * BB, 16, g, j);
    Cn = f16::load_t(C + (L - 2) * BB, 16, g, j);
  }
  for (int64_t i = L - 2; i >= 0; --i) {
    const Frag<T> Si = Sn, Ci = Cn;
    if (i >= 1) {
      Sn = f16::load_t(st + (i - 1) * BB, 16, g, j);
      Cn = f16::load_t(C + (i - 1) * BB, 16, g, j);
    }
    const Frag<T> X = f16::mm<T>(Ci, Si, f16::zero<T>());   // C_i Sinv_i
    const Frag<T> V = f16::mm<T>(G, X, f16::zero<T>());     // G_{i+1} X
    f16::store(Gl + i * BB, 16, -V, g, j);                  // G_{i+1,i}
    G = f16::mm<T>(X, V, Si);                               // Sinv_i + X^T V
    f16::store_t(Gd + i * BB, 16, G, g, j);
  }
  if (lane == 0) {
    logdet[m] = ld;
    if (info) info[m] = 0;
  }
}

}  // namespace

template <typename T>
hipError_t chain16_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                          T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  hipLaunchKernelGGL(chain16_kernel<T>, dim3(static_cast<unsigned>(B)), dim3(64), 0, s, L, diag,
                     lower, G_diag, G_lower, logdet, info, static_cast<T *>(ws));
  return hipGetLastError();
}

template hipError_t chain16_launch<float>(int64_t, int64_t, const float *, const float *, float *,
                                          float *, double *, int32_t *, void *, hipStream_t);
template hipError_t chain16_launch<double>(int64_t, int64_t, const double *, const double *,
                                           double *, double *, double *, int32_t *, void *,
                                           hipStream_t);

}  // namespace selinv
