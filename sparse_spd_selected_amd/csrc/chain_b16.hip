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
// the distribute pass (workspace: its packed lower triangle, 136 entries per
// block); C_i is re-read.
// Every product has its left factor available as O(A^T): C_i is loaded
// transposed (one 16/32-byte vector per lane), and Sinv_i, G are symmetric.
#include "frag16.h"
#include "internal.h"

namespace selinv {

namespace {

using f16::Frag;

#ifndef SELINV_CHAIN16_WAVES
#define SELINV_CHAIN16_WAVES 4
#endif

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SELINV_CHAIN16_WAVES, 8)))
void chain16_kernel(int L, const T *__restrict__ diag, const T *__restrict__ lower,
                    T *__restrict__ G_diag, T *__restrict__ G_lower, double *__restrict__ logdet,
                    int32_t *__restrict__ info, T *__restrict__ state) {
  constexpr int BB = 256, PB = f16::kPacked16;
  __shared__ __align__(32) T col[16];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * BB;
  // with L == 1 there is no off-diagonal block (lower may be null); the
  // unconditional prefetch below then reads diagonal data it never uses
  const T *C = L > 1 ? lower + m * (L - 1) * BB : D;
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
  T *st = state + m * L * PB;
  const f16::SymOffsets<T> so(16, g, j);
  const f16::PackedOffsets<T> po(g, j);

  double ld = 0.0;
  int32_t fail = 0;
  Frag<T> S = so.load(D);
  // Collect.  The inputs of the next block (C_{i+1}, D_{i+2}) are loaded
  // while block i is swept; two register sets alternate (the loop is
  // unrolled by two) so that no copy of an in-flight register forces an
  // early wait on the load counter.
  Frag<T> C0 = f16::zero<T>(), D0 = f16::zero<T>(), C1 = f16::zero<T>(), D1 = f16::zero<T>();
  if (L > 1) {
    C0 = f16::load_t(C, 16, g, j);
    D0 = so.load(D + BB);
  }
  // The prefetch is unconditional (block indices clamped into range) so that
  // no register merge forces a wait on loads still in flight.
  auto collect = [&](int i, const Frag<T> &Cu, const Frag<T> &Du, Frag<T> &Cn,
                     Frag<T> &Dn) -> bool {
    const int ic = min(i + 1, max(L - 2, 0)), id = min(i + 2, L - 1);
    Cn = f16::load_t(C + ic * BB, 16, g, j);
    Dn = so.load(D + id * BB);
    f16::PivotLog pl;
    if (f16::gj_inverse(S, col, g, j, pl)) {
      fail = i + 1;
      return true;
    }
    ld += pl.log();
    if (i == L - 1) return true;
    po.store(st + i * PB, S);
    const Frag<T> Y = f16::mm<T>(S, Cu, f16::zero<T>());  // Sinv_i C_i^T
    S = Du - f16::mm<T>(Cu, Y, f16::zero<T>());           // D_{i+1} - C_i Sinv_i C_i^T
    return false;
  };
  for (int i = 0;; i += 2) {
    if (collect(i, C0, D0, C1, D1)) break;
    if (collect(i + 1, C1, D1, C0, D0)) break;
  }
  if (fail) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = lane; e < static_cast<int64_t>(L) * BB; e += 64) Gd[e] = nan;
    for (int64_t e = lane; e < static_cast<int64_t>(L - 1) * BB; e += 64) Gl[e] = nan;
    if (lane == 0) {
      logdet[m] = __builtin_nan("");
      if (info) info[m] = fail;
    }
    return;
  }
  Frag<T> G = S;  // G_{L-1,L-1} = Sinv_{L-1}
  f16::store_t(Gd + (L - 1) * BB, 16, G, g, j);
  // Distribute, with the packed Sinv and C of the next block in flight (same
  // alternating register sets).
  Frag<T> S0 = f16::zero<T>(), S1 = f16::zero<T>();
  if (L > 1) {
    S0 = po.load(st + (L - 2) * PB);
    C0 = f16::load_t(C + (L - 2) * BB, 16, g, j);
  }
  auto distribute = [&](int i, const Frag<T> &Si, const Frag<T> &Ci, Frag<T> &Sn,
                        Frag<T> &Cn) -> bool {
    if (i < 0) return true;
    const int in = max(i - 1, 0);
    Sn = po.load(st + in * PB);
    Cn = f16::load_t(C + in * BB, 16, g, j);
    const Frag<T> X = f16::mm<T>(Ci, Si, f16::zero<T>());  // C_i Sinv_i
    const Frag<T> V = f16::mm<T>(G, X, f16::zero<T>());    // G_{i+1} X
    f16::store(Gl + i * BB, 16, -V, g, j);                 // G_{i+1,i}
    G = f16::mm<T>(X, V, Si);                              // Sinv_i + X^T V
    f16::store_t(Gd + i * BB, 16, G, g, j);
    return false;
  };
  for (int i = L - 2;; i -= 2) {
    if (distribute(i, S0, C0, S1, C1)) break;
    if (distribute(i - 1, S1, C1, S0, C0)) break;
  }
  if (lane == 0) {
    logdet[m] = ld;
    if (info) info[m] = 0;
  }
}

}  // namespace

size_t chain16_workspace_bytes(int dtype_bytes, int64_t B, int64_t L) {
  return align_up(static_cast<size_t>(B) * L * f16::kPacked16 * dtype_bytes);
}

template <typename T>
hipError_t chain16_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                          T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  hipLaunchKernelGGL(chain16_kernel<T>, dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     static_cast<int>(L), diag, lower, G_diag, G_lower, logdet, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

template hipError_t chain16_launch<float>(int64_t, int64_t, const float *, const float *, float *,
                                          float *, double *, int32_t *, void *, hipStream_t);
template hipError_t chain16_launch<double>(int64_t, int64_t, const double *, const double *,
                                           double *, double *, double *, int32_t *, void *,
                                           hipStream_t);

}  // namespace selinv
