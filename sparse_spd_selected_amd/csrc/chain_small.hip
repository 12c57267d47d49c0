// chain_small.hip -- block-tridiagonal selected inverse for block sizes
// b <= 8: eight chains per wavefront, one block row per lane (rows8.h).
// Per chain (gabp-sparse-inv 0.3.2 page, item Chain of "Implemented and
// tested kernels"; the chain is the path rooted at its last block), with
// C_i = lower[i] = A_{i+1,i}:
//   collect  i = 0 .. L-2:   Sinv_i = S_i^{-1},  X = C_i Sinv_i,
//                            S_{i+1} = D_{i+1} - X C_i^T
//   root:                    G_{L-1} = Sinv_{L-1}
//   distribute i = L-2 .. 0: X = C_i Sinv_i,  V = G_{i+1} X,
//                            G_lower[i] = -V,  G_i = Sinv_i + X^T V
// Sinv_i (padded 8 x 8) is the only state kept between the passes.
#include "internal.h"
#include "rows8.h"

namespace selinv {

namespace {

constexpr int kWaves = 4;

template <typename T>
__global__ __launch_bounds__(256) void chain_small_kernel(
    int64_t B, int L, int b, const T *__restrict__ diag, const T *__restrict__ lower,
    T *__restrict__ G_diag, T *__restrict__ G_lower, double *__restrict__ logdet,
    int32_t *__restrict__ info, T *__restrict__ state) {
  __shared__ __align__(32) T lds[kWaves][2][8 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = lane >> 3, i = lane & 7;
  const r8::Stage<T> sa{lds[wave][0]}, sb{lds[wave][1]};
  const int64_t m = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * 8 + s;
  const bool valid = m < B;
  const int bb = b * b;
  const int64_t mc = valid ? m : 0;  // inactive slots shadow chain 0 and store nothing
  const T *D = diag + mc * L * bb;
  const T *C = L > 1 ? lower + mc * (L - 1) * bb : D;
  T *Gd = G_diag + mc * L * bb;
  T *Gl = G_lower + mc * (L - 1) * bb;
  T *st = state + mc * L * 64;

  double ld = 0.0;
  int32_t fail = 0;
  r8::Row<T> S = r8::load_sym(D, b, i);
  // Collect.  C_k and D_{k+1} are loaded one step ahead; two register sets
  // alternate (loop unrolled by two, clamped in-range indices) so that no
  // register copy waits on a load in flight.
  const int lc = max(L - 2, 0);
  r8::Row<T> C0 = r8::load(C, b, i), D0 = r8::load_sym(D + min(1, L - 1) * bb, b, i);
  r8::Row<T> C1, D1;
  auto collect = [&](int k, const r8::Row<T> &Ck, const r8::Row<T> &Dn, r8::Row<T> &Cn,
                     r8::Row<T> &Dnn) -> bool {
    Cn = r8::load(C + min(k + 1, lc) * bb, b, i);
    Dnn = r8::load_sym(D + min(k + 2, L - 1) * bb, b, i);
    f16::PivotLog pl;
    const bool bad = r8::gj_inverse(S, sa, s, i, pl);
    if (bad && !fail) fail = k + 1;
    ld += pl.log();
    if (k == L - 1) return true;
    if (valid) r8::store8(st + k * 64, i, S);
    f16::wave_sync();
    sa.put(s, i, S);
    sb.put(s, i, Ck);
    f16::wave_sync();
    const r8::Row<T> X = r8::mul(Ck, sa, s, r8::zero<T>());  // C_k Sinv_k
    const r8::Row<T> M = r8::mul_t(X, sb, s, r8::zero<T>());  // X C_k^T
#pragma unroll
    for (int c = 0; c < 8; ++c) S.v[c] = Dn.v[c] - M.v[c];
    return false;
  };
  for (int k = 0;; k += 2) {
    if (collect(k, C0, D0, C1, D1)) break;
    if (collect(k + 1, C1, D1, C0, D0)) break;
  }
  if (fail) {
    if (valid) {
      r8::Row<T> nan;
#pragma unroll
      for (int c = 0; c < 8; ++c) nan.v[c] = static_cast<T>(__builtin_nan(""));
      for (int k = 0; k < L; ++k) r8::store(Gd + k * bb, b, i, nan);
      for (int k = 0; k + 1 < L; ++k) r8::store(Gl + k * bb, b, i, nan);
      if (i == 0) {
        logdet[m] = __builtin_nan("");
        if (info) info[m] = fail;
      }
    }
    return;  // only this slot's lanes leave; the other slots' staging is disjoint
  }
  r8::Row<T> G = S;  // G_{L-1} = Sinv_{L-1}
  if (valid) r8::store(Gd + (L - 1) * bb, b, i, G);
  // Distribute, with Sinv and C of the next block in flight.
  r8::Row<T> S0 = r8::load8(st + lc * 64, i), S1;
  C0 = r8::load(C + lc * bb, b, i);
  auto distribute = [&](int k, const r8::Row<T> &Si, const r8::Row<T> &Ck, r8::Row<T> &Sn,
                        r8::Row<T> &Cn) -> bool {
    if (k < 0) return true;
    const int kn = max(k - 1, 0);
    Sn = r8::load8(st + kn * 64, i);
    Cn = r8::load(C + kn * bb, b, i);
    f16::wave_sync();
    sa.put(s, i, Si);
    f16::wave_sync();
    const r8::Row<T> X = r8::mul(Ck, sa, s, r8::zero<T>());  // C_k Sinv_k
    sb.put(s, i, X);
    f16::wave_sync();
    const r8::Row<T> V = r8::mul(G, sb, s, r8::zero<T>());   // G_{k+1} X
    f16::wave_sync();
    sa.put(s, i, V);
    f16::wave_sync();
    G = r8::mul_tn(sb, sa, s, i, Si);                        // Sinv_k + X^T V
    if (valid) {
      r8::store(Gl + k * bb, b, i, r8::neg(V));
      r8::store(Gd + k * bb, b, i, G);
    }
    return false;
  };
  for (int k = L - 2;; k -= 2) {
    if (distribute(k, S0, C0, S1, C1)) break;
    if (distribute(k - 1, S1, C1, S0, C0)) break;
  }
  if (valid && i == 0) {
    logdet[m] = ld;
    if (info) info[m] = 0;
  }
}

}  // namespace

size_t chain_small_workspace_bytes(int dtype_bytes, int64_t B, int64_t L) {
  return align_up(static_cast<size_t>(B) * L * 64 * dtype_bytes);
}

template <typename T>
hipError_t chain_small_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                              T *G_diag, T *G_lower, double *logdet, int32_t *info, void *ws,
                              hipStream_t s) {
  const int64_t per_block = kWaves * 8;
  const unsigned grid = static_cast<unsigned>((B + per_block - 1) / per_block);
  hipLaunchKernelGGL(chain_small_kernel<T>, dim3(grid), dim3(256), 0, s, B,
                     static_cast<int>(L), b, diag, lower, G_diag, G_lower, logdet, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

template hipError_t chain_small_launch<float>(int64_t, int64_t, int32_t, const float *,
                                              const float *, float *, float *, double *,
                                              int32_t *, void *, hipStream_t);
template hipError_t chain_small_launch<double>(int64_t, int64_t, int32_t, const double *,
                                               const double *, double *, double *, double *,
                                               int32_t *, void *, hipStream_t);

}  // namespace selinv
