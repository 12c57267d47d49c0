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
//
// Every global access is a 16-byte-per-lane vector over consecutive bytes
// (io16.h): blocks arrive in natural order one step ahead of their use and
// are permuted into fragments in a per-wavefront LDS tile; results leave the
// same way.  C_i is read from its tile transposed, giving O(C_i^T), the form
// in which it enters the products as the left factor (Sinv_i and G are
// symmetric, so O(X) = O(X^T) for those).
#include "frag16.h"
#include "internal.h"
#include "io16.h"

namespace selinv {

namespace {

using f16::Frag;

#ifndef SELINV_CHAIN16_WAVES
#define SELINV_CHAIN16_WAVES 4
#endif

// kFactor: the collect pass only (the shared factor of the solve and the
// sampler): packed Sinv_i of every block, root included, goes to `state`
// ([B][L][136]; null = log det and info only) and G_diag, G_lower are unused.
template <typename T, bool kFactor>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SELINV_CHAIN16_WAVES, 8)))
void chain16_kernel(int L, const T *__restrict__ diag, const T *__restrict__ lower,
                    T *__restrict__ G_diag, T *__restrict__ G_lower, double *__restrict__ logdet,
                    int32_t *__restrict__ info, T *__restrict__ state) {
  using Tr = io16::Traits<T>;
  constexpr int BB = 256, PB = f16::kPacked16;
  __shared__ __align__(16) T col[16];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  __shared__ __align__(16) T tP[PB];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * BB;
  // with L == 1 there is no off-diagonal block (lower may be null); the
  // unconditional prefetch below then reads diagonal data it never uses
  const T *C = L > 1 ? lower + m * (L - 1) * BB : D;
  T *st = state ? state + m * L * PB : nullptr;
  const bool keep = !kFactor || st;  // the packed Sinv_i are stored
  const io16::SymLanes<T> sl(g, j, lane);

  f16::PivotLog pl;  // product of all pivots of the chain (log taken once)
  int32_t fail = 0;
  Frag<T> S;
  {
    const io16::Nat<T> d0 = io16::load(D, lane);
    io16::put(tA, lane, d0);
    f16::wave_sync();
    S = sl.get_sym(tA);
    f16::wave_sync();
  }
  // Collect.  The inputs of the next block (C_{i+1}, D_{i+2}) are loaded
  // while block i is swept; two register sets alternate (the loop is
  // unrolled by two) and the block indices are clamped into range, so that
  // no register copy or merge forces an early wait on loads in flight.  The
  // loops have a single exit: a failed pivot is recorded and the sweep runs
  // on (its output is discarded), which keeps the waits on the prefetched
  // registers exact.
  const int lc = max(L - 2, 0);
  io16::Nat<T> C0 = io16::load(C, lane), D0 = io16::load(D + min(1, L - 1) * BB, lane);
  io16::Nat<T> C1, D1;
  auto collect = [&](int i, const io16::Nat<T> &Cu, const io16::Nat<T> &Du, io16::Nat<T> &Cn,
                     io16::Nat<T> &Dn) {
    Cn = io16::load(C + min(i + 1, lc) * BB, lane);
    Dn = io16::load(D + min(i + 2, L - 1) * BB, lane);
    if (f16::gj_inverse(S, col, g, j, pl) && !fail) fail = i + 1;
    // Sinv_i -> packed triangle in the workspace; C_i, D_{i+1} -> fragments
    f16::wave_sync();
    io16::put_frag(tA, g, j, S);
    io16::put(tB, lane, Cu);
    f16::wave_sync();
    const io16::Nat<T> pk = sl.gather_packed(tA);
    const Frag<T> Ct = io16::get_frag_t(tB, g, j);  // O(C_i^T)
    f16::wave_sync();
    io16::put(tA, lane, Du);
    if (keep) io16::store_packed(st + i * PB, lane, pk);
    f16::wave_sync();
    const Frag<T> Dn1 = sl.get_sym(tA);
    const Frag<T> Y = f16::mm<T>(S, Ct, f16::zero<T>());  // Sinv_i C_i^T
    S = Dn1 - f16::mm<T>(Ct, Y, f16::zero<T>());          // D_{i+1} - C_i Sinv_i C_i^T
  };
  int i = 0;
  for (; i + 1 < L - 1; i += 2) {
    collect(i, C0, D0, C1, D1);
    collect(i + 1, C1, D1, C0, D0);
  }
  if (i < L - 1) collect(i, C0, D0, C1, D1);
  if (f16::gj_inverse(S, col, g, j, pl) && !fail) fail = L;  // the root block
  if constexpr (kFactor) {
    if (st) {
      f16::wave_sync();
      io16::put_frag(tA, g, j, S);
      f16::wave_sync();
      io16::store_packed(st + (L - 1) * PB, lane, sl.gather_packed(tA));
    }
    if (lane == 0) {
      logdet[m] = fail ? __builtin_nan("") : pl.log();
      if (info) info[m] = fail;
    }
    return;
  }
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
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
  const double ld = pl.log();
  Frag<T> G = S;  // G_{L-1,L-1} = Sinv_{L-1}
  f16::wave_sync();
  io16::put_frag(tA, g, j, G);
  f16::wave_sync();
  io16::store(Gd + (L - 1) * BB, lane, io16::get(tA, lane));
  // Distribute, with the packed Sinv and C of the next block in flight (same
  // alternating register sets).
  io16::Nat<T> S0 = io16::load_packed(st + lc * PB, lane), S1;
  C0 = io16::load(C + lc * BB, lane);
  auto distribute = [&](int i, const io16::Nat<T> &Sp, const io16::Nat<T> &Cu, io16::Nat<T> &Sn,
                        io16::Nat<T> &Cn) {
    const int in = max(i - 1, 0);
    Sn = io16::load_packed(st + in * PB, lane);
    Cn = io16::load(C + in * BB, lane);
    f16::wave_sync();
    io16::put_packed(tP, lane, Sp);
    io16::put(tB, lane, Cu);
    f16::wave_sync();
    const Frag<T> Si = sl.get_packed(tP);
    const Frag<T> Ct = io16::get_frag_t(tB, g, j);        // O(C_i^T)
    const Frag<T> X = f16::mm<T>(Ct, Si, f16::zero<T>());  // C_i Sinv_i
    const Frag<T> V = f16::mm<T>(G, X, f16::zero<T>());    // G_{i+1} X
    G = f16::mm<T>(X, V, Si);                              // Sinv_i + X^T V
    f16::wave_sync();
    io16::put_frag(tA, g, j, -V);
    io16::put_frag(tB, g, j, G);
    f16::wave_sync();
    io16::store(Gl + i * BB, lane, io16::get(tA, lane));  // G_{i+1,i}
    io16::store(Gd + i * BB, lane, io16::get(tB, lane));
  };
  i = L - 2;
  for (; i >= 1; i -= 2) {
    distribute(i, S0, C0, S1, C1);
    distribute(i - 1, S1, C1, S0, C0);
  }
  if (i == 0) distribute(0, S0, C0, S1, C1);
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
  hipLaunchKernelGGL((chain16_kernel<T, false>), dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     static_cast<int>(L), diag, lower, G_diag, G_lower, logdet, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

template <typename T>
hipError_t chain16_factor_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *factor,
                                 double *logdet, int32_t *info, hipStream_t s) {
  hipLaunchKernelGGL((chain16_kernel<T, true>), dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     static_cast<int>(L), diag, lower, nullptr, nullptr, logdet, info, factor);
  return hipGetLastError();
}

template hipError_t chain16_launch<float>(int64_t, int64_t, const float *, const float *, float *,
                                          float *, double *, int32_t *, void *, hipStream_t);
template hipError_t chain16_factor_launch<float>(int64_t, int64_t, const float *, const float *,
                                                 float *, double *, int32_t *, hipStream_t);
template hipError_t chain16_factor_launch<double>(int64_t, int64_t, const double *,
                                                  const double *, double *, double *, int32_t *,
                                                  hipStream_t);
template hipError_t chain16_launch<double>(int64_t, int64_t, const double *, const double *,
                                           double *, double *, double *, int32_t *, void *,
                                           hipStream_t);

}  // namespace selinv
