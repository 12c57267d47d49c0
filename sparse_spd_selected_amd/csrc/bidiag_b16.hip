// bidiag_b16.hip -- selected inverse of block lower-bidiagonal matrices with
// 16x16 blocks: one wavefront per matrix, blocks in the MFMA 16x16 register
// layout (frag16.h), products on the matrix cores.
//
// The non-symmetric chain of the gabp-sparse-inv page ("Implemented and
// tested kernels", item Non-symmetric chain): on M's pattern
//   G_ii = M_ii^{-1},   G_{i+1,i} = -G_{i+1,i+1} M_{i+1,i} G_ii,
// fully local.  Walking i = 0 .. L-1 keeps G_{i-1,i-1} in registers, so every
// block is inverted once and every input block read once: the kernel streams
// 2 blocks in and 2 blocks out per step.  Blocks are inverted by Gauss-Jordan
// without pivoting (the page's setting, safe for block-diagonally dominant M).
// A zero or non-finite pivot sets info = 1 + the first failing block and
// every output of that matrix becomes NaN.
#include "frag16.h"
#include "internal.h"
#include "io16.h"

namespace selinv {

namespace {

using f16::Frag;

// In-place inverse of a general 16x16 block held as O(A), Gauss-Jordan
// without pivoting: pivot k (d = a_kk) maps a_ij -> a_ij - a_ik a_kj / d
// (i, j != k), a_kj -> a_kj / d, a_ik -> -a_ik / d, a_kk -> 1 / d; after the 16
// pivots the block holds A^{-1}.  Column k and row k are broadcast through 32
// entries of LDS private to the wavefront (`rc`: column k at rc[4 g + r] for
// row row(g, r), row k at rc[16 + j]).  Returns true if a pivot is zero or
// not finite.
template <typename T>
__device__ __forceinline__ bool gen_inverse16(Frag<T> &a, T *rc, int g, int j) {
  bool bad = false;
#pragma unroll 1
  for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
    for (int kr = 0; kr < 4; ++kr) {
      const int k = f16::row<T>(kq, kr);
      const bool colk = j == k, own = g == kq;
      if (colk) *reinterpret_cast<Frag<T> *>(rc + 4 * g) = a;  // A[row(g, r)][k]
      if (own) rc[16 + j] = a[kr];                             // A[k][j]
      f16::wave_sync();
      const T d = rc[16 + k];
      const Frag<T> ci = *reinterpret_cast<const Frag<T> *>(rc + 4 * g);
      const T rj = rc[16 + j];
      f16::wave_sync();
      bad |= !(d != T(0)) || !__builtin_isfinite(d);
      const T inv = f16::rcp<T>(d);
      const T sj = rj * inv;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = colk ? -ci[r] * inv : a[r] - ci[r] * sj;
      if (own) a[kr] = colk ? inv : sj;
    }
  }
  return bad;
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8)))
void bidiag16_kernel(int L, const T *__restrict__ diag, const T *__restrict__ lower,
                     T *__restrict__ G_diag, T *__restrict__ G_lower, int32_t *__restrict__ info) {
  using Tr = io16::Traits<T>;
  constexpr int BB = 256;
  __shared__ __align__(16) T rc[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * BB;
  // with L == 1 there is no lower block (lower may be null): the clamped
  // prefetch then reads a diagonal block it never uses
  const T *C = L > 1 ? lower + m * (L - 1) * BB : D;
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
  const int lc = max(L - 2, 0);
  int32_t fail = 0;
  Frag<T> Gp = f16::zero<T>();  // G_{i-1,i-1}
  // step i consumes D_i and C_{i-1} (= lower[i-1]); the next pair is loaded
  // while this one is processed, two register sets alternating
  io16::Nat<T> D0 = io16::load(D, lane), C0 = io16::load(C, lane), D1, C1;
  auto step = [&](int i, const io16::Nat<T> &Du, const io16::Nat<T> &Cu, io16::Nat<T> &Dn,
                  io16::Nat<T> &Cn) {
    Dn = io16::load(D + min(i + 1, L - 1) * BB, lane);
    Cn = io16::load(C + min(i, lc) * BB, lane);
    f16::wave_sync();
    io16::put(tA, lane, Du);
    io16::put(tB, lane, Cu);
    f16::wave_sync();
    Frag<T> A = io16::get_frag(tA, g, j);
    const Frag<T> Mt = io16::get_frag_t(tB, g, j);  // O(M_{i,i-1}^T)
    f16::wave_sync();
    if (gen_inverse16(A, rc, g, j) && !fail) fail = i + 1;
    io16::put_frag(tA, g, j, A);
    f16::wave_sync();
    io16::store(Gd + i * BB, lane, io16::get(tA, lane));
    if (i > 0) {
      const Frag<T> Gt = io16::get_frag_t(tA, g, j);             // O(G_ii^T)
      const Frag<T> X = f16::mm<T>(Mt, Gp, f16::zero<T>());      // M_{i,i-1} G_{i-1,i-1}
      const Frag<T> Y = f16::mm<T>(Gt, X, f16::zero<T>());       // G_ii X
      io16::put_frag(tB, g, j, -Y);
      f16::wave_sync();
      io16::store(Gl + (i - 1) * BB, lane, io16::get(tB, lane));
    }
    Gp = A;
  };
  int i = 0;
  for (; i + 1 < L; i += 2) {
    step(i, D0, C0, D1, C1);
    step(i + 1, D1, C1, D0, C0);
  }
  if (i < L) step(i, D0, C0, D1, C1);
  if (fail) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = lane; e < static_cast<int64_t>(L) * BB; e += 64) Gd[e] = nan;
    for (int64_t e = lane; e < static_cast<int64_t>(L - 1) * BB; e += 64) Gl[e] = nan;
  }
  if (lane == 0 && info) info[m] = fail;
}

}  // namespace

template <typename T>
hipError_t bidiag16_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                           T *G_lower, int32_t *info, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(bidiag16_kernel<T>, dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     static_cast<int>(L), diag, lower, G_diag, G_lower, info);
  return hipGetLastError();
}

template hipError_t bidiag16_launch<float>(int64_t, int64_t, const float *, const float *, float *,
                                           float *, int32_t *, hipStream_t);
template hipError_t bidiag16_launch<double>(int64_t, int64_t, const double *, const double *,
                                            double *, double *, int32_t *, hipStream_t);

}  // namespace selinv
