// block_wg.h -- b x b block algebra shared by all threads of one workgroup,
// blocks held in LDS (row-major).  Used by the kernels for any b <= 32; the
// specialised kernels keep their blocks in registers instead.
//
// Every function starts from synchronised LDS and ends with __syncthreads(),
// so calls can be chained without extra barriers.
//
// With b = 32 and 256 threads the products run on the matrix cores: each of
// the four wavefronts forms one 16 x 16 quadrant of the result with eight
// 16x16x4 MFMA steps, reading its operands straight from the row-major
// blocks (frag16.h gives the operand and result layouts), and the SPD inverse
// is the register-resident blocked Gauss-Jordan of frag32.h on one wavefront.
#pragma once

#include <hip/hip_runtime.h>

#include "frag32.h"

namespace selinv {
namespace wg {

__device__ inline int tid() { return threadIdx.x; }
__device__ inline int nthreads() { return blockDim.x; }

// the b = 32 matrix-core path applies
__device__ inline bool mfma32(int b) { return b == 32 && blockDim.x == 256; }

// Quadrant (I, J) of op(A) op(B) for 32 x 32 row-major A, B (op = transpose
// when TA / TB), in the MFMA result layout: lane (g, j) register r holds
// entry (16 I + row(g, r), 16 J + j).  Step s of the 16x16x4 product takes
// lane l's A operand op(A)[16 I + l % 16][4 s + l / 16] and its B operand
// op(B)[4 s + l / 16][16 J + l % 16].
template <typename T, bool TA, bool TB>
__device__ __forceinline__ f16::Frag<T> quad32(const T *A, const T *B, int I, int J, int lane) {
  const int i = lane & 15, kk = lane >> 4, r = 16 * I + i, c = 16 * J + i;
  f16::Frag<T> acc = f16::zero<T>();
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int k = 4 * s + kk;
    const T a = TA ? A[k * 32 + r] : A[r * 32 + k];
    const T x = TB ? B[c * 32 + k] : B[k * 32 + c];
    acc = f16::Mfma<T>::op(a, x, acc);
  }
  return acc;
}

template <typename T>
__device__ inline T qnan() {
  return __builtin_nan("");
}
template <>
__device__ inline float qnan<float>() {
  return __builtin_nanf("");
}

// dst = src (b*b entries); either side may be global or LDS
template <typename T>
__device__ inline void copy(T *dst, const T *src, int bb) {
  for (int e = tid(); e < bb; e += nthreads()) dst[e] = src[e];
  __syncthreads();
}

// dst = sign * src
template <typename T>
__device__ inline void copy_scaled(T *dst, const T *src, int bb, T sign) {
  for (int e = tid(); e < bb; e += nthreads()) dst[e] = sign * src[e];
  __syncthreads();
}

// dst = symmetric block from the LOWER triangle of src (mirrored)
template <typename T>
__device__ inline void load_sym_lower(T *dst, const T *src, int b) {
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    dst[e] = r >= c ? src[r * b + c] : src[c * b + r];
  }
  __syncthreads();
}

template <typename T>
__device__ inline void fill(T *dst, int bb, T v) {
  for (int e = tid(); e < bb; e += nthreads()) dst[e] = v;
  __syncthreads();
}

// Out = op(A) op(B), op = transpose when TA/TB.  Out must not alias A or B.
template <typename T, bool TA, bool TB>
__device__ inline void gemm(T *Out, const T *A, const T *B, int b) {
  if (mfma32(b)) {
    const int w = tid() >> 6, lane = tid() & 63, I = w >> 1, J = w & 1;
    const f16::Frag<T> p = quad32<T, TA, TB>(A, B, I, J, lane);
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) Out[(16 * I + f16::row<T>(g, r)) * 32 + 16 * J + j] = p[r];
    __syncthreads();
    return;
  }
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    T acc = T(0);
    for (int k = 0; k < b; ++k) {
      const T a = TA ? A[k * b + r] : A[r * b + k];
      const T x = TB ? B[c * b + k] : B[k * b + c];
      acc += a * x;
    }
    Out[e] = acc;
  }
  __syncthreads();
}

// Out = Base + sign * op(A) op(B), computed on the lower triangle and
// mirrored, so Out is exactly symmetric (for products that are symmetric in
// exact arithmetic).  Base may be null (taken as 0) and may alias Out.
template <typename T, bool TA, bool TB>
__device__ inline void gemm_sym(T *Out, const T *Base, const T *A, const T *B, int b, T sign) {
  if (mfma32(b)) {  // quadrants on and below the diagonal
    const int w = tid() >> 6, lane = tid() & 63, I = w >> 1, J = w & 1;
    if (I >= J) {
      const f16::Frag<T> p = quad32<T, TA, TB>(A, B, I, J, lane);
      const int g = lane >> 4, j = lane & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * I + f16::row<T>(g, q), c = 16 * J + j;
        if (r < c) continue;
        const T v = (Base ? Base[r * 32 + c] : T(0)) + sign * p[q];
        Out[r * 32 + c] = v;
        Out[c * 32 + r] = v;
      }
    }
    __syncthreads();
    return;
  }
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    if (r < c) continue;
    T acc = T(0);
    for (int k = 0; k < b; ++k) {
      const T a = TA ? A[k * b + r] : A[r * b + k];
      const T x = TB ? B[c * b + k] : B[k * b + c];
      acc += a * x;
    }
    const T v = (Base ? Base[r * b + c] : T(0)) + sign * acc;
    Out[r * b + c] = v;
    Out[c * b + r] = v;
  }
  __syncthreads();
}

// dst = (src + src^T) / 2; dst must not alias src
template <typename T>
__device__ inline void sym_part(T *dst, const T *src, int b) {
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    dst[e] = T(0.5) * (src[r * b + c] + src[c * b + r]);
  }
  __syncthreads();
}

// Out = beta * Base + alpha * op(A) op(B), every entry.  Base may alias Out;
// Out must not alias A or B.
template <typename T, bool TA, bool TB>
__device__ inline void gemm_axpby(T *Out, T beta, const T *Base, T alpha, const T *A, const T *B,
                                  int b) {
  if (mfma32(b)) {
    const int w = tid() >> 6, lane = tid() & 63, I = w >> 1, J = w & 1;
    const f16::Frag<T> p = quad32<T, TA, TB>(A, B, I, J, lane);
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = (16 * I + f16::row<T>(g, q)) * 32 + 16 * J + j;
      Out[e] = beta * Base[e] + alpha * p[q];
    }
    __syncthreads();
    return;
  }
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    T acc = T(0);
    for (int k = 0; k < b; ++k) {
      const T a = TA ? A[k * b + r] : A[r * b + k];
      const T x = TB ? B[c * b + k] : B[k * b + c];
      acc += a * x;
    }
    Out[e] = beta * Base[e] + alpha * acc;
  }
  __syncthreads();
}

// Out = Base + sign * (P + P^T) / 2 with P = op(A) op(B): the symmetric part
// of a product that is not symmetric by itself, exactly symmetric.  Base
// (symmetric; only its lower triangle is read) may be null or alias Out.
template <typename T, bool TA, bool TB>
__device__ inline void gemm_symmetrized(T *Out, const T *Base, const T *A, const T *B, int b,
                                        T sign) {
  if (mfma32(b)) {
    // quadrant (I, J) of P and of P^T = op(B)^T op(A)^T, on and below the diagonal
    const int w = tid() >> 6, lane = tid() & 63, I = w >> 1, J = w & 1;
    if (I >= J) {
      const f16::Frag<T> p = quad32<T, TA, TB>(A, B, I, J, lane);
      const f16::Frag<T> pt = quad32<T, !TB, !TA>(B, A, I, J, lane);
      const int g = lane >> 4, j = lane & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * I + f16::row<T>(g, q), c = 16 * J + j;
        if (r < c) continue;
        const T v = (Base ? Base[r * 32 + c] : T(0)) + sign * (T(0.5) * (p[q] + pt[q]));
        Out[r * 32 + c] = v;
        Out[c * 32 + r] = v;
      }
    }
    __syncthreads();
    return;
  }
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    if (r < c) continue;
    T prc = T(0), pcr = T(0);
    for (int k = 0; k < b; ++k) {
      prc += (TA ? A[k * b + r] : A[r * b + k]) * (TB ? B[c * b + k] : B[k * b + c]);
      pcr += (TA ? A[k * b + c] : A[c * b + k]) * (TB ? B[r * b + k] : B[k * b + r]);
    }
    const T v = (Base ? Base[r * b + c] : T(0)) + sign * (T(0.5) * (prc + pcr));
    Out[r * b + c] = v;
    Out[c * b + r] = v;
  }
  __syncthreads();
}

// Packed lower triangle of a symmetric block: entry (r, c), r >= c, at
// r (r + 1) / 2 + c.  packed_entries(b) rounds the count up to a multiple of
// four elements so that consecutive packed blocks stay 16-byte aligned.
__host__ __device__ inline int packed_entries(int b) { return (b * (b + 1) / 2 + 3) / 4 * 4; }

// dst = packed lower triangle of the symmetric block src (read from its
// lower triangle)
template <typename T>
__device__ inline void pack_lower(T *dst, const T *src, int b) {
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    if (r >= c) dst[r * (r + 1) / 2 + c] = src[r * b + c];
  }
  __syncthreads();
}

// dst = the full symmetric block of a packed lower triangle
template <typename T>
__device__ inline void unpack_sym(T *dst, const T *src, int b) {
  for (int e = tid(); e < b * b; e += nthreads()) {
    const int r = e / b, c = e % b;
    dst[e] = r >= c ? src[r * (r + 1) / 2 + c] : src[c * (c + 1) / 2 + r];
  }
  __syncthreads();
}

// Block times a block of vectors: Out (b x kc, row stride ldo) =
// beta * Base + alpha * op(A) V, A b x b, V b x kc with row stride ldv, Base
// with row stride ldo (may alias Out; null = 0).  Out must not alias A or V.
template <typename T, bool TA>
__device__ inline void bmv(T *Out, int ldo, T beta, const T *Base, T alpha, const T *A,
                           const T *V, int ldv, int b, int kc) {
  for (int e = tid(); e < b * kc; e += nthreads()) {
    const int r = e / kc, c = e % kc;
    T acc = T(0);
    for (int t = 0; t < b; ++t) acc += (TA ? A[t * b + r] : A[r * b + t]) * V[t * ldv + c];
    Out[r * ldo + c] = (Base ? beta * Base[r * ldo + c] : T(0)) + alpha * acc;
  }
  __syncthreads();
}

// U = the upper triangular factor of a symmetric positive definite block S
// with U U^T = S and a positive diagonal (Cholesky in reversed index order:
// columns j = b-1 .. 0, each from the columns to its right).  U is written in
// full, zeros below the diagonal.  For S = A^{-1} with A = R R^T (R lower
// triangular), U = R^{-T}.
template <typename T>
__device__ inline void rev_cholesky(T *U, const T *S, int b) {
  for (int e = tid(); e < b * b; e += nthreads()) U[e] = T(0);
  __syncthreads();
  for (int j = b - 1; j >= 0; --j) {
    if (tid() == 0) {
      T d = S[j * b + j];
      for (int t = j + 1; t < b; ++t) d -= U[j * b + t] * U[j * b + t];
      U[j * b + j] = sqrt(d);
    }
    __syncthreads();
    const T ujj = U[j * b + j];
    for (int i = tid(); i < j; i += nthreads()) {
      T s = S[i * b + j];
      for (int t = j + 1; t < b; ++t) s -= U[i * b + t] * U[j * b + t];
      U[i * b + j] = s / ujj;
    }
    __syncthreads();
  }
}

// In-place inverse of a general block by Gauss-Jordan elimination without
// pivoting: pivot k maps a_kk -> 1/d, a_kj -> a_kj / d and a_ik -> -a_ik / d
// (i, j != k), a_ij -> a_ij - a_ik a_kj / d, with d = a_kk.  `rowk`, `colk`
// are LDS scratch of b entries.  Returns 1 (uniformly across the workgroup)
// if a pivot is zero or not finite; then A holds garbage.
template <typename T>
__device__ inline int gen_inverse(T *A, int b, T *rowk, T *colk) {
  for (int k = 0; k < b; ++k) {
    const T d = A[k * b + k];
    if (d == T(0) || !__builtin_isfinite(d)) return 1;
    if (tid() < b) {
      rowk[tid()] = A[k * b + tid()];
      colk[tid()] = A[tid() * b + k];
    }
    __syncthreads();
    const T inv = T(1) / d;
    for (int e = tid(); e < b * b; e += nthreads()) {
      const int i = e / b, j = e % b;
      T a;
      if (i == k && j == k)
        a = inv;
      else if (i == k)
        a = rowk[j] * inv;
      else if (j == k)
        a = -colk[i] * inv;
      else
        a = A[e] - colk[i] * (rowk[j] * inv);
      A[e] = a;
    }
    __syncthreads();
  }
  return 0;
}

// In-place inverse of a symmetric positive definite block by the symmetric
// Gauss-Jordan sweep, without pivoting.  Sweeping pivot k maps
//   a_ij -> a_ij - a_ik a_kj / d   (i, j != k),   a_ik -> a_ik / d,
//   a_kk -> -1/d,   with d = a_kk,
// so that sweeping every pivot leaves -A^{-1}; the sign is flipped at the end.
// Each pivot d is the diagonal of the current Schur complement (the D of an
// LDL^T factorisation), so A is positive definite iff every d > 0 and
// ln det A = sum_k ln d.  `col` is LDS scratch of b entries.
// Returns 0, or 1 (uniformly across the workgroup) if a pivot is not > 0 or
// is NaN; then A holds garbage.  *logdet receives sum ln d (float64).
template <typename T>
__device__ inline int spd_inverse(T *A, int b, T *col, double *logdet) {
  if (mfma32(b)) {  // one wavefront, blocked Gauss-Jordan in registers (frag32.h)
    __shared__ int s_bad;
    __shared__ double s_ld;
    if (tid() < 64) {
      const int lane = tid(), g = lane >> 4, j = lane & 15;
      f32t::Blk<T> a = f32t::load(A, g, j);
      f16::PivotLog pl;
      const bool bad = f32t::gj_inverse(a, col, g, j, pl);
      f32t::store(A, a, g, j);
      if (lane == 0) {
        s_bad = bad ? 1 : 0;
        s_ld = pl.log();
      }
    }
    __syncthreads();
    *logdet = s_ld;
    const int bad = s_bad;
    __syncthreads();
    return bad;
  }
  double ld = 0.0;
  for (int k = 0; k < b; ++k) {
    const T d = A[k * b + k];
    if (!(d > T(0))) return 1;
    ld += log(static_cast<double>(d));
    if (tid() < b) col[tid()] = tid() == k ? T(-1) : A[tid() * b + k];
    __syncthreads();
    const T inv = T(1) / d;
    for (int e = tid(); e < b * b; e += nthreads()) {
      const int i = e / b, j = e % b;
      const T a = (i == k || j == k) ? T(0) : A[e];
      A[e] = a - (col[i] * col[j]) * inv;
    }
    __syncthreads();
  }
  for (int e = tid(); e < b * b; e += nthreads()) A[e] = -A[e];
  __syncthreads();
  *logdet = ld;
  return 0;
}

}  // namespace wg
}  // namespace selinv
