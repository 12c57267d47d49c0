// frag16.h -- 16x16 blocks held by one wavefront in the register layout of
// the CDNA MFMA 16x16x4 result, and block products on the matrix cores.
//
// Layout "O(P)": lane l = 16 g + j (g = l / 16, j = l % 16) holds, in
// element r = 0..3, P[row(g, r)][j].  This is the accumulator layout of the
// 16x16x4 MFMA: for v_mfma_f32_16x16x4f32 row(g, r) = 4 g + r, for
// v_mfma_f64_16x16x4f64 row(g, r) = 4 r + g (measured on gfx950).  In both,
// lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16].
//
// A 16x16x16 product is four 16x16x4 steps.  The contraction index of step s
// in lane group g is taken as k = row(g, s).  Then the B operand of step s is
// element s of O(B) and the A operand is element s of O(A^T): no data
// movement is needed when the left factor is available as O(A^T).  So
//     O(A B) = mm(O(A^T), O(B)).
// For symmetric A, O(A^T) = O(A); loading a row-major block "transposed"
// (lane (g, x) reads P[x][row(g, r)]) yields O(P^T).
#pragma once

#include <hip/hip_runtime.h>

namespace selinv {
namespace f16 {

template <typename T>
struct Mfma;

template <>
struct Mfma<double> {
  typedef double v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 op(double a, double b, v4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static constexpr __device__ __forceinline__ int row(int g, int r) { return 4 * r + g; }
  // position of row i inside a lane group's 4 contiguous LDS entries
  static constexpr __device__ __forceinline__ int pos(int i) { return 4 * (i & 3) + (i >> 2); }
  static constexpr bool kRowContiguous = false;
};

template <>
struct Mfma<float> {
  typedef float v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 op(float a, float b, v4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static constexpr __device__ __forceinline__ int row(int g, int r) { return 4 * g + r; }
  static constexpr __device__ __forceinline__ int pos(int i) { return i; }
  static constexpr bool kRowContiguous = true;
};

template <typename T>
using Frag = typename Mfma<T>::v4;

template <typename T>
__device__ __forceinline__ Frag<T> zero() {
  Frag<T> z = {T(0), T(0), T(0), T(0)};
  return z;
}

// O(A B) + acc from O(A^T) and O(B)
template <typename T>
__device__ __forceinline__ Frag<T> mm(Frag<T> At, Frag<T> Bf, Frag<T> acc) {
  acc = Mfma<T>::op(At[0], Bf[0], acc);
  acc = Mfma<T>::op(At[1], Bf[1], acc);
  acc = Mfma<T>::op(At[2], Bf[2], acc);
  acc = Mfma<T>::op(At[3], Bf[3], acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ int row(int g, int r) {
  return Mfma<T>::row(g, r);
}

// O(P^T) of a row-major block with leading dimension ld (one vector load
// when the layout's rows are contiguous per lane group)
template <typename T>
__device__ __forceinline__ Frag<T> load_t(const T *P, int ld, int g, int x) {
  if constexpr (Mfma<T>::kRowContiguous) {
    return *reinterpret_cast<const Frag<T> *>(P + x * ld + 4 * g);
  } else {
    Frag<T> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = P[x * ld + row<T>(g, r)];
    return f;
  }
}

// O(P) of a symmetric block, reading only its lower triangle
template <typename T>
__device__ __forceinline__ Frag<T> load_sym(const T *P, int ld, int g, int j) {
  Frag<T> f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = row<T>(g, r);
    f[r] = i >= j ? P[i * ld + j] : P[j * ld + i];
  }
  return f;
}

// Lane offsets of a symmetric block read from its lower triangle: element r
// of lane (g, j) is P[off[r]] (row-major, leading dimension ld).
template <typename T>
struct SymOffsets {
  int off[4];
  __device__ __forceinline__ SymOffsets(int ld, int g, int j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = row<T>(g, r);
      off[r] = i >= j ? i * ld + j : j * ld + i;
    }
  }
  __device__ __forceinline__ Frag<T> load(const T *P) const {
    Frag<T> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = P[off[r]];
    return f;
  }
};

// Packed lower triangle of a symmetric 16x16 block (136 entries, row i at
// offset i (i + 1) / 2): the element of lane (g, j) register r sits at
// off[r]; lanes whose element is in the upper triangle do not store it.
constexpr int kPacked16 = 136;
template <typename T>
struct PackedOffsets {
  int off[4];
  unsigned lower_mask;  // bit r: element r lies on or below the diagonal
  __device__ __forceinline__ PackedOffsets(int g, int j) : lower_mask(0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = row<T>(g, r);
      const int a = i >= j ? i : j, b = i >= j ? j : i;
      off[r] = a * (a + 1) / 2 + b;
      if (i >= j) lower_mask |= 1u << r;
    }
  }
  __device__ __forceinline__ Frag<T> load(const T *P) const {
    Frag<T> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = P[off[r]];
    return f;
  }
  __device__ __forceinline__ void store(T *P, Frag<T> f) const {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lower_mask & (1u << r)) P[off[r]] = f[r];
  }
};

// O(P) row-major store
template <typename T>
__device__ __forceinline__ void store(T *P, int ld, Frag<T> f, int g, int j) {
#pragma unroll
  for (int r = 0; r < 4; ++r) P[row<T>(g, r) * ld + j] = f[r];
}

// store of O(P) as P^T; equals a plain store when P is symmetric.
// store_t followed by load_t returns the same fragment.
template <typename T>
__device__ __forceinline__ void store_t(T *P, int ld, Frag<T> f, int g, int j) {
  if constexpr (Mfma<T>::kRowContiguous) {
    *reinterpret_cast<Frag<T> *>(P + j * ld + 4 * g) = f;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) P[j * ld + row<T>(g, r)] = f[r];
  }
}

// Orders LDS accesses between the lanes of one wavefront (a wavefront
// executes its LDS instructions in order, so a compiler-level barrier with
// wavefront-scope fences is enough; no workgroup barrier is involved, so
// wavefronts of one workgroup may call it different numbers of times).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T rcp(T d);

// 1/d: hardware estimate plus two Newton steps (error ~1 ulp)
template <>
__device__ __forceinline__ double rcp<double>(double d) {
  double x = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, x, 1.0);
  x = __builtin_fma(x, e, x);
  e = __builtin_fma(-d, x, 1.0);
  return __builtin_fma(x, e, x);
}

template <>
__device__ __forceinline__ float rcp<float>(float d) {
  float x = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, x, 1.0f);
  return __builtin_fmaf(x, e, x);
}

// 1/sqrt(d) for d > 0: the hardware estimate refined by Newton-Raphson steps
// for the reciprocal square root, y <- y (3/2 - (d/2) y^2), each of which
// doubles the correct bits (two steps for double, one for float).
template <typename T>
__device__ __forceinline__ T rsqrt(T d);

template <>
__device__ __forceinline__ double rsqrt<double>(double d) {
  double y = __builtin_amdgcn_rsq(d);
  const double h = 0.5 * d;
  y = y * __builtin_fma(-h * y, y, 1.5);
  return y * __builtin_fma(-h * y, y, 1.5);
}

template <>
__device__ __forceinline__ float rsqrt<float>(float d) {
  const float y = __builtin_amdgcn_rsqf(d);
  return y * __builtin_fmaf(-0.5f * d * y, y, 1.5f);
}

// Running product of pivots kept as mantissa * 2^exponent.  Pivots are
// multiplied in groups of four and renormalised once per group, so any four
// consecutive pivots with magnitudes in [2^-255, 2^255] are safe; ln of the
// product is taken once per block.
struct PivotLog {
  double mant = 1.0;
  int expo = 0;
  __device__ __forceinline__ void mul4(double d0, double d1, double d2, double d3) {
    int e;
    mant = frexp(mant * ((d0 * d1) * (d2 * d3)), &e);
    expo += e;
  }
  __device__ __forceinline__ double log() const {
    return ::log(mant) + expo * 0.69314718055994530941723212145818;
  }
};

// In-place inverse of a symmetric positive definite 16x16 block held as
// O(A), by the symmetric Gauss-Jordan sweep without pivoting: sweeping
// pivot k maps a_ij -> a_ij - a_ik a_kj / d (i, j != k), a_ik -> a_ik / d,
// a_kk -> -1 / d with d = a_kk; after all 16 pivots the block holds -A^{-1}
// and the sign is flipped.  The pivots are the diagonal of the Schur
// complements (the D of LDL^T): A is positive definite iff all are > 0, and
// their product is det A.  Column k is broadcast through 16 entries of LDS
// (`col`, private to this wavefront): the lanes holding column k store their
// four entries contiguously at col[4 g ..], so row i sits at col[pos(i)].
// Returns true if some pivot is not > 0.
template <typename T>
__device__ __forceinline__ bool gj_inverse(Frag<T> &a, T *col, int g, int j, PivotLog &pl) {
  bool bad = false;
  const int pj = Mfma<T>::pos(j);
#pragma unroll 1
  for (int kq = 0; kq < 4; ++kq) {
    double dq[4];
    const bool own = g == kq;  // this lane group holds the quad's pivot rows
#pragma unroll
    for (int kr = 0; kr < 4; ++kr) {
      // pivot k = row(kq, kr): the element of lane group kq, register kr
      const int k = Mfma<T>::row(kq, kr);
      const bool colk = j == k;  // this lane holds column k
      if (colk) {  // broadcast column k, then clear it (its new value is u_i u_k / d)
        *reinterpret_cast<Frag<T> *>(col + 4 * g) = a;
        a = zero<T>();
      }
      wave_sync();
      const T d = col[4 * kq + kr];
      const Frag<T> ci = *reinterpret_cast<const Frag<T> *>(col + 4 * g);
      const T cj = col[pj];
      wave_sync();
      bad |= !(d > T(0));
      dq[kr] = static_cast<double>(d);
      const T inv = rcp<T>(d);
      const T sj = (colk ? T(-1) : cj) * inv;  // u_j / d
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] -= ci[r] * sj;
      if (own) a[kr] = sj;  // row k: u_k = -1 on a cleared entry gives u_j / d
    }
    pl.mul4(dq[0], dq[1], dq[2], dq[3]);
  }
  a = -a;
  return bad;
}

}  // namespace f16
}  // namespace selinv
