// rows8.h -- blocks of size b <= 8 held "one row per lane": lane l of a
// wavefront works on slot s = l / 8 (up to 8 independent blocks per
// wavefront) and holds row i = l % 8 of that slot's block in 8 registers.
// Blocks smaller than 8 are padded to 8 x 8: diagonal (SPD) blocks with the
// identity, off-diagonal blocks with zeros, so every operation below is an
// 8 x 8 one (padded pivots equal 1 and add nothing to log det).
//
// Products read the right-hand operand's rows (or columns) from LDS; each
// wavefront owns an 8 x 8 x 8 staging area per operand (`Stage`).
#pragma once

#include <hip/hip_runtime.h>

#include "frag16.h"

namespace selinv {
namespace r8 {

template <typename T>
struct Row {
  T v[8];
};

template <typename T>
__device__ __forceinline__ Row<T> zero() {
  Row<T> r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = T(0);
  return r;
}

// Row i of an 8 x 8 block stored densely (stride 8): two or four vector loads.
template <typename T>
__device__ __forceinline__ Row<T> load8(const T *P, int i) {
  Row<T> r;
  typedef T v4 __attribute__((ext_vector_type(4)));
  const v4 a = *reinterpret_cast<const v4 *>(P + i * 8);
  const v4 c = *reinterpret_cast<const v4 *>(P + i * 8 + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r.v[k] = a[k];
    r.v[4 + k] = c[k];
  }
  return r;
}

// Row i of a b x b row-major block (1 <= b <= 8; zero beyond b).  b == 8 takes vector
// loads; otherwise every lane loads from clamped in-range addresses and
// padding is selected afterwards (no divergent loads).
template <typename T>
__device__ __forceinline__ Row<T> load(const T *P, int b, int i) {
  if (b == 8) return load8(P, i);
  Row<T> r;
  const int ic = min(i, b - 1);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const T x = P[ic * b + min(k, b - 1)];
    r.v[k] = (i < b && k < b) ? x : T(0);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void store8(T *P, int i, const Row<T> &r) {
  typedef T v4 __attribute__((ext_vector_type(4)));
  v4 a, c;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = r.v[k];
    c[k] = r.v[4 + k];
  }
  *reinterpret_cast<v4 *>(P + i * 8) = a;
  *reinterpret_cast<v4 *>(P + i * 8 + 4) = c;
}

// Row i of a symmetric b x b block read from its lower triangle, identity
// padded beyond b (clamped in-range addresses, padding selected afterwards).
template <typename T>
__device__ __forceinline__ Row<T> load_sym(const T *P, int b, int i) {
  Row<T> r;
  const int ic = min(i, b - 1);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int kc = min(k, b - 1);
    const T x = P[k <= i ? ic * b + kc : kc * b + ic];
    r.v[k] = (i < b && k < b) ? x : ((k == i) ? T(1) : T(0));
  }
  return r;
}

// Store the first b entries of row i (rows i >= b are padding: skipped).
template <typename T>
__device__ __forceinline__ void store(T *P, int b, int i, const Row<T> &r) {
  if (b == 8) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 a, c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = r.v[k];
      c[k] = r.v[4 + k];
    }
    *reinterpret_cast<v4 *>(P + i * 8) = a;
    *reinterpret_cast<v4 *>(P + i * 8 + 4) = c;
    return;
  }
  if (i >= b) return;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < b) P[i * b + k] = r.v[k];
}

template <typename T>
__device__ __forceinline__ Row<T> neg(Row<T> r) {
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = -r.v[k];
  return r;
}

// Per-wavefront LDS area holding one 8 x 8 block per slot (rows contiguous).
template <typename T>
struct Stage {
  T *base;  // 8 slots x 64 entries
  __device__ __forceinline__ void put(int s, int i, const Row<T> &r) const {
    store8(base + s * 64, i, r);
  }
  __device__ __forceinline__ Row<T> row(int s, int k) const { return load8(base + s * 64, k); }
  __device__ __forceinline__ T at(int s, int k, int c) const { return base[s * 64 + k * 8 + c]; }
};

// out_i = a_i B  (row i of A B), B staged in `sb` (wave_sync between put and use)
template <typename T>
__device__ __forceinline__ Row<T> mul(const Row<T> &a, const Stage<T> &sb, int s, Row<T> acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const Row<T> bk = sb.row(s, k);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc.v[c] += a.v[k] * bk.v[c];
  }
  return acc;
}

// out_i = a_i B^T: entry c is the dot product of a_i with row c of B
template <typename T>
__device__ __forceinline__ Row<T> mul_t(const Row<T> &a, const Stage<T> &sb, int s, Row<T> acc) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const Row<T> bc = sb.row(s, c);
    T d = T(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) d += a.v[k] * bc.v[k];
    acc.v[c] += d;
  }
  return acc;
}

// out_i = (A^T B)_i = sum_k A[k][i] B[k][:], A and B staged
template <typename T>
__device__ __forceinline__ Row<T> mul_tn(const Stage<T> &sa, const Stage<T> &sb, int s, int i,
                                         Row<T> acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const T aki = sa.at(s, k, i);
    const Row<T> bk = sb.row(s, k);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc.v[c] += aki * bk.v[c];
  }
  return acc;
}

// In-place inverse of the SPD 8 x 8 block of each slot (row i per lane) by the
// symmetric Gauss-Jordan sweep without pivoting (see frag16.h): pivot k maps
// a_ij -> a_ij - a_ik a_kj / d (i, j != k), a_ik -> a_ik / d, a_kk -> -1/d; the
// sign is flipped at the end.  Row k is broadcast through `st` (slot s, row
// k).  Returns true if a pivot of this lane's slot is not > 0; `pl` receives
// the product of the slot's pivots.
template <typename T>
__device__ __forceinline__ bool gj_inverse(Row<T> &a, const Stage<T> &st, int s, int i,
                                           f16::PivotLog &pl) {
  bool bad = false;
  double dq[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (i == k) st.put(s, k, a);
    f16::wave_sync();
    const Row<T> rk = st.row(s, k);
    f16::wave_sync();
    const T d = rk.v[k];
    bad |= !(d > T(0));
    dq[k & 3] = static_cast<double>(d);
    if ((k & 3) == 3) pl.mul4(dq[0], dq[1], dq[2], dq[3]);
    const T inv = f16::rcp<T>(d);
    const bool pivot_row = i == k;
    // u_i = a_ik (or -1 on the pivot row); w_c = a_kc (or -1 at c = k)
    const T si = (pivot_row ? T(-1) : a.v[k]) * inv;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const T wc = c == k ? T(-1) : rk.v[c];
      const T base = (pivot_row || c == k) ? T(0) : a.v[c];
      a.v[c] = base - si * wc;
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) a.v[c] = -a.v[c];
  return bad;
}

// U with U U^T = A and a positive diagonal, U upper triangular, for the
// symmetric positive definite b x b block A of each slot (row i per lane;
// rows and columns from b on are left zero): the Cholesky factorisation in
// reversed index order, k = b-1 .. 0, each step taking u_kk = sqrt(a_kk),
// u_ik = a_ik / u_kk (i < k) and a_ij -= u_ik u_jk (i, j < k).  Row k is
// broadcast through `st`.  For A = S^-1 with S = R R^T, U = R^-T.
template <typename T>
__device__ __forceinline__ Row<T> rev_cholesky(Row<T> a, const Stage<T> &st, int s, int i, int b) {
  Row<T> u = zero<T>();
#pragma unroll
  for (int k = 7; k >= 0; --k) {
    if (k < b) {
      if (i == k) st.put(s, k, a);
      f16::wave_sync();
      const Row<T> rk = st.row(s, k);
      f16::wave_sync();
      const T d = __builtin_sqrt(rk.v[k]);
      const T inv = f16::rcp<T>(d);
      const T uk = i == k ? d : (i < k ? a.v[k] * inv : T(0));  // u_ik
      u.v[k] = uk;
      const T f = uk * inv;
#pragma unroll
      for (int j = 0; j < k; ++j) a.v[j] -= f * rk.v[j];  // u_ik u_jk, u_jk = a_kj / d
    }
  }
  return u;
}

}  // namespace r8
}  // namespace selinv
