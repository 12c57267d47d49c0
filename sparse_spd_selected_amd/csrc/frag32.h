// frag32.h -- 32x32 blocks held by one wavefront as 2 x 2 tiles of the
// 16x16 MFMA accumulator layout of frag16.h (16 entries per lane), with
// block products on the matrix cores and a register-resident Gauss-Jordan
// inverse.
//
// Tile (I, J) of "O32(P)" is O(P_IJ), P_IJ = P[16I .. 16I+15][16J .. 16J+15].
// Products: O32(A B) tile (I, J) = sum_K mm(O(A^T) tile (K, I), O(B) tile (K, J)),
// i.e. O32(A B) = mm32(O32(A^T), O32(B)) exactly as for 16x16 blocks.
#pragma once

#include "frag16.h"

namespace selinv {
namespace f32t {

using f16::Frag;
using f16::Mfma;
using f16::row;

template <typename T>
struct Blk {
  Frag<T> t[2][2];
};

template <typename T>
__device__ __forceinline__ Blk<T> zero() {
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) b.t[I][J] = f16::zero<T>();
  return b;
}

// O32(A B) + acc from O32(A^T) and O32(B)
template <typename T>
__device__ __forceinline__ Blk<T> mm(const Blk<T> &At, const Blk<T> &Bf, Blk<T> acc) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) {
      acc.t[I][J] = f16::mm<T>(At.t[0][I], Bf.t[0][J], acc.t[I][J]);
      acc.t[I][J] = f16::mm<T>(At.t[1][I], Bf.t[1][J], acc.t[I][J]);
    }
  return acc;
}

// Symmetric variant: only the tiles on and below the diagonal are formed and
// the upper tile is taken as the transpose of the lower one's layout-twin,
// which is valid when the exact product is symmetric.  The (0,1) tile is
// returned as the (1,0) tile's layout transposition is not available in
// registers, so it is computed too but with the cheaper of the two
// contractions shared; callers that only store the lower triangle can skip it.
template <typename T>
__device__ __forceinline__ Blk<T> mm_lower(const Blk<T> &At, const Blk<T> &Bf, Blk<T> acc) {
  acc.t[0][0] = f16::mm<T>(At.t[0][0], Bf.t[0][0], acc.t[0][0]);
  acc.t[0][0] = f16::mm<T>(At.t[1][0], Bf.t[1][0], acc.t[0][0]);
  acc.t[1][0] = f16::mm<T>(At.t[0][1], Bf.t[0][0], acc.t[1][0]);
  acc.t[1][0] = f16::mm<T>(At.t[1][1], Bf.t[1][0], acc.t[1][0]);
  acc.t[1][1] = f16::mm<T>(At.t[0][1], Bf.t[0][1], acc.t[1][1]);
  acc.t[1][1] = f16::mm<T>(At.t[1][1], Bf.t[1][1], acc.t[1][1]);
  return acc;
}

// The other symmetric variant: tiles (0,0), (0,1) and (1,1) are formed and
// (1,0) is left as acc.t[1][0] (for consumers such as the blocked inverse
// below, which reads the upper off-diagonal tile only).
template <typename T>
__device__ __forceinline__ Blk<T> mm_upper(const Blk<T> &At, const Blk<T> &Bf, Blk<T> acc) {
  acc.t[0][0] = f16::mm<T>(At.t[0][0], Bf.t[0][0], acc.t[0][0]);
  acc.t[0][0] = f16::mm<T>(At.t[1][0], Bf.t[1][0], acc.t[0][0]);
  acc.t[0][1] = f16::mm<T>(At.t[0][0], Bf.t[0][1], acc.t[0][1]);
  acc.t[0][1] = f16::mm<T>(At.t[1][0], Bf.t[1][1], acc.t[0][1]);
  acc.t[1][1] = f16::mm<T>(At.t[0][1], Bf.t[0][1], acc.t[1][1]);
  acc.t[1][1] = f16::mm<T>(At.t[1][1], Bf.t[1][1], acc.t[1][1]);
  return acc;
}

// O32(P^T) of a row-major 32x32 block
template <typename T>
__device__ __forceinline__ Blk<T> load_t(const T *P, int g, int x) {
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) b.t[I][J] = f16::load_t(P + 16 * J * 32 + 16 * I, 32, g, x);
  return b;
}

// O32(P) of a row-major 32x32 block
template <typename T>
__device__ __forceinline__ Blk<T> load(const T *P, int g, int j) {
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.t[I][J][r] = P[(16 * I + row<T>(g, r)) * 32 + 16 * J + j];
  return b;
}

template <typename T>
__device__ __forceinline__ void store(T *P, const Blk<T> &b, int g, int j) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) f16::store(P + 16 * I * 32 + 16 * J, 32, b.t[I][J], g, j);
}

// store of O32(P) as P^T (a plain store when P is symmetric)
template <typename T>
__device__ __forceinline__ void store_t(T *P, const Blk<T> &b, int g, int j) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) f16::store_t(P + 16 * J * 32 + 16 * I, 32, b.t[I][J], g, j);
}

// Largest |entry| of a block, the same value in every lane of the wavefront.
template <typename T>
__device__ __forceinline__ T max_abs(const Blk<T> &b) {
  T m = T(0);
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmax(m, fabs(b.t[I][J][r]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
  return m;
}

// True in every lane when every entry of the block has |entry| <= bound.
template <typename T>
__device__ __forceinline__ bool all_below(const Blk<T> &b, T bound) {
  bool ok = true;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) ok = ok && fabs(b.t[I][J][r]) <= bound;
  return __all(ok);
}

template <typename T>
__device__ __forceinline__ Blk<T> neg(Blk<T> b) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) b.t[I][J] = -b.t[I][J];
  return b;
}

template <typename T>
__device__ __forceinline__ Blk<T> sub(Blk<T> a, const Blk<T> &b) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) a.t[I][J] = a.t[I][J] - b.t[I][J];
  return a;
}

// Lane offsets for a symmetric 32x32 block read from its lower triangle.
// Off-diagonal tiles are always wholly below ((1,0)) or above ((0,1)) the
// diagonal, so their offsets are affine in the register index; only the
// diagonal tiles need one lane offset per register (shared by both tiles).
template <typename T>
struct SymOffsets {
  int dg[4];  // tile (0,0); tile (1,1) adds 16 * 33
  int g_, j_;
  __device__ __forceinline__ SymOffsets(int g, int j) : g_(g), j_(j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = row<T>(g, r);
      dg[r] = a >= j ? a * 32 + j : j * 32 + a;
    }
  }
  __device__ __forceinline__ Blk<T> load(const T *P) const {
    Blk<T> b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = row<T>(g_, r);
      b.t[0][0][r] = P[dg[r]];
      b.t[1][1][r] = P[dg[r] + 16 * 33];
      b.t[1][0][r] = P[(16 + a) * 32 + j_];   // below the diagonal
      b.t[0][1][r] = P[(16 + j_) * 32 + a];   // above: read the mirrored entry
    }
    return b;
  }
};

// Packed lower triangle of a symmetric 32x32 block (528 entries, row i at
// offset i (i + 1) / 2).
constexpr int kPacked32 = 528;
template <typename T>
struct PackedOffsets {
  int d0[4];   // tile (0,0) entry offsets (hi, lo = max, min of row and column)
  int hi0[4];  // max(row, column) inside the diagonal tiles
  int r10[4];  // tile (1,0): (16 + row)(17 + row) / 2 + column
  int g_, j_;
  unsigned diag_lower;  // bit r: diagonal-tile entry r lies on or below the diagonal
  __device__ __forceinline__ PackedOffsets(int g, int j) : g_(g), j_(j), diag_lower(0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = row<T>(g, r);
      const int hi = a >= j ? a : j, lo = a >= j ? j : a;
      d0[r] = hi * (hi + 1) / 2 + lo;
      hi0[r] = hi;
      r10[r] = (16 + a) * (17 + a) / 2 + j;
      if (a >= j) diag_lower |= 1u << r;
    }
  }
  // tile (1,1): (16+hi)(17+hi)/2 + 16 + lo = d0 + 16 hi + 152
  __device__ __forceinline__ int d1(int r) const { return d0[r] + 16 * hi0[r] + 152; }
  // tile (0,1): entry (row, 16 + j) mirrors (16 + j, row)
  __device__ __forceinline__ int u01(int r) const {
    return (16 + j_) * (17 + j_) / 2 + row<T>(g_, r);
  }
  __device__ __forceinline__ Blk<T> load(const T *P) const {
    Blk<T> b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      b.t[0][0][r] = P[d0[r]];
      b.t[1][1][r] = P[d1(r)];
      b.t[1][0][r] = P[r10[r]];
      b.t[0][1][r] = P[u01(r)];
    }
    return b;
  }
  __device__ __forceinline__ void store(T *P, const Blk<T> &b) const {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      P[r10[r]] = b.t[1][0][r];
      if (diag_lower & (1u << r)) {
        P[d0[r]] = b.t[0][0][r];
        P[d1(r)] = b.t[1][1][r];
      }
    }
  }
};

// In-place inverse of a symmetric positive definite 32x32 block held as
// O32(A): the symmetric Gauss-Jordan sweep of frag16.h over 32 pivots.
// Column k is broadcast through 32 entries of LDS (`col`, private to this
// wavefront): the lanes holding column k store tile row I's four entries at
// col[16 I + 4 g ..], so row i sits at col[16 (i / 16) + pos(i % 16)].
// Pivots of tile kt are swept with kt a compile-time constant so that every
// register choice is static; row k and column k are cleared under the lane
// masks that own them, then one FMA per entry applies
//     a_ij <- a_ij - u_i (u_j / d),  u = column k with u_k = -1.
template <int kt, typename T>
__device__ __forceinline__ bool gj_tile(Blk<T> &a, T *col, int g, int j, f16::PivotLog &pl) {
  bool bad = false;
  const int pj = Mfma<T>::pos(j);
#pragma unroll 1
  for (int kq = 0; kq < 4; ++kq) {
    double dq[4];
    const bool own = g == kq;  // this lane group holds the pivot rows of this quad
#pragma unroll
    for (int kr = 0; kr < 4; ++kr) {
      const int kl = Mfma<T>::row(kq, kr);  // pivot row inside tile kt
      const bool colk = j == kl;            // this lane holds column k
      if (colk) {
        *reinterpret_cast<Frag<T> *>(col + 4 * g) = a.t[0][kt];
        *reinterpret_cast<Frag<T> *>(col + 16 + 4 * g) = a.t[1][kt];
        a.t[0][kt] = f16::zero<T>();
        a.t[1][kt] = f16::zero<T>();
      }
      f16::wave_sync();
      const T d = col[16 * kt + 4 * kq + kr];
      Frag<T> ci0 = *reinterpret_cast<const Frag<T> *>(col + 4 * g);
      Frag<T> ci1 = *reinterpret_cast<const Frag<T> *>(col + 16 + 4 * g);
      T cj0 = col[pj], cj1 = col[16 + pj];
      f16::wave_sync();
      bad |= !(d > T(0));
      dq[kr] = static_cast<double>(d);
      const T inv = f16::rcp<T>(d);
      if (own) {  // row k: cleared, and u_k = -1
        a.t[kt][0][kr] = T(0);
        a.t[kt][1][kr] = T(0);
        if (kt == 0)
          ci0[kr] = T(-1);
        else
          ci1[kr] = T(-1);
      }
      if (colk) {
        if (kt == 0)
          cj0 = T(-1);
        else
          cj1 = T(-1);
      }
      const T s0 = cj0 * inv, s1 = cj1 * inv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a.t[0][0][r] -= ci0[r] * s0;
        a.t[0][1][r] -= ci0[r] * s1;
        a.t[1][0][r] -= ci1[r] * s0;
        a.t[1][1][r] -= ci1[r] * s1;
      }
    }
    pl.mul4(dq[0], dq[1], dq[2], dq[3]);
  }
  return bad;
}

// Returns true if some pivot is not > 0.  (Scalar sweep over all 32
// pivots; gj_inverse below does the same elimination in 16x16 blocks.)
template <typename T>
__device__ __forceinline__ bool gj_inverse_scalar(Blk<T> &a, T *col, int g, int j,
                                                  f16::PivotLog &pl) {
  bool bad = gj_tile<0>(a, col, g, j, pl);
  bad |= gj_tile<1>(a, col, g, j, pl);
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) a.t[I][J] = -a.t[I][J];
  return bad;
}

// In-place inverse of an SPD 32x32 block by one level of block elimination
// on its 16x16 tiles: sweep A00 (16 pivots), form the Schur complement
// S = A11 - A10 A00^-1 A01 on the matrix cores, sweep S (the other 16
// pivots), then
//     G11 = S^-1,  G10 = -S^-1 X,  G00 = A00^-1 + X^T S^-1 X,  X = A10 A00^-1.
// The pivots are those of the scalar sweep in the same order (the LDL^T
// pivots), so the positive-definiteness test and the determinant are
// unchanged; the work moves from 32 broadcast steps to 16 + 16 on a quarter
// of the entries plus six tile products.  `col` needs 16 entries.
template <typename T>
__device__ __forceinline__ bool gj_inverse(Blk<T> &a, T *col, int g, int j, f16::PivotLog &pl) {
  Frag<T> i00 = a.t[0][0];
  bool bad = f16::gj_inverse(i00, col, g, j, pl);
  const Frag<T> a01 = a.t[0][1];                              // O(A01) = O(A10^T)
  const Frag<T> Xt = f16::mm<T>(i00, a01, f16::zero<T>());    // O(A00^-1 A01) = O(X^T)
  const Frag<T> X = f16::mm<T>(a01, i00, f16::zero<T>());     // O(A10 A00^-1) = O(X)
  Frag<T> S = a.t[1][1] - f16::mm<T>(Xt, a01, f16::zero<T>());  // A11 - X A01
  bad |= f16::gj_inverse(S, col, g, j, pl);
  const Frag<T> G10 = -f16::mm<T>(S, X, f16::zero<T>());     // -S^-1 X
  a.t[1][1] = S;
  a.t[1][0] = G10;
  a.t[0][1] = -f16::mm<T>(X, S, f16::zero<T>());            // -X^T S^-1 = G10^T
  a.t[0][0] = i00 - f16::mm<T>(X, G10, f16::zero<T>());     // A00^-1 + X^T S^-1 X
  return bad;
}

// One elimination step with a 32x32 SPD pivot S and the block C that couples
// it to the next pivot: S is replaced by S^-1 (tiles (0,0), (1,0) and (1,1);
// tile (0,1) is left as it was) and the message C S^-1 C^T is added to tiles
// (0,0), (0,1) and (1,1) of M (tile (1,0) is not touched).  `Ct` is O32(C^T).
// With the block LDL^T of S,
//     S = L diag(S00, Sc) L^T,  L = [[I, 0], [X, I]],  X = S10 S00^-1,
//     Sc = S11 - X S01,
// the message is M = W^T diag(S00^-1, Sc^-1) W with W = L^-1 C^T, whose tile
// row 0 is that of C^T and tile row 1 is (C^T)_1 - X (C^T)_0.  That takes 12
// tile products where forming C S^-1 and then M takes 14, and the explicit
// inverse needs three more (X, P = Sc^-1 X, S00^-1 + X^T P) where gj_inverse
// takes six; after the second sweep only three products stand between Sc^-1
// and M.  The pivots are gj_inverse's, in the same order.
template <typename T>
__device__ __forceinline__ bool gj_congruence(Blk<T> &a, const Blk<T> &Ct, Blk<T> &M, T *col,
                                              int g, int j, f16::PivotLog &pl) {
  const Frag<T> z = f16::zero<T>();
  Frag<T> i00 = a.t[0][0];
  bool bad = f16::gj_inverse(i00, col, g, j, pl);
  const Frag<T> a01 = a.t[0][1];                        // O(S01) = O(S10^T)
  const Frag<T> nXt = -f16::mm<T>(i00, a01, z);         // O(-X^T)
  Frag<T> s11 = f16::mm<T>(nXt, a01, a.t[1][1]);        // O(S11 - X S01)
  const Frag<T> W10 = f16::mm<T>(nXt, Ct.t[0][0], Ct.t[1][0]);
  const Frag<T> W11 = f16::mm<T>(nXt, Ct.t[0][1], Ct.t[1][1]);
  const Frag<T> Z00 = f16::mm<T>(i00, Ct.t[0][0], z);   // S00^-1 W_00
  const Frag<T> Z01 = f16::mm<T>(i00, Ct.t[0][1], z);
  const Frag<T> X = f16::mm<T>(a01, i00, z);            // O(X)
  bad |= f16::gj_inverse(s11, col, g, j, pl);           // Sc^-1
  const Frag<T> Z10 = f16::mm<T>(s11, W10, z);          // Sc^-1 W_10
  const Frag<T> Z11 = f16::mm<T>(s11, W11, z);
  M.t[0][0] = f16::mm<T>(W10, Z10, f16::mm<T>(Ct.t[0][0], Z00, M.t[0][0]));
  M.t[0][1] = f16::mm<T>(W10, Z11, f16::mm<T>(Ct.t[0][0], Z01, M.t[0][1]));
  M.t[1][1] = f16::mm<T>(W11, Z11, f16::mm<T>(Ct.t[0][1], Z01, M.t[1][1]));
  const Frag<T> P = f16::mm<T>(s11, X, z);              // O(Sc^-1 X)
  a.t[0][0] = f16::mm<T>(X, P, i00);                    // S00^-1 + X^T Sc^-1 X
  a.t[1][0] = -P;                                       // -Sc^-1 X
  a.t[1][1] = s11;
  return bad;
}

}  // namespace f32t
}  // namespace selinv
