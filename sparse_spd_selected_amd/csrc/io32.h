// io32.h -- coalesced transfers of 32x32 blocks between global memory and
// the 2 x 2-tile fragment layout of frag32.h, staged through a per-wavefront
// LDS tile (the 32x32 counterpart of io16.h).
//
// Global memory is touched only with 16-byte vectors in natural order: lane
// l handles vectors l, l + 64, ... of the row-major block, so each
// instruction covers 1 KiB of consecutive bytes (eight per f64 block, four
// per f32 block).  The permutation into the fragment layout happens in LDS.
// Rows of a tile are padded to kLd elements.  Input and output blocks are
// streamed (non-temporal); the packed workspace triangles are not, so that
// they can stay cached between the passes.
//
// All calls are per wavefront; the caller separates a tile's writes from the
// reads that depend on them with f16::wave_sync().
#pragma once

#include <hip/hip_runtime.h>

#include "frag32.h"

namespace selinv {
namespace io32 {

using f32t::Blk;
using f16::row;

template <typename T>
struct Traits {
  static constexpr int kVec = 16 / sizeof(T);        // elements per 16-byte vector
  static constexpr int kChunks = 1024 / (64 * kVec);  // vectors per lane per block
  static constexpr int kLd = 32 + kVec;              // padded LDS row
  static constexpr int kTile = 32 * kLd;
  static constexpr int kPacked = f32t::kPacked32;  // 528
  static constexpr int kPackedVecs = kPacked / kVec;  // 264 (f64) or 132 (f32)
  static constexpr int kPackedChunks = (kPackedVecs + 63) / 64;
  typedef T vec __attribute__((ext_vector_type(16 / sizeof(T))));
};

template <typename T>
struct Nat {
  typename Traits<T>::vec c[Traits<T>::kChunks];
};

template <typename T>
struct NatP {  // packed triangle, natural vectors (surplus lanes repeat the last)
  typename Traits<T>::vec c[Traits<T>::kPackedChunks];
};

template <typename T>
__device__ __forceinline__ Nat<T> load(const T *P, int lane) {
  using Tr = Traits<T>;
  Nat<T> n;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    n.c[c] = __builtin_nontemporal_load(
        reinterpret_cast<const typename Tr::vec *>(P + Tr::kVec * (64 * c + lane)));
  return n;
}

template <typename T>
__device__ __forceinline__ void store(T *P, int lane, const Nat<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    __builtin_nontemporal_store(n.c[c],
                                reinterpret_cast<typename Tr::vec *>(P + Tr::kVec * (64 * c + lane)));
}

// Workspace blocks that are written in one pass and read back in the next
// use ordinary (cacheable) accesses.
template <typename T>
__device__ __forceinline__ Nat<T> load_ws(const T *P, int lane) {
  using Tr = Traits<T>;
  Nat<T> n;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    n.c[c] = *reinterpret_cast<const typename Tr::vec *>(P + Tr::kVec * (64 * c + lane));
  return n;
}

template <typename T>
__device__ __forceinline__ void store_ws(T *P, int lane, const Nat<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    *reinterpret_cast<typename Tr::vec *>(P + Tr::kVec * (64 * c + lane)) = n.c[c];
}

template <typename T>
__device__ __forceinline__ constexpr int nat_pos(int v) {
  using Tr = Traits<T>;
  return (v * Tr::kVec / 32) * Tr::kLd + (v * Tr::kVec) % 32;
}

template <typename T>
__device__ __forceinline__ void put(T *tile, int lane, const Nat<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    *reinterpret_cast<typename Tr::vec *>(tile + nat_pos<T>(64 * c + lane)) = n.c[c];
}

template <typename T>
__device__ __forceinline__ Nat<T> get(const T *tile, int lane) {
  using Tr = Traits<T>;
  Nat<T> n;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c)
    n.c[c] = *reinterpret_cast<const typename Tr::vec *>(tile + nat_pos<T>(64 * c + lane));
  return n;
}

// O32(M) of the block in the tile
template <typename T>
__device__ __forceinline__ Blk<T> get_blk(const T *tile, int g, int j) {
  constexpr int ld = Traits<T>::kLd;
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.t[I][J][r] = tile[(16 * I + row<T>(g, r)) * ld + 16 * J + j];
  return b;
}

// O32(M^T) of the block in the tile
template <typename T>
__device__ __forceinline__ Blk<T> get_blk_t(const T *tile, int g, int j) {
  constexpr int ld = Traits<T>::kLd;
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.t[I][J][r] = tile[(16 * J + j) * ld + 16 * I + row<T>(g, r)];
  return b;
}

// write O32(M) as M
template <typename T>
__device__ __forceinline__ void put_blk(T *tile, int g, int j, const Blk<T> &b) {
  constexpr int ld = Traits<T>::kLd;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(16 * I + row<T>(g, r)) * ld + 16 * J + j] = b.t[I][J][r];
}

// write tiles (0,0), (1,0) and (1,1) of O32(M) (enough for its lower triangle)
template <typename T>
__device__ __forceinline__ void put_blk_low(T *tile, int g, int j, const Blk<T> &b) {
  constexpr int ld = Traits<T>::kLd;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = row<T>(g, r);
    tile[a * ld + j] = b.t[0][0][r];
    tile[(16 + a) * ld + j] = b.t[1][0][r];
    tile[(16 + a) * ld + 16 + j] = b.t[1][1][r];
  }
}

// write O32(M) as M^T
template <typename T>
__device__ __forceinline__ void put_blk_t(T *tile, int g, int j, const Blk<T> &b) {
  constexpr int ld = Traits<T>::kLd;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(16 * J + j) * ld + 16 * I + row<T>(g, r)] = b.t[I][J][r];
}

// Write a symmetric result of which only tiles (0,0), (1,0) and (1,1) are
// formed: the (0,1) tile is the transpose of the (1,0) tile.
template <typename T>
__device__ __forceinline__ void put_sym(T *tile, int g, int j, const Blk<T> &b) {
  constexpr int ld = Traits<T>::kLd;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = row<T>(g, r);
    tile[a * ld + j] = b.t[0][0][r];
    tile[(16 + a) * ld + 16 + j] = b.t[1][1][r];
    tile[(16 + a) * ld + j] = b.t[1][0][r];
    tile[j * ld + 16 + a] = b.t[1][0][r];
  }
}

// Write a symmetric result of which only tiles (0,0), (0,1) and (1,1) are
// formed: the (1,0) tile is the transpose of the (0,1) tile.
template <typename T>
__device__ __forceinline__ void put_sym_u(T *tile, int g, int j, const Blk<T> &b) {
  constexpr int ld = Traits<T>::kLd;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = row<T>(g, r);
    tile[a * ld + j] = b.t[0][0][r];
    tile[(16 + a) * ld + 16 + j] = b.t[1][1][r];
    tile[a * ld + 16 + j] = b.t[0][1][r];
    tile[(16 + j) * ld + a] = b.t[0][1][r];
  }
}

// Per-lane LDS offsets that are not affine in (g, j):
//   dg[r]      element r of the diagonal tiles of O32(M) read from the lower
//              triangle of a tile (tile (1,1) adds 16 (kLd + 1))
//   pk[t][r]   the same elements in a packed lower triangle (row a at
//              a (a + 1) / 2): t = 0 tile (0,0), 1 tile (1,0), 2 tile (1,1);
//              tile (0,1) is (16 + j)(17 + j) / 2 + row(g, r)
//   src[c][e]  tile offset of packed entry kVec v + e, v = min(64 c + lane,
//              kPackedVecs - 1), for gathering the packed triangle
template <typename T>
struct SymLanes {
  using Tr = Traits<T>;
  int dg[4];
  int pk[3][4];
  int pk01;
  int src[Tr::kPackedChunks][Tr::kVec];
  int g_, j_;
  __device__ __forceinline__ SymLanes(int g, int j, int lane) : g_(g), j_(j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = row<T>(g, r);
      const int hi = a >= j ? a : j, lo = a >= j ? j : a;
      dg[r] = hi * Tr::kLd + lo;
      pk[0][r] = hi * (hi + 1) / 2 + lo;
      pk[2][r] = (16 + hi) * (17 + hi) / 2 + 16 + lo;
      pk[1][r] = (16 + a) * (17 + a) / 2 + j;
    }
    pk01 = (16 + j) * (17 + j) / 2;
#pragma unroll
    for (int c = 0; c < Tr::kPackedChunks; ++c) {
      const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
#pragma unroll
      for (int e = 0; e < Tr::kVec; ++e) {
        const int q = Tr::kVec * v + e;
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= q) ++a;
        src[c][e] = a * Tr::kLd + (q - a * (a + 1) / 2);
      }
    }
  }
  // O32(M) of a symmetric block from the lower triangle of a tile
  __device__ __forceinline__ Blk<T> get_sym(const T *tile) const {
    constexpr int ld = Tr::kLd;
    Blk<T> b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = row<T>(g_, r);
      b.t[0][0][r] = tile[dg[r]];
      b.t[1][1][r] = tile[dg[r] + 16 * (ld + 1)];
      b.t[1][0][r] = tile[(16 + a) * ld + j_];
      b.t[0][1][r] = tile[(16 + j_) * ld + a];
    }
    return b;
  }
  // O32(M) of a symmetric block from a packed-triangle tile
  __device__ __forceinline__ Blk<T> get_packed(const T *ptile) const {
    Blk<T> b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      b.t[0][0][r] = ptile[pk[0][r]];
      b.t[1][0][r] = ptile[pk[1][r]];
      b.t[1][1][r] = ptile[pk[2][r]];
      b.t[0][1][r] = ptile[pk01 + row<T>(g_, r)];
    }
    return b;
  }
  // packed lower triangle of the block in a tile, natural vectors
  __device__ __forceinline__ NatP<T> gather_packed(const T *tile) const {
    NatP<T> n;
#pragma unroll
    for (int c = 0; c < Tr::kPackedChunks; ++c)
#pragma unroll
      for (int e = 0; e < Tr::kVec; ++e) n.c[c][e] = tile[src[c][e]];
    return n;
  }
};

template <typename T>
__device__ __forceinline__ NatP<T> load_packed(const T *P, int lane) {
  using Tr = Traits<T>;
  NatP<T> n;
#pragma unroll
  for (int c = 0; c < Tr::kPackedChunks; ++c) {
    const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
    n.c[c] = *reinterpret_cast<const typename Tr::vec *>(P + Tr::kVec * v);
  }
  return n;
}

template <typename T>
__device__ __forceinline__ void store_packed(T *P, int lane, const NatP<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kPackedChunks; ++c) {
    const int v = 64 * c + lane;
    if (v < Tr::kPackedVecs) *reinterpret_cast<typename Tr::vec *>(P + Tr::kVec * v) = n.c[c];
  }
}

// registers -> packed-triangle tile (surplus lanes rewrite the last vector
// with the same data)
template <typename T>
__device__ __forceinline__ void put_packed(T *ptile, int lane, const NatP<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kPackedChunks; ++c) {
    const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
    *reinterpret_cast<typename Tr::vec *>(ptile + Tr::kVec * v) = n.c[c];
  }
}

}  // namespace io32
}  // namespace selinv
