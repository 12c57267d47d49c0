// io16.h -- coalesced transfers of 16x16 blocks between global memory and
// the MFMA fragment layout of frag16.h, staged through a per-wavefront LDS
// tile.
//
// Global memory is only touched with 16-byte vectors in "natural" order:
// vector v of a row-major block covers elements kVec * v .. kVec * v +
// kVec - 1, and lane l handles vectors l, l + 64, ... .  A whole f64 block
// is two such loads or stores per lane (one for f32), each instruction
// covering 1 KiB of consecutive bytes.  The permutation into (or out of) the
// fragment layout happens in LDS, where scattered 8- or 4-byte accesses are
// cheap.  Rows of a tile are padded to kLd elements to spread LDS banks.
//
// All calls are per wavefront; the caller separates a tile's writes from the
// reads that depend on them with f16::wave_sync().
#pragma once

#include <hip/hip_runtime.h>

#include "frag16.h"

namespace selinv {
namespace io16 {

template <typename T>
struct Traits {
  static constexpr int kVec = 16 / sizeof(T);           // elements per 16-byte vector
  static constexpr int kChunks = 256 / (64 * kVec);     // vectors per lane per block
  static constexpr int kLd = 16 + kVec;                 // padded LDS row (multiple of kVec)
  static constexpr int kTile = 16 * kLd;                // elements per LDS tile
  static constexpr int kPackedVecs = f16::kPacked16 / kVec;  // 68 (f64) or 34 (f32)
  typedef T vec __attribute__((ext_vector_type(16 / sizeof(T))));
};

// One block in natural order, kChunks vectors per lane (8 VGPRs for f64 and
// 4 for f32).
template <typename T>
struct Nat {
  typename Traits<T>::vec c[Traits<T>::kChunks];
};

// Row-major 16x16 block (leading dimension 16) -> registers.  Input and
// output blocks are touched once per pass, so they are loaded and stored
// non-temporally (streaming), which leaves the caches to the workspace.
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

// Workspace blocks are written and read back by the same kernel: ordinary
// (temporal) accesses, so that they can stay in the caches in between.
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

// Tile position of natural vector v (16-byte aligned: kLd is a multiple of kVec).
template <typename T>
__device__ __forceinline__ constexpr int nat_pos(int v) {
  using Tr = Traits<T>;
  return (v * Tr::kVec / 16) * Tr::kLd + (v * Tr::kVec) % 16;
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

// O(M) of the block in the tile
template <typename T>
__device__ __forceinline__ f16::Frag<T> get_frag(const T *tile, int g, int j) {
  f16::Frag<T> f;
#pragma unroll
  for (int r = 0; r < 4; ++r) f[r] = tile[f16::row<T>(g, r) * Traits<T>::kLd + j];
  return f;
}

// O(M^T) of the block in the tile
template <typename T>
__device__ __forceinline__ f16::Frag<T> get_frag_t(const T *tile, int g, int j) {
  f16::Frag<T> f;
#pragma unroll
  for (int r = 0; r < 4; ++r) f[r] = tile[j * Traits<T>::kLd + f16::row<T>(g, r)];
  return f;
}

// write O(M) as M
template <typename T>
__device__ __forceinline__ void put_frag(T *tile, int g, int j, f16::Frag<T> f) {
#pragma unroll
  for (int r = 0; r < 4; ++r) tile[f16::row<T>(g, r) * Traits<T>::kLd + j] = f[r];
}

// Per-lane tile offsets that do not follow from (g, j) affinely: the
// symmetric read from the lower triangle, and the packed lower triangle.
//   sym[r]     tile offset of the element of O(M) in register r, taken from
//              the lower triangle of M
//   pk[r]      offset of that element in a packed lower triangle (row a at
//              a (a + 1) / 2), for reading a fragment from a packed tile
//   src[c][t]  tile offset of packed entry kVec * v + t, v = min(64 c + lane,
//              kPackedVecs - 1), for gathering the packed triangle of a block
template <typename T>
struct SymLanes {
  using Tr = Traits<T>;
  int sym[4];
  int pk[4];
  int src[Tr::kChunks][Tr::kVec];
  __device__ __forceinline__ SymLanes(int g, int j, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = f16::row<T>(g, r);
      const int a = i >= j ? i : j, b = i >= j ? j : i;
      sym[r] = a * Tr::kLd + b;
      pk[r] = a * (a + 1) / 2 + b;
    }
#pragma unroll
    for (int c = 0; c < Tr::kChunks; ++c) {
      const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
#pragma unroll
      for (int t = 0; t < Tr::kVec; ++t) {
        const int e = Tr::kVec * v + t;
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= e) ++a;
        src[c][t] = a * Tr::kLd + (e - a * (a + 1) / 2);
      }
    }
  }
  // O(M) of a symmetric block from the lower triangle of the tile
  __device__ __forceinline__ f16::Frag<T> get_sym(const T *tile) const {
    f16::Frag<T> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = tile[sym[r]];
    return f;
  }
  // O(M) of a symmetric block from a packed-triangle tile
  __device__ __forceinline__ f16::Frag<T> get_packed(const T *ptile) const {
    f16::Frag<T> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = ptile[pk[r]];
    return f;
  }
  // packed lower triangle of the block in the tile, natural vectors
  __device__ __forceinline__ Nat<T> gather_packed(const T *tile) const {
    Nat<T> n;
#pragma unroll
    for (int c = 0; c < Tr::kChunks; ++c)
#pragma unroll
      for (int t = 0; t < Tr::kVec; ++t) n.c[c][t] = tile[src[c][t]];
    return n;
  }
};

// Packed triangle (kPacked16 entries, 16-byte aligned) <-> registers.  Lanes
// beyond the last vector re-read the last one; only the owners store.
template <typename T>
__device__ __forceinline__ Nat<T> load_packed(const T *P, int lane) {
  using Tr = Traits<T>;
  Nat<T> n;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c) {
    const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
    n.c[c] = *reinterpret_cast<const typename Tr::vec *>(P + Tr::kVec * v);
  }
  return n;
}

template <typename T>
__device__ __forceinline__ void store_packed(T *P, int lane, const Nat<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c) {
    const int v = 64 * c + lane;
    if (v < Tr::kPackedVecs) *reinterpret_cast<typename Tr::vec *>(P + Tr::kVec * v) = n.c[c];
  }
}

// registers -> packed-triangle tile (surplus lanes write the last vector
// again, with the same data)
template <typename T>
__device__ __forceinline__ void put_packed(T *ptile, int lane, const Nat<T> &n) {
  using Tr = Traits<T>;
#pragma unroll
  for (int c = 0; c < Tr::kChunks; ++c) {
    const int v = min(64 * c + lane, Tr::kPackedVecs - 1);
    *reinterpret_cast<typename Tr::vec *>(ptile + Tr::kVec * v) = n.c[c];
  }
}

}  // namespace io16
}  // namespace selinv
