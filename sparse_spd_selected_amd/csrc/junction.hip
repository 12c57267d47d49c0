// junction.hip -- selected inverse of general sparse SPD matrices on their
// filled (chordal) pattern, batched over matrices that share the pattern
// (gabp-sparse-inv page, junction-tree section: sparse block Cholesky, then
// the multi-neighbour Takahashi recurrence, level by level).
//
// Fat nodes.  The plan groups the elimination into chunks J of consecutive
// supernode columns (their pivot is one dense (s b) x (s b) block) and the
// recurrences run on chunks.  In Cholesky form, with A = L~ L~^T, the
// chunk's diagonal factor R_J (lower triangular) and its later rows
// W_{N,J} = C_{N,J} R_J^-T:
//   factor (chunk levels upward): for every block (t, j) of J's panel
//       C_{t,j} = A_{t,j} - sum_u W_{t,u} W_{j,u}^T
//   over the earlier columns u outside J with j and t in N(u); then
//       R_J = chol(C_JJ) (dense),  W_{N,J} = C_{N,J} R_J^-T,
//       log det += 2 sum ln diag(R_J)
//   Takahashi (chunk levels downward, root first), N = N_J:
//       G_{N,J} = -(G_{N,N} W_{N,J}) R_J^-1
//       G_JJ    = R_J^-T (R_J^-1 - W_{N,J}^T G_{N,J})
// (the page's LDL^T recurrences for the fat node, L_{N,J} = W_{N,J} R_J^-1,
// D_J = R_J R_J^T).  Every block read lies in S because N_J is a clique;
// the blocks inside a chunk are in S because a supernode's columns are dense.
// One G_{N,N} block now serves s columns at once.
//
// Work decomposition, each workgroup owning what it writes for one matrix:
// per level the Schur sums (one workgroup per panel block, or one wavefront
// per panel block for b <= 8), the dense pivots (one per chunk: R_J^-1, the
// log det term), the scaling of the later rows (one per row, or one per tile
// of 64 / b rows for b = 4, 8, 16), and in the Takahashi pass the rows
// G_{w,J} (one per tile of rows) and the chunk's own blocks (one per block
// column); on levels with few tiles or columns the last two split their sums
// over several workgroups and add the parts in a fixed order.  For b = 4, 8,
// 16 the scaling, row and diagonal products run on the matrix cores
// (16x16x4, one 16-row block per wavefront; s b <= 48 gives three 16-column
// blocks).  Sums run in a fixed order, so results are deterministic; the
// only atomic is the first-failure index.  Without G outputs only the
// factorisation runs (the log det call).
// Operands are staged through LDS in rounds; every thread issues a batch of
// loads before storing them, so a round costs about one memory latency.  The
// level kernels take their workgroups in XCD-contiguous ranges (xcd_wg).
#include <hip/hip_runtime.h>

#include <climits>

#include "block_wg.h"
#include "frag16.h"
#include "internal.h"

namespace selinv {
namespace {

constexpr int kJT = 256;  // threads per workgroup

// Pairs per staging round: buffers of 2048 elements (1024 for b > 16), so
// that with the four extra blocks a workgroup stays under 64 KB of LDS.
__host__ __device__ inline int stage_pairs(int bb) {
  const int c = (bb <= 256 ? 2048 : 1024) / bb;
  return c < 1 ? 1 : (c > 64 ? 64 : c);
}

// LDS: the pair table of a staging round (two block pointers and a flag
// byte per pair), two staging buffers, a reduction buffer of kJT and four
// blocks.
constexpr int kMaxPairs = 64;
constexpr size_t kTableBytes = kMaxPairs * (2 * sizeof(void *) + 1);
constexpr int kMaxLoads = 8;  // staged elements per thread and buffer (2048 / kJT)

template <typename T>
size_t lds_bytes(int b) {
  const int bb = b * b;
  return kTableBytes + sizeof(T) * (2 * size_t(stage_pairs(bb)) * bb + kJT + 4 * size_t(bb));
}

template <typename T>
struct Lds {
  const T **pa, **pb;
  unsigned char *tr;
  T *sa, *sb, *red, *blk;
};

template <typename T>
__device__ inline Lds<T> lds_carve(int b) {
  extern __shared__ char smem_raw[];
  Lds<T> l;
  l.pa = reinterpret_cast<const T **>(smem_raw);
  l.pb = l.pa + kMaxPairs;
  l.tr = reinterpret_cast<unsigned char *>(l.pb + kMaxPairs);
  const int bb = b * b, CH = stage_pairs(bb);
  l.sa = reinterpret_cast<T *>(smem_raw + kTableBytes);
  l.sb = l.sa + CH * bb;
  l.red = l.sb + CH * bb;
  l.blk = l.red + kJT;
  return l;
}

enum Mode { kABt = 0, kAB = 1, kAtB = 2 };

template <int MODE, typename T>
__device__ inline T dot_block(const T *A, const T *Bm, int b, int r, int c) {
  T s = T(0);
  for (int k = 0; k < b; ++k) {
    const T a = MODE == kAtB ? A[k * b + r] : A[r * b + k];
    const T x = MODE == kABt ? Bm[c * b + k] : Bm[k * b + c];
    s += a * x;
  }
  return s;
}

// Sum over q < count of op(A_q) op(B_q) into `out` (LDS, bb entries).
// src(q, A, ta, B, tb) names the two blocks of pair q (global memory) and
// whether each is to be read transposed.  Each round first puts the pair
// table in LDS, then every thread issues all its element loads before it
// stores any (one memory latency per round, not one per element), then the
// groups of bb threads multiply.  Deterministic: fixed pair-to-group map and
// fixed reduction order.
template <int MODE, typename T, typename Src>
__device__ inline void staged_sum(T *out, int count, int b, const Lds<T> &l, Src src) {
  const int bb = b * b, t = threadIdx.x;
  const int CH = stage_pairs(bb);
  const bool small = bb <= kJT;
  const int G = small ? kJT / bb : 1;
  const int g = small ? t / bb : 0;
  T acc[4] = {T(0), T(0), T(0), T(0)};
  for (int q0 = 0; q0 < count; q0 += CH) {
    const int cnt = count - q0 < CH ? count - q0 : CH;
    if (t < cnt) {
      const T *A, *Bp;
      int ta, tb;
      src(q0 + t, A, ta, Bp, tb);
      l.pa[t] = A;
      l.pb[t] = Bp;
      l.tr[t] = static_cast<unsigned char>(ta | (tb << 1));
    }
    __syncthreads();
    const int tot = cnt * bb;
    T va[kMaxLoads], vb[kMaxLoads];
#pragma unroll
    for (int j = 0; j < kMaxLoads; ++j) {
      const int idx = t + j * kJT;
      if (idx < tot) {
        const int q = idx / bb, el = idx - q * bb, r = el / b, c = el - r * b;
        const int f = l.tr[q];
        va[j] = l.pa[q][(f & 1) ? c * b + r : el];
        vb[j] = l.pb[q][(f & 2) ? c * b + r : el];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxLoads; ++j) {
      const int idx = t + j * kJT;
      if (idx < tot) {
        l.sa[idx] = va[j];
        l.sb[idx] = vb[j];
      }
    }
    __syncthreads();
    if (small) {
      if (g < G) {
        const int e = t - g * bb, r = e / b, c = e - r * b;
        for (int q = g; q < cnt; q += G)
          acc[0] += dot_block<MODE>(l.sa + q * bb, l.sb + q * bb, b, r, c);
      }
    } else {
      for (int i = 0; i < 4; ++i) {
        const int e = t + i * kJT;
        if (e >= bb) break;
        const int r = e / b, c = e - r * b;
        for (int q = 0; q < cnt; ++q) acc[i] += dot_block<MODE>(l.sa + q * bb, l.sb + q * bb, b, r, c);
      }
    }
    __syncthreads();
  }
  if (small) {
    l.red[t] = acc[0];
    __syncthreads();
    if (t < bb) {
      T s = T(0);
      for (int gg = 0; gg < G; ++gg) s += l.red[gg * bb + t];
      out[t] = s;
    }
  } else {
    for (int i = 0; i < 4; ++i) {
      const int e = t + i * kJT;
      if (e < bb) out[e] = acc[i];
    }
  }
  __syncthreads();
}


// Row tiles of the row kernel, pairs per round of the chunk kernel (a b x sb
// row and a block each), and the LDS of every kernel.
constexpr size_t kLdsMax = 64 * 1024;
constexpr int kTileTable = 256;  // G block pointers per staging round of a row tile
constexpr size_t kTileTableBytes = kTileTable * (sizeof(void *) + 1);

// rows per tile: H = R b <= 64 scalar rows (16 threads x 4 rows)
__host__ __device__ inline int tile_rows(int b) { return b >= 64 ? 1 : 64 / b; }
// staging steps (x values) per round: about 4096 elements, table-limited
__host__ __device__ inline int tile_steps(int b, int s) {
  const int R = tile_rows(b), per = R * b * b + b * s * b;
  int c = 4096 / per;
  c = c < 1 ? 1 : c;
  c = c > kTileTable / R ? kTileTable / R : c;
  return c < 1 ? 1 : c;
}

__host__ __device__ inline int diag_pairs(int b, int s) {
  const int per = b * s * b + b * b;
  const int c = 4096 / per;
  return c < 1 ? 1 : (c > kMaxPairs ? kMaxPairs : c);
}
template <typename T>
size_t fac_lds(int b, int sm) {
  const size_t sb = size_t(sm) * b;
  return sizeof(T) * (2 * sb * sb + sb * b);
}
template <typename T>
size_t scale_lds(int b, int sm) {
  const size_t sb = size_t(sm) * b;
  return sizeof(T) * (sb * sb + b * sb);
}
// the chunk size varies (s <= sm); the largest need over s bounds the launch
template <typename T>
size_t rows_lds(int b, int sm) {
  size_t best = 0;
  const size_t H = size_t(tile_rows(b)) * b;
  for (int s = 1; s <= sm; ++s) {
    const size_t sb = size_t(s) * b;
    const size_t stage = size_t(tile_steps(b, s)) * (H * b + b * sb);
    const size_t epi = H * sb + sb * sb + (size_t(tile_rows(b)) * s * 4 + sizeof(T) - 1) / sizeof(T);
    const size_t e = stage > epi ? stage : epi;
    best = e > best ? e : best;
  }
  return kTileTableBytes + sizeof(T) * best;
}
template <typename T>
size_t diag_lds(int b, int sm) {
  size_t best = 0;
  for (int s = 1; s <= sm; ++s) {
    const size_t sb = size_t(s) * b, wr = b * sb;
    size_t stage = size_t(diag_pairs(b, s)) * (wr + b * b);
    // later X and Y (sb x b each) and the s output codes of the block column
    const size_t xy = 2 * sb * b + (size_t(s) * 4 + sizeof(T) - 1) / sizeof(T);
    stage = stage < xy ? xy : stage;
    const size_t e = sb * sb + stage;
    best = e > best ? e : best;
  }
  return sizeof(T) * best;
}

// Copies tot elements into LDS dst, element e = src(e) (a global load),
// each thread issuing up to eight loads before it stores them.
template <typename T, typename F>
__device__ inline void gather_lds(T *dst, int tot, F src) {
  for (int base = 0; base < tot; base += 8 * kJT) {
    T v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + threadIdx.x + j * kJT;
      if (e < tot) v[j] = src(e);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + threadIdx.x + j * kJT;
      if (e < tot) dst[e] = v[j];
    }
  }
}

// Cholesky step sequence of chol_inverse for n <= NM on one wavefront (lane i
// holds row i of the matrix padded to NM x NM with the identity, so that the
// code is straight-line with static register indices; padded pivots are 1 and
// leave the rest unchanged).  Column j is broadcast through LDS with
// wavefront-scope ordering only.  On return row i of S (LDS, n x n) holds, for
// l <= i, entry (i, l) as it was at pivot step l.  Returns 0 or 1 + the first
// column whose pivot is not > 0 (the same in every lane); the steps after a
// failure run on, their results unused.
template <int NM, typename T>
__device__ __forceinline__ int chol_wave(T *S, int n) {
  __shared__ T colbuf[64];
  const int t = threadIdx.x;
  T r[NM];
#pragma unroll
  for (int l = 0; l < NM; ++l)
    r[l] = (t < n && l < n) ? (l <= t ? S[t * n + l] : T(0)) : (l == t ? T(1) : T(0));
  int fail = 0;
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    colbuf[t] = r[j];  // column j (lanes below j hold S_ij; the rest is unused)
    f16::wave_sync();
    const T dj = colbuf[j];
    if (fail == 0 && !(dj > T(0))) fail = j + 1;
    const T sj = r[j] * f16::rcp<T>(dj);
#pragma unroll
    for (int l = j + 1; l < NM; ++l) r[l] -= sj * colbuf[l];
    f16::wave_sync();
  }
#pragma unroll
  for (int l = 0; l < NM; ++l)
    if (t < n && l < n && l <= t) S[t * n + l] = r[l];
  return fail;
}

// S (LDS, n x n with n = s b; lower triangle read) = R R^T: R overwrites
// the lower triangle of S, and X (LDS) receives R^-1 (lower, zero above);
// tmp is LDS scratch of n b entries.  Returns 0, or 1 + the first column
// whose pivot is not > 0 (NaN included), uniformly; *logdet = ln det S.
// Cholesky: right-looking on unscaled columns (S_il -= S_ij S_lj / d_j for
// j < l <= i), scaled at the end.  For n <= 48 (always the case for chunks)
// one wavefront runs it (chol_wave); larger n: one barrier per column.
// Inverse:
// block forward substitution with b x b blocks -- the diagonal blocks'
// inverses, then one block diagonal of R^-1 at a time,
// X_ik = -X_ii sum_{k <= q < i} R_iq X_qk.
template <typename T>
__device__ __forceinline__ int chol_inverse(T *S, T *X, T *tmp, int n, int b, double *logdet) {
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  if (n <= 48) {
    __shared__ int fail_s;
    if (t < 64) {  // the first wavefront; lane i holds row i
      int fail;
      if (n <= 8)
        fail = chol_wave<8>(S, n);
      else if (n <= 16)
        fail = chol_wave<16>(S, n);
      else if (n <= 24)
        fail = chol_wave<24>(S, n);
      else if (n <= 32)
        fail = chol_wave<32>(S, n);
      else
        fail = chol_wave<48>(S, n);
      if (t == 0) fail_s = fail;
    }
    __syncthreads();
    if (fail_s) return fail_s;
  } else {
    for (int j = 0; j < n; ++j) {
      const T dj = S[j * n + j];
      if (!(dj > T(0))) return j + 1;
      const T inv = T(1) / dj;
      for (int i = j + 1 + ty; i < n; i += 16) {
        const T sij = S[i * n + j] * inv;
        for (int l = j + 1 + tx; l <= i; l += 16) S[i * n + l] -= sij * S[l * n + j];
      }
      __syncthreads();
    }
  }
  double ld = 0.0;
  if (n <= 48) {  // the pivots' logs in parallel, summed in column order
    __shared__ double lg[48];
    if (t < n) lg[t] = log(static_cast<double>(S[t * n + t]));
    __syncthreads();
    for (int j = 0; j < n; ++j) ld += lg[j];
  } else {
    for (int j = 0; j < n; ++j) ld += log(static_cast<double>(S[j * n + j]));
  }
  for (int e = t; e < n * n; e += kJT) {
    const int i = e / n, j = e - i * n;
    if (i > j) S[e] /= sqrt(S[j * n + j]);
    X[e] = T(0);
  }
  __syncthreads();
  for (int j = t; j < n; j += kJT) S[j * n + j] = sqrt(S[j * n + j]);
  __syncthreads();
  const int bb = b * b, s = n / b;
  for (int kc = t; kc < n; kc += kJT) {  // diagonal blocks, one column each
    const int o = (kc / b) * b, c = kc - o;
    for (int r = c; r < b; ++r) {
      T v = r == c ? T(1) : T(0);
      for (int u = c; u < r; ++u) v -= S[(o + r) * n + o + u] * X[(o + u) * n + o + c];
      X[(o + r) * n + o + c] = v / S[(o + r) * n + o + r];
    }
  }
  __syncthreads();
  for (int m = 1; m < s; ++m) {
    const int cnt = (s - m) * bb;
    for (int e = t; e < cnt; e += kJT) {
      const int k = e / bb, rem = e - k * bb, r = rem / b, c = rem - r * b, i0 = (k + m) * b;
      T v = T(0);
      for (int K = k * b; K < i0; ++K) v += S[(i0 + r) * n + K] * X[K * n + k * b + c];
      tmp[e] = v;
    }
    __syncthreads();
    for (int e = t; e < cnt; e += kJT) {
      const int k = e / bb, rem = e - k * bb, r = rem / b, c = rem - r * b, i0 = (k + m) * b;
      T v = T(0);
      for (int u = 0; u <= r; ++u) v += X[(i0 + r) * n + i0 + u] * tmp[k * bb + u * b + c];
      X[(i0 + r) * n + k * b + c] = -v;
    }
    __syncthreads();
  }
  *logdet = ld;
  return 0;
}

struct Dims {
  int64_t n, m, nnz, nch, npanel, nrinv;
  int b;
};

template <typename T>
__global__ void __launch_bounds__(kJT) jt_init(int32_t *info_ws, int64_t B) {
  const int64_t m = blockIdx.x * int64_t(kJT) + threadIdx.x;
  if (m < B) info_ws[m] = INT_MAX;
}

// Schur sums of the panel blocks [tbase, tbase + gridDim.x), matrix blockIdx.y
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_update(JunctionPlanDev P, Dims d, int64_t tbase,
                                                     const T *__restrict__ diag,
                                                     const T *__restrict__ edge_val, T *W) {
  const int b = BC ? BC : d.b, bb = b * b;
  const Lds<T> l = lds_carve<T>(b);
  T *acc = l.blk;
  const int64_t tg = tbase + blockIdx.x, mat = blockIdx.y;
  const int id = P.tg_chunk[tg], rc = P.tg_rc[tg], r = rc >> 6, col = rc & 63;
  const int32_t f0 = P.fptr[tg], f1 = P.fptr[tg + 1];
  const T *Wm = W + mat * d.npanel * bb;
  const int32_t *fp = P.fpair;
  staged_sum<kABt>(acc, f1 - f0, b, l, [&](int q, const T *&A, int &ta, const T *&Bp, int &tb) {
    A = Wm + int64_t(fp[2 * (f0 + q)]) * bb;
    Bp = Wm + int64_t(fp[2 * (f0 + q) + 1]) * bb;
    ta = tb = 0;
  });
  const int32_t enc = P.ain[tg];
  T *dst = W + (mat * d.npanel + P.ch_pbase[id] + int64_t(r) * P.ch_s[id] + col) * bb;
  if (r == col) {
    const T *D = diag + (mat * d.n + enc) * bb;
    for (int e = threadIdx.x; e < bb; e += kJT) {
      const int i = e / b, j = e - i * b;
      dst[e] = (i >= j ? D[i * b + j] : D[j * b + i]) - acc[e];
    }
  } else {
    const T *E = enc < 0 ? nullptr : edge_val + (mat * d.m + (enc >> 1)) * bb;
    const bool tr = enc >= 0 && (enc & 1);
    for (int e = threadIdx.x; e < bb; e += kJT) {
      const int i = e / b, j = e - i * b;
      dst[e] = (E ? (tr ? E[j * b + i] : E[e]) : T(0)) - acc[e];
    }
  }
}

// C_{t,j} = A_{t,j} - acc for lane e < bb of the wavefront (entry e of the
// panel block of target tg)
template <typename T, int BC>
__device__ __forceinline__ void write_target(const JunctionPlanDev &P, const Dims &d, int64_t tg,
                                             int64_t mat, int e, T acc, const T *diag,
                                             const T *edge_val, T *W) {
  constexpr int b = BC, bb = b * b;
  const int er = e / b, ec = e - er * b;
  const int id = P.tg_chunk[tg], rc = P.tg_rc[tg], r = rc >> 6, col = rc & 63;
  const int32_t enc = P.ain[tg];
  T *dst = W + (mat * d.npanel + P.ch_pbase[id] + int64_t(r) * P.ch_s[id] + col) * bb;
  T base;
  if (r == col) {
    const T *D = diag + (mat * d.n + enc) * bb;
    base = er >= ec ? D[er * b + ec] : D[ec * b + er];
  } else {
    const T *E = enc < 0 ? nullptr : edge_val + (mat * d.m + (enc >> 1)) * bb;
    base = E ? ((enc & 1) ? E[ec * b + er] : E[e]) : T(0);
  }
  dst[e] = base - acc;
}

// Schur sums for b <= 8 (bb <= 64): one wavefront per work item (a run of at
// most 64 pairs of one panel block's list), four per workgroup, no
// workgroup barrier.  Lane e owns entry e of the b x b sum (b = 8) or, for
// smaller b, the 64 / bb lane groups take every (64 / bb)-th pair and are
// added at the end.  Each round stages up to 512 / bb pairs of blocks through
// the wavefront's LDS.  A target with one item is finished here; the items
// of a longer list leave partial sums in their slots of Spart for
// jt_fwd_update_sum.
// Workgroup (x, matrix) of a 2-D launch, remapped so that each of the eight
// XCDs (the dispatcher deals workgroups to them round-robin by linear index)
// runs one contiguous range of linear indices: neighbouring work items, which
// read many of the same panel blocks, then share that XCD's L2.  A bijection
// of the grid, so the result does not depend on the real dispatch.
struct WgXM {
  int64_t x, mat;
};
__device__ inline WgXM xcd_wg() {
  const int64_t nx = gridDim.x, n = nx * gridDim.y, w = int64_t(blockIdx.y) * nx + blockIdx.x;
  const int64_t xcd = w % 8, k = w / 8, q = n / 8, r = n % 8;
  const int64_t l = xcd * q + (xcd < r ? xcd : r) + k;
  return {l % nx, l / nx};
}

template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_update_wave(JunctionPlanDev P, Dims d,
                                                          int64_t ibase, int64_t iend,
                                                          int64_t nslots, T *Spart,
                                                          const T *__restrict__ diag,
                                                          const T *__restrict__ edge_val, T *W) {
  constexpr int b = BC, bb = b * b, CH = (512 / bb) > 32 ? 32 : 512 / bb, G = 64 / bb;
  constexpr int NL = CH * bb / 64;  // staged elements per lane and operand
  __shared__ __align__(16) T sa[4][CH * bb];
  __shared__ __align__(16) T sb[4][CH * bb];
  __shared__ T red[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const WgXM wg = xcd_wg();
  const int64_t it = ibase + wg.x * 4 + wave, mat = wg.mat;
  if (it >= iend) return;
  const int64_t tg = P.it_tg[it];
  const int32_t f0 = P.it_lo[it], f1 = P.it_hi[it], slot = P.it_slot[it];
  const T *Wm = W + mat * d.npanel * bb;
  const int grp = lane / bb, e = lane - grp * bb, er = e / b, ec = e - er * b;
  T acc = T(0);
  // Rounds of CH pairs, pipelined one round ahead: round r + 1's blocks are
  // loaded (their pair codes read a round earlier still, lane l < 2 CH
  // holding code l) while round r's products run.  Wavefront-scope
  // synchronisation only, so nothing waits on the loads in flight.
  const int nround = (f1 - f0 + CH - 1) / CH;
  auto cnt_of = [&](int r) { const int32_t q0 = f0 + r * CH; return f1 - q0 < CH ? f1 - q0 : CH; };
  auto codes = [&](int r) -> int32_t {
    return r < nround && lane < 2 * cnt_of(r) ? P.fpair[2 * int64_t(f0 + r * CH) + lane] : 0;
  };
  T va[NL], vb[NL];
  auto load = [&](int r, int32_t code) {
    const int cnt = cnt_of(r);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = lane + 64 * u, q = idx / bb, el = idx - q * bb;
      const int32_t ca = __shfl(code, 2 * q < 64 ? 2 * q : 0), cb = __shfl(code, 2 * q + 1 < 64 ? 2 * q + 1 : 0);
      if (q < cnt) {
        va[u] = Wm[int64_t(ca) * bb + el];
        vb[u] = Wm[int64_t(cb) * bb + el];
      }
    }
  };
  int32_t code = codes(0);
  if (nround > 0) load(0, code);
  code = codes(1);
  for (int r = 0; r < nround; ++r) {
    const int cnt = cnt_of(r);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = lane + 64 * u;
      if (idx / bb < cnt) {
        sa[wave][idx] = va[u];
        sb[wave][idx] = vb[u];
      }
    }
    f16::wave_sync();
    if (r + 1 < nround) {
      load(r + 1, code);
      code = codes(r + 2);
    }
    if (grp < G)
      for (int q = grp; q < cnt; q += G) {
        const T *A = sa[wave] + q * bb + er * b, *Bq = sb[wave] + q * bb + ec * b;
#pragma unroll
        for (int k = 0; k < b; ++k) acc += A[k] * Bq[k];
      }
    f16::wave_sync();
  }
  if (G > 1) {
    red[wave][lane] = acc;
    f16::wave_sync();
    if (lane < bb) {
      T v = T(0);
      for (int gg = 0; gg < G; ++gg) v += red[wave][gg * bb + lane];
      acc = v;
    }
  }
  if (lane >= bb) return;
  if (slot < 0)
    write_target<T, BC>(P, d, tg, mat, e, acc, diag, edge_val, W);
  else
    Spart[(mat * nslots + slot) * bb + e] = acc;
}

// Targets with several work items: their partial sums added in item order
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_update_sum(JunctionPlanDev P, Dims d,
                                                         int64_t mbase, int64_t mend,
                                                         int64_t nslots, const T *Spart,
                                                         const T *__restrict__ diag,
                                                         const T *__restrict__ edge_val, T *W) {
  constexpr int bb = BC * BC;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t k = mbase + int64_t(blockIdx.x) * 4 + wave, mat = blockIdx.y;
  if (k >= mend || lane >= bb) return;
  const int64_t tg = P.multi_tg[k];
  const int32_t i0 = P.it_ptr[tg], i1 = P.it_ptr[tg + 1], s0 = P.it_slot[i0];
  T acc = T(0);
  for (int32_t i = 0; i < i1 - i0; ++i) acc += Spart[(mat * nslots + s0 + i) * bb + lane];
  write_target<T, BC>(P, d, tg, mat, lane, acc, diag, edge_val, W);
}

// Dense pivot of every chunk of the level: R_J^-1 (into RJ), the log det
// term, the first failing column
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_factor(JunctionPlanDev P, Dims d, int64_t cbase,
                                                     const T *W, T *RJ, double *ld_ws,
                                                     int32_t *info_ws) {
  extern __shared__ char smem_raw[];
  T *M = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b;
  const int64_t id = cbase + blockIdx.x, mat = blockIdx.y;
  const int s = P.ch_s[id], sb = s * b;
  T *X = M + sb * sb;  // then n b entries of scratch
  const T *Wp = W + (mat * d.npanel + P.ch_pbase[id]) * bb;
  gather_lds(M, sb * sb, [&](int e) {
    const int I = e / sb, J = e - I * sb;
    return I >= J ? Wp[(int64_t(I / b) * s + J / b) * bb + (I % b) * b + (J % b)] : T(0);
  });
  __syncthreads();
  double ld = 0.0;
  const int fail = chol_inverse(M, X, X + sb * sb, sb, b, &ld);
  if (fail) wg::fill(X, sb * sb, wg::qnan<T>());
  T *Rout = RJ + (mat * d.nrinv + P.ch_rbase[id]) * bb;
  for (int e = threadIdx.x; e < sb * sb; e += kJT) Rout[e] = X[e];
  if (threadIdx.x == 0) {
    ld_ws[mat * d.nch + id] = fail ? static_cast<double>(wg::qnan<T>()) : ld;
    if (fail) atomicMin(info_ws + mat, P.ch_first[id] + (fail - 1) / b);
  }
}

// Later rows of the level: W_{w,J} = C_{w,J} R_J^-T in place
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_scale(JunctionPlanDev P, Dims d, int64_t rbase0,
                                                    T *W, const T *RJ) {
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b;
  const int64_t ri = rbase0 + blockIdx.x, mat = blockIdx.y;
  const int id = P.row_chunk[ri], a = static_cast<int>(ri - P.rows_ptr[id]);
  const int s = P.ch_s[id], sb = s * b, wr = b * sb;
  T *C = Ri + sb * sb;
  const T *Rj = RJ + (mat * d.nrinv + P.ch_rbase[id]) * bb;
  T *Wrow = W + (mat * d.npanel + P.ch_pbase[id] + int64_t(s + a) * s) * bb;
  gather_lds(Ri, sb * sb, [&](int e) { return Rj[e]; });
  // C as a dense b x sb row: element (i, cc) is block cc / b, entry (i, cc % b)
  gather_lds(C, wr, [&](int e) {
    const int i = e / sb, cc = e - i * sb;
    return Wrow[(cc / b) * bb + i * b + cc % b];
  });
  __syncthreads();
  for (int e = threadIdx.x; e < wr; e += kJT) {
    const int i = e / sb, cc = e - i * sb;
    T v = T(0);
    for (int kk = 0; kk <= cc; ++kk) v += C[i * sb + kk] * Ri[cc * sb + kk];
    Wrow[(cc / b) * bb + i * b + cc % b] = v;
  }
}

// The same scaling for b = 4, 8, 16, a tile of up to 64 / b later rows of one
// chunk per workgroup (the tiles of the backward row products): R_J^-1 is
// staged once per tile, and W_tile = C_tile R_J^-T runs on the matrix cores,
// wavefront w owning rows 16 w .. 16 w + 15 and three 16-column blocks; lane
// (lk, lr) supplies C[16 w + lr][k] and R_J^-1[16 cb + lr][k], k = 4 kk + lk.
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_fwd_scale_tiles(JunctionPlanDev P, Dims d,
                                                          int64_t tbase, T *W, const T *RJ) {
  static_assert(BC % 4 == 0, "matrix-core scaling needs b a multiple of 4");
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  constexpr int b = BC, bb = b * b, R = 64 / b, H = 64;
  const int t = threadIdx.x;
  const WgXM wg = xcd_wg();
  const int64_t tile = tbase + wg.x, mat = wg.mat;
  const int id = P.tile_chunk[tile];
  const int a0 = static_cast<int>(tile - P.tiles_ptr[id]) * R;
  const int s = P.ch_s[id], nr = P.ch_n[id], sb = s * b;
  const int rows = nr - a0 < R ? nr - a0 : R;
  T *Cs = Ri + sb * sb;  // H x sb
  const T *Rj = RJ + (mat * d.nrinv + P.ch_rbase[id]) * bb;
  T *Wp = W + (mat * d.npanel + P.ch_pbase[id]) * bb;
  gather_lds(Ri, sb * sb, [&](int e) { return Rj[e]; });
  gather_lds(Cs, H * sb, [&](int e) {
    const int h = e / sb, cc = e - h * sb, ra = h / b, i = h - ra * b;
    return ra < rows ? Wp[(int64_t(s + a0 + ra) * s + cc / b) * bb + i * b + cc % b] : T(0);
  });
  __syncthreads();
  const int wv = t >> 6, ln = t & 63, lr = ln & 15, lk = ln >> 4;
  f16::Frag<T> acc[3] = {f16::zero<T>(), f16::zero<T>(), f16::zero<T>()};
  for (int kk = 0; kk < sb / 4; ++kk) {
    const int k = 4 * kk + lk;
    const T a = Cs[(16 * wv + lr) * sb + k];
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) {
      const int cc = 16 * cb + lr;
      const T bv = cc < sb ? Ri[cc * sb + k] : T(0);
      acc[cb] = f16::Mfma<T>::op(a, bv, acc[cb]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < 3; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * wv + f16::Mfma<T>::row(lk, r), cc = 16 * cb + lr;
      const int ra = h / b, i = h - ra * b;
      if (cc < sb && ra < rows)
        Wp[(int64_t(s + a0 + ra) * s + cc / b) * bb + i * b + cc % b] = acc[cb][r];
    }
}

// Row tiles of the level: for R consecutive later rows w of a chunk (H = R b
// scalar rows), G_{w,J} = -(sum_x G_{w,x} W_{x,J}) R_J^-1.  The sum is a
// gathered product (H x n b) (n b x s b): each step stages, for one x, the
// R blocks G_{w,x} and the row W_{x,J} once for all R rows; every thread
// keeps a 4 x 3 register tile of the H x s b result.
// Tt (LDS, H x sb, the tile's sum) -> -Tt R_J^-1 into the output rows;
// Ri is LDS scratch of sb * sb entries.
// The output codes of the tile's blocks are staged in LDS with R_J^-1, so
// that no store waits on a dependent load.  Ri is LDS scratch of sb * sb
// entries followed by room for rows * s codes.
template <int BC, typename T>
__device__ inline void rows_epilogue(const JunctionPlanDev &P, const Dims &d, int64_t mat, int id,
                                     int a0, int rows, const T *Tt, T *Ri, const T *RJ,
                                     T *G_lower) {
  const int b = BC ? BC : d.b, bb = b * b, s = P.ch_s[id], sb = s * b;
  const int64_t pb = P.ch_pbase[id];
  int32_t *codes = reinterpret_cast<int32_t *>(Ri + sb * sb);
  for (int e = threadIdx.x; e < rows * s; e += kJT)
    codes[e] = P.poutenc[pb + int64_t(s + a0) * s + e];
  gather_lds(Ri, sb * sb, [&](int e) { return RJ[(mat * d.nrinv + P.ch_rbase[id]) * bb + e]; });
  __syncthreads();
  if constexpr (BC != 0 && BC % 4 == 0) {
    // on the matrix cores (the tile is 64 rows): wavefront w owns rows
    // 16 w .. 16 w + 15 and three 16-column blocks; lane (lk, lr) supplies
    // T[16 w + lr][k] and R_J^-1[k][16 cb + lr], k = 4 kk + lk
    const int t = threadIdx.x, wv = t >> 6, ln = t & 63, lr = ln & 15, lk = ln >> 4;
    f16::Frag<T> acc[3] = {f16::zero<T>(), f16::zero<T>(), f16::zero<T>()};
    for (int kk = 0; kk < sb / 4; ++kk) {
      const int k = 4 * kk + lk;
      const T a = Tt[(16 * wv + lr) * sb + k];
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) {
        const int cc = 16 * cb + lr;
        const T bv = cc < sb ? Ri[k * sb + cc] : T(0);
        acc[cb] = f16::Mfma<T>::op(a, bv, acc[cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < 3; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * wv + f16::Mfma<T>::row(lk, r), cc = 16 * cb + lr;
        const int ra = h / b, i = h - ra * b, j = cc % b;
        if (cc < sb && ra < rows) {
          const int32_t o = codes[ra * s + cc / b];
          T *dst = G_lower + (mat * d.nnz + (o >> 1)) * bb;
          dst[(o & 1) ? j * b + i : i * b + j] = -acc[cb][r];
        }
      }
    return;
  }
  for (int e = threadIdx.x; e < rows * b * sb; e += kJT) {
    const int h = e / sb, cc = e - h * sb;
    T v = T(0);
#pragma unroll 4
    for (int kk = cc; kk < sb; ++kk) v += Tt[h * sb + kk] * Ri[kk * sb + cc];
    const int ra = h / b, i = h - ra * b, j = cc % b;
    const int32_t o = codes[ra * s + cc / b];
    T *dst = G_lower + (mat * d.nnz + (o >> 1)) * bb;
    dst[(o & 1) ? j * b + i : i * b + j] = -v;
  }
}

// Partial sums of a split row tile: kTilePart entries per (tile, part)
constexpr int kTilePart = 64 * 48;

template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_bwd_rows(JunctionPlanDev P, Dims d, int64_t tbase,
                                                   int nsplit, T *Tpart,
                                                   const T *__restrict__ W,
                                                   const T *__restrict__ RJ, const T *G_diag,
                                                   T *G_lower) {
  extern __shared__ char smem_raw[];
  const T **tab = reinterpret_cast<const T **>(smem_raw);
  unsigned char *fl = reinterpret_cast<unsigned char *>(tab + kTileTable);
  T *stage = reinterpret_cast<T *>(smem_raw + kTileTableBytes);
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  const int R = tile_rows(b), H = R * b;
  const WgXM wg = xcd_wg();
  const int64_t bx = wg.x, tl = bx / nsplit, mat = wg.mat;
  const int part = static_cast<int>(bx - tl * nsplit);
  const int64_t tile = tbase + tl;
  const int id = P.tile_chunk[tile];
  const int a0 = static_cast<int>(tile - P.tiles_ptr[id]) * R;
  const int s = P.ch_s[id], nr = P.ch_n[id], sb = s * b;
  const int rows = nr - a0 < R ? nr - a0 : R;  // valid rows of this tile
  // this part's range of the sum over x (all of it without a split)
  const int qlo = static_cast<int>(int64_t(nr) * part / nsplit);
  const int qhi = static_cast<int>(int64_t(nr) * (part + 1) / nsplit);
  const int CQ = tile_steps(b, s);
  T *sA = stage, *sB = sA + CQ * H * b;
  const int64_t pb = P.ch_pbase[id];
  const T *Wp = W + (mat * d.npanel + pb) * bb;
  const T *Gd = G_diag + mat * d.n * bb, *Gl = G_lower + mat * d.nnz * bb;
  const int32_t *gt = P.gtab + P.ch_gptr[id];
  const int ty = t / 16, tx = t % 16;  // rows 4 ty .. 4 ty + 3, columns tx + 16 j
  // b a multiple of 4 (compile time): the products run on the matrix cores,
  // wavefront w owning rows 16 w .. 16 w + 15 of the tile and the column
  // blocks 16 cb .. 16 cb + 15 (cb < 3); otherwise a 4 x 3 register tile per
  // thread on the vector units
  constexpr bool kMfma = BC != 0 && BC % 4 == 0;
  const int wv = t >> 6, ln = t & 63, lr = ln & 15, lk = ln >> 4;
  f16::Frag<T> accm[3] = {f16::zero<T>(), f16::zero<T>(), f16::zero<T>()};
  T acc[4][3];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[r][j] = T(0);
  for (int q0 = qlo; q0 < qhi; q0 += CQ) {
    const int cnt = qhi - q0 < CQ ? qhi - q0 : CQ;
    // table: block G_{w_{a0+ra}, x_{q0+q}} for ra < rows, q < cnt
    for (int e = t; e < cnt * R; e += kJT) {
      const int q = e / R, ra = e - q * R;
      if (ra < rows) {
        const int32_t enc = gt[int64_t(a0 + ra) * nr + q0 + q];
        tab[e] = enc < 0 ? Gd + int64_t(-enc - 1) * bb : Gl + int64_t(enc >> 1) * bb;
        fl[e] = enc >= 0 && (enc & 1);
      } else {
        tab[e] = nullptr;
        fl[e] = 0;
      }
    }
    __syncthreads();
    // sA[q][h][k] = G_{w(h), x_q}[h % b][k]  (H x b per step)
    gather_lds(sA, cnt * H * b, [&](int e) {
      const int q = e / (H * b), rem = e - q * H * b, h = rem / b, k = rem - h * b;
      const int ra = h / b, i = h - ra * b;
      const T *src = tab[q * R + ra];
      return src ? src[fl[q * R + ra] ? k * b + i : i * b + k] : T(0);
    });
    // sB[q][k][cc] = W_{x_q,J}[k][cc]  (b x sb per step, panel row s + q0 + q)
    gather_lds(sB, cnt * b * sb, [&](int e) {
      const int q = e / (b * sb), rem = e - q * b * sb, k = rem / sb, cc = rem - k * sb;
      return Wp[(int64_t(s + q0 + q) * s + cc / b) * bb + k * b + cc % b];
    });
    __syncthreads();
    if constexpr (kMfma) {
      // one MFMA step per 4 of the b inner indices: lane (lk, lr) supplies
      // A[16 w + lr][4 kk + lk] and B[4 kk + lk][16 cb + lr]
      for (int q = 0; q < cnt; ++q) {
        const T *A = sA + q * H * b, *Bq = sB + q * b * sb;
#pragma unroll
        for (int kk = 0; kk < BC / 4; ++kk) {
          const int k = 4 * kk + lk;
          const T a = A[(16 * wv + lr) * b + k];
#pragma unroll
          for (int cb = 0; cb < 3; ++cb) {
            const int cc = 16 * cb + lr;
            const T bv = cc < sb ? Bq[k * sb + cc] : T(0);
            accm[cb] = f16::Mfma<T>::op(a, bv, accm[cb]);
          }
        }
      }
      __syncthreads();
      continue;
    }
    for (int q = 0; q < cnt; ++q) {
      const T *A = sA + q * H * b, *Bq = sB + q * b * sb;
      for (int k = 0; k < b; ++k) {
        T av[4], bv[3];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * ty + r;
          av[r] = h < H ? A[h * b + k] : T(0);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int cc = tx + 16 * j;
          bv[j] = cc < sb ? Bq[k * sb + cc] : T(0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int j = 0; j < 3; ++j) acc[r][j] += av[r] * bv[j];
      }
    }
    __syncthreads();
  }
  // the tile's H x sb result, row-major, to dst
  auto put_tile = [&](T *dst) {
    if constexpr (kMfma) {
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 16 * wv + f16::Mfma<T>::row(lk, r), cc = 16 * cb + lr;
          if (cc < sb) dst[h * sb + cc] = accm[cb][r];
        }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int h = 4 * ty + r, cc = tx + 16 * j;
          if (h < H && cc < sb) dst[h * sb + cc] = acc[r][j];
        }
    }
  };
  if (nsplit > 1) {  // partial sum to the workspace; jt_bwd_rows_sum finishes the tile
    put_tile(Tpart + ((mat * gridDim.x + bx)) * int64_t(kTilePart));
    return;
  }
  // epilogue: T (H x sb) and R_J^-1 in LDS, then -T R_J^-1 to the output
  T *Tt = stage, *Ri = Tt + H * sb;
  put_tile(Tt);
  rows_epilogue<BC>(P, d, mat, id, a0, rows, Tt, Ri, RJ, G_lower);
}

// Split row tiles: sum the parts in a fixed order, then the epilogue
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_bwd_rows_sum(JunctionPlanDev P, Dims d, int64_t tbase,
                                                       int nsplit, const T *Tpart,
                                                       const T *__restrict__ RJ, T *G_lower) {
  extern __shared__ char smem_raw[];
  T *Tt = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, R = tile_rows(b), H = R * b;
  const int64_t tl = blockIdx.x, mat = blockIdx.y;
  const int64_t tile = tbase + tl;
  const int id = P.tile_chunk[tile];
  const int a0 = static_cast<int>(tile - P.tiles_ptr[id]) * R;
  const int nr = P.ch_n[id], sb = P.ch_s[id] * b;
  const int rows = nr - a0 < R ? nr - a0 : R;
  const T *src = Tpart + (mat * int64_t(gridDim.x) * nsplit + tl * nsplit) * int64_t(kTilePart);
  // each thread owns at most 12 entries (H sb <= 3072): one batch of loads
  // per part, added in part order
  T v[12];
#pragma unroll
  for (int u = 0; u < 12; ++u) v[u] = T(0);
  for (int p = 0; p < nsplit; ++p) {
    T x[12];
#pragma unroll
    for (int u = 0; u < 12; ++u) {
      const int e = threadIdx.x + u * kJT;
      x[u] = e < H * sb ? src[p * int64_t(kTilePart) + e] : T(0);
    }
#pragma unroll
    for (int u = 0; u < 12; ++u) v[u] += x[u];
  }
#pragma unroll
  for (int u = 0; u < 12; ++u) {
    const int e = threadIdx.x + u * kJT;
    if (e < H * sb) Tt[e] = v[u];
  }
  // (rows_epilogue's first gather is followed by a barrier before Tt is read)
  rows_epilogue<BC>(P, d, mat, id, a0, rows, Tt, Tt + H * sb, RJ, G_lower);
}

// Epilogue of a chunk block column: X (LDS, sb x b) = (R_J^-1 - W^T G)_{:,col}
// is mapped to G_{J,col} = R_J^-T X; the blocks on and below the diagonal are
// written (the diagonal block symmetrised).  Y is LDS scratch of sb b entries
// followed by room for s codes.
template <int BC, typename T>
__device__ inline void diag_epilogue(const JunctionPlanDev &P, const Dims &d, int64_t mat, int id,
                                     int col, const T *Ri, const T *X, T *Y, T *G_diag,
                                     T *G_lower) {
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  const int s = P.ch_s[id], sb = s * b, ob = sb * b, f = P.ch_first[id];
  const int64_t pb = P.ch_pbase[id];
  int32_t *codes = reinterpret_cast<int32_t *>(Y + ob);  // block (r, col), r < s
  for (int r = t; r < s; r += kJT) codes[r] = P.poutenc[pb + int64_t(r) * s + col];
  // rows I >= col b: sum over K >= I of Ri[K][I] X[K][j]
  for (int e = t; e < ob; e += kJT) {
    const int I = e / b, j = e - I * b;
    if (I < col * b) continue;
    T y = T(0);
    for (int K = I; K < sb; ++K) y += Ri[K * sb + I] * X[K * b + j];
    Y[e] = y;
  }
  __syncthreads();
  for (int e = t; e < ob; e += kJT) {
    const int I = e / b, j = e - I * b, r = I / b, i = I - r * b;
    if (r < col) continue;
    if (r == col) {
      if (i < j) continue;
      const T v = T(0.5) * (Y[I * b + j] + Y[(col * b + j) * b + i]);
      T *dst = G_diag + (mat * d.n + P.order[f + r]) * bb;
      dst[i * b + j] = v;
      dst[j * b + i] = v;
    } else {
      const int32_t o = codes[r];
      T *dst = G_lower + (mat * d.nnz + (o >> 1)) * bb;
      dst[(o & 1) ? j * b + i : i * b + j] = Y[e];
    }
  }
}

// Partial sums of a split block column: kDiagPart entries per (column, part)
constexpr int kDiagPart = 48 * 32;

// The chunk's own blocks, one workgroup per block column col of the chunk:
// G_{J,col} = R_J^-T (R_J^-1 - W_{N,J}^T G_{N,J})_{:,col}.  On levels with
// few columns the sum over the later rows is split into nsplit parts whose
// partial sums go to Dpart; jt_bwd_diag_sum finishes those columns.
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_bwd_diag(JunctionPlanDev P, Dims d, int64_t fcbase,
                                                   int nsplit, T *Dpart,
                                                   const T *__restrict__ W,
                                                   const T *__restrict__ RJ, T *G_diag,
                                                   T *G_lower) {
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  const WgXM wg = xcd_wg();
  const int64_t bx = wg.x, fcl = bx / nsplit, mat = wg.mat;
  const int part = static_cast<int>(bx - fcl * nsplit);
  const int64_t fc = fcbase + fcl;
  const int id = P.col_chunk[fc], col = static_cast<int>(fc - P.ch_cptr[id]);
  const int s = P.ch_s[id], nr = P.ch_n[id], sb = s * b, wr = b * sb;
  const int CH = diag_pairs(b, s), ob = sb * b;  // output: sb x b
  T *sA = Ri + sb * sb, *sB = sA + CH * wr;
  const int64_t pb = P.ch_pbase[id];
  const T *Wp = W + (mat * d.npanel + pb) * bb;
  const T *Gl = G_lower + mat * d.nnz * bb;
  const int qlo = static_cast<int>(int64_t(nr) * part / nsplit);
  const int qhi = static_cast<int>(int64_t(nr) * (part + 1) / nsplit);
  T acc[6] = {T(0), T(0), T(0), T(0), T(0), T(0)};
  // b a multiple of 4 (compile time): the sum runs on the matrix cores
  constexpr bool kMfma = BC != 0 && BC % 4 == 0;
  const int wv = t >> 6, ln = t & 63, lr = ln & 15, lk = ln >> 4;
  f16::Frag<T> accm = f16::zero<T>();
  for (int q0 = qlo; q0 < qhi; q0 += CH) {
    const int cnt = qhi - q0 < CH ? qhi - q0 : CH;
    // W_{x_q,J} as dense b x sb rows; G_{x_q, f+col} blocks
    gather_lds(sA, cnt * wr, [&](int e) {
      const int q = e / wr, rem = e - q * wr, k = rem / sb, cc = rem - k * sb;
      return Wp[(int64_t(s + q0 + q) * s + cc / b) * bb + k * b + cc % b];
    });
    gather_lds(sB, cnt * bb, [&](int e) {
      const int q = e / bb, el = e - q * bb, k = el / b, j = el - k * b;
      const int32_t o = P.poutenc[pb + int64_t(s + q0 + q) * s + col];
      return Gl[int64_t(o >> 1) * bb + ((o & 1) ? j * b + k : el)];
    });
    __syncthreads();
    if constexpr (kMfma) {
      // wavefront w < 3 owns rows 16 w .. 16 w + 15 of the sb x b result;
      // lane (lk, lr) supplies W_q[k][16 w + lr] and G_q[k][lr], k = 4 kk + lk
      if (wv < 3 && 16 * wv < sb) {
        for (int q = 0; q < cnt; ++q) {
          const T *A = sA + q * wr, *Bq = sB + q * bb;
#pragma unroll
          for (int kk = 0; kk < BC / 4; ++kk) {
            const int k = 4 * kk + lk, I = 16 * wv + lr;
            const T a = I < sb ? A[k * sb + I] : T(0);
            const T bv = lr < b ? Bq[k * b + lr] : T(0);
            accm = f16::Mfma<T>::op(a, bv, accm);
          }
        }
      }
    } else {
      for (int u = 0; u < 6; ++u) {
        const int e = t + u * kJT;
        if (e >= ob) break;
        const int I = e / b, j = e - I * b;
        for (int q = 0; q < cnt; ++q) {
          const T *A = sA + q * wr + I, *Bq = sB + q * bb + j;
          T v = T(0);
          for (int k = 0; k < b; ++k) v += A[k * sb] * Bq[k * b];
          acc[u] += v;
        }
      }
    }
    __syncthreads();
  }
  if constexpr (kMfma) {  // the matrix-core result to acc[] in the vector layout, through sA
    if (wv < 3)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int I = 16 * wv + f16::Mfma<T>::row(lk, r);
        if (I < sb && lr < b) sA[I * b + lr] = accm[r];
      }
    __syncthreads();
    for (int u = 0; u < 6; ++u) {
      const int e = t + u * kJT;
      if (e < ob) acc[u] = sA[e];
    }
    __syncthreads();
  }
  if (nsplit > 1) {
    T *dst = Dpart + (mat * gridDim.x + bx) * int64_t(kDiagPart);
    for (int u = 0; u < 6; ++u) {
      const int e = t + u * kJT;
      if (e < ob) dst[e] = acc[u];
    }
    return;
  }
  gather_lds(Ri, sb * sb, [&](int e) { return RJ[(mat * d.nrinv + P.ch_rbase[id]) * bb + e]; });
  __syncthreads();
  T *X = sA;  // sb x b column block of R^-1 - W^T G
  for (int u = 0; u < 6; ++u) {
    const int e = t + u * kJT;
    if (e >= ob) break;
    const int I = e / b, j = e - I * b;
    X[e] = Ri[I * sb + col * b + j] - acc[u];
  }
  __syncthreads();
  diag_epilogue<BC>(P, d, mat, id, col, Ri, X, sA + ob, G_diag, G_lower);
}

// Split block columns: the parts added in a fixed order, then the epilogue
template <typename T, int BC>
__global__ void __launch_bounds__(kJT) jt_bwd_diag_sum(JunctionPlanDev P, Dims d, int64_t fcbase,
                                                       int nsplit, const T *Dpart,
                                                       const T *__restrict__ RJ, T *G_diag,
                                                       T *G_lower) {
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  const int64_t fcl = blockIdx.x, mat = blockIdx.y, fc = fcbase + fcl;
  const int id = P.col_chunk[fc], col = static_cast<int>(fc - P.ch_cptr[id]);
  const int sb = P.ch_s[id] * b, ob = sb * b;
  T *X = Ri + sb * sb;
  const T *src = Dpart + (mat * int64_t(gridDim.x) * nsplit + fcl * nsplit) * int64_t(kDiagPart);
  T v[6] = {T(0), T(0), T(0), T(0), T(0), T(0)};
  for (int p = 0; p < nsplit; ++p) {
    T x[6];
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int e = t + u * kJT;
      x[u] = e < ob ? src[p * int64_t(kDiagPart) + e] : T(0);
    }
#pragma unroll
    for (int u = 0; u < 6; ++u) v[u] += x[u];
  }
  gather_lds(Ri, sb * sb, [&](int e) { return RJ[(mat * d.nrinv + P.ch_rbase[id]) * bb + e]; });
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int e = t + u * kJT;
    if (e < ob) {
      const int I = e / b, j = e - I * b;
      X[e] = Ri[I * sb + col * b + j] - v[u];
    }
  }
  __syncthreads();
  diag_epilogue<BC>(P, d, mat, id, col, Ri, X, X + ob, G_diag, G_lower);
}

template <typename T>
__global__ void __launch_bounds__(kJT) jt_finish(JunctionPlanDev P, int64_t nch,
                                                 const double *ld_ws, const int32_t *info_ws,
                                                 double *logdet, int32_t *info) {
  __shared__ double red[kJT];
  const int64_t mat = blockIdx.x;
  double s = 0.0;
  for (int64_t c = threadIdx.x; c < nch; c += kJT) s += ld_ws[mat * nch + c];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kJT / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t f = info_ws[mat];
    logdet[mat] = f == INT_MAX ? red[0] : __builtin_nan("");
    if (info) info[mat] = f == INT_MAX ? 0 : 1 + P.order[f];
  }
}

// Parts of the sum over x for the row tiles of a level: enough workgroups
// to occupy the chip (about 1024) when a level has few tiles.
int rows_split(int64_t tiles, int64_t B) {
  const int64_t wgs = tiles * B;
  if (wgs <= 0 || wgs >= 1024) return 1;
  const int64_t p = (1024 + wgs - 1) / wgs;
  return static_cast<int>(p > 8 ? 8 : p);
}

int64_t max_split_cols(const selinv_junction_plan *plan, int64_t B) {
  int64_t best = 0;
  for (int32_t l = 0; l < plan->levels; ++l) {
    const int64_t c = plan->ch_cptr[plan->level_off[l + 1]] - plan->ch_cptr[plan->level_off[l]];
    const int p = rows_split(c, B);
    if (p > 1 && c * p > best) best = c * p;
  }
  return best;
}

int64_t max_split_tiles(const selinv_junction_plan *plan, int64_t B) {
  int64_t best = 0;
  for (int32_t l = 0; l < plan->levels; ++l) {
    const int64_t t = plan->tiles_ptr[plan->level_off[l + 1]] - plan->tiles_ptr[plan->level_off[l]];
    const int p = rows_split(t, B);
    if (p > 1 && t * p > best) best = t * p;
  }
  return best;
}

struct JtWs {
  void *W, *RJ, *Tpart, *Dpart, *Spart;
  double *ld;
  int32_t *info;
  size_t bytes;
};

// ext_factor: W and RJ live in a caller-owned factor buffer (not carved)
JtWs carve(const selinv_junction_plan *plan, int64_t B, void *ws, bool ext_factor = false) {
  const size_t bb = size_t(plan->b) * plan->b, es = plan->dtype_bytes;
  Carve cv(ws);
  JtWs w;
  w.W = ext_factor ? nullptr : cv.take<char>(B * plan->npanel * bb * es);
  w.RJ = ext_factor ? nullptr : cv.take<char>(B * plan->nrinv * bb * es);
  w.Tpart = cv.take<char>(B * max_split_tiles(plan, B) * kTilePart * es);
  w.Dpart = cv.take<char>(B * max_split_cols(plan, B) * kDiagPart * es);
  w.Spart = cv.take<char>(B * plan->max_slots * bb * es);
  w.ld = cv.take<double>(B * plan->nch);
  w.info = cv.take<int32_t>(B);
  w.bytes = cv.off;
  return w;
}

}  // namespace

size_t junction_workspace_bytes(const selinv_junction_plan *plan, int64_t B) {
  return carve(plan, B, nullptr).bytes;
}

size_t junction_factor_workspace_bytes(const selinv_junction_plan *plan, int64_t B) {
  return carve(plan, B, nullptr, true).bytes;
}

// The factor a solve or a sample reads: every chunk's panel (the later rows
// W_{N,J}; the pivot rows hold C_JJ) [B][npanel][b][b], then every chunk's
// R_J^-1 (dense, row-major s b x s b) [B][nrinv][b][b].
size_t junction_factor_bytes(const selinv_junction_plan *plan, int64_t B) {
  return size_t(B) * (plan->npanel + plan->nrinv) * plan->b * plan->b * plan->dtype_bytes;
}

// G_diag == nullptr: the factorisation alone (log det and info); factor !=
// nullptr: W and R_J^-1 are kept there (junction_factor_bytes layout)
template <typename T, int BC>
hipError_t junction_run(const selinv_junction_plan *plan, int64_t B, const T *diag,
                           const T *edge_val, T *G_diag, T *G_lower, double *logdet,
                           int32_t *info, void *ws, hipStream_t s, T *factor = nullptr) {
  const int b = plan->b, sm = plan->smax;
  const Dims d{plan->n, plan->m, plan->nnz, plan->nch, plan->npanel, plan->nrinv, b};
  const JunctionPlanDev &P = plan->dev;
  const JtWs w = carve(plan, B, ws, factor != nullptr);
  T *W = factor ? factor : static_cast<T *>(w.W);
  T *RJ = factor ? factor + B * plan->npanel * int64_t(b) * b : static_cast<T *>(w.RJ);
  const size_t l_upd = lds_bytes<T>(b), l_fac = fac_lds<T>(b, sm), l_scl = scale_lds<T>(b, sm),
               l_row = rows_lds<T>(b, sm), l_dia = diag_lds<T>(b, sm),
               l_sum = sizeof(T) * (size_t(kTilePart) + size_t(sm) * b * sm * b) +
                       4 * size_t(tile_rows(b)) * sm,
               l_dsum = sizeof(T) * (size_t(sm) * b * sm * b + 3 * size_t(sm) * b * b) + 4 * sm;
  const size_t l_sct = sizeof(T) * (size_t(sm) * b * sm * b + 64 * size_t(sm) * b);
  if (l_upd > kLdsMax || l_fac > kLdsMax || l_scl > kLdsMax || l_sct > kLdsMax || l_row > kLdsMax ||
      l_dia > kLdsMax || l_sum > kLdsMax || l_dsum > kLdsMax)
    return hipErrorInvalidValue;
  const auto &lo = plan->level_off;
  const auto &tp = plan->ch_tptr;
  const auto &rp = plan->rows_ptr;
  const unsigned By = static_cast<unsigned>(B);
  const dim3 blk(kJT);
  jt_init<T><<<dim3(static_cast<unsigned>((B + kJT - 1) / kJT)), blk, 0, s>>>(w.info, B);
  for (int32_t l = 0; l < plan->levels; ++l) {
    const int64_t c0 = lo[l], c1 = lo[l + 1];
    if constexpr (BC == 4 || BC == 8) {
      const auto &ip = plan->it_ptr;
      const int64_t i0 = ip[tp[c0]], i1 = ip[tp[c1]];
      T *Sp = static_cast<T *>(w.Spart);
      jt_fwd_update_wave<T, BC><<<dim3(static_cast<unsigned>((i1 - i0 + 3) / 4), By), blk, 0, s>>>(
          P, d, i0, i1, plan->max_slots, Sp, diag, edge_val, W);
      const int64_t m0 = plan->multi_off[l], m1 = plan->multi_off[l + 1];
      if (m1 > m0)
        jt_fwd_update_sum<T, BC><<<dim3(static_cast<unsigned>((m1 - m0 + 3) / 4), By), blk, 0, s>>>(
            P, d, m0, m1, plan->max_slots, Sp, diag, edge_val, W);
    } else {
      jt_fwd_update<T, BC><<<dim3(static_cast<unsigned>(tp[c1] - tp[c0]), By), blk, l_upd, s>>>(
          P, d, tp[c0], diag, edge_val, W);
    }
    jt_fwd_factor<T, BC><<<dim3(static_cast<unsigned>(c1 - c0), By), blk, l_fac, s>>>(
        P, d, c0, W, RJ, w.ld, w.info);
    if constexpr (BC == 4 || BC == 8 || BC == 16) {
      const auto &tl = plan->tiles_ptr;
      const int64_t nt = tl[c1] - tl[c0];
      if (nt > 0)
        jt_fwd_scale_tiles<T, BC><<<dim3(static_cast<unsigned>(nt), By), blk, l_sct, s>>>(
            P, d, tl[c0], W, RJ);
    } else if (rp[c1] > rp[c0]) {
      jt_fwd_scale<T, BC><<<dim3(static_cast<unsigned>(rp[c1] - rp[c0]), By), blk, l_scl, s>>>(
          P, d, rp[c0], W, RJ);
    }
  }
  for (int32_t l = G_diag ? plan->levels - 1 : -1; l >= 0; --l) {
    const int64_t c0 = lo[l], c1 = lo[l + 1];
    const auto &tl = plan->tiles_ptr;
    const int64_t nt = tl[c1] - tl[c0];
    if (nt > 0) {
      const int sp = rows_split(nt, B);
      jt_bwd_rows<T, BC><<<dim3(static_cast<unsigned>(nt * sp), By), blk, l_row, s>>>(
          P, d, tl[c0], sp, static_cast<T *>(w.Tpart), W, RJ, G_diag, G_lower);
      if (sp > 1)
        jt_bwd_rows_sum<T, BC><<<dim3(static_cast<unsigned>(nt), By), blk, l_sum, s>>>(
            P, d, tl[c0], sp, static_cast<const T *>(w.Tpart), RJ, G_lower);
    }
    const int64_t f0 = plan->ch_cptr[c0], f1 = plan->ch_cptr[c1];
    const int dsp = rows_split(f1 - f0, B);
    jt_bwd_diag<T, BC><<<dim3(static_cast<unsigned>((f1 - f0) * dsp), By), blk, l_dia, s>>>(
        P, d, f0, dsp, static_cast<T *>(w.Dpart), W, RJ, G_diag, G_lower);
    if (dsp > 1)
      jt_bwd_diag_sum<T, BC><<<dim3(static_cast<unsigned>(f1 - f0), By), blk, l_dsum, s>>>(
          P, d, f0, dsp, static_cast<const T *>(w.Dpart), RJ, G_diag, G_lower);
  }
  jt_finish<T><<<dim3(By), blk, 0, s>>>(P, plan->nch, w.ld, w.info, logdet, info);
  return hipGetLastError();
}

// Compile-time block sizes for the common b (fully unrolled inner loops),
// the runtime b otherwise
template <typename T>
hipError_t junction_launch(const selinv_junction_plan *plan, int64_t B, const T *diag,
                           const T *edge_val, T *G_diag, T *G_lower, double *logdet,
                           int32_t *info, void *ws, hipStream_t s) {
  switch (plan->b) {
    case 4: return junction_run<T, 4>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, ws, s);
    case 8: return junction_run<T, 8>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, ws, s);
    case 16: return junction_run<T, 16>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, ws, s);
    default: return junction_run<T, 0>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, ws, s);
  }
}

// The factorisation alone, keeping W and R_J^-1 in `factor` for the sweeps
template <typename T>
hipError_t junction_factor_launch(const selinv_junction_plan *plan, int64_t B, const T *diag,
                                  const T *edge_val, T *factor, double *logdet, int32_t *info,
                                  void *ws, hipStream_t s) {
  switch (plan->b) {
    case 4: return junction_run<T, 4>(plan, B, diag, edge_val, nullptr, nullptr, logdet, info, ws, s, factor);
    case 8: return junction_run<T, 8>(plan, B, diag, edge_val, nullptr, nullptr, logdet, info, ws, s, factor);
    case 16: return junction_run<T, 16>(plan, B, diag, edge_val, nullptr, nullptr, logdet, info, ws, s, factor);
    default: return junction_run<T, 0>(plan, B, diag, edge_val, nullptr, nullptr, logdet, info, ws, s, factor);
  }
}

template hipError_t junction_factor_launch<double>(const selinv_junction_plan *, int64_t,
                                                   const double *, const double *, double *,
                                                   double *, int32_t *, void *, hipStream_t);
template hipError_t junction_factor_launch<float>(const selinv_junction_plan *, int64_t,
                                                  const float *, const float *, float *, double *,
                                                  int32_t *, void *, hipStream_t);
template hipError_t junction_launch<double>(const selinv_junction_plan *, int64_t, const double *,
                                            const double *, double *, double *, double *,
                                            int32_t *, void *, hipStream_t);
template hipError_t junction_launch<float>(const selinv_junction_plan *, int64_t, const float *,
                                           const float *, float *, float *, double *, int32_t *,
                                           void *, hipStream_t);

}  // namespace selinv
