// chain_solve_b16.hip -- solve with the shared factor of b = 16 chains
// ("Factor once, do everything" on the gabp-sparse-inv 0.3.2 page: the
// factor of the collect pass is reused for solves): one wavefront per chain
// and chunk of up to 16 right-hand sides (one wavefront per chain when there
// are at most 4).
//
// With the chain rooted at its last block, A = L D L^T, D = blockdiag(S_i),
// L_{i+1,i} = C_i S_i^-1 (C_i = lower[i]); the factor holds the packed lower
// triangle of every S_i^-1 (entry (a, c), a >= c, at a (a + 1) / 2 + c):
//   forward:  u_0 = y_0,  u_i = y_i - C_{i-1} w_{i-1},  w_i = Sinv_i u_i
//   backward: x_{L-1} = w_{L-1},  x_i = w_i - Sinv_i C_i^T x_{i+1}
// Lane (r, q) = (lane % 16, lane / 16) owns row r of every block and the
// columns q, q + 4, q + 8, q + 12 of the chunk.  The packed Sinv_i and the
// coupling block are loaded with coalesced accesses one step ahead, staged in
// LDS, and each lane takes row r of Sinv_i and row r (forward) or column r
// (backward) of the coupling from there; the vector being multiplied is read
// from LDS too, so each step waits only on LDS and arithmetic.
#include "frag16.h"
#include "internal.h"

namespace selinv {

namespace {

constexpr int kCols = 16;    // right-hand sides per wavefront
constexpr int kPerLane = 4;  // columns per lane
constexpr int kPB = 136;     // packed 16 x 16 triangle

template <typename T>
struct Rows {
  T v[16];
};

// A step's factor and coupling blocks, loaded coalesced (packed Sinv: entries
// lane, lane + 64, lane + 128 < 136; coupling: entries 4 lane .. 4 lane + 3)
// and handed to the lanes' rows through LDS.
template <typename T>
struct Raw {
  T p[3];
  T c[4];
};

// Cb == nullptr (a chain of one block): no coupling block, zeros
template <typename T>
__device__ __forceinline__ void load_raw(Raw<T> &w, const T *P, const T *Cb, int lane) {
#pragma unroll
  for (int t = 0; t < 3; ++t) w.p[t] = (lane + 64 * t < kPB) ? P[lane + 64 * t] : T(0);
#pragma unroll
  for (int t = 0; t < 4; ++t) w.c[t] = Cb ? Cb[4 * lane + t] : T(0);
}

template <typename T>
__device__ __forceinline__ void put_raw(T *sP, T *sC, const Raw<T> &w, int lane) {
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (lane + 64 * t < kPB) sP[lane + 64 * t] = w.p[t];
#pragma unroll
  for (int t = 0; t < 4; ++t) sC[4 * lane + t] = w.c[t];
}

template <typename T>
__device__ __forceinline__ Rows<T> sinv_row(const T *P, int r) {
  Rows<T> s;
#pragma unroll
  for (int c = 0; c < 16; ++c) s.v[c] = P[c <= r ? r * (r + 1) / 2 + c : c * (c + 1) / 2 + r];
  return s;
}

template <typename T>
__device__ __forceinline__ Rows<T> block_row(const T *P, int r) {
  Rows<T> s;
#pragma unroll
  for (int c = 0; c < 16; ++c) s.v[c] = P[r * 16 + c];
  return s;
}

template <typename T>
__device__ __forceinline__ Rows<T> block_col(const T *P, int r) {
  Rows<T> s;
#pragma unroll
  for (int c = 0; c < 16; ++c) s.v[c] = P[c * 16 + r];
  return s;
}

// this lane's entries of row r of a b x kc vector block (row stride k)
template <typename T>
__device__ __forceinline__ void load_vec(T (&out)[kPerLane], const T *row, int q, int kc) {
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) {
    const int c = q + 4 * t;
    out[t] = c < kc ? row[c] : T(0);
  }
}

template <typename T>
__device__ __forceinline__ void store_vec(T *row, const T (&v)[kPerLane], int q, int kc) {
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) {
    const int c = q + 4 * t;
    if (c < kc) row[c] = v[t];
  }
}

// out_t = sum_j a_j V[j][q + 4 t]  (V in LDS, [16][kCols])
template <typename T>
__device__ __forceinline__ void row_times(T (&out)[kPerLane], const Rows<T> &a, const T *V, int q) {
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) out[t] = T(0);
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) out[t] += a.v[j] * V[j * kCols + q + 4 * t];
}

template <typename T>
__device__ __forceinline__ void put(T *V, int r, int q, const T (&v)[kPerLane]) {
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) V[r * kCols + q + 4 * t] = v[t];
}

template <typename T>
__global__ __launch_bounds__(64) void chain16_solve(int L, int64_t k, int nch,
                                                   const T *__restrict__ lower,
                                                   const T *__restrict__ factor,
                                                   const T *__restrict__ y, T *__restrict__ x) {
  __shared__ __align__(16) T bufA[16 * kCols];
  __shared__ __align__(16) T bufB[16 * kCols];
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T sC[256];
  const int lane = threadIdx.x, r = lane & 15, q = lane >> 4;
  const int64_t m = blockIdx.x / nch;
  const int64_t c0 = int64_t(blockIdx.x % nch) * kCols;
  const int kc = static_cast<int>(min<int64_t>(kCols, k - c0));
  const T *F = factor + m * L * kPB;
  // with L == 1 there is no coupling block (lower may be null) and none is read
  const T *C = L > 1 ? lower + m * (L - 1) * 256 : nullptr;
  const int lc = L > 1 ? L - 2 : 0;
  auto vrow = [&](const T *base, int i) { return base + ((m * L + i) * 16 + r) * k + c0; };
  auto vrow_w = [&](T *base, int i) { return base + ((m * L + i) * 16 + r) * k + c0; };
  auto coupling = [&](int i) -> const T * {
    return C ? C + int64_t(min(max(i, 0), lc)) * 256 : nullptr;
  };

  // forward: L D w = y.  Step i uses Sinv_i and C_{i-1}.
  Raw<T> nx;
  load_raw(nx, F, coupling(-1), lane);
  T yn[kPerLane];
  load_vec(yn, vrow(y, 0), q, kc);
  for (int i = 0; i < L; ++i) {
    put_raw(sP, sC, nx, lane);
    T u[kPerLane];
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) u[t] = yn[t];
    if (i + 1 < L) {  // prefetch step i + 1: Sinv_{i+1}, C_i, y_{i+1}
      load_raw(nx, F + int64_t(i + 1) * kPB, coupling(i), lane);
      load_vec(yn, vrow(y, i + 1), q, kc);
    }
    f16::wave_sync();
    const Rows<T> Si = sinv_row(sP, r);
    if (i > 0) {  // u_i = y_i - C_{i-1} w_{i-1}, w_{i-1} in bufB
      const Rows<T> Cp = block_row(sC, r);
      T t2[kPerLane];
      row_times(t2, Cp, bufB, q);
#pragma unroll
      for (int t = 0; t < kPerLane; ++t) u[t] -= t2[t];
    }
    put(bufA, r, q, u);
    f16::wave_sync();
    T w[kPerLane];
    row_times(w, Si, bufA, q);  // w_i = Sinv_i u_i
    store_vec(vrow_w(x, i), w, q, kc);
    put(bufB, r, q, w);
    f16::wave_sync();
  }

  // backward: L^T x = w (x_{L-1} = w_{L-1} is already in place and in bufB).
  // Step i uses Sinv_i and C_i.
  if (L == 1) return;
  load_raw(nx, F + int64_t(L - 2) * kPB, coupling(L - 2), lane);
  load_vec(yn, vrow(x, L - 2), q, kc);  // w_{L-2}
  for (int i = L - 2; i >= 0; --i) {
    put_raw(sP, sC, nx, lane);
    T w[kPerLane];
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) w[t] = yn[t];
    if (i > 0) {  // prefetch step i - 1
      load_raw(nx, F + int64_t(i - 1) * kPB, coupling(i - 1), lane);
      load_vec(yn, vrow(x, i - 1), q, kc);
    }
    f16::wave_sync();
    const Rows<T> Si = sinv_row(sP, r);
    const Rows<T> Ct = block_col(sC, r);
    T t2[kPerLane];
    row_times(t2, Ct, bufB, q);  // C_i^T x_{i+1}, x_{i+1} in bufB
    put(bufA, r, q, t2);
    f16::wave_sync();
    T v[kPerLane];
    row_times(v, Si, bufA, q);  // Sinv_i C_i^T x_{i+1}
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) w[t] -= v[t];
    store_vec(vrow_w(x, i), w, q, kc);
    put(bufB, r, q, w);
    f16::wave_sync();
  }
}

// Up to four right-hand sides: lane (r, q) owns row r and the quarter
// j = 4q .. 4q + 3 of every dot product; the partial sums of the four lanes
// of a row are added by two cross-lane exchanges, after which all four hold
// the row's result.  That reads 4 (not 16) entries of each matrix row and of
// each vector column from LDS per product.
constexpr int kNarrow = 4;
// the solve runs column groups up to this k (measured: two groups beat the
// chunked kernel, four lose to it), the chunked kernel beyond
constexpr int64_t kGroupedMax = 8;

template <typename T>
__device__ __forceinline__ T row_sum(T v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <typename T>
__global__ __launch_bounds__(64) void chain16_solve_narrow(int L, int64_t k,
                                                          const T *__restrict__ lower,
                                                          const T *__restrict__ factor,
                                                          const T *__restrict__ y,
                                                          T *__restrict__ x) {
  __shared__ __align__(16) T bufA[16 * kNarrow];
  __shared__ __align__(16) T bufB[16 * kNarrow];
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T sC[256];
  const int lane = threadIdx.x, r = lane & 15, q = lane >> 4;
  // workgroup (m, grp) takes columns 4 grp .. 4 grp + 3 of chain m
  const int64_t ngrp = (k + kNarrow - 1) / kNarrow;
  const int64_t m = blockIdx.x / ngrp, k0 = (blockIdx.x - m * ngrp) * kNarrow;
  const int kc = static_cast<int>(k - k0 < kNarrow ? k - k0 : kNarrow);
  const T *F = factor + m * L * kPB;
  const T *C = L > 1 ? lower + m * (L - 1) * 256 : nullptr;  // none for one block
  const int lc = L > 1 ? L - 2 : 0;
  auto vrow = [&](const T *base, int i) { return base + ((m * L + i) * 16 + r) * k + k0; };
  auto vrow_w = [&](T *base, int i) { return base + ((m * L + i) * 16 + r) * k + k0; };
  auto coupling = [&](int i) -> const T * {
    return C ? C + int64_t(min(max(i, 0), lc)) * 256 : nullptr;
  };
  // this lane's quarter of row r of Sinv (packed) and of row r / column r of C
  auto sinv_q = [&](T (&o)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * q + t;
      o[t] = sP[c <= r ? r * (r + 1) / 2 + c : c * (c + 1) / 2 + r];
    }
  };
  // sum over this lane's quarter of a_j V[j][c], then over the row's lanes
  auto dot = [&](T (&o)[kNarrow], const T (&a)[4], const T *V) {
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) {
      T acc = T(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += a[t] * V[(4 * q + t) * kNarrow + c];
      o[c] = c < kc ? row_sum(acc) : T(0);
    }
  };
  auto put_row = [&](T *V, const T (&v)[kNarrow]) {
    if (q == 0)
#pragma unroll
      for (int c = 0; c < kNarrow; ++c) V[r * kNarrow + c] = v[c];
  };
  auto load_row = [&](T (&o)[kNarrow], const T *row) {
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) o[c] = c < kc ? row[c] : T(0);
  };
  auto store_row = [&](T *row, const T (&v)[kNarrow]) {
    if (q == 0)
#pragma unroll
      for (int c = 0; c < kNarrow; ++c)
        if (c < kc) row[c] = v[c];
  };

  Raw<T> nx;
  load_raw(nx, F, coupling(-1), lane);
  T yn[kNarrow];
  load_row(yn, vrow(y, 0));
  for (int i = 0; i < L; ++i) {  // forward: L D w = y
    put_raw(sP, sC, nx, lane);
    T u[kNarrow];
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) u[c] = yn[c];
    if (i + 1 < L) {
      load_raw(nx, F + int64_t(i + 1) * kPB, coupling(i), lane);
      load_row(yn, vrow(y, i + 1));
    }
    f16::wave_sync();
    T si[4];
    sinv_q(si);
    if (i > 0) {  // u_i = y_i - C_{i-1} w_{i-1}, w_{i-1} in bufB
      T cr[4], t2[kNarrow];
#pragma unroll
      for (int t = 0; t < 4; ++t) cr[t] = sC[r * 16 + 4 * q + t];
      dot(t2, cr, bufB);
#pragma unroll
      for (int c = 0; c < kNarrow; ++c) u[c] -= t2[c];
    }
    put_row(bufA, u);
    f16::wave_sync();
    T w[kNarrow];
    dot(w, si, bufA);  // w_i = Sinv_i u_i
    store_row(vrow_w(x, i), w);
    put_row(bufB, w);
    f16::wave_sync();
  }
  if (L == 1) return;
  load_raw(nx, F + int64_t(L - 2) * kPB, coupling(L - 2), lane);
  load_row(yn, vrow(x, L - 2));
  for (int i = L - 2; i >= 0; --i) {  // backward: L^T x = w
    put_raw(sP, sC, nx, lane);
    T w[kNarrow];
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) w[c] = yn[c];
    if (i > 0) {
      load_raw(nx, F + int64_t(i - 1) * kPB, coupling(i - 1), lane);
      load_row(yn, vrow(x, i - 1));
    }
    f16::wave_sync();
    T si[4], cc[4], t2[kNarrow];
    sinv_q(si);
#pragma unroll
    for (int t = 0; t < 4; ++t) cc[t] = sC[(4 * q + t) * 16 + r];
    dot(t2, cc, bufB);  // C_i^T x_{i+1}
    put_row(bufA, t2);
    f16::wave_sync();
    T v[kNarrow];
    dot(v, si, bufA);  // Sinv_i C_i^T x_{i+1}
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) w[c] -= v[c];
    store_row(vrow_w(x, i), w);
    put_row(bufB, w);
    f16::wave_sync();
  }
}

// Sampling, x = L^-T D^-1/2 z with D^-1/2 = blockdiag(U_i), U_i U_i^T =
// Sinv_i, U_i upper triangular (up to four right-hand sides): parents
// first, w_i = U_i z_i, x_{L-1} = w_{L-1}, x_i = w_i - Sinv_i C_i^T x_{i+1}.
// U_i is formed in registers, one block per step: lane (r, q) holds entries
// (r, q + 4t) of Sinv_i and turns them into those of U_i by the reversed
// (upper-lower) Cholesky, columns 15 down to 0: u_jj = sqrt(a_jj),
// u_rj = a_rj / u_jj (r < j), then a_rl -= u_rj u_lj for r, l < j.  Column j
// is broadcast through LDS.  Dot products use the same strided column sets.
// Any k: workgroup (m, grp) takes columns 4 grp .. 4 grp + 3 of chain m
// (grid B ceil(k / 4)); every group forms its chain's U_i itself.
// Sampling, x = L^-T D^-1/2 z with D^-1/2_i = U_i (U_i U_i^T = Sinv_i, U_i
// upper triangular), in two launches.  First w_i = U_i z_i for every block at
// once (one wavefront per block: U_i by the reversed Cholesky of Sinv_i,
// columns 15 down to 0, each broadcast through LDS, then the columns of z_i
// in groups of four), written to x; then the sequential backward sweep
// x_i = w_i - Sinv_i C_i^T x_{i+1}, which reads w_i from x and overwrites it.
template <typename T>
__global__ __launch_bounds__(64) void chain16_sample_w(int64_t k, const T *__restrict__ factor,
                                                       const T *__restrict__ z,
                                                       T *__restrict__ x) {
  __shared__ __align__(16) T bufA[16 * kNarrow];
  __shared__ __align__(16) T colj[16];
  __shared__ __align__(16) T sP[kPB];
  const int lane = threadIdx.x, r = lane & 15, q = lane >> 4;
  const int64_t blk = blockIdx.x;
  const T *P = factor + blk * kPB;
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (lane + 64 * t < kPB) sP[lane + 64 * t] = P[lane + 64 * t];
  f16::wave_sync();
  T u[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = q + 4 * t;
    u[t] = sP[c <= r ? r * (r + 1) / 2 + c : c * (c + 1) / 2 + r];
  }
  // reversed Cholesky of Sinv_i into u (entries (r, q + 4t) of U_i): column
  // j = sqrt(a_jj) on the diagonal, a_rj / u_jj above it; one reciprocal
  // square root per column
#pragma unroll
  for (int j = 15; j >= 0; --j) {
    const int tj = j >> 2;
    if ((j & 3) == q) colj[r] = u[tj];  // column j, current values
    f16::wave_sync();
    const T inv = f16::rsqrt<T>(colj[j]);  // 1 / u_jj
    const T ujj = colj[j] * inv;
    const T urj = colj[r] * inv;
    const T f = urj * inv;  // u_rj / u_jj: a_cj u_rj / u_jj = u_rj u_cj
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = q + 4 * t;
      if (c < j && r < j) u[t] -= f * colj[c];
    }
    if ((j & 3) == q) u[tj] = r < j ? urj : (r == j ? ujj : T(0));
    f16::wave_sync();
  }
  // w = U_i z_i, columns in groups of four: this lane's quarter of row r,
  // summed over the row's lanes
  const int64_t row = (blk * 16 + r) * k;
  for (int64_t k0 = 0; k0 < k; k0 += kNarrow) {
    const int kc = static_cast<int>(k - k0 < kNarrow ? k - k0 : kNarrow);
    if (q == 0)
#pragma unroll
      for (int c = 0; c < kNarrow; ++c) bufA[r * kNarrow + c] = c < kc ? z[row + k0 + c] : T(0);
    f16::wave_sync();
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) {
      T acc = T(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += u[t] * bufA[(q + 4 * t) * kNarrow + c];
      acc = row_sum(acc);
      if (q == 0 && c < kc) x[row + k0 + c] = acc;
    }
    f16::wave_sync();
  }
}

template <typename T>
__global__ __launch_bounds__(64) void chain16_sample_bwd(int L, int64_t k,
                                                         const T *__restrict__ lower,
                                                         const T *__restrict__ factor, T *x) {
  __shared__ __align__(16) T bufB[16 * kNarrow];
  __shared__ __align__(16) T bufC[16 * kNarrow];
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T sC[256];
  const int lane = threadIdx.x, r = lane & 15, q = lane >> 4;
  const int64_t ngrp = (k + kNarrow - 1) / kNarrow;
  const int64_t m = blockIdx.x / ngrp, k0 = (blockIdx.x - m * ngrp) * kNarrow;
  const int kc = static_cast<int>(k - k0 < kNarrow ? k - k0 : kNarrow);
  const T *F = factor + m * L * kPB;
  const T *C = L > 1 ? lower + m * (L - 1) * 256 : nullptr;  // none for one block
  const int lc = L > 1 ? L - 2 : 0;
  auto vrow = [&](int i) { return x + ((m * L + i) * 16 + r) * k + k0; };
  auto coupling = [&](int i) -> const T * {
    return C ? C + int64_t(min(max(i, 0), lc)) * 256 : nullptr;
  };
  // sum over this lane's columns q + 4t of a_t V[q + 4t][c], then over the row's lanes
  auto dot = [&](T (&o)[kNarrow], const T (&a)[4], const T *V) {
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) {
      T acc = T(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += a[t] * V[(q + 4 * t) * kNarrow + c];
      o[c] = c < kc ? row_sum(acc) : T(0);
    }
  };
  auto put_row = [&](T *V, const T (&v)[kNarrow]) {
    if (q == 0)
#pragma unroll
      for (int c = 0; c < kNarrow; ++c) V[r * kNarrow + c] = v[c];
  };
  auto load_row = [&](T (&o)[kNarrow], const T *row) {
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) o[c] = c < kc ? row[c] : T(0);
  };

  Raw<T> nx;
  load_raw(nx, F + int64_t(L - 1) * kPB, coupling(L - 1), lane);
  T wn[kNarrow];
  load_row(wn, vrow(L - 1));
  for (int i = L - 1; i >= 0; --i) {
    put_raw(sP, sC, nx, lane);
    T w[kNarrow];
#pragma unroll
    for (int c = 0; c < kNarrow; ++c) w[c] = wn[c];
    if (i > 0) {  // the next step's blocks and w (row i - 1, not written yet)
      load_raw(nx, F + int64_t(i - 1) * kPB, coupling(i - 1), lane);
      load_row(wn, vrow(i - 1));
    }
    f16::wave_sync();
    if (i < L - 1) {  // x_i = w_i - Sinv_i C_i^T x_{i+1}, x_{i+1} in bufB
      T si[4], cc[4], t2[kNarrow];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = q + 4 * t;
        si[t] = sP[c <= r ? r * (r + 1) / 2 + c : c * (c + 1) / 2 + r];
        cc[t] = sC[c * 16 + r];
      }
      dot(t2, cc, bufB);
      put_row(bufC, t2);
      f16::wave_sync();
      T v[kNarrow];
      dot(v, si, bufC);
#pragma unroll
      for (int c = 0; c < kNarrow; ++c) w[c] -= v[c];
    }
    if (q == 0)
#pragma unroll
      for (int c = 0; c < kNarrow; ++c)
        if (c < kc) vrow(i)[c] = w[c];
    put_row(bufB, w);
    f16::wave_sync();
  }
}

}  // namespace

template <typename T>
hipError_t chain16_sample_launch(int64_t B, int64_t L, int64_t k, const T *lower,
                                 const T *factor, const T *z, T *x, hipStream_t s) {
  if (B == 0 || k == 0) return hipSuccess;
  const int64_t groups = B * ((k + kNarrow - 1) / kNarrow);
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  if (B * L > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chain16_sample_w<T>, dim3(static_cast<unsigned>(B * L)), dim3(64), 0, s, k,
                     factor, z, x);
  hipLaunchKernelGGL(chain16_sample_bwd<T>, dim3(static_cast<unsigned>(groups)), dim3(64), 0, s,
                     static_cast<int>(L), k, lower, factor, x);
  return hipGetLastError();
}

template hipError_t chain16_sample_launch<float>(int64_t, int64_t, int64_t, const float *,
                                                 const float *, const float *, float *,
                                                 hipStream_t);
template hipError_t chain16_sample_launch<double>(int64_t, int64_t, int64_t, const double *,
                                                  const double *, const double *, double *,
                                                  hipStream_t);

template <typename T>
hipError_t chain16_solve_launch(int64_t B, int64_t L, int64_t k, const T *lower, const T *factor,
                                const T *y, T *x, hipStream_t s) {
  if (B == 0 || k == 0) return hipSuccess;
  if (k <= kGroupedMax) {  // groups of four columns on the one-wavefront kernel
    const int64_t groups = B * ((k + kNarrow - 1) / kNarrow);
    hipLaunchKernelGGL(chain16_solve_narrow<T>, dim3(static_cast<unsigned>(groups)), dim3(64), 0,
                       s, static_cast<int>(L), k, lower, factor, y, x);
    return hipGetLastError();
  }
  const int nch = static_cast<int>((k + kCols - 1) / kCols);
  hipLaunchKernelGGL(chain16_solve<T>, dim3(static_cast<unsigned>(B * nch)), dim3(64), 0, s,
                     static_cast<int>(L), k, nch, lower, factor, y, x);
  return hipGetLastError();
}

template hipError_t chain16_solve_launch<float>(int64_t, int64_t, int64_t, const float *,
                                                const float *, const float *, float *,
                                                hipStream_t);
template hipError_t chain16_solve_launch<double>(int64_t, int64_t, int64_t, const double *,
                                                 const double *, const double *, double *,
                                                 hipStream_t);

}  // namespace selinv
