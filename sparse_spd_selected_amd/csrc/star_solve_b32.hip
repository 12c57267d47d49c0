// star_solve_b32.hip -- solve and sampling with the shared factor of b = 32
// stars ("Factor once, do everything" on the gabp-sparse-inv 0.3.2 page), up
// to four right-hand sides: one wavefront per leaf, one workgroup per centre.
//
// The centre is the parent of every leaf, E_j = A_{0,j} = coupling[j]^T; the
// factor holds the packed lower triangle of every Sinv (leaves [B][K], then
// centres [B]; entry (a, c), a >= c, at a (a + 1) / 2 + c).
//   solve:  leaves  w_j = Sinv_j y_j, message E_j w_j;
//           centre  x_0 = Sinv_0 (y_0 - sum_j E_j w_j)  (messages in leaf order);
//           leaves  x_j = w_j - Sinv_j coupling[j] x_0
//   sample: centre  x_0 = U_0 z_0;  leaves  x_j = U_j z_j - Sinv_j coupling[j] x_0,
//           U U^T = Sinv with U upper triangular
// Lane (r, h) = (lane % 32, lane / 32) owns row r and the columns h, h + 2,
// ..., h + 30 of every dot product; the two halves are added by one
// cross-lane exchange.  A leaf's packed Sinv and coupling block are staged in
// LDS with coalesced loads (the coupling with row stride 33 against bank
// conflicts), and U is formed in registers by the reversed Cholesky, columns
// 31 down to 0, each column broadcast through LDS.
#include <climits>

#include "frag16.h"
#include "internal.h"

namespace selinv {

namespace {

constexpr int kB = 32, kPB = 528, kCS = 33;  // block, packed entries, coupling LDS stride
constexpr int kN = 4;                        // right-hand sides handled here

template <typename T>
__device__ __forceinline__ T half_sum(T v) {
  return v + __shfl_xor(v, 32);
}

template <typename T>
struct Lane {
  int r, h, kc;
  // this lane's half of row r of the packed symmetric block in sP
  __device__ __forceinline__ void sinv_half(T (&o)[16], const T *sP) const {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int c = h + 2 * t;
      o[t] = sP[c <= r ? r * (r + 1) / 2 + c : c * (c + 1) / 2 + r];
    }
  }
  // o_c = sum_t a_t V[h + 2t][c] over the row's two lanes (V is [32][kN] in LDS)
  __device__ __forceinline__ void dot(T (&o)[kN], const T (&a)[16], const T *V) const {
#pragma unroll
    for (int c = 0; c < kN; ++c) {
      T acc = T(0);
#pragma unroll
      for (int t = 0; t < 16; ++t) acc += a[t] * V[(h + 2 * t) * kN + c];
      o[c] = c < kc ? half_sum(acc) : T(0);
    }
  }
  __device__ __forceinline__ void put(T *V, const T (&v)[kN]) const {
    if (h == 0)
#pragma unroll
      for (int c = 0; c < kN; ++c) V[r * kN + c] = v[c];
  }
  __device__ __forceinline__ void load_row(T (&o)[kN], const T *row) const {
#pragma unroll
    for (int c = 0; c < kN; ++c) o[c] = c < kc ? row[c] : T(0);
  }
  __device__ __forceinline__ void store_row(T *row, const T (&v)[kN]) const {
    if (h == 0)
#pragma unroll
      for (int c = 0; c < kN; ++c)
        if (c < kc) row[c] = v[c];
  }
  // u (this lane's half of row r of Sinv) -> the same entries of U, U U^T = Sinv
  __device__ __forceinline__ void rev_cholesky(T (&u)[16], T *colj) const {
#pragma unroll
    for (int j = kB - 1; j >= 0; --j) {
      const int tj = j >> 1;
      if ((j & 1) == h) colj[r] = u[tj];
      f16::wave_sync();
      const T inv = f16::rsqrt<T>(colj[j]);  // 1 / u_jj, one per column
      const T ujj = colj[j] * inv;
      const T urj = colj[r] * inv;
      const T f = urj * inv;  // a_cj u_rj / u_jj = u_rj u_cj
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int c = h + 2 * t;
        if (c < j && r < j) u[t] -= f * colj[c];
      }
      if ((j & 1) == h) u[tj] = r < j ? urj : (r == j ? ujj : T(0));
      f16::wave_sync();
    }
  }
};

// one wavefront stages a packed block (and optionally a coupling block)
template <typename T>
__device__ __forceinline__ void stage(T *sP, const T *P, T *sC, const T *Cb, int lane) {
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const int e = lane + 64 * t;
    if (e < kPB) sP[e] = P[e];
  }
  if (Cb)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = lane + 64 * t;
      sC[(e >> 5) * kCS + (e & 31)] = Cb[e];
    }
}

// Solve, leaves first: w_j = Sinv_j y_j to x, message E_j w_j = coupling[j]^T w_j
template <typename T>
__global__ __launch_bounds__(64) void star32_solve_leaf_fwd(int64_t k,
                                                           const T *__restrict__ coupling,
                                                           const T *__restrict__ factor,
                                                           const T *__restrict__ y_leaves,
                                                           T *__restrict__ x_leaves,
                                                           T *__restrict__ msg) {
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T sC[kB * kCS];
  __shared__ __align__(16) T V[kB * kN];
  __shared__ __align__(16) T W[kB * kN];
  const int lane = threadIdx.x;
  const Lane<T> ln{lane & 31, lane >> 5, static_cast<int>(k)};
  const int64_t leaf = blockIdx.x;
  stage(sP, factor + leaf * kPB, sC, coupling + leaf * kB * kB, lane);
  T y[kN];
  ln.load_row(y, y_leaves + (leaf * kB + ln.r) * k);
  ln.put(V, y);
  f16::wave_sync();
  T si[16], w[kN];
  ln.sinv_half(si, sP);
  ln.dot(w, si, V);
  ln.store_row(x_leaves + (leaf * kB + ln.r) * k, w);
  ln.put(W, w);
  f16::wave_sync();
  T cc[16], mo[kN];
#pragma unroll
  for (int t = 0; t < 16; ++t) cc[t] = sC[(ln.h + 2 * t) * kCS + ln.r];  // coupling[c][r]
  ln.dot(mo, cc, W);
  ln.store_row(msg + (leaf * kB + ln.r) * k, mo);
}

// Centre, one workgroup of 256 per matrix: u_0 = y_0 - sum_j messages (solve;
// each thread adds a contiguous range of leaves in order, the ranges are then
// added in order) and x_0 = Sinv_0 u_0, or x_0 = U_0 z_0 (sample).
template <typename T, bool kSample>
__global__ __launch_bounds__(256) void star32_apply_center(int64_t B, int64_t K, int64_t k,
                                                          const T *__restrict__ factor,
                                                          const T *__restrict__ in_center,
                                                          const T *__restrict__ msg,
                                                          T *__restrict__ x_center) {
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T V[kB * kN];
  __shared__ __align__(16) T part[256];
  __shared__ __align__(16) T colj[kB];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int kc = static_cast<int>(k);
  const int ne = kB * kc;        // entries of the centre's vector block
  const int parts = 256 / ne;    // >= 2
  T sum = T(0);
  if (!kSample && tid < parts * ne) {
    const int e = tid % ne, p = tid / ne;
    const int64_t j0 = K * p / parts, j1 = K * (p + 1) / parts;
    for (int64_t j = j0; j < j1; ++j) sum += msg[(m * K + j) * kB * k + e];
  }
  part[tid] = sum;
  __syncthreads();
  if (tid >= 64) return;
  const Lane<T> ln{tid & 31, tid >> 5, kc};
  stage(sP, factor + (B * K + m) * kPB, static_cast<T *>(nullptr), static_cast<const T *>(nullptr),
        tid);
  T u[kN];
  ln.load_row(u, in_center + (m * kB + ln.r) * k);
  if (!kSample)
#pragma unroll
    for (int c = 0; c < kN; ++c)
      if (c < kc)
        for (int p = 0; p < parts; ++p) u[c] -= part[p * ne + ln.r * kc + c];
  ln.put(V, u);
  f16::wave_sync();
  T a[16], w[kN];
  ln.sinv_half(a, sP);
  if (kSample) ln.rev_cholesky(a, colj);
  ln.dot(w, a, V);
  ln.store_row(x_center + (m * kB + ln.r) * k, w);
}

// Leaves, parents first: x_j = w_j - Sinv_j coupling[j] x_0, with w_j the
// forward result (solve) or U_j z_j (sample)
template <typename T, bool kSample>
__global__ __launch_bounds__(64) void star32_apply_leaf_bwd(int64_t K, int64_t k,
                                                           const T *__restrict__ coupling,
                                                           const T *__restrict__ factor,
                                                           const T *__restrict__ z_leaves,
                                                           const T *__restrict__ x_center,
                                                           T *__restrict__ x_leaves) {
  __shared__ __align__(16) T sP[kPB];
  __shared__ __align__(16) T sC[kB * kCS];
  __shared__ __align__(16) T V0[kB * kN];
  __shared__ __align__(16) T Z[kB * kN];
  __shared__ __align__(16) T Tt[kB * kN];
  __shared__ __align__(16) T colj[kB];
  const int lane = threadIdx.x;
  const Lane<T> ln{lane & 31, lane >> 5, static_cast<int>(k)};
  const int64_t leaf = blockIdx.x, m = leaf / K;
  stage(sP, factor + leaf * kPB, sC, coupling + leaf * kB * kB, lane);
  T x0[kN], w[kN];
  ln.load_row(x0, x_center + (m * kB + ln.r) * k);
  ln.put(V0, x0);
  if (kSample) {
    T z[kN];
    ln.load_row(z, z_leaves + (leaf * kB + ln.r) * k);
    ln.put(Z, z);
  } else {
    ln.load_row(w, x_leaves + (leaf * kB + ln.r) * k);
  }
  f16::wave_sync();
  T si[16];
  ln.sinv_half(si, sP);
  if (kSample) {
    T u[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) u[t] = si[t];
    ln.rev_cholesky(u, colj);
    ln.dot(w, u, Z);  // U_j z_j
  }
  T cr[16], t2[kN];
#pragma unroll
  for (int t = 0; t < 16; ++t) cr[t] = sC[ln.r * kCS + ln.h + 2 * t];  // coupling[r][c]
  ln.dot(t2, cr, V0);  // coupling[j] x_0
  ln.put(Tt, t2);
  f16::wave_sync();
  T v[kN];
  ln.dot(v, si, Tt);
#pragma unroll
  for (int c = 0; c < kN; ++c) w[c] -= v[c];
  ln.store_row(x_leaves + (leaf * kB + ln.r) * k, w);
}

}  // namespace

template <typename T>
hipError_t star32_apply_launch(int64_t B, int64_t K, int64_t k, bool sample, const T *coupling,
                               const T *factor, const T *in_center, const T *in_leaves,
                               T *x_center, T *x_leaves, void *ws, hipStream_t s) {
  if (B == 0 || k == 0) return hipSuccess;
  const size_t nl = static_cast<size_t>(B) * K;
  T *msg = static_cast<T *>(ws);
  if (!sample && nl)
    hipLaunchKernelGGL(star32_solve_leaf_fwd<T>, dim3(static_cast<unsigned>(nl)), dim3(64), 0, s,
                       k, coupling, factor, in_leaves, x_leaves, msg);
  if (sample)
    hipLaunchKernelGGL((star32_apply_center<T, true>), dim3(static_cast<unsigned>(B)), dim3(256),
                       0, s, B, K, k, factor, in_center, msg, x_center);
  else
    hipLaunchKernelGGL((star32_apply_center<T, false>), dim3(static_cast<unsigned>(B)),
                       dim3(256), 0, s, B, K, k, factor, in_center, msg, x_center);
  if (nl) {
    if (sample)
      hipLaunchKernelGGL((star32_apply_leaf_bwd<T, true>), dim3(static_cast<unsigned>(nl)),
                         dim3(64), 0, s, K, k, coupling, factor, in_leaves, x_center, x_leaves);
    else
      hipLaunchKernelGGL((star32_apply_leaf_bwd<T, false>), dim3(static_cast<unsigned>(nl)),
                         dim3(64), 0, s, K, k, coupling, factor, in_leaves, x_center, x_leaves);
  }
  return hipGetLastError();
}

template hipError_t star32_apply_launch<float>(int64_t, int64_t, int64_t, bool, const float *,
                                               const float *, const float *, const float *,
                                               float *, float *, void *, hipStream_t);
template hipError_t star32_apply_launch<double>(int64_t, int64_t, int64_t, bool, const double *,
                                                const double *, const double *, const double *,
                                                double *, double *, void *, hipStream_t);

}  // namespace selinv
