// star_b32.hip -- block-arrowhead selected inverse for 32x32 blocks on the
// matrix cores (gabp-sparse-inv 0.3.2 page, "Implemented and tested
// kernels", item Star: one centre coupled to K leaves, no leaf-leaf coupling,
// leaves eliminated in parallel).  With F_j = coupling[j] = A_{j,0} the
// centre is every leaf's parent and E_j = A_{0,j} = F_j^T:
//
//   collect (per leaf):  Dinv_j = D_j^{-1},  Z_j = Dinv_j F_j,
//                        M_j = E_j Dinv_j E_j^T = F_j^T Z_j
//   centre:              S_0 = A_00 - sum_j M_j,  G_00 = S_0^{-1}
//   distribute (per leaf): X_j = E_j Dinv_j = F_j^T Dinv_j,  V = G_00 X_j,
//                        G_cross[j] = G_{j,0} = -V^T,  G_leaf[j] = Dinv_j + X_j^T V
//
// Three launches.  A wavefront owns LPW consecutive leaves of one matrix and
// sums their messages in its MFMA accumulators, so the centre reduction reads
// ceil(K / LPW) partial blocks per matrix, in a fixed order (deterministic).
// Only the packed lower triangle of Dinv_j (528 entries) crosses from collect
// to distribute; F_j is re-read.
#include <climits>

#include "frag32.h"
#include "internal.h"
#include "io32.h"

namespace selinv {

namespace {

using f32t::Blk;
constexpr int kLPW = 16;  // leaves per wavefront
constexpr int BB = 1024, PB = f32t::kPacked32;

template <typename T>
__device__ __forceinline__ void store_sym_u(T *P, const Blk<T> &b, int g, int j) {
  // symmetric result with tiles (0,0), (0,1), (1,1) formed: the (1,0) block is
  // the transpose of the (0,1) block
  f16::store_t(P, 32, b.t[0][0], g, j);
  f16::store(P + 16, 32, b.t[0][1], g, j);
  f16::store_t(P + 16 * 32, 32, b.t[0][1], g, j);
  f16::store_t(P + 16 * 32 + 16, 32, b.t[1][1], g, j);
}

// kFactor: the collect pass of the shared factor; st_dinv is then the factor's
// leaf part ([B][K][528]) and may be null (log det only).
template <typename T, bool kFactor>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void star32_collect(
    int K, int nw, const T *__restrict__ leaves, const T *__restrict__ coupling,
    T *__restrict__ st_dinv, T *__restrict__ st_mpart, double *__restrict__ st_ld,
    int32_t *__restrict__ st_fail) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / nw;
  const int w = blockIdx.x % nw;
  const int j0 = w * kLPW, j1 = min(j0 + kLPW, K);
  const T *Dm = leaves + m * K * BB;
  const T *Fm = coupling + m * K * BB;
  const bool keep = !kFactor || st_dinv;  // the packed Dinv_j are stored
  T *dinv = keep ? st_dinv + m * K * PB : nullptr;
  const io32::SymLanes<T> sl(g, j, lane);

  Blk<T> Macc = f32t::zero<T>();  // sum of F_j^T Dinv_j F_j, tiles (0,0), (0,1), (1,1)
  f16::PivotLog pl;  // product of all pivots of this wavefront's leaves
  int32_t first_bad = 0;
  Blk<T> S, Fo;
  {
    io32::put(tA, lane, io32::load(Dm + j0 * BB, lane));
    io32::put(tB, lane, io32::load(Fm + j0 * BB, lane));
    f16::wave_sync();
    S = sl.get_sym(tA);
    Fo = io32::get_blk(tB, g, j);  // O32(F_j0)
  }
  // Per leaf: the next leaf's blocks are loaded first and staged after the
  // step (single-exit loop).  With C = F_j^T the step's message C Dinv_j C^T
  // is F_j^T Dinv_j F_j, and O32(C^T) = O32(F_j).
  for (int jj = j0; jj < j1; ++jj) {
    const int jn = min(jj + 1, j1 - 1);
    const io32::Nat<T> Fn = io32::load(Fm + jn * BB, lane);
    const io32::Nat<T> Dn = io32::load(Dm + jn * BB, lane);
    if (f32t::gj_congruence(S, Fo, Macc, col, g, j, pl) && !first_bad) first_bad = jj + 1;
    if (keep) {  // Dinv_j -> packed workspace triangle
      f16::wave_sync();
      io32::put_blk_low(tA, g, j, S);
      f16::wave_sync();
      const io32::NatP<T> pk = sl.gather_packed(tA);
      io32::store_packed(dinv + jj * PB, lane, pk);
    }
    f16::wave_sync();
    io32::put(tA, lane, Dn);
    io32::put(tB, lane, Fn);
    f16::wave_sync();
    S = sl.get_sym(tA);
    Fo = io32::get_blk(tB, g, j);
  }
  store_sym_u(st_mpart + (m * nw + w) * BB, Macc, g, j);
  if (lane == 0) {
    st_ld[m * nw + w] = pl.log();
    st_fail[m * nw + w] = first_bad;
  }
}

// kFactor: G_center is the factor's centre part ([B][528], packed S_0^{-1})
// and may be null; mat_fail is unused.
template <typename T, bool kFactor>
__global__ __launch_bounds__(64) void star32_center(int nw, const T *__restrict__ center,
                                                    const T *__restrict__ st_mpart,
                                                    const double *__restrict__ st_ld,
                                                    const int32_t *__restrict__ st_fail,
                                                    T *__restrict__ G_center,
                                                    double *__restrict__ logdet,
                                                    int32_t *__restrict__ info,
                                                    int32_t *__restrict__ mat_fail) {
  __shared__ __align__(32) T col[32];
  __shared__ __align__(16) T tile[kFactor ? io32::Traits<T>::kTile : 1];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const f32t::SymOffsets<T> so(g, j);
  Blk<T> S = so.load(center + m * BB);
  int32_t fail = 0;
  double ld = 0.0;
  for (int w = 0; w < nw; ++w) {  // fixed order: leaves ascending
    S = f32t::sub(S, so.load(st_mpart + (m * nw + w) * BB));
    if (!fail && st_fail[m * nw + w]) fail = st_fail[m * nw + w] - 1 + 2;  // leaf j -> j+2
    ld += st_ld[m * nw + w];
  }
  f16::PivotLog pl;
  const bool bad = f32t::gj_inverse(S, col, g, j, pl);
  if (!fail && bad) fail = 1;
  if constexpr (kFactor) {
    if (G_center) {
      const io32::SymLanes<T> sl(g, j, lane);
      io32::put_blk(tile, g, j, S);
      f16::wave_sync();
      io32::store_packed(G_center + m * PB, lane, sl.gather_packed(tile));
    }
    if (lane == 0) {
      logdet[m] = fail ? __builtin_nan("") : ld + pl.log();
      if (info) info[m] = fail;
    }
    return;
  }
  if (fail) {
    S = f32t::zero<T>();
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
      for (int J = 0; J < 2; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) S.t[I][J][r] = static_cast<T>(__builtin_nan(""));
  }
  f32t::store_t(G_center + m * BB, S, g, j);
  if (lane == 0) {
    logdet[m] = fail ? __builtin_nan("") : ld + pl.log();
    if (info) info[m] = fail;
    mat_fail[m] = fail;
  }
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void star32_distribute(
    int K, int nw, const T *__restrict__ coupling, const T *__restrict__ G_center,
    const T *__restrict__ st_dinv, const int32_t *__restrict__ mat_fail, T *__restrict__ G_leaf,
    T *__restrict__ G_cross) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / nw;
  const int w = blockIdx.x % nw;
  const int j0 = w * kLPW, j1 = min(j0 + kLPW, K);
  const T *Fm = coupling + m * K * BB;
  const T *dinv = st_dinv + m * K * PB;
  T *Glm = G_leaf + m * K * BB;
  T *Gxm = G_cross + m * K * BB;
  if (mat_fail[m]) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = static_cast<int64_t>(j0) * BB + lane; e < static_cast<int64_t>(j1) * BB;
         e += 64) {
      Glm[e] = nan;
      Gxm[e] = nan;
    }
    return;
  }
  const io32::SymLanes<T> sl(g, j, lane);
  Blk<T> G;
  {
    const io32::Nat<T> gc = io32::load(G_center + m * BB, lane);
    io32::put(tA, lane, gc);
    f16::wave_sync();
    G = io32::get_blk(tA, g, j);
  }
  // The packed Dinv and the coupling of the next leaf are loaded into the
  // registers just freed by staging the current leaf's in LDS.
  io32::NatP<T> Pc = io32::load_packed(dinv + j0 * PB, lane);
  io32::Nat<T> Fc = io32::load(Fm + j0 * BB, lane);
  for (int jj = j0; jj < j1; ++jj) {
    f16::wave_sync();
    io32::put_packed(tA, lane, Pc);
    io32::put(tB, lane, Fc);
    const int jn = min(jj + 1, j1 - 1);
    Pc = io32::load_packed(dinv + jn * PB, lane);
    Fc = io32::load(Fm + jn * BB, lane);
    f16::wave_sync();
    const Blk<T> Di = sl.get_packed(tA);
    const Blk<T> Fo = io32::get_blk(tB, g, j);
    const Blk<T> X = f32t::mm(Fo, Di, f32t::zero<T>());  // F_j^T Dinv_j
    const Blk<T> V = f32t::mm(G, X, f32t::zero<T>());    // G_00 X_j = -G_{0,j}
    const Blk<T> Gl = f32t::mm_lower(X, V, Di);          // Dinv_j + X_j^T V
    f16::wave_sync();
    io32::put_blk_t(tA, g, j, f32t::neg(V));  // G_{j,0} = -V^T
    io32::put_sym(tB, g, j, Gl);
    f16::wave_sync();
    io32::store(Gxm + jj * BB, lane, io32::get(tA, lane));
    io32::store(Glm + jj * BB, lane, io32::get(tB, lane));
  }
}

}  // namespace

size_t star32_workspace_bytes(int dtype_bytes, int64_t B, int64_t K) {
  const size_t nw = (K + kLPW - 1) / kLPW;
  return align_up(static_cast<size_t>(B) * K * PB * dtype_bytes) +
         align_up(static_cast<size_t>(B) * nw * BB * dtype_bytes) +
         align_up(static_cast<size_t>(B) * nw * sizeof(double)) +
         align_up(static_cast<size_t>(B) * nw * sizeof(int32_t)) +
         align_up(static_cast<size_t>(B) * sizeof(int32_t));
}

template <typename T>
hipError_t star32_launch(int64_t B, int64_t K, const T *center, const T *leaves, const T *coupling,
                         T *G_center, T *G_leaf, T *G_cross, double *logdet, int32_t *info,
                         void *ws, hipStream_t s) {
  const int nw = static_cast<int>((K + kLPW - 1) / kLPW);
  Carve cv(ws);
  T *dinv = cv.take<T>(static_cast<size_t>(B) * K * PB);
  T *mpart = cv.take<T>(static_cast<size_t>(B) * nw * BB);
  double *ldp = cv.take<double>(static_cast<size_t>(B) * nw);
  int32_t *failp = cv.take<int32_t>(static_cast<size_t>(B) * nw);
  int32_t *matfail = cv.take<int32_t>(B);
  if (nw > 0)
    hipLaunchKernelGGL((star32_collect<T, false>), dim3(static_cast<unsigned>(B * nw)), dim3(64),
                       0, s, static_cast<int>(K), nw, leaves, coupling, dinv, mpart, ldp, failp);
  hipLaunchKernelGGL((star32_center<T, false>), dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     nw, center, mpart, ldp, failp, G_center, logdet, info, matfail);
  if (nw > 0)
    hipLaunchKernelGGL(star32_distribute<T>, dim3(static_cast<unsigned>(B * nw)), dim3(64), 0, s,
                       static_cast<int>(K), nw, coupling, G_center, dinv, matfail, G_leaf,
                       G_cross);
  return hipGetLastError();
}

size_t star32_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K) {
  const size_t nw = (K + kLPW - 1) / kLPW;
  return align_up(static_cast<size_t>(B) * nw * BB * dtype_bytes) +
         align_up(static_cast<size_t>(B) * nw * sizeof(double)) +
         align_up(static_cast<size_t>(B) * nw * sizeof(int32_t));
}

template <typename T>
hipError_t star32_factor_launch(int64_t B, int64_t K, const T *center, const T *leaves,
                                const T *coupling, T *factor, double *logdet, int32_t *info,
                                void *ws, hipStream_t s) {
  const int nw = static_cast<int>((K + kLPW - 1) / kLPW);
  Carve cv(ws);
  T *mpart = cv.take<T>(static_cast<size_t>(B) * nw * BB);
  double *ldp = cv.take<double>(static_cast<size_t>(B) * nw);
  int32_t *failp = cv.take<int32_t>(static_cast<size_t>(B) * nw);
  T *fc = factor ? factor + static_cast<size_t>(B) * K * PB : nullptr;
  if (nw > 0)
    hipLaunchKernelGGL((star32_collect<T, true>), dim3(static_cast<unsigned>(B * nw)), dim3(64),
                       0, s, static_cast<int>(K), nw, leaves, coupling, factor, mpart, ldp,
                       failp);
  hipLaunchKernelGGL((star32_center<T, true>), dim3(static_cast<unsigned>(B)), dim3(64), 0, s, nw,
                     center, mpart, ldp, failp, fc, logdet, info, nullptr);
  return hipGetLastError();
}

template hipError_t star32_factor_launch<float>(int64_t, int64_t, const float *, const float *,
                                                const float *, float *, double *, int32_t *,
                                                void *, hipStream_t);
template hipError_t star32_factor_launch<double>(int64_t, int64_t, const double *,
                                                 const double *, const double *, double *,
                                                 double *, int32_t *, void *, hipStream_t);
template hipError_t star32_launch<float>(int64_t, int64_t, const float *, const float *,
                                         const float *, float *, float *, float *, double *,
                                         int32_t *, void *, hipStream_t);
template hipError_t star32_launch<double>(int64_t, int64_t, const double *, const double *,
                                          const double *, double *, double *, double *, double *,
                                          int32_t *, void *, hipStream_t);

}  // namespace selinv
