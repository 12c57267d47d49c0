// vjp_star_b32.hip -- reverse mode of the block-arrowhead selected inverse
// for 32x32 blocks on the matrix cores (the backward of gabp-sparse-inv
// 0.3.2, "Implemented and tested kernels", items Star and Differentiable
// tree: a second collect / distribute pair on the same tree).  With
// F_j = coupling[j] = A_{j,0}, the centre is every leaf's parent and the edge
// block is E_j = F_j^T; the cotangent of G_{0,j} is Gx_j^T (Gx = the
// cotangent of G_cross), that of G_jj is Gv_j, that of G_00 is Gc.
//
//   collect (per leaf; a leaf has no children, so GG_j = sym(Gv_j)):
//     Dinv_j = D_j^{-1},  O32(X_j^T) = Dinv_j F_j,  M_j = F_j^T Dinv_j F_j
//     W^T = GG_j X_j^T,  Y1^T = W^T - Gx_j,  Y2^T = W^T + Y1^T
//     Z_j = Y2 Dinv_j,  N_j = Y1 X_j^T,  P_j = lb Dinv_j - Dinv_j GG_j Dinv_j
//   centre:  S_0 = A_00 - sum_j M_j,  G_00 = S_0^{-1},
//            GG_0 = sym(Gc) + sym(sum_j N_j),
//            center_bar = P_0 = lb G_00 - G_00 GG_0 G_00
//   distribute (per leaf):  A1 = G_00 Z_j,  T2 = center_bar X_j,
//            Q = A1 - T2,  coupling_bar[j] = (A1 - 2 T2)^T,
//            leaves_bar[j] = P_j - sym(X_j^T Q)
//
// Three launches, as in the forward kernel: a wavefront owns kLPW leaves of
// one matrix and sums their M and N in its accumulators, and the centre
// reduces the partial sums in a fixed order.  Workspace per leaf (written by
// the collect launch, read by the distribute launch): X_j^T, Z_j and the
// packed P_j.
#include <climits>

#include "frag32.h"
#include "internal.h"
#include "io32.h"

namespace selinv {

namespace {

using f32t::Blk;
constexpr int kLPW = 16;  // leaves per wavefront
constexpr int BB = 1024, PB = f32t::kPacked32;
// The f64 leaf kernels hold about seven 32x32 blocks (32 VGPRs each) plus
// the blocks in flight: one wave per SIMD; f32 fits two.
template <typename T>
constexpr int kStarVjpWaves = sizeof(T) == 8 ? 1 : 2;

template <typename T>
__device__ __forceinline__ Blk<T> lin(T a, const Blk<T> &x, T b, const Blk<T> &y) {
  Blk<T> r;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) r.t[I][J] = a * x.t[I][J] + b * y.t[I][J];
  return r;
}

template <typename T>
__device__ __forceinline__ Blk<T> scale(T a, const Blk<T> &x) {
  Blk<T> r;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) r.t[I][J] = a * x.t[I][J];
  return r;
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kStarVjpWaves<T>, 8)))
void star32_vjp_collect(int K, int nw, const T *__restrict__ leaves,
                        const T *__restrict__ coupling, const T *__restrict__ gleaf,
                        const T *__restrict__ gcross, const double *__restrict__ ld_bar,
                        T *__restrict__ st_xt, T *__restrict__ st_z, T *__restrict__ st_p,
                        T *__restrict__ st_mpart, T *__restrict__ st_npart,
                        int32_t *__restrict__ st_fail) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / nw;
  const int w = blockIdx.x % nw;
  const int j0 = w * kLPW, j1 = min(j0 + kLPW, K);
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const int64_t base = m * K;
  const io32::SymLanes<T> sl(g, j, lane);

  Blk<T> Macc = f32t::zero<T>(), Nacc = f32t::zero<T>();
  f16::PivotLog pl;  // pivots are only tested here
  int32_t first_bad = 0;
  Blk<T> S;
  {
    const io32::Nat<T> d0 = io32::load(leaves + (base + j0) * BB, lane);
    io32::put(tA, lane, d0);
    f16::wave_sync();
    S = sl.get_sym(tA);
  }
  // Single-exit loop: a failed pivot is recorded and the leaf's (discarded)
  // work runs on.  The leaf's three other input blocks are loaded before the
  // sweep; the next diagonal block once they are staged.
  for (int jj = j0; jj < j1; ++jj) {
    const int64_t lf = base + jj;
    const io32::Nat<T> Fn = io32::load(coupling + lf * BB, lane);
    const io32::Nat<T> Hn = io32::load(gleaf + lf * BB, lane);
    const io32::Nat<T> Xn = io32::load(gcross + lf * BB, lane);
    if (f32t::gj_inverse(S, col, g, j, pl) && !first_bad) first_bad = jj + 1;
    f16::wave_sync();
    io32::put(tA, lane, Fn);
    io32::put(tB, lane, Hn);
    f16::wave_sync();
    const Blk<T> Fo = io32::get_blk(tA, g, j);
    const Blk<T> GG = lin(T(0.5), io32::get_blk(tB, g, j), T(0.5), io32::get_blk_t(tB, g, j));
    f16::wave_sync();
    io32::put(tB, lane, Xn);  // Gx_j waits in tB
    const io32::Nat<T> Dn = io32::load(leaves + (base + min(jj + 1, j1 - 1)) * BB, lane);
    const Blk<T> Z0 = f32t::mm(S, Fo, f32t::zero<T>());  // O32(X^T) = Dinv F
    Macc = f32t::mm_lower(Fo, Z0, Macc);                  // += F^T Dinv F
    const Blk<T> U = f32t::mm(GG, S, f32t::zero<T>());    // GG Dinv
    const Blk<T> Wt = f32t::mm(GG, Z0, f32t::zero<T>());  // GG X^T
    const Blk<T> P = f32t::mm_lower(f32t::neg(U), S, scale(lb, S));
    f16::wave_sync();
    io32::put_sym(tA, g, j, P);
    f16::wave_sync();
    io32::store_packed(st_p + lf * PB, lane, sl.gather_packed(tA));
    const Blk<T> Y1t = f32t::sub(Wt, io32::get_blk(tB, g, j));  // W^T - Gx
    const Blk<T> Z = f32t::mm(lin(T(1), Wt, T(1), Y1t), S, f32t::zero<T>());  // Y2 Dinv
    Nacc = f32t::mm(Y1t, Z0, Nacc);                                          // += Y1 X^T
    f16::wave_sync();
    io32::put_blk(tA, g, j, Z0);
    io32::put_blk(tB, g, j, Z);
    f16::wave_sync();
    io32::store_ws(st_xt + lf * BB, lane, io32::get(tA, lane));
    io32::store_ws(st_z + lf * BB, lane, io32::get(tB, lane));
    f16::wave_sync();
    io32::put(tA, lane, Dn);
    f16::wave_sync();
    S = sl.get_sym(tA);
  }
  // partial sums: M (symmetric, lower tiles formed) and N (full)
  T *mp = st_mpart + (m * nw + w) * BB;
  f16::wave_sync();
  io32::put_sym(tA, g, j, Macc);
  io32::put_blk(tB, g, j, Nacc);
  f16::wave_sync();
  io32::store_ws(mp, lane, io32::get(tA, lane));
  io32::store_ws(st_npart + (m * nw + w) * BB, lane, io32::get(tB, lane));
  if (lane == 0) st_fail[m * nw + w] = first_bad;
}

template <typename T>
__global__ __launch_bounds__(64) void star32_vjp_center(
    int nw, const T *__restrict__ center, const T *__restrict__ gcenter,
    const double *__restrict__ ld_bar, const T *__restrict__ st_mpart,
    const T *__restrict__ st_npart, const int32_t *__restrict__ st_fail, T *__restrict__ G00,
    T *__restrict__ center_bar, int32_t *__restrict__ info, int32_t *__restrict__ mat_fail) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const f32t::SymOffsets<T> so(g, j);
  const io32::SymLanes<T> sl(g, j, lane);
  Blk<T> S = so.load(center + m * BB);
  Blk<T> N = f32t::zero<T>();
  int32_t fail = 0;
  for (int w = 0; w < nw; ++w) {  // fixed order: leaves ascending
    S = f32t::sub(S, so.load(st_mpart + (m * nw + w) * BB));
    N = lin(T(1), N, T(1), f32t::load(st_npart + (m * nw + w) * BB, g, j));
    if (!fail && st_fail[m * nw + w]) fail = st_fail[m * nw + w] - 1 + 2;  // leaf j -> j+2
  }
  f16::PivotLog pl;
  const bool bad = f32t::gj_inverse(S, col, g, j, pl);
  if (!fail && bad) fail = 1;
  if (lane == 0) {
    if (info) info[m] = fail;
    mat_fail[m] = fail;
  }
  if (fail) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int e = lane; e < BB; e += 64) center_bar[m * BB + e] = nan;
    return;
  }
  f32t::store_t(G00 + m * BB, S, g, j);
  // GG_0 = sym(Gc) + sym(N)
  f16::wave_sync();
  io32::put_blk(tA, g, j, N);
  f16::wave_sync();
  const Blk<T> Nt = io32::get_blk_t(tA, g, j);
  const Blk<T> gc = f32t::load(gcenter + m * BB, g, j), gct = f32t::load_t(gcenter + m * BB, g, j);
  const Blk<T> GG = lin(T(0.5), lin(T(1), gc, T(1), gct), T(0.5), lin(T(1), N, T(1), Nt));
  const Blk<T> U = f32t::mm(GG, S, f32t::zero<T>());
  const Blk<T> P = f32t::mm_lower(f32t::neg(U), S, scale(lb, S));
  // exactly symmetric output: mirror the lower triangle
  f16::wave_sync();
  io32::put_sym(tA, g, j, P);
  f16::wave_sync();
  const Blk<T> Ps = sl.get_sym(tA);
  f16::wave_sync();
  io32::put_blk(tA, g, j, Ps);
  f16::wave_sync();
  io32::store(center_bar + m * BB, lane, io32::get(tA, lane));
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kStarVjpWaves<T>, 8)))
void star32_vjp_distribute(int K, int nw, const T *__restrict__ G00,
                           const T *__restrict__ center_bar, const T *__restrict__ st_xt,
                           const T *__restrict__ st_z, const T *__restrict__ st_p,
                           const int32_t *__restrict__ mat_fail, T *__restrict__ leaves_bar,
                           T *__restrict__ coupling_bar) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  __shared__ __align__(16) T tP[PB];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / nw;
  const int w = blockIdx.x % nw;
  const int j0 = w * kLPW, j1 = min(j0 + kLPW, K);
  const int64_t base = m * K;
  if (mat_fail[m]) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = (base + j0) * BB + lane; e < (base + j1) * BB; e += 64) {
      leaves_bar[e] = nan;
      coupling_bar[e] = nan;
    }
    return;
  }
  const io32::SymLanes<T> sl(g, j, lane);
  Blk<T> G, Db;
  {
    const io32::Nat<T> a = io32::load_ws(G00 + m * BB, lane);
    const io32::Nat<T> b = io32::load_ws(center_bar + m * BB, lane);
    io32::put(tA, lane, a);
    io32::put(tB, lane, b);
    f16::wave_sync();
    G = io32::get_blk(tA, g, j);
    Db = io32::get_blk(tB, g, j);
  }
  io32::Nat<T> Xc = io32::load_ws(st_xt + (base + j0) * BB, lane);
  io32::Nat<T> Zc = io32::load_ws(st_z + (base + j0) * BB, lane);
  io32::NatP<T> Pc = io32::load_packed(st_p + (base + j0) * PB, lane);
  for (int jj = j0; jj < j1; ++jj) {
    f16::wave_sync();
    io32::put(tA, lane, Xc);
    io32::put(tB, lane, Zc);
    io32::put_packed(tP, lane, Pc);
    const int64_t ln = base + min(jj + 1, j1 - 1);
    Xc = io32::load_ws(st_xt + ln * BB, lane);
    Zc = io32::load_ws(st_z + ln * BB, lane);
    Pc = io32::load_packed(st_p + ln * PB, lane);
    f16::wave_sync();
    const Blk<T> Xo = io32::get_blk_t(tA, g, j);  // the tile holds X^T
    const Blk<T> A1 = f32t::mm(G, io32::get_blk(tB, g, j), f32t::zero<T>());  // G_00 Z
    const Blk<T> T2 = f32t::mm(Db, Xo, f32t::zero<T>());                     // Dbar_0 X
    const Blk<T> Q = f32t::sub(A1, T2);
    const Blk<T> Eb = f32t::sub(Q, T2);
    const Blk<T> R = f32t::mm(Xo, Q, f32t::zero<T>());  // X^T Q
    f16::wave_sync();
    io32::put_blk_t(tB, g, j, Eb);  // coupling_bar = Ebar^T
    io32::put_blk(tA, g, j, R);
    f16::wave_sync();
    const int64_t lf = base + jj;
    io32::store(coupling_bar + lf * BB, lane, io32::get(tB, lane));
    const Blk<T> Lb = lin(T(1), sl.get_packed(tP), T(-0.5), lin(T(1), R, T(1), io32::get_blk_t(tA, g, j)));
    f16::wave_sync();
    io32::put_blk(tA, g, j, Lb);
    f16::wave_sync();
    io32::store(leaves_bar + lf * BB, lane, io32::get(tA, lane));
  }
}

}  // namespace

size_t star32_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K) {
  const size_t nw = (K + kLPW - 1) / kLPW, nl = static_cast<size_t>(B) * K;
  return 2 * align_up(nl * BB * dtype_bytes) + align_up(nl * PB * dtype_bytes) +
         2 * align_up(static_cast<size_t>(B) * nw * BB * dtype_bytes) +
         align_up(static_cast<size_t>(B) * BB * dtype_bytes) +
         align_up(static_cast<size_t>(B) * nw * sizeof(int32_t)) +
         align_up(static_cast<size_t>(B) * sizeof(int32_t));
}

template <typename T>
hipError_t star32_vjp_launch(int64_t B, int64_t K, const T *center, const T *leaves,
                             const T *coupling, const T *gc, const T *gleaf, const T *gcross,
                             const double *ld_bar, T *center_bar, T *leaves_bar, T *coupling_bar,
                             int32_t *info, void *ws, hipStream_t s) {
  const int nw = static_cast<int>((K + kLPW - 1) / kLPW);
  const size_t nl = static_cast<size_t>(B) * K;
  Carve cv(ws);
  T *xt = cv.take<T>(nl * BB);
  T *z = cv.take<T>(nl * BB);
  T *p = cv.take<T>(nl * PB);
  T *mpart = cv.take<T>(static_cast<size_t>(B) * nw * BB);
  T *npart = cv.take<T>(static_cast<size_t>(B) * nw * BB);
  T *g00 = cv.take<T>(static_cast<size_t>(B) * BB);
  int32_t *failp = cv.take<int32_t>(static_cast<size_t>(B) * nw);
  int32_t *matfail = cv.take<int32_t>(B);
  if (nw > 0)
    hipLaunchKernelGGL(star32_vjp_collect<T>, dim3(static_cast<unsigned>(B * nw)), dim3(64), 0, s,
                       static_cast<int>(K), nw, leaves, coupling, gleaf, gcross, ld_bar, xt, z, p,
                       mpart, npart, failp);
  hipLaunchKernelGGL(star32_vjp_center<T>, dim3(static_cast<unsigned>(B)), dim3(64), 0, s, nw,
                     center, gc, ld_bar, mpart, npart, failp, g00, center_bar, info, matfail);
  if (nw > 0)
    hipLaunchKernelGGL(star32_vjp_distribute<T>, dim3(static_cast<unsigned>(B * nw)), dim3(64), 0,
                       s, static_cast<int>(K), nw, g00, center_bar, xt, z, p, matfail, leaves_bar,
                       coupling_bar);
  return hipGetLastError();
}

template hipError_t star32_vjp_launch<float>(int64_t, int64_t, const float *, const float *,
                                             const float *, const float *, const float *,
                                             const float *, const double *, float *, float *,
                                             float *, int32_t *, void *, hipStream_t);
template hipError_t star32_vjp_launch<double>(int64_t, int64_t, const double *, const double *,
                                              const double *, const double *, const double *,
                                              const double *, const double *, double *, double *,
                                              double *, int32_t *, void *, hipStream_t);

}  // namespace selinv
