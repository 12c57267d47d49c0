// vjp_chain_b16.hip -- reverse mode of the block-tridiagonal selected inverse
// for 16x16 blocks: one wavefront per chain, blocks in registers in the MFMA
// 16x16 layout (frag16.h), products on the matrix cores, coalesced I/O
// through per-wavefront LDS tiles (io16.h).
//
// The backward is a second collect / distribute pair on the same chain
// (gabp-sparse-inv 0.3.2 page, "Implemented and tested kernels", item
// Differentiable tree); the chain is the path rooted at its last block, with
// C_i = lower[i] = A_{i+1,i} the edge block of block i.  Cotangents: Gd_i on
// G_diag[i] (only its symmetric part counts), Gl_i on G_lower[i] =
// G_{i+1,i}, lb on log det A.
//   collect  i = 0 .. L-1 (GG_0 = sym(Gd_0)):
//     Sinv_i = S_i^{-1}
//     P_i    = lb Sinv_i - Sinv_i GG_i Sinv_i
//     Y      = Sinv_i C_i^T  (= X_i^T)
//     S_{i+1}  = D_{i+1} - C_i Y
//     W^T    = GG_i Y,  Y1^T = W^T - Gl_i^T,  Y2^T = W^T + Y1^T
//     Z_i    = Y2 Sinv_i
//     GG_{i+1} = sym(Gd_{i+1}) + sym(Y1 X_i^T)
//   distribute i = L-2 .. 0 (G = Sinv_{L-1}, Dbar_{L-1} = P_{L-1}), with
//   X_i, Z_i and P_i rebuilt from Sinv_i, GG_i, C_i and Gl_i:
//     Q          = G Z_i - Dbar_{i+1} X_i
//     lower_bar[i] = Q - Dbar_{i+1} X_i
//     Dbar_i     = P_i - sym(X_i^T Q)
//     G          = Sinv_i + X_i^T G X_i
// Workspace per block (temporal accesses, written by the collect pass and
// read back by the distribute pass of the same wavefront): the packed
// symmetric Sinv_i and GG_i only.  The distribute pass re-reads C_i and
// Gl_i and rebuilds X_i = C_i Sinv_i, Z_i and P_i on the matrix cores, which
// moves less data than storing X_i, Z_i and P_i.
#include "frag16.h"
#include "internal.h"
#include "io16.h"

namespace selinv {

namespace {

using f16::Frag;

constexpr int kBB = 256, kPB = f16::kPacked16;
constexpr int kStateBlock = 2 * kPB;  // elements of workspace per block

// Occupancy per element type: the f64 kernel needs about 200 VGPRs (two
// waves per SIMD), the f32 one about 130 (three) to run without spills.
template <typename T>
constexpr int kVjpWaves = sizeof(T) == 8 ? 2 : 3;

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kVjpWaves<T>, 8)))
void chain16_vjp_kernel(int L, const T *__restrict__ diag, const T *__restrict__ lower,
                        const T *__restrict__ gd, const T *__restrict__ gl,
                        const double *__restrict__ ld_bar, T *__restrict__ d_bar,
                        T *__restrict__ l_bar, int32_t *__restrict__ info, T *__restrict__ state) {
  using Tr = io16::Traits<T>;
  __shared__ __align__(16) T col[16];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  __shared__ __align__(16) T tC[Tr::kTile];
  __shared__ __align__(16) T tP[kPB];
  __shared__ __align__(16) T tQ[kPB];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const T *D = diag + m * L * kBB;
  const T *Gd = gd + m * L * kBB;
  // with L == 1 there is no edge block (lower, gl may be null); the
  // unconditional prefetches then read diagonal data they never use
  const T *C = L > 1 ? lower + m * (L - 1) * kBB : D;
  const T *Gl = L > 1 ? gl + m * (L - 1) * kBB : Gd;
  T *Db = d_bar + m * L * kBB;
  T *Cb = l_bar + m * (L - 1) * kBB;
  T *st = state + m * L * kStateBlock;
  const io16::SymLanes<T> sl(g, j, lane);
  const Frag<T> zero = f16::zero<T>();

  f16::PivotLog pl;  // pivots are only tested here; the log-det is not an output
  int32_t fail = 0;
  Frag<T> S, GG;
  {
    const io16::Nat<T> d0 = io16::load(D, lane), g0 = io16::load(Gd, lane);
    io16::put(tA, lane, d0);
    io16::put(tB, lane, g0);
    f16::wave_sync();
    S = sl.get_sym(tA);
    GG = T(0.5) * (io16::get_frag(tB, g, j) + io16::get_frag_t(tB, g, j));
    f16::wave_sync();
  }
  // Sinv_i = S^{-1} and GG_i, both packed to the workspace.  Leaves Sinv in S.
  auto invert = [&](int i) {
    if (f16::gj_inverse(S, col, g, j, pl) && !fail) fail = i + 1;
    f16::wave_sync();
    io16::put_frag(tA, g, j, S);
    io16::put_frag(tB, g, j, GG);
    f16::wave_sync();
    io16::store_packed(st + i * kStateBlock, lane, sl.gather_packed(tA));
    io16::store_packed(st + i * kStateBlock + kPB, lane, sl.gather_packed(tB));
  };
  // Collect with the next step's four input blocks in flight (two register
  // sets alternate, indices clamped; single-exit loop, see chain_b16.hip).
  const int lc = max(L - 2, 0);
  io16::Nat<T> C0 = io16::load(C, lane), E0 = io16::load(Gl, lane);
  io16::Nat<T> D0 = io16::load(D + min(1, L - 1) * kBB, lane);
  io16::Nat<T> H0 = io16::load(Gd + min(1, L - 1) * kBB, lane);
  io16::Nat<T> C1, E1, D1, H1;
  auto collect = [&](int i, const io16::Nat<T> &Cu, const io16::Nat<T> &Eu,
                     const io16::Nat<T> &Du, const io16::Nat<T> &Hu, io16::Nat<T> &Cn,
                     io16::Nat<T> &En, io16::Nat<T> &Dn, io16::Nat<T> &Hn) {
    Cn = io16::load(C + min(i + 1, lc) * kBB, lane);
    En = io16::load(Gl + min(i + 1, lc) * kBB, lane);
    Dn = io16::load(D + min(i + 2, L - 1) * kBB, lane);
    Hn = io16::load(Gd + min(i + 2, L - 1) * kBB, lane);
    invert(i);
    f16::wave_sync();
    io16::put(tA, lane, Cu);
    io16::put(tB, lane, Eu);
    io16::put(tC, lane, Hu);
    f16::wave_sync();
    const Frag<T> Ct = io16::get_frag_t(tA, g, j);   // O(C_i^T)
    const Frag<T> Glt = io16::get_frag_t(tB, g, j);  // O(Gl_i^T)
    const Frag<T> Gdn = T(0.5) * (io16::get_frag(tC, g, j) + io16::get_frag_t(tC, g, j));
    f16::wave_sync();
    io16::put(tA, lane, Du);
    f16::wave_sync();
    const Frag<T> Dn1 = sl.get_sym(tA);
    const Frag<T> Y = f16::mm<T>(S, Ct, zero);      // O(X_i^T)
    const Frag<T> Wt = f16::mm<T>(GG, Y, zero);     // O(W^T)
    const Frag<T> N = f16::mm<T>(Wt - Glt, Y, zero);  // O(Y1 X_i^T)
    S = Dn1 - f16::mm<T>(Ct, Y, zero);                // S_{i+1}
    f16::wave_sync();
    io16::put_frag(tA, g, j, N);
    f16::wave_sync();
    GG = Gdn + T(0.5) * (N + io16::get_frag_t(tA, g, j));
  };
  int i = 0;
  for (; i + 1 < L - 1; i += 2) {
    collect(i, C0, E0, D0, H0, C1, E1, D1, H1);
    collect(i + 1, C1, E1, D1, H1, C0, E0, D0, H0);
  }
  if (i < L - 1) collect(i, C0, E0, D0, H0, C1, E1, D1, H1);
  invert(L - 1);  // the root block
  if (fail) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t e = lane; e < static_cast<int64_t>(L) * kBB; e += 64) Db[e] = nan;
    for (int64_t e = lane; e < static_cast<int64_t>(L - 1) * kBB; e += 64) Cb[e] = nan;
    if (lane == 0 && info) info[m] = fail;
    return;
  }
  Frag<T> G = S;  // Sinv_{L-1}
  Frag<T> Dbar;
  {
    // Dbar_{L-1} = P_{L-1} = lb Sinv - Sinv GG Sinv, symmetrised
    const Frag<T> U = f16::mm<T>(GG, S, zero);
    const Frag<T> Pr = f16::mm<T>(-U, S, lb * S);
    f16::wave_sync();
    io16::put_frag(tA, g, j, Pr);
    f16::wave_sync();
    Dbar = T(0.5) * (Pr + io16::get_frag_t(tA, g, j));
    f16::wave_sync();
    io16::put_frag(tA, g, j, Dbar);
    f16::wave_sync();
    io16::store(Db + (L - 1) * kBB, lane, io16::get(tA, lane));
  }
  // Distribute, with the next block's packed Sinv, GG and its C, Gl in flight.
  auto ld_s = [&](int k) { return io16::load_packed(st + k * kStateBlock, lane); };
  auto ld_g = [&](int k) { return io16::load_packed(st + k * kStateBlock + kPB, lane); };
  io16::Nat<T> S0 = ld_s(lc), Q0 = ld_g(lc), C2 = io16::load(C + lc * kBB, lane),
               E2 = io16::load(Gl + lc * kBB, lane);
  io16::Nat<T> S1, Q1, C3, E3;
  auto distribute = [&](int i, const io16::Nat<T> &Su, const io16::Nat<T> &Qu,
                        const io16::Nat<T> &Cu, const io16::Nat<T> &Eu, io16::Nat<T> &Sn,
                        io16::Nat<T> &Qn, io16::Nat<T> &Cn, io16::Nat<T> &En) {
    const int in = max(i - 1, 0);
    Sn = ld_s(in);
    Qn = ld_g(in);
    Cn = io16::load(C + in * kBB, lane);
    En = io16::load(Gl + in * kBB, lane);
    f16::wave_sync();
    io16::put_packed(tP, lane, Su);
    io16::put_packed(tQ, lane, Qu);
    io16::put(tA, lane, Cu);
    io16::put(tB, lane, Eu);
    f16::wave_sync();
    const Frag<T> Si = sl.get_packed(tP);
    const Frag<T> GGf = sl.get_packed(tQ);
    const Frag<T> Ct = io16::get_frag_t(tA, g, j);   // O(C_i^T)
    const Frag<T> Glt = io16::get_frag_t(tB, g, j);  // O(Gl_i^T)
    const Frag<T> Xf = f16::mm<T>(Ct, Si, zero);     // O(X_i), X_i = C_i Sinv_i
    const Frag<T> Yt = f16::mm<T>(Si, Ct, zero);     // O(X_i^T)
    const Frag<T> Wt = f16::mm<T>(GGf, Yt, zero);    // O(W^T)
    const Frag<T> Zf = f16::mm<T>(Wt + Wt - Glt, Si, zero);  // O(Z_i), Y2^T = 2 W^T - Gl^T
    const Frag<T> U = f16::mm<T>(GGf, Si, zero);             // O(GG Sinv)
    const Frag<T> Pf = f16::mm<T>(-U, Si, lb * Si);          // O(P_i)
    const Frag<T> T2 = f16::mm<T>(Dbar, Xf, zero);  // Dbar_{i+1} X_i
    const Frag<T> Q = f16::mm<T>(G, Zf, -T2);       // G Z_i - Dbar X_i
    const Frag<T> R = f16::mm<T>(Xf, Q, zero);      // X_i^T Q
    const Frag<T> V = f16::mm<T>(G, Xf, zero);      // G X_i
    G = f16::mm<T>(Xf, V, Si);                      // Sinv_i + X_i^T V
    f16::wave_sync();
    io16::put_frag(tA, g, j, Pf - R);
    io16::put_frag(tB, g, j, Q - T2);
    f16::wave_sync();
    Dbar = T(0.5) * ((Pf - R) + io16::get_frag_t(tA, g, j));  // P_i - sym(X_i^T Q)
    io16::store(Cb + i * kBB, lane, io16::get(tB, lane));
    f16::wave_sync();
    io16::put_frag(tC, g, j, Dbar);
    f16::wave_sync();
    io16::store(Db + i * kBB, lane, io16::get(tC, lane));
  };
  i = L - 2;
  for (; i >= 1; i -= 2) {
    distribute(i, S0, Q0, C2, E2, S1, Q1, C3, E3);
    distribute(i - 1, S1, Q1, C3, E3, S0, Q0, C2, E2);
  }
  if (i == 0) distribute(0, S0, Q0, C2, E2, S1, Q1, C3, E3);
  if (lane == 0 && info) info[m] = 0;
}

}  // namespace

size_t chain16_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L) {
  return align_up(static_cast<size_t>(B) * L * kStateBlock * dtype_bytes);
}

template <typename T>
hipError_t chain16_vjp_launch(int64_t B, int64_t L, const T *diag, const T *lower, const T *gd,
                              const T *gl, const double *ld_bar, T *d_bar, T *l_bar,
                              int32_t *info, void *ws, hipStream_t s) {
  hipLaunchKernelGGL(chain16_vjp_kernel<T>, dim3(static_cast<unsigned>(B)), dim3(64), 0, s,
                     static_cast<int>(L), diag, lower, gd, gl, ld_bar, d_bar, l_bar, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

template hipError_t chain16_vjp_launch<float>(int64_t, int64_t, const float *, const float *,
                                              const float *, const float *, const double *,
                                              float *, float *, int32_t *, void *, hipStream_t);
template hipError_t chain16_vjp_launch<double>(int64_t, int64_t, const double *, const double *,
                                               const double *, const double *, const double *,
                                               double *, double *, int32_t *, void *,
                                               hipStream_t);

}  // namespace selinv
