// chain_b32.hip -- block-tridiagonal selected inverse for 32x32 blocks with a
// two-sided sweep: the chain is rooted at its middle block r = L / 2 instead
// of its last block.  The gabp-sparse-inv 0.3.2 page notes that the root of a
// tree does not change the result (Quickstart, root-invariance remark), so
// the left part 0 .. r-1 (parent i+1) and the right part r+1 .. L-1 (parent
// i-1) are eliminated concurrently by two wavefronts of one workgroup, which
// meet at the root through LDS and then distribute outward.
//
// For a left node i:  E_i = A_{i+1,i} = lower[i];  for a right node i:
// E_i = A_{i-1,i} = lower[i-1]^T.  Per node (item Chain of "Implemented and
// tested kernels"; frag32.h layouts):
//   collect:    Sinv_i = S_i^{-1},  Y = Sinv_i E_i^T,  M_i = E_i Y,
//               S_parent = D_parent - M_i
//   root:       S_r = D_r - M_{r-1} - M_{r+1},  G_rr = S_r^{-1}
//   distribute: X = E_i Sinv_i,  V = G_pp X,  G_{p,i} = -V,
//               G_ii = Sinv_i + X^T V
// Left:  G_lower[i] = G_{i+1,i} = -V.   Right: G_lower[i-1] = G_{i,i-1} = -V^T.
// Only the packed Sinv_i (528 entries) crosses from collect to distribute.
#include "frag32.h"
#include "internal.h"

namespace selinv {

namespace {

using f32t::Blk;
constexpr int BB = 1024, PB = f32t::kPacked32;

template <typename T>
__device__ __forceinline__ Blk<T> nan_blk() {
  Blk<T> b;
  const T nan = static_cast<T>(__builtin_nan(""));
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.t[I][J][r] = nan;
  return b;
}

// O32 of E^T for node i: left E^T = lower[i]^T (loaded transposed),
// right E^T = lower[i-1] (loaded as is).  As a left factor, O32(E^T)
// serves products with E on the left: O32(E B) = mm(O32(E^T), O32(B)).
template <bool RIGHT, typename T>
__device__ __forceinline__ Blk<T> load_et(const T *C, int i, int g, int j) {
  if (RIGHT) return f32t::load(C + (i - 1) * BB, g, j);
  return f32t::load_t(C + i * BB, g, j);
}

template <typename T>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 2)))
void chain32_kernel(int L, const T *__restrict__ diag, const T *__restrict__ lower,
                    T *__restrict__ G_diag, T *__restrict__ G_lower, double *__restrict__ logdet,
                    int32_t *__restrict__ info, T *__restrict__ state) {
  __shared__ __align__(32) T col[2][32];
  __shared__ __align__(32) T msg[2][BB];  // messages into the root, O32 lane order
  __shared__ int32_t s_fail[2];
  __shared__ double s_ld[2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x;
  const T *D = diag + m * L * BB;
  const T *C = lower + m * (L - 1) * BB;
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
  T *st = state + m * L * PB;
  const int r = L / 2;  // root
  const f32t::SymOffsets<T> so(g, j);
  const f32t::PackedOffsets<T> po(g, j);
  T *mycol = col[wave];

  // ---------------------------------------------------------------- collect
  // wave 0: i = 0 .. r-1 (parent i+1); wave 1: i = L-1 .. r+1 (parent i-1)
  const bool right = wave == 1;
  const int n = right ? L - 1 - r : r;  // nodes of this part
  double ld = 0.0;
  int32_t fail = 0;
  Blk<T> M = f32t::zero<T>();
  if (n > 0) {
    Blk<T> S = so.load(D + (right ? L - 1 : 0) * BB);
    for (int t = 0; t < n; ++t) {
      const int i = right ? L - 1 - t : t;
      const int ip = right ? i - 1 : i + 1;  // parent
      // inputs consumed after this sweep: E_i^T and D_parent
      const Blk<T> Et = right ? load_et<true>(C, i, g, j) : load_et<false>(C, i, g, j);
      const Blk<T> Dp = so.load(D + ip * BB);
      f16::PivotLog pl;
      if (f32t::gj_inverse(S, mycol, g, j, pl)) {
        fail = i + 1;
        break;
      }
      ld += pl.log();
      po.store(st + i * PB, S);
      const Blk<T> Y = f32t::mm(S, Et, f32t::zero<T>());  // Sinv_i E_i^T
      M = f32t::mm(Et, Y, f32t::zero<T>());               // E_i Sinv_i E_i^T
      if (t + 1 < n) S = f32t::sub(Dp, M);
    }
  }
  // hand the message to the root through LDS
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
      *reinterpret_cast<f16::Frag<T> *>(&msg[wave][((I * 2 + J) * 64 + lane) * 4]) = M.t[I][J];
  if (lane == 0) {
    s_fail[wave] = fail;
    s_ld[wave] = ld;
  }
  __syncthreads();
  // ------------------------------------------------------------------ root
  // both wavefronts form S_r and invert it (identical work, no extra barrier)
  Blk<T> G = so.load(D + r * BB);
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
      for (int J = 0; J < 2; ++J)
        G.t[I][J] = G.t[I][J] - *reinterpret_cast<const f16::Frag<T> *>(
                                    &msg[w][((I * 2 + J) * 64 + lane) * 4]);
  f16::PivotLog plr;
  const bool root_bad = f32t::gj_inverse(G, mycol, g, j, plr);
  int32_t any_fail = s_fail[0] ? s_fail[0] : (s_fail[1] ? s_fail[1] : (root_bad ? r + 1 : 0));
  if (any_fail) {
    // outputs of a failed matrix are NaN
    const Blk<T> nb = nan_blk<T>();
    if (wave == 0) {
      for (int i = 0; i <= r; ++i) f32t::store(Gd + i * BB, nb, g, j);
      for (int i = 0; i < r; ++i) f32t::store(Gl + i * BB, nb, g, j);
    } else {
      for (int i = r + 1; i < L; ++i) {
        f32t::store(Gd + i * BB, nb, g, j);
        f32t::store(Gl + (i - 1) * BB, nb, g, j);
      }
      if (lane == 0) {
        logdet[m] = __builtin_nan("");
        if (info) info[m] = any_fail;
      }
    }
    return;
  }
  if (wave == 0) {
    f32t::store_t(Gd + r * BB, G, g, j);
    if (lane == 0) {
      logdet[m] = s_ld[0] + s_ld[1] + plr.log();
      if (info) info[m] = 0;
    }
  }
  // -------------------------------------------------------------- distribute
  if (n == 0) return;
  {
    const int i0 = right ? r + 1 : r - 1;
    Blk<T> Sa = po.load(st + i0 * PB), Sb = f32t::zero<T>();
    Blk<T> Ea = right ? load_et<true>(C, i0, g, j) : load_et<false>(C, i0, g, j);
    Blk<T> Eb = f32t::zero<T>();
    auto node = [&](int t, const Blk<T> &Si, const Blk<T> &Et, Blk<T> &Sn, Blk<T> &En) -> bool {
      if (t >= n) return true;
      const int i = right ? r + 1 + t : r - 1 - t;
      const int tn = min(t + 1, n - 1);
      const int in = right ? r + 1 + tn : r - 1 - tn;
      Sn = po.load(st + in * PB);
      En = right ? load_et<true>(C, in, g, j) : load_et<false>(C, in, g, j);
      const Blk<T> X = f32t::mm(Et, Si, f32t::zero<T>());  // E_i Sinv_i
      const Blk<T> V = f32t::mm(G, X, f32t::zero<T>());    // G_pp X = -G_{p,i}
      if (right)
        f32t::store_t(Gl + (i - 1) * BB, f32t::neg(V), g, j);  // G_{i,i-1} = -V^T
      else
        f32t::store(Gl + i * BB, f32t::neg(V), g, j);          // G_{i+1,i} = -V
      G = f32t::mm(X, V, Si);                              // Sinv_i + X^T V
      f32t::store_t(Gd + i * BB, G, g, j);
      return false;
    };
    for (int t = 0;; t += 2) {
      if (node(t, Sa, Ea, Sb, Eb)) break;
      if (node(t + 1, Sb, Eb, Sa, Ea)) break;
    }
  }
}

}  // namespace

size_t chain32_workspace_bytes(int dtype_bytes, int64_t B, int64_t L) {
  return align_up(static_cast<size_t>(B) * L * PB * dtype_bytes);
}

template <typename T>
hipError_t chain32_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                          T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s) {
  hipLaunchKernelGGL(chain32_kernel<T>, dim3(static_cast<unsigned>(B)), dim3(128), 0, s,
                     static_cast<int>(L), diag, lower, G_diag, G_lower, logdet, info,
                     static_cast<T *>(ws));
  return hipGetLastError();
}

template hipError_t chain32_launch<float>(int64_t, int64_t, const float *, const float *, float *,
                                          float *, double *, int32_t *, void *, hipStream_t);
template hipError_t chain32_launch<double>(int64_t, int64_t, const double *, const double *,
                                           double *, double *, double *, int32_t *, void *,
                                           hipStream_t);

}  // namespace selinv
