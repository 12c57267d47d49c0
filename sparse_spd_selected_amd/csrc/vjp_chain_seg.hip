// vjp_chain_seg.hip -- reverse mode of the chain selected inverse for a few
// long chains, parallel over segments of each chain.
//
// The two-pass reverse mode (vjp_generic.hip; the analytic backward of the
// gabp-sparse-inv 0.3.2 page's differentiable tree) is sequential along a
// chain.  With C_i = lower[i], X_i = C_i Sinv_i and the forward selected
// inverse G already computed (here by the segment-parallel forward), every
// recurrence it needs can be cut into segments:
//   * Sinv at a segment start a comes from G alone:  X_a = -G_{a+1,a+1}^{-1}
//     G_{a+1,a} and Sinv_a = G_aa - G_{a+1,a}^T G_{a+1,a+1}^{-1} G_{a+1,a}
//     (from G_{a+1,a} = -G_{a+1,a+1} X_a and G_aa = Sinv_a + X_a^T G_{a+1,a+1}
//     X_a); inside the segment the ordinary collect recurrence continues;
//   * the cotangent of G_ii obeys GG_{i+1} = X_i GG_i X_i^T + c_i with
//     c_i = sym(Gd_{i+1}) - sym(Gl_i X_i^T), an affine congruence: a segment
//     maps GG_a to GG_e = Phi GG_a Phi^T + Cm (Phi = X_{e-1} ... X_a);
//   * the input cotangent obeys Dbar_i = X_i^T Dbar_{i+1} X_i + r_i with
//     r_i = P_i - sym(X_i^T G_{i+1,i+1} Z_i), the same congruence run
//     backwards: Dbar_a = Phi^T Dbar_e Phi + R, R = sum_i Pi_i^T r_i Pi_i,
//     Pi_i = X_{i-1} ... X_a.
// Passes (b = 32; prep, mid and out are one wavefront per segment with the
// blocks in the MFMA 32 x 32 register layout of frag32.h, the two scans one
// workgroup per chain with the blocks in LDS):
//   forward selected inverse (any forward path) -> G, info
//   prep:  Sinv_i, X_i per block; the GG map (Phi, Cm) per segment
//   scan:  one workgroup per chain, GG at every segment start
//   mid:   P_i = lb Sinv_i - Sinv_i GG_i Sinv_i, Z_i = (2 X_i GG_i - Gl_i) Sinv_i,
//          the Dbar map's R per segment
//   scan:  one workgroup per chain, Dbar at every segment end (from P_{L-1})
//   out:   Dbar_i and lower_bar_i = G_{i+1,i+1} Z_i - 2 Dbar_{i+1} X_i, descending
// Decay.  Phi and Pi_i are products of the X's from the segment start; on a
// diagonally dominant chain they shrink geometrically (2^-3.6 per block on
// the b = 32 workload), as the forward's fill block does.  Once every entry
// of Phi (prep) or Pi_i (mid) is at most 2^-100 (both start as I), it is set
// to zero and no longer updated: what is lost is Pi_d^T R' Pi_d (R' the map of
// the rest of the segment) in R, and the corresponding Phi_d GG_a Phi_d^T
// term in the GG map, 2^-200 relative to terms of the same shape.  A product
// that does not decay is never dropped.
#include <algorithm>
#include <climits>

#include "block_wg.h"
#include "frag32.h"
#include "internal.h"
#include "io32.h"

namespace selinv {

namespace {

inline int cvs_threads(int b) { return b <= 8 ? 64 : 256; }

struct SegRange {
  int64_t a0, a1;
};
__device__ inline SegRange seg_range(int64_t L, int P, int s) {
  return {static_cast<int64_t>(s) * L / P, static_cast<int64_t>(s + 1) * L / P};
}

// GG at every segment start, one workgroup per chain
template <typename T>
__global__ void cvs_gg_scan(int b, int P, int64_t L, const T *__restrict__ gd,
                            const T *__restrict__ phi, const T *__restrict__ cmap,
                            T *__restrict__ gg_start) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *GG = smem, *T2 = GG + bb, *Ph = T2 + bb;
  const int64_t m = blockIdx.x;
  wg::sym_part(GG, gd + m * L * bb, b);
  for (int s = 0; s < P; ++s) {
    const int64_t q = m * P + s;
    wg::copy(gg_start + q * bb, GG, bb);
    wg::copy(Ph, phi + q * bb, bb);
    wg::gemm<T, false, false>(T2, Ph, GG, b);
    wg::gemm_sym<T, false, true>(GG, cmap + q * bb, T2, Ph, b, T(1));  // base read once
  }
}

// Dbar at every segment end (the first block after the segment; the root for
// the last one), one workgroup per chain
template <typename T>
__global__ void cvs_db_scan(int b, int P, int64_t L, const T *__restrict__ p_ws,
                            const T *__restrict__ phi, const T *__restrict__ rmap,
                            T *__restrict__ db_end) {
  extern __shared__ unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);
  const int bb = b * b;
  T *Db = smem, *T2 = Db + bb, *Ph = T2 + bb;
  const int64_t m = blockIdx.x;
  wg::copy(Db, p_ws + (m * L + L - 1) * bb, bb);
  for (int s = P - 1; s >= 0; --s) {
    const int64_t q = m * P + s;
    wg::copy(db_end + q * bb, Db, bb);
    wg::copy(Ph, phi + q * bb, bb);
    wg::gemm<T, false, false>(T2, Db, Ph, b);
    wg::gemm_sym<T, true, false>(Db, rmap + q * bb, Ph, T2, b, T(1));
  }
}

// ------------------------------------------------------ wave kernels, b = 32
// O32(M) is the register layout of frag32.h; f32t::mm(O(A^T), O(B)) = O(A B).
// Workspace blocks: Sinv_i as its packed lower triangle, X_i stored as X_i^T
// (row-major), P_i and Z_i row-major.
using f32t::Blk;
constexpr int kBB32 = 1024;

template <typename T>
__device__ __forceinline__ Blk<T> lin32(T a, const Blk<T> &x, T c, const Blk<T> &y) {
  Blk<T> r;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) r.t[I][J] = a * x.t[I][J] + c * y.t[I][J];
  return r;
}

template <typename T>
__device__ __forceinline__ Blk<T> scale32(T a, const Blk<T> &x) {
  Blk<T> r;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) r.t[I][J] = a * x.t[I][J];
  return r;
}

template <typename T>
__device__ __forceinline__ Blk<T> identity32(int g, int j) {
  Blk<T> r = f32t::zero<T>();
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int q = 0; q < 4; ++q) r.t[I][I][q] = f16::row<T>(g, q) == j ? T(1) : T(0);
  return r;
}

// row-major block -> its O32 (and, optionally, the O32 of its transpose)
// through the wavefront's tile; `ws` selects cacheable workspace loads
template <typename T>
struct Io32 {
  T *tile;
  int lane, g, j;
  __device__ __forceinline__ void stage(const T *P, bool ws) const {
    f16::wave_sync();
    io32::put(tile, lane, ws ? io32::load_ws(P, lane) : io32::load(P, lane));
    f16::wave_sync();
  }
  // a block already loaded into registers
  __device__ __forceinline__ void stage(const io32::Nat<T> &n) const {
    f16::wave_sync();
    io32::put(tile, lane, n);
    f16::wave_sync();
  }
  __device__ __forceinline__ Blk<T> blk() const { return io32::get_blk(tile, g, j); }
  __device__ __forceinline__ Blk<T> blk_t() const { return io32::get_blk_t(tile, g, j); }
  // row-major store of the block b (all four tiles formed)
  __device__ __forceinline__ void store(T *P, const Blk<T> &b, bool ws) const {
    f16::wave_sync();
    io32::put_blk(tile, g, j, b);
    f16::wave_sync();
    if (ws)
      io32::store_ws(P, lane, io32::get(tile, lane));
    else
      io32::store(P, lane, io32::get(tile, lane));
  }
  // (M + M^T) / 2 of a block with all four tiles formed: exactly symmetric
  // (entries (a, c) and (c, a) are the same two terms added)
  __device__ __forceinline__ Blk<T> symmetrize(const Blk<T> &b) const {
    f16::wave_sync();
    io32::put_blk(tile, g, j, b);
    f16::wave_sync();
    return lin32(T(0.5), io32::get_blk(tile, g, j), T(0.5), io32::get_blk_t(tile, g, j));
  }
  // row-major store of a symmetric result of which tiles (0,0), (1,0), (1,1)
  // are formed, made exactly symmetric; returns the full block in registers
  __device__ __forceinline__ Blk<T> store_sym(T *P, const Blk<T> &b, bool ws) const {
    f16::wave_sync();
    io32::put_sym(tile, g, j, b);
    f16::wave_sync();
    const Blk<T> f = lin32(T(0.5), io32::get_blk(tile, g, j), T(0.5), io32::get_blk_t(tile, g, j));
    store(P, f, ws);
    return f;
  }
};

// prep: Sinv_i (packed) and X_i^T per block, the segment's GG map (Phi, Cm)
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void cvs32_prep(
    int64_t L, int P, const T *__restrict__ diag, const T *__restrict__ lower,
    const T *__restrict__ gd, const T *__restrict__ gl, const T *__restrict__ Gd,
    const T *__restrict__ Gl, T *__restrict__ sinv_ws, T *__restrict__ x_ws,
    T *__restrict__ phi, T *__restrict__ cmap) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const Io32<T> io{tA, lane, g, j};
  const io32::SymLanes<T> sl(g, j, lane);
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange r = seg_range(L, P, s);
  const T *D = diag + m * L * kBB32, *C = lower + m * (L - 1) * kBB32;
  const T *GDm = Gd + m * L * kBB32, *GLm = Gl + m * (L - 1) * kBB32;
  const T *gdm = gd + m * L * kBB32, *glm = gl + m * (L - 1) * kBB32;
  f16::PivotLog pl;  // pivots unused here
  Blk<T> S;
  if (s == 0) {
    f16::wave_sync();
    io32::put(tA, lane, io32::load(D, lane));
    f16::wave_sync();
    S = sl.get_sym(tA);
  } else {  // Sinv_a = G_aa - G_{a+1,a}^T G_{a+1,a+1}^{-1} G_{a+1,a}
    f16::wave_sync();
    io32::put(tA, lane, io32::load_ws(GDm + (r.a0 + 1) * kBB32, lane));
    f16::wave_sync();
    Blk<T> Gn = sl.get_sym(tA);
    f32t::gj_inverse(Gn, col, g, j, pl);
    io.stage(GLm + r.a0 * kBB32, true);
    const Blk<T> GLa = io.blk();                                 // O(G_{a+1,a})
    const Blk<T> T2 = f32t::mm(Gn, GLa, f32t::zero<T>());        // G_{a+1,a+1}^-1 G_{a+1,a}
    f16::wave_sync();
    io32::put(tA, lane, io32::load_ws(GDm + r.a0 * kBB32, lane));
    f16::wave_sync();
    S = f32t::sub(sl.get_sym(tA), f32t::mm(GLa, T2, f32t::zero<T>()));
  }
  Blk<T> Ph = identity32<T>(g, j), Cm = f32t::zero<T>();
  bool decayed = false;  // Phi dropped
  for (int64_t i = r.a0; i < r.a1; ++i) {
    if (i > r.a0 || s == 0) f32t::gj_inverse(S, col, g, j, pl);  // S <- Sinv_i
    f16::wave_sync();
    io32::put_blk(tA, g, j, S);
    f16::wave_sync();
    io32::store_packed(sinv_ws + (m * L + i) * kBB32, lane, sl.gather_packed(tA));
    if (i == L - 1) break;
    // the step's four input blocks, loaded together
    const io32::Nat<T> nC = io32::load(C + i * kBB32, lane);
    const io32::Nat<T> nD = io32::load(D + (i + 1) * kBB32, lane);
    const io32::Nat<T> nGl = io32::load(glm + i * kBB32, lane);
    const io32::Nat<T> nGd = io32::load(gdm + (i + 1) * kBB32, lane);
    io.stage(nC);
    const Blk<T> Ct = io.blk_t();                                // O(C_i^T)
    const Blk<T> XT = f32t::mm(S, Ct, f32t::zero<T>());          // O(X_i^T) = O(Sinv C_i^T)
    io.store(x_ws + (m * L + i) * kBB32, XT, true);              // X_i^T, row-major
    // S_{i+1} = D_{i+1} - C_i Sinv_i C_i^T (tile (1,0) not formed)
    io.stage(nD);
    S = f32t::sub(sl.get_sym(tA), f32t::mm_upper(Ct, XT, f32t::zero<T>()));
    // c_i = sym(gd_{i+1}) - sym(gl_i X_i^T) = sym(gd_{i+1} - gl_i X_i^T)
    io.stage(nGl);
    const Blk<T> GLtn = f32t::neg(io.blk_t());                   // -O(gl_i^T)
    io.stage(nGd);
    const Blk<T> c = io.symmetrize(f32t::mm(GLtn, XT, io.blk()));
    if (!decayed) {
      Ph = f32t::mm(XT, Ph, f32t::zero<T>());                    // Phi <- X_i Phi
      if (f32t::all_below(Ph, T(0x1p-100))) {
        decayed = true;
        Ph = f32t::zero<T>();
      }
    }
    const Blk<T> W = f32t::mm(Cm, XT, f32t::zero<T>());          // Cm X^T
    Cm = f32t::mm(XT, W, c);                                     // X Cm X^T + c
  }
  io.store(phi + (m * P + s) * kBB32, Ph, true);
  io.store(cmap + (m * P + s) * kBB32, Cm, true);
}

// mid: P_i, Z_i per block and the segment's Dbar map R, from GG at the start
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void cvs32_mid(
    int64_t L, int P, const T *__restrict__ gd, const T *__restrict__ gl,
    const double *__restrict__ ld_bar, const T *__restrict__ Gd, const T *__restrict__ sinv_ws,
    const T *__restrict__ x_ws, const T *__restrict__ gg_start, T *__restrict__ p_ws,
    T *__restrict__ z_ws, T *__restrict__ rmap) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tP[Tr::kPacked];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const Io32<T> io{tA, lane, g, j};
  const io32::SymLanes<T> sl(g, j, lane);
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange rg = seg_range(L, P, s);
  const T lb = ld_bar ? static_cast<T>(ld_bar[m]) : T(0);
  const T *gdm = gd + m * L * kBB32, *glm = gl + m * (L - 1) * kBB32, *GDm = Gd + m * L * kBB32;
  io.stage(gg_start + (m * P + s) * kBB32, true);
  Blk<T> GG = io.blk(), Pi = identity32<T>(g, j), R = f32t::zero<T>();
  bool decayed = false;  // Pi dropped
  for (int64_t i = rg.a0; i < rg.a1; ++i) {
    // the step's input blocks, loaded together (the last block has only Sinv)
    const bool more = i < L - 1;
    const int64_t inx = more ? i + 1 : i;
    const io32::NatP<T> nS = io32::load_packed(sinv_ws + (m * L + i) * kBB32, lane);
    const io32::Nat<T> nX = io32::load_ws(x_ws + (m * L + (more ? i : 0)) * kBB32, lane);
    const io32::Nat<T> nGl = io32::load(glm + (more ? i : 0) * kBB32, lane);
    const io32::Nat<T> nGd = io32::load(gdm + inx * kBB32, lane);
    const io32::Nat<T> nG = io32::load_ws(GDm + inx * kBB32, lane);
    f16::wave_sync();
    io32::put_packed(tP, lane, nS);
    f16::wave_sync();
    const Blk<T> Si = sl.get_packed(tP);
    // P_i = lb Sinv - Sinv GG Sinv (lower tiles), stored and read back in full
    const Blk<T> A = f32t::mm(GG, Si, f32t::zero<T>());          // GG Sinv
    const Blk<T> Pf = io.store_sym(p_ws + (m * L + i) * kBB32,
                                   f32t::mm_lower(f32t::neg(A), Si, scale32(lb, Si)), true);
    if (!more) break;
    io.stage(nX);                                                // X_i^T
    const Blk<T> XT = io.blk(), Xo = io.blk_t();                 // O(X^T), O(X)
    io.stage(nGl);
    const Blk<T> GLt = io.blk_t();                               // O(gl_i^T)
    const Blk<T> Wt = f32t::mm(GG, XT, f32t::zero<T>());         // O(W^T), W = X GG
    const Blk<T> Y1t = f32t::sub(Wt, GLt);                       // O((W - gl)^T)
    const Blk<T> Y2t = lin32(T(2), Wt, T(-1), GLt);              // O((2W - gl)^T)
    // GG <- sym(gd_{i+1}) + sym(Y1 X^T) = sym(gd_{i+1} + Y1 X^T)
    io.stage(nGd);
    GG = io.symmetrize(f32t::mm(Y1t, XT, io.blk()));
    const Blk<T> Z = f32t::mm(Y2t, Si, f32t::zero<T>());         // Z_i = Y2 Sinv
    io.store(z_ws + (m * L + i) * kBB32, Z, true);
    // r_i = P_i - sym(X^T G_{i+1,i+1} Z_i) = sym(P_i - X^T G Z)  (P_i symmetric)
    io.stage(nG);
    const Blk<T> Vn = f32t::neg(f32t::mm(io.blk_t(), Z, f32t::zero<T>()));  // -G Z
    const Blk<T> rr = io.symmetrize(f32t::mm(Xo, Vn, Pf));
    // R += Pi^T r Pi, Pi <- X_i Pi
    if (!decayed) {
      const Blk<T> A2 = f32t::mm(rr, Pi, f32t::zero<T>());       // r Pi
      R = f32t::mm(Pi, A2, R);
      Pi = f32t::mm(XT, Pi, f32t::zero<T>());
      decayed = f32t::all_below(Pi, T(0x1p-100));
    }
  }
  io.store(rmap + (m * P + s) * kBB32, R, true);
}

// out: Dbar_i and lower_bar_i = G_{i+1,i+1} Z_i - 2 Dbar_{i+1} X_i, descending
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void cvs32_out(
    int64_t L, int P, const T *__restrict__ Gd, const T *__restrict__ x_ws,
    const T *__restrict__ z_ws, const T *__restrict__ p_ws, const T *__restrict__ db_end,
    const int32_t *__restrict__ info_ws, T *__restrict__ d_bar, T *__restrict__ l_bar,
    int32_t *__restrict__ info) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T tA[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const Io32<T> io{tA, lane, g, j};
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const SegRange rg = seg_range(L, P, s);
  const int64_t e = s == P - 1 ? L - 1 : rg.a1;
  T *Dbm = d_bar + m * L * kBB32, *Lbm = l_bar + m * (L - 1) * kBB32;
  if (s == 0 && lane == 0 && info) info[m] = info_ws[m];
  if (info_ws[m]) {
    const T nan = static_cast<T>(__builtin_nan(""));
    for (int64_t q = rg.a0 * kBB32 + lane; q < rg.a1 * kBB32; q += 64) Dbm[q] = nan;
    for (int64_t q = rg.a0 * kBB32 + lane; q < min(rg.a1, L - 1) * kBB32; q += 64) Lbm[q] = nan;
    return;
  }
  io.stage(db_end + (m * P + s) * kBB32, true);
  Blk<T> Db = io.blk();
  if (s == P - 1) io.store(Dbm + (L - 1) * kBB32, Db, false);  // Dbar_{L-1} = P_{L-1}
  for (int64_t i = e - 1; i >= rg.a0; --i) {
    // the step's input blocks, loaded together
    const io32::Nat<T> nX = io32::load_ws(x_ws + (m * L + i) * kBB32, lane);
    const io32::Nat<T> nZ = io32::load_ws(z_ws + (m * L + i) * kBB32, lane);
    const io32::Nat<T> nG = io32::load_ws(Gd + (m * L + i + 1) * kBB32, lane);
    const io32::Nat<T> nP = io32::load_ws(p_ws + (m * L + i) * kBB32, lane);
    io.stage(nX);
    const Blk<T> Xo = io.blk_t();                                // O(X_i)
    io.stage(nZ);
    const Blk<T> Z = io.blk();
    io.stage(nG);
    const Blk<T> Gt = io.blk_t();                                // O(G^T)
    const Blk<T> T2 = f32t::mm(Db, Xo, f32t::zero<T>());         // Dbar_{i+1} X_i (Dbar sym)
    const Blk<T> Q = f32t::mm(Gt, Z, f32t::neg(T2));             // G Z - Dbar X
    io.store(Lbm + i * kBB32, f32t::sub(Q, T2), false);          // lower_bar_i = Q - T2
    io.stage(nP);
    // Dbar_i = P_i - sym(X^T Q) = sym(P_i - X^T Q)  (P_i symmetric)
    const Blk<T> Dn = io.symmetrize(f32t::mm(Xo, f32t::neg(Q), io.blk()));
    io.store(Dbm + i * kBB32, Dn, false);
    Db = Dn;
  }
}

struct CvsLayout {
  size_t gd, gl, ld, info, fwd, sinv, x, p, z, phi, cmap, rmap, ggs, dbe, total;
};

CvsLayout cvs_layout(int dtype_bytes, int64_t B, int64_t L, int32_t b, int P) {
  CvsLayout o{};
  const size_t bb = static_cast<size_t>(b) * b, w = dtype_bytes;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  o.gd = take(B * L * bb * w);
  o.gl = take(B * (L - 1) * bb * w);
  o.ld = take(B * sizeof(double));
  o.info = take(B * sizeof(int32_t));
  o.fwd = take(chain_workspace_bytes(dtype_bytes, B, L, b));
  o.sinv = take(B * L * bb * w);
  o.x = take(B * L * bb * w);
  o.p = take(B * L * bb * w);
  o.z = take(B * L * bb * w);
  o.phi = take(B * P * bb * w);
  o.cmap = take(B * P * bb * w);
  o.rmap = take(B * P * bb * w);
  o.ggs = take(B * P * bb * w);
  o.dbe = take(B * P * bb * w);
  o.total = off;
  return o;
}

}  // namespace

int chain_vjp_segments(int64_t B, int64_t L, int32_t b) {
  if (b != 32 || B >= 512 || L < 512) return 0;
  return static_cast<int>(std::min<int64_t>(L / 128, 16384 / B));
}

size_t chain_vjp_seg_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b, int P) {
  return cvs_layout(dtype_bytes, B, L, b, P).total;
}

template <typename T>
hipError_t chain_vjp_seg_launch(int64_t B, int64_t L, int32_t b, int P, const T *diag,
                                const T *lower, const T *gd, const T *gl, const double *ld_bar,
                                T *d_bar, T *l_bar, int32_t *info, void *ws, hipStream_t s) {
  const CvsLayout o = cvs_layout(sizeof(T), B, L, b, P);
  char *base = static_cast<char *>(ws);
  T *Gd = reinterpret_cast<T *>(base + o.gd), *Gl = reinterpret_cast<T *>(base + o.gl);
  double *ld = reinterpret_cast<double *>(base + o.ld);
  int32_t *info_ws = reinterpret_cast<int32_t *>(base + o.info);
  T *sinv = reinterpret_cast<T *>(base + o.sinv), *x = reinterpret_cast<T *>(base + o.x);
  T *p = reinterpret_cast<T *>(base + o.p), *z = reinterpret_cast<T *>(base + o.z);
  T *phi = reinterpret_cast<T *>(base + o.phi), *cmap = reinterpret_cast<T *>(base + o.cmap);
  T *rmap = reinterpret_cast<T *>(base + o.rmap), *ggs = reinterpret_cast<T *>(base + o.ggs);
  T *dbe = reinterpret_cast<T *>(base + o.dbe);
  hipError_t e = chain_launch<T>(B, L, b, diag, lower, Gd, Gl, ld, info_ws, base + o.fwd, s);
  if (e != hipSuccess) return e;
  if (b != 32) return hipErrorInvalidValue;  // segments are planned for b = 32 only
  const int nt = cvs_threads(b);
  const size_t bb = static_cast<size_t>(b) * b;
  const dim3 segs(static_cast<unsigned>(B * P)), chains(static_cast<unsigned>(B));
  hipLaunchKernelGGL(cvs32_prep<T>, segs, dim3(64), 0, s, L, P, diag, lower, gd, gl, Gd, Gl,
                     sinv, x, phi, cmap);
  hipLaunchKernelGGL(cvs_gg_scan<T>, chains, dim3(nt), 3 * bb * sizeof(T), s, b, P, L, gd, phi,
                     cmap, ggs);
  hipLaunchKernelGGL(cvs32_mid<T>, segs, dim3(64), 0, s, L, P, gd, gl, ld_bar, Gd, sinv, x, ggs,
                     p, z, rmap);
  hipLaunchKernelGGL(cvs_db_scan<T>, chains, dim3(nt), 3 * bb * sizeof(T), s, b, P, L, p, phi,
                     rmap, dbe);
  hipLaunchKernelGGL(cvs32_out<T>, segs, dim3(64), 0, s, L, P, Gd, x, z, p, dbe, info_ws, d_bar,
                     l_bar, info);
  return hipGetLastError();
}

template hipError_t chain_vjp_seg_launch<float>(int64_t, int64_t, int32_t, int, const float *,
                                                const float *, const float *, const float *,
                                                const double *, float *, float *, int32_t *,
                                                void *, hipStream_t);
template hipError_t chain_vjp_seg_launch<double>(int64_t, int64_t, int32_t, int, const double *,
                                                 const double *, const double *, const double *,
                                                 const double *, double *, double *, int32_t *,
                                                 void *, hipStream_t);

}  // namespace selinv
