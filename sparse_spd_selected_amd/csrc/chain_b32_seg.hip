// chain_b32_seg.hip -- block-tridiagonal selected inverse for 32x32 blocks
// when there are too few chains to occupy the GPU with one sweep per chain.
//
// The selected inverse does not depend on the elimination order (any order is
// a Cholesky of a symmetric permutation of A; the gabp-sparse-inv 0.3.2 page
// makes the same point for the choice of root, Quickstart).  Each chain of L
// blocks is cut into P segments [a_s, a_{s+1}); the last block t_s of every
// segment is a separator.  Elimination order: the interiors of all segments
// (in parallel, each from its first block on), then the separators.
//
// Collect, segment s >= 1 with left separator t = t_{s-1}: eliminating the
// interior block i (neighbours i+1 and t) with S_i its Schur block,
// F_i = A'_{i,t} the fill block to t, C_i = lower[i] = A_{i+1,i}:
//     Sinv = S_i^-1,  S_{i+1} = D_{i+1} - C_i Sinv C_i^T,
//     F_{i+1} = -C_i Sinv F_i   (F_{a_s} = A_{a_s,t} = lower[a_s - 1]),
//     U_s += F_i^T Sinv F_i     (update of the separator t).
// Segment 0 has no left separator (F = U = 0).  What remains is a chain of
// the P separators: diagonal S_{t_s} - U_{s+1}, off-diagonal F_{t_{s+1}}
// (= A'_{t_{s+1}, t_s}); it is solved by the two-sided b = 32 chain kernel.
// Distribute, with the 2x2 block G_NN of the neighbours N = {i+1, t} known:
//     X1 = C_i Sinv,  X2 = F_i^T Sinv,
//     V1 = G_{i+1,i+1} X1 + G_{i+1,t} X2 = -G_{i+1,i},
//     V2 = G_{t,i+1}  X1 + G_{t,t}  X2 = -G_{t,i},
//     G_ii = Sinv + X1^T V1 + X2^T V2
// (the Takahashi step of the chain item, "Implemented and tested kernels",
// with a two-block parent set).  G_lower[i] = -V1; G_{t,i} is carried to the
// next (lower) block and G_{a_s,t} becomes G_lower[a_s - 1].
//
// Work per block: one 32x32 inverse, five block products forward and eight
// backward (against two and three for the plain sweep), in exchange for B*P
// independent sweeps instead of B.
//
// Fill decay.  F_{i+1} = -C_i Sinv F_i shrinks geometrically along a
// diagonally dominant segment (by |C_i S_i^-1| per block: 2^-3.6 on the
// b = 32 workload).  Once every entry of F_{i+1} is at most 2^-100 times the
// largest entry of the segment's first coupling block A_{a,t}, the collect
// stops carrying it: F_j = 0 for j > i, which is exactly the elimination of
// A + E with E one block at (i+1, t) (and its transpose) equal to the F_{i+1}
// just computed.  max|E| <= 2^-100 max|A|, 47 bits below the rounding of A's
// own entries, so the result is the selected inverse of A to within the
// rounding error the computation has anyway.  From there on every step of
// the segment is the plain sweep (two products forward, three backward):
// with F = 0 the update of t stops, the segment's final fill block is zero,
// so G_{t_s,t} = 0 comes out of the separator chain exactly and G_{t,j} = 0
// for every j past the drop.  A fill that does not decay is never dropped.
#include <algorithm>
#include <cmath>

#include "frag32.h"
#include "internal.h"
#include "io32.h"

namespace selinv {

namespace {

using f32t::Blk;
constexpr int BB = 1024, PB = f32t::kPacked32;

__device__ __forceinline__ int seg_begin(int s, int L, int P) {
  return static_cast<int>(static_cast<int64_t>(s) * L / P);
}

// A block's register image (16 entries per lane) in the workspace, entry r
// of tile (I, J) of lane l at ((2 I + J) 4 + r) 64 + l: each access
// instruction covers 64 consecutive entries.
template <typename T>
__device__ __forceinline__ void store_image(T *P, int lane, const Blk<T> &b) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) P[((2 * I + J) * 4 + r) * 64 + lane] = b.t[I][J][r];
}

template <typename T>
__device__ __forceinline__ Blk<T> load_image(const T *P, int lane) {
  Blk<T> b;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.t[I][J][r] = P[((2 * I + J) * 4 + r) * 64 + lane];
  return b;
}

// The collect runs in two kernels.  seg32_fill takes each segment from its
// first block while the fill block is carried (until it is dropped, or to the
// separator if it never decays) and hands the current Schur block over;
// seg32_plain continues with the plain sweep to the separator.  The plain
// sweep holds no fill state, so it fits in half the registers and runs two
// wavefronts per SIMD, which hides much of its dependent latency; the fill
// phase is short (about 28 blocks per segment on the b = 32 workload).  The
// fill kernel is held to two wavefronts per SIMD (a few registers spill), so
// that 2048 segments run in one round rather than two.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void seg32_fill(
    int L, int P, const T *__restrict__ diag, const T *__restrict__ lower,
    T *__restrict__ st_sinv, T *__restrict__ st_f, T *__restrict__ r_F, T *__restrict__ r_U,
    T *__restrict__ st_hand, double *__restrict__ seg_ld, int32_t *__restrict__ seg_fail,
    int32_t *__restrict__ seg_fill_end) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int a = seg_begin(s, L, P), ts = seg_begin(s + 1, L, P) - 1;
  const bool left = s > 0;
  const T *D = diag + m * L * BB;
  const T *C = lower + m * (L - 1) * BB;
  T *sinv = st_sinv + m * L * PB;
  T *fst = st_f + m * L * BB;
  const io32::SymLanes<T> sl(g, j, lane);

  Blk<T> S, F = f32t::zero<T>(), U = f32t::zero<T>();
  {
    const io32::Nat<T> d0 = io32::load(D + a * BB, lane);
    io32::put(tA, lane, d0);
    if (left) io32::put(tB, lane, io32::load(C + (a - 1) * BB, lane));  // F_a = A_{a,t}
    f16::wave_sync();
    S = sl.get_sym(tA);
    if (left) F = io32::get_blk(tB, g, j);
  }
  // fill is carried while `fill`; fe = the first block whose fill is dropped
  bool fill = left;
  int fe = left ? ts : a;
  const T drop_below = left ? f32t::max_abs(F) * T(0x1p-100) : T(0);
  if (left && f32t::all_below(F, drop_below)) {  // a zero coupling block: no fill
    fill = false;
    fe = a;
    F = f32t::zero<T>();
  }
  f16::PivotLog pl;
  int32_t fail = 0;
  for (int i = a; i < ts && fill; ++i) {
    // C_i and D_{i+1} are consumed after the sweep of block i
    const io32::Nat<T> Cn = io32::load(C + i * BB, lane);
    const io32::Nat<T> Dn = io32::load(D + (i + 1) * BB, lane);
    if (f32t::gj_inverse(S, col, g, j, pl) && !fail) fail = i + 1;
    f16::wave_sync();
    io32::put_blk(tA, g, j, S);
    io32::put_blk(tB, g, j, F);
    f16::wave_sync();
    const io32::NatP<T> pk = sl.gather_packed(tA);
    const io32::Nat<T> fn = io32::get(tB, lane);
    f16::wave_sync();
    io32::store_packed(sinv + i * PB, lane, pk);
    io32::store_ws(fst + i * BB, lane, fn);
    io32::put(tA, lane, Cn);
    io32::put(tB, lane, Dn);
    f16::wave_sync();
    const Blk<T> Ct = io32::get_blk_t(tA, g, j);  // O32(C_i^T)
    const Blk<T> Dd = sl.get_sym(tB);
    const Blk<T> Y2 = f32t::mm(S, F, f32t::zero<T>());  // Sinv F_i
    U = f32t::mm_lower(F, Y2, U);                       // += F_i^T Sinv F_i
    F = f32t::neg(f32t::mm(Ct, Y2, f32t::zero<T>()));   // -C_i Sinv F_i
    if (f32t::all_below(F, drop_below)) {               // dropped from i + 1 on
      fill = false;
      fe = i + 1;
      F = f32t::zero<T>();
    }
    const Blk<T> Y1 = f32t::mm(S, Ct, f32t::zero<T>());  // Sinv C_i^T
    // D_{i+1} - C_i Sinv C_i^T; the (1,0) tile is not formed (the blocked
    // inverse reads only the upper off-diagonal tile)
    S = f32t::sub(Dd, f32t::mm_upper(Ct, Y1, f32t::zero<T>()));
  }
  // hand-over (block fe's Schur block), the segment's fill block and update of t
  const int64_t q = m * P + s;
  store_image(st_hand + q * BB, lane, S);
  if (left) {
    f16::wave_sync();
    io32::put_blk(tA, g, j, F);
    io32::put_sym(tB, g, j, U);
    f16::wave_sync();
    io32::store_ws(r_F + q * BB, lane, io32::get(tA, lane));
    io32::store_ws(r_U + q * BB, lane, io32::get(tB, lane));
  }
  if (lane == 0) {
    seg_ld[q] = pl.log();
    seg_fail[q] = fail;
    seg_fill_end[q] = fe;
  }
}

// The plain sweep from block fe to the separator, then the separator's
// partial Schur block.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void seg32_plain(
    int L, int P, const T *__restrict__ diag, const T *__restrict__ lower,
    T *__restrict__ st_sinv, const T *__restrict__ st_hand, T *__restrict__ r_S,
    double *__restrict__ seg_ld, int32_t *__restrict__ seg_fail,
    const int32_t *__restrict__ seg_fill_end) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T col[32];
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t q = m * P + s;
  const int a = seg_begin(s, L, P), ts = seg_begin(s + 1, L, P) - 1;
  const int fe = seg_fill_end[q];
  const T *D = diag + m * L * BB;
  const T *C = lower + m * (L - 1) * BB;
  T *sinv = st_sinv + m * L * PB;
  const io32::SymLanes<T> sl(g, j, lane);
  Blk<T> S = load_image(st_hand + q * BB, lane);
  f16::PivotLog pl;
  int32_t fail = 0;
  // C_i^T is staged one block ahead; C_{i+1} and D_{i+1} load during step i
  if (fe < ts) io32::put(tA, lane, io32::load(C + fe * BB, lane));
  f16::wave_sync();
  Blk<T> Ct = io32::get_blk_t(tA, g, j);  // O32(C_fe^T)
  for (int i = fe; i < ts; ++i) {
    const io32::Nat<T> Cn = io32::load(C + min(i + 1, ts - 1) * BB, lane);
    const io32::Nat<T> Dn = io32::load(D + (i + 1) * BB, lane);
    Blk<T> M = f32t::zero<T>();  // C_i Sinv C_i^T
    if (f32t::gj_congruence(S, Ct, M, col, g, j, pl) && !fail) fail = i + 1;
    f16::wave_sync();
    io32::put_blk_low(tA, g, j, S);
    f16::wave_sync();
    const io32::NatP<T> pk = sl.gather_packed(tA);
    f16::wave_sync();
    io32::store_packed(sinv + i * PB, lane, pk);
    io32::put(tA, lane, Cn);
    io32::put(tB, lane, Dn);
    f16::wave_sync();
    Ct = io32::get_blk_t(tA, g, j);  // O32(C_{i+1}^T)
    S = f32t::sub(sl.get_sym(tB), M);
  }
  // separator t_s: its partial Schur block (its (1,0) tile was formed only if
  // no block of the segment was eliminated)
  f16::wave_sync();
  if (ts > a)
    io32::put_sym_u(tA, g, j, S);
  else
    io32::put_blk(tA, g, j, S);
  f16::wave_sync();
  io32::store_ws(r_S + q * BB, lane, io32::get(tA, lane));
  if (lane == 0) {
    seg_ld[q] += pl.log();
    if (!seg_fail[q]) seg_fail[q] = fail;
  }
}

// Separator chain: diag_r[s] = S_{t_s} - U_{s+1}, lower_r[s] = F_{t_{s+1}}.
// One wavefront per (matrix, separator), natural-order vectors.
template <typename T>
__global__ __launch_bounds__(64) void seg32_reduce(int P, const T *__restrict__ r_S,
                                                   const T *__restrict__ r_F,
                                                   const T *__restrict__ r_U,
                                                   T *__restrict__ diag_r, T *__restrict__ lower_r) {
  using Tr = io32::Traits<T>;
  const int lane = threadIdx.x;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t q = m * P + s;
  io32::Nat<T> d = io32::load_ws(r_S + q * BB, lane);
  if (s + 1 < P) {
    const io32::Nat<T> u = io32::load_ws(r_U + (q + 1) * BB, lane);
#pragma unroll
    for (int c = 0; c < Tr::kChunks; ++c) d.c[c] = d.c[c] - u.c[c];
    io32::store_ws(lower_r + (m * (P - 1) + s) * BB, lane, io32::load_ws(r_F + (q + 1) * BB, lane));
  }
  io32::store_ws(diag_r + q * BB, lane, d);
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void seg32_distribute(
    int L, int P, const T *__restrict__ lower, const T *__restrict__ st_sinv,
    const T *__restrict__ st_f, const T *__restrict__ Gr_d, const T *__restrict__ Gr_l,
    const int32_t *__restrict__ seg_fill_end, T *__restrict__ G_diag, T *__restrict__ G_lower) {
  using Tr = io32::Traits<T>;
  __shared__ __align__(16) T tA[Tr::kTile];
  __shared__ __align__(16) T tB[Tr::kTile];
  __shared__ __align__(16) T tC[Tr::kTile];
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int64_t m = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int a = seg_begin(s, L, P), ts = seg_begin(s + 1, L, P) - 1;
  const bool left = s > 0;
  // blocks [a, fe) carry fill to t; past fe the steps are the plain sweep
  const int fe = seg_fill_end[m * P + s];
  const T *C = lower + m * (L - 1) * BB;
  const T *sinv = st_sinv + m * L * PB;
  const T *fst = st_f + m * L * BB;
  T *Gd = G_diag + m * L * BB;
  T *Gl = G_lower + m * (L - 1) * BB;
  const io32::SymLanes<T> sl(g, j, lane);

  // separator blocks from the separator chain
  Blk<T> Gnn, Gnt = f32t::zero<T>(), Gtn = f32t::zero<T>(), Gtt = f32t::zero<T>();
  {
    const io32::Nat<T> gs = io32::load_ws(Gr_d + (m * P + s) * BB, lane);
    io32::store(Gd + ts * BB, lane, gs);
    io32::put(tA, lane, gs);
    if (left) {
      const io32::Nat<T> gl = io32::load_ws(Gr_l + (m * (P - 1) + s - 1) * BB, lane);  // G_{ts,t}
      if (a == ts) io32::store(Gl + (a - 1) * BB, lane, gl);
      io32::put(tB, lane, gl);
      io32::put(tC, lane, io32::load_ws(Gr_d + (m * P + s - 1) * BB, lane));
    }
    f16::wave_sync();
    Gnn = io32::get_blk(tA, g, j);
    if (left && fe == ts) {  // fill carried to the end: G_{ts,t} couples the step
      Gnt = io32::get_blk(tB, g, j);    // O32(G_{i+1,t})
      Gtn = io32::get_blk_t(tB, g, j);  // O32(G_{t,i+1})
    }  // else the final fill block was dropped and G_{ts,t} = 0 exactly
    if (left) Gtt = io32::get_blk(tC, g, j);
  }
  if (ts == a) return;
  // Block i's packed Sinv, C_i and F_i are staged in LDS, then the next
  // block's are loaded into the freed registers.
  io32::NatP<T> Pc = io32::load_packed(sinv + (ts - 1) * PB, lane);
  io32::Nat<T> Cc = io32::load(C + (ts - 1) * BB, lane);
  io32::Nat<T> Fc;
  if (ts - 1 < fe) Fc = io32::load_ws(fst + (ts - 1) * BB, lane);
  for (int i = ts - 1; i >= a; --i) {
    const int in = max(i - 1, a);
    const bool two = i < fe;  // block i carries fill (implies left)
    f16::wave_sync();
    io32::put_packed(tA, lane, Pc);
    io32::put(tB, lane, Cc);
    if (two) io32::put(tC, lane, Fc);
    Pc = io32::load_packed(sinv + in * PB, lane);
    Cc = io32::load(C + in * BB, lane);
    if (in < fe) Fc = io32::load_ws(fst + in * BB, lane);
    f16::wave_sync();
    const Blk<T> Si = sl.get_packed(tA);
    const Blk<T> Ct = io32::get_blk_t(tB, g, j);            // O32(C_i^T)
    const Blk<T> X1 = f32t::mm(Ct, Si, f32t::zero<T>());     // C_i Sinv
    Blk<T> V1 = f32t::mm(Gnn, X1, f32t::zero<T>());
    Blk<T> Gii;
    if (two) {
      const Blk<T> Fb = io32::get_blk(tC, g, j);             // O32(F_i)
      const Blk<T> X2 = f32t::mm(Fb, Si, f32t::zero<T>());   // F_i^T Sinv
      V1 = f32t::mm(Gtn, X2, V1);                            // + G_{i+1,t} X2
      const Blk<T> V2 = f32t::mm(Gnt, X1, f32t::mm(Gtt, X2, f32t::zero<T>()));
      // Sinv + X1^T V1 + X2^T V2, lower tiles (the result is symmetric)
      Gii = f32t::mm_lower(X1, V1, f32t::mm_lower(X2, V2, Si));
      Gtn = f32t::neg(V2);                                   // O32(G_{t,i})
    } else {
      Gii = f32t::mm_lower(X1, V1, Si);                      // Sinv + X1^T V1
    }
    f16::wave_sync();
    io32::put_blk(tA, g, j, f32t::neg(V1));  // G_{i+1,i}
    io32::put_sym(tB, g, j, Gii);
    if (two) io32::put_blk_t(tC, g, j, Gtn);  // G_{i,t} = G_{t,i}^T
    f16::wave_sync();
    io32::store(Gl + i * BB, lane, io32::get(tA, lane));
    io32::store(Gd + i * BB, lane, io32::get(tB, lane));
    Gnn = io32::get_blk(tB, g, j);
    if (two) Gnt = io32::get_blk(tC, g, j);
    if (left && i == a) {  // G_{a,t}; zero when the segment carried no fill
      if (two)
        io32::store(Gl + (a - 1) * BB, lane, io32::get(tC, lane));
      else
        io32::store(Gl + (a - 1) * BB, lane, io32::Nat<T>{});
    }
  }
}

// logdet = interior pivots of all segments + separator chain; info: the
// first failing interior block of any segment, else the separator chain's.
__global__ void seg32_finish(int64_t B, int L, int P, const double *__restrict__ seg_ld,
                             const int32_t *__restrict__ seg_fail,
                             const double *__restrict__ logdet_r,
                             const int32_t *__restrict__ info_r, double *__restrict__ logdet,
                             int32_t *__restrict__ info) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (m >= B) return;
  double ld = 0.0;
  int32_t fail = 0;
  for (int s = 0; s < P; ++s) {
    ld += seg_ld[m * P + s];
    const int32_t f = seg_fail[m * P + s];
    if (f && (!fail || f < fail)) fail = f;
  }
  if (!fail && info_r[m]) {
    const int s = info_r[m] - 1;  // separator s is block t_s
    fail = static_cast<int32_t>(static_cast<int64_t>(s + 1) * L / P);
  }
  logdet[m] = fail ? __builtin_nan("") : ld + logdet_r[m];
  if (info) info[m] = fail;
}

struct SegLayout {
  size_t sinv, f, rS, rF, rU, hand, diag_r, lower_r, gr_d, gr_l, seg_ld, seg_fail, seg_fe, ld_r,
      info_r, ws_r, total;
};

SegLayout seg_layout(int dtype_bytes, int64_t B, int64_t L, int P) {
  SegLayout o{};
  const size_t w = dtype_bytes;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  o.sinv = take(B * L * PB * w);
  o.f = take(B * L * BB * w);
  o.rS = take(B * P * BB * w);
  o.rF = take(B * P * BB * w);
  o.rU = take(B * P * BB * w);
  o.hand = take(B * P * BB * w);
  o.diag_r = take(B * P * BB * w);
  o.lower_r = take(B * P * BB * w);
  o.gr_d = take(B * P * BB * w);
  o.gr_l = take(B * P * BB * w);
  o.seg_ld = take(B * P * sizeof(double));
  o.seg_fail = take(B * P * sizeof(int32_t));
  o.seg_fe = take(B * P * sizeof(int32_t));
  o.ld_r = take(B * sizeof(double));
  o.info_r = take(B * sizeof(int32_t));
  o.ws_r = take(chain32_workspace_bytes(dtype_bytes, B, P));
  o.total = off;
  return o;
}

}  // namespace

int chain32_segments(int64_t B, int64_t L) {
  if (B <= 0 || B >= 512 || L < 64) return 0;
  // two wavefronts per SIMD for the plain sweep (seg32_plain)
  const int64_t by_occupancy = std::max<int64_t>(2, 2048 / B);
  const int64_t by_length = L / 8;
  const int64_t by_balance = static_cast<int64_t>(std::sqrt(8.0 * static_cast<double>(L)));
  return static_cast<int>(std::max<int64_t>(2, std::min({by_occupancy, by_length, by_balance})));
}

size_t chain32_seg_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int P) {
  return seg_layout(dtype_bytes, B, L, P).total;
}

template <typename T>
hipError_t chain32_seg_launch(int64_t B, int64_t L, int P, const T *diag, const T *lower,
                              T *G_diag, T *G_lower, double *logdet, int32_t *info, void *ws,
                              hipStream_t s) {
  const SegLayout o = seg_layout(sizeof(T), B, L, P);
  char *base = static_cast<char *>(ws);
  T *sinv = reinterpret_cast<T *>(base + o.sinv);
  T *f = reinterpret_cast<T *>(base + o.f);
  T *rS = reinterpret_cast<T *>(base + o.rS);
  T *rF = reinterpret_cast<T *>(base + o.rF);
  T *rU = reinterpret_cast<T *>(base + o.rU);
  T *hand = reinterpret_cast<T *>(base + o.hand);
  T *diag_r = reinterpret_cast<T *>(base + o.diag_r);
  T *lower_r = reinterpret_cast<T *>(base + o.lower_r);
  T *gr_d = reinterpret_cast<T *>(base + o.gr_d);
  T *gr_l = reinterpret_cast<T *>(base + o.gr_l);
  double *seg_ld = reinterpret_cast<double *>(base + o.seg_ld);
  int32_t *seg_fail = reinterpret_cast<int32_t *>(base + o.seg_fail);
  int32_t *seg_fe = reinterpret_cast<int32_t *>(base + o.seg_fe);
  double *ld_r = reinterpret_cast<double *>(base + o.ld_r);
  int32_t *info_r = reinterpret_cast<int32_t *>(base + o.info_r);
  const unsigned grid = static_cast<unsigned>(B * P);
  hipLaunchKernelGGL(seg32_fill<T>, dim3(grid), dim3(64), 0, s, static_cast<int>(L), P, diag,
                     lower, sinv, f, rF, rU, hand, seg_ld, seg_fail, seg_fe);
  hipLaunchKernelGGL(seg32_plain<T>, dim3(grid), dim3(64), 0, s, static_cast<int>(L), P, diag,
                     lower, sinv, hand, rS, seg_ld, seg_fail, seg_fe);
  hipLaunchKernelGGL(seg32_reduce<T>, dim3(grid), dim3(64), 0, s, P, rS, rF, rU, diag_r, lower_r);
  hipError_t e = chain32_launch<T>(B, P, diag_r, lower_r, gr_d, gr_l, ld_r, info_r, base + o.ws_r, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seg32_distribute<T>, dim3(grid), dim3(64), 0, s, static_cast<int>(L), P,
                     lower, sinv, f, gr_d, gr_l, seg_fe, G_diag, G_lower);
  hipLaunchKernelGGL(seg32_finish, dim3(static_cast<unsigned>((B + 255) / 256)), dim3(256), 0, s,
                     B, static_cast<int>(L), P, seg_ld, seg_fail, ld_r, info_r, logdet, info);
  return hipGetLastError();
}

template hipError_t chain32_seg_launch<float>(int64_t, int64_t, int, const float *, const float *,
                                              float *, float *, double *, int32_t *, void *,
                                              hipStream_t);
template hipError_t chain32_seg_launch<double>(int64_t, int64_t, int, const double *,
                                               const double *, double *, double *, double *,
                                               int32_t *, void *, hipStream_t);

}  // namespace selinv
