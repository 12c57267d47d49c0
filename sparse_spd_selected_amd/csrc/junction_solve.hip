// junction_solve.hip -- solve and Gaussian sampling on the filled pattern of
// a junction plan, from the factor its factorisation leaves behind
// (gabp-sparse-inv page, junction-tree section: junction_solve with one or
// several right-hand sides, and Gaussian sampling, both reusing the
// factorisation of the selected inverse).
//
// The factor is the Cholesky form the factorisation kernels compute,
// A = L~ L~^T with, per chunk J (s consecutive supernode columns), the dense
// pivot factor R_J (kept as R_J^-1) and the later rows W_{N,J} = C_{N,J} R_J^-T:
//   forward, chunk levels upward (children first):
//       z_J = R_J^-1 (y_J - sum_K W_{J,K} z_K)
//   over the earlier chunks K whose later rows hold nodes of J;
//   backward, chunk levels downward (root first):
//       x_J = R_J^-T (v_J - W_{N,J}^T x_N)
// with v = z for a solve (x = A^-1 y) and v = the caller's z for a sample
// (x = L~^-T z, so Cov x = L~^-T L~^-1 = A^-1 for z ~ N(0, I)).  L~'s
// diagonal blocks are the Cholesky factors R_v of the node pivots D_v (the
// Cholesky factor of A in the elimination order is unique), so the sample is
// x = L^-T D^-1/2 z with D^-1/2_v = R_v^-T, as for chains, stars and trees.
//
// Forward as producer and consumer: once chunk K has z_K, the same
// workgroup multiplies it into every later row a of K's panel and stores
// u_a = W_{a,K} z_K (b x k) in a row buffer (one slot per later row, so no
// two workgroups write one slot).  A later chunk J then only adds, for each
// of its nodes, the b-vectors of the rows that hold that node (occ_ptr /
// occ_row, in a fixed order); the matrix-vector work runs where the rows are
// produced, spread over all rows of a level instead of serialised on the
// few separator chunks whose nodes occur in many panels.
//
// One workgroup per (chunk, matrix, tile of right-hand sides).  Thread e of
// the first s b kt threads owns entry (I, kc) of the chunk's s b x kt tile;
// the workgroup's other threads form further groups that split the sum over
// occurrences (forward) or later rows (backward), and the groups' partial sums
// are added in a fixed order, so results are deterministic.  Vectors are
// [B][n][b][k] by label, k fastest: consecutive threads read consecutive
// right-hand sides.  The solve keeps z in the output (the backward pass of
// chunk J reads z_J before any thread writes x_J, and no chunk that runs
// before J has written x_J reads J's nodes).
//
// Schedules.  The solve runs each sweep as one launch over all chunks
// (kDF): workgroups in chunk-id order for the forward sweep (children have
// lower chunk levels, hence lower ids) and in reverse for the backward sweep.
// A workgroup first issues every load that needs no other chunk (its plan
// entries, y or z, R_J^-1), then waits for the flags of the chunks it reads
// (fdep: those whose later rows hold its nodes; bdep: those holding the nodes
// of its later rows), computes, stores and sets its own flag once its stores
// have completed.  Rows and x that cross workgroups are written and read with
// device-coherent accesses, and every wait is bounded, as in dataflow.h; a
// call whose wait gives up writes NaN into every x entry computed after that.
// With four or more right-hand sides per tile, a chunk with long sums (many
// occurrences or later rows; the plan fixes its number of parts) is split
// over several workgroups: each part adds every P-th term into a slot of
// its own, and the part that arrives last at the chunk's counter adds the
// slots in part order and finishes the chunk (results stay deterministic;
// no part waits for another).  Its workspace is the row buffer
// [B][rows][b][k], then the flags and counters, the give-up word and the
// parts' slots.  The sample has no workspace: it runs the backward
// sweep as one launch per chunk level (levels downward), which orders the
// chunks by kernel boundaries instead.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "dataflow.h"
#include "internal.h"

namespace selinv {
namespace {

constexpr int kST = 256;   // threads per workgroup
constexpr int kIdx = 1024;  // row indices per LDS staging batch
constexpr int kSplitMinCols = 4;  // right-hand sides per tile from which chunks are split

struct SDims {
  int64_t n, npanel, nrinv, nrows, k;
  int kt, b;
  int64_t nch, B, nkt;  // chunks, matrices, tiles of right-hand sides
  int64_t nparts;       // parts of all chunks (split chunks count several)
  bool split;           // single-launch sweeps: one workgroup per part, else per chunk
};

// Reads of a region that other workgroups of the same launch write (kDF:
// at the point of coherence, several in flight), or plain loads.
template <bool kDF, typename T>
struct Reader {
  const T *p;
  __device__ __forceinline__ Reader(const T *base, int64_t) : p(base) {}
  __device__ __forceinline__ T operator[](int64_t i) const { return p[i]; }
};

template <typename T>
struct Reader<true, T> : df::CoherentReader<T> {
  __device__ __forceinline__ Reader(const T *base, int64_t n) : df::CoherentReader<T>(base, n) {}
};

template <bool kDF, typename T>
__device__ __forceinline__ void st(T *p, T v) {
  if constexpr (kDF)
    df::store_coherent(p, v);
  else
    *p = v;
}

// Waits (bounded) until flags[dep[e] * per + off] >= 1 for every e in
// [d0, d1), the workgroup's threads sharing the list; then no load of the
// workgroup moves above the waits.
__device__ inline void wait_deps(const int32_t *flags, const int32_t *dep, int32_t d0, int32_t d1,
                                 int64_t per, int64_t off, int32_t *timeout, uint64_t ticks) {
  const uint64_t deadline = df::deadline_after(ticks);
  for (int32_t e = d0 + static_cast<int32_t>(threadIdx.x); e < d1; e += kST) {
    const int32_t *f = flags + int64_t(dep[e]) * per + off;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 1) {
      if (df::timed_out(timeout)) break;
      if (static_cast<uint64_t>(wall_clock64()) >= deadline) {
        __hip_atomic_store(timeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  df::acquire();
}

// The workgroup's (chunk id, part, parts, matrix, tile of right-hand sides):
// one launch per level (blockIdx = (chunk in level, matrix, tile), one part),
// or one launch over all parts of all chunks, part-major, ascending (forward)
// or descending (backward); the parts of a chunk are consecutive.
template <bool kDF>
__device__ inline void workgroup_item(const JunctionPlanDev &P, const SDims &d, int64_t cbase,
                                      bool descending, int64_t &id, int &part, int &nparts,
                                      int64_t &mat, int64_t &kz) {
  if constexpr (kDF) {
    const int64_t per = d.B * d.nkt, w = blockIdx.x, c = w / per, r = w - c * per;
    if (d.split) {
      const int64_t gp = descending ? d.nparts - 1 - c : c;
      id = P.part_chunk[gp];
      const int32_t p0 = P.part_off[id];
      part = static_cast<int>(gp - p0);
      nparts = P.part_off[id + 1] - p0;
    } else {
      id = descending ? d.nch - 1 - c : c;
      part = 0;
      nparts = 1;
    }
    mat = r / d.nkt;
    kz = r - mat * d.nkt;
  } else {
    id = cbase + blockIdx.x;
    part = 0;
    nparts = 1;
    mat = blockIdx.y;
    kz = blockIdx.z;
  }
}

// A part of a split chunk hands over its partial sums (thread t < ne holds
// entry t): it stores them in its slot at the point of coherence, and the
// part that arrives last at the chunk's counter (when every other part's
// slot is complete) goes on.  Returns true in that part.
template <typename T>
__device__ inline bool arrive_last(T *slot, T v, bool has, int32_t *cnt, int nparts,
                                   int32_t *lds_word) {
  if (has) df::store_coherent(slot + threadIdx.x, v);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    *lds_word = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nparts - 1;
  __syncthreads();
  const bool last = *lds_word != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return last;
}

// dst[0 .. n) = src[0 .. n) by the workgroup, n >= 1: each thread issues up to
// kR loads (at clamped, in-range addresses) before it waits for any of them,
// so a long copy costs a few memory round trips instead of one per element.
template <typename T>
__device__ inline void stage(T *dst, const T *src, int n) {
  constexpr int kR = 8;
  for (int base = threadIdx.x; base < n; base += kR * kST) {
    T v[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) v[r] = src[min(base + r * kST, n - 1)];
#pragma unroll
    for (int r = 0; r < kR; ++r)
      if (base + r * kST < n) dst[base + r * kST] = v[r];
  }
}

// The chunk's tile: its plan entries, the thread's entry and group.
struct Tile {
  int64_t id, mat, koff, rbase, pbase, rows, cptr;
  int s, sb, f, nr, kt, ne, G, g, I, kc, c, i;
};

// All plan entries of the chunk are read here, together, before any of them
// is waited for.
template <int BC>
__device__ inline Tile tile_setup(const JunctionPlanDev &P, const SDims &d, int64_t id,
                                  int64_t mat, int64_t kz) {
  Tile q;
  const int b = BC ? BC : d.b, t = threadIdx.x;
  q.id = id;
  q.mat = mat;
  const int64_t k0 = kz * d.kt;
  q.kt = d.k - k0 < d.kt ? static_cast<int>(d.k - k0) : d.kt;
  q.s = P.ch_s[q.id];
  q.f = P.ch_first[q.id];
  q.nr = P.ch_n[q.id];
  q.rbase = P.ch_rbase[q.id];
  q.pbase = P.ch_pbase[q.id];
  q.rows = P.rows_ptr[q.id];
  q.cptr = P.ch_cptr[q.id];
  q.sb = q.s * b;
  q.ne = q.sb * q.kt;
  q.G = kST / q.ne;
  q.g = t / q.ne;
  const int e = t - q.g * q.ne;
  q.I = e / q.kt;
  q.kc = e - q.I * q.kt;
  q.c = q.I / b;
  q.i = q.I - q.c * b;
  q.koff = k0 + q.kc;
  return q;
}

// Forward: z_J = R_J^-1 (y_J - sum of the row vectors of J's nodes), then
// u_a = W_{a,J} z_J for every later row a of J into the row buffer U
template <typename T, int BC, bool kDF>
__global__ void __launch_bounds__(kST) js_forward(JunctionPlanDev P, SDims d, int64_t cbase,
                                                  const T *__restrict__ W,
                                                  const T *__restrict__ RJ,
                                                  const T *__restrict__ y, T *z, T *U,
                                                  int32_t *flags, int32_t *cnt, T *slots,
                                                  int32_t *timeout, uint64_t ticks) {
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  int64_t id, mat, kz;
  int part, nparts;
  workgroup_item<kDF>(P, d, cbase, false, id, part, nparts, mat, kz);
  const Tile q = tile_setup<BC>(P, d, id, mat, kz);
  T *part_s = Ri + q.sb * q.sb, *rs = part_s + kST;
  int32_t *idx = reinterpret_cast<int32_t *>(rs + kST);
  const int64_t k = d.k, k0 = q.koff - q.kc;
  const T *Um = U + q.mat * d.nrows * b * k;
  // the occurrences of the chunk's nodes are one contiguous range of occ_row
  // (flat columns of a chunk are consecutive)
  const int32_t ob = P.occ_ptr[q.cptr], oe = P.occ_ptr[q.cptr + q.s];
  const int32_t o0 = P.occ_ptr[q.cptr + q.c], o1 = P.occ_ptr[q.cptr + q.c + 1];
  const int64_t node = P.order[q.f + q.c];
  const int64_t at = ((q.mat * d.n + node) * b + q.i) * k + q.koff;
  const T yv = t < q.ne ? y[at] : T(0);
  stage(Ri, RJ + (q.mat * d.nrinv + q.rbase) * bb, q.sb * q.sb);
  const int64_t per_ch = d.B * d.nkt, self = q.mat * d.nkt + kz;
  if constexpr (kDF)  // the chunks whose later rows hold J's nodes
    wait_deps(flags, P.fdep, P.fdep_ptr[q.id], P.fdep_ptr[q.id + 1], per_ch, self, timeout,
              ticks);
  {
    // the occurrences' row indices are staged in LDS in batches, so that the
    // row-vector loads do not wait on index loads
    const Reader<kDF, T> Ur(Um, d.nrows * b * k);  // this matrix's row buffer
    const int64_t ui = int64_t(q.i) * k + q.koff;
    T acc = T(0);
    for (int32_t b0 = ob; b0 < oe; b0 += kIdx) {
      const int32_t b1 = oe - b0 < kIdx ? oe : b0 + kIdx;
      __syncthreads();  // the previous batch has been read
      stage(idx, P.occ_row + b0, b1 - b0);
      __syncthreads();
      if (q.g < q.G) {  // this part's groups take every stride-th occurrence
        const int32_t lo = o0 > b0 ? o0 : b0, hi = o1 < b1 ? o1 : b1;
        const int32_t stride = nparts * q.G;
        int32_t o = o0 + part * q.G + q.g;
        if (o < lo) o += (lo - o + stride - 1) / stride * stride;
#pragma unroll 8
        for (; o < hi; o += stride) acc += Ur[int64_t(idx[o - b0]) * b * k + ui];
      }
    }
    if (q.g < q.G) part_s[q.g * q.ne + (t - q.g * q.ne)] = acc;
  }
  __syncthreads();
  T v = T(0);
  if (t < q.ne)
    for (int gg = 0; gg < q.G; ++gg) v += part_s[gg * q.ne + t];
  if constexpr (kDF) {
    if (nparts > 1) {  // the last part to arrive adds the parts' sums in order
      const int64_t sl = P.split_off[q.id];
      T *my = slots + ((sl + part) * per_ch + self) * kST;
      if (!arrive_last(my, v, t < q.ne, cnt + q.id * per_ch + self, nparts, idx)) return;
      const df::CoherentReader<T> sr(slots + sl * per_ch * kST,
                                     int64_t(nparts) * per_ch * kST);
      v = T(0);
      if (t < q.ne)
        for (int pp = 0; pp < nparts; ++pp) v += sr[(pp * per_ch + self) * kST + t];
    }
  }
  if (t < q.ne) rs[t] = yv - v;
  __syncthreads();
  T zv = T(0);
  if (t < q.ne) {
    for (int K = 0; K <= q.I; ++K) zv += Ri[q.I * q.sb + K] * rs[K * q.kt + q.kc];
    z[at] = zv;
  }
  __syncthreads();
  if (t < q.ne) rs[t] = zv;  // z_J, s b x kt
  __syncthreads();
  // the later rows' vectors: entry (a, i, kc) = sum_I W_{a,J}[i][I] z_J[I][kc]
  const int nr = q.nr, per = b * q.kt;
  const T *Wp = W + (q.mat * d.npanel + q.pbase + int64_t(q.s) * q.s) * bb;
  T *Ur = U + (q.mat * d.nrows + q.rows) * b * k + k0;
  for (int e = t; e < nr * per; e += kST) {
    const int a = e / per, rem = e - a * per, i = rem / q.kt, kc = rem - i * q.kt;
    const T *Wa = Wp + int64_t(a) * q.s * bb + i * b;
    T acc = T(0);
    for (int c = 0; c < q.s; ++c) {
      const T *Wb = Wa + c * bb, *zc = rs + c * b * q.kt + kc;
#pragma unroll
      for (int l = 0; l < b; ++l) acc += Wb[l] * zc[l * q.kt];
    }
    st<kDF>(Ur + (int64_t(a) * b + i) * k + kc, acc);
  }
  if constexpr (kDF) df::publish(flags, q.id * per_ch + self, t == 0, 1);
}

// Backward: x_J = R_J^-T (v_J - W_{N,J}^T x_N).  v may be x itself (the
// solve): the tile reads v_J before it writes x_J, and the chunks that read
// J's nodes (its descendants) run after it.
template <typename T, int BC, bool kDF>
__global__ void __launch_bounds__(kST) js_backward(JunctionPlanDev P, SDims d, int64_t cbase,
                                                   const T *__restrict__ W,
                                                   const T *__restrict__ RJ, const T *v,
                                                   T *x, int32_t *flags, int32_t *cnt,
                                                   T *slots, int32_t *timeout, uint64_t ticks) {
  extern __shared__ char smem_raw[];
  T *Ri = reinterpret_cast<T *>(smem_raw);
  const int b = BC ? BC : d.b, bb = b * b, t = threadIdx.x;
  int64_t id, mat, kz;
  int part, nparts;
  workgroup_item<kDF>(P, d, cbase, true, id, part, nparts, mat, kz);
  const Tile q = tile_setup<BC>(P, d, id, mat, kz);
  T *part_s = Ri + q.sb * q.sb, *rs = part_s + kST;
  int32_t *idx = reinterpret_cast<int32_t *>(rs + kST);
  const int64_t k = d.k;
  const int l = q.i;  // entry I = c b + l of the chunk's columns
  const int64_t node = P.order[q.f + q.c];
  const int64_t at = ((q.mat * d.n + node) * b + l) * k + q.koff;
  const T vv = t < q.ne ? v[at] : T(0);  // read before any write of x (v may be x)
  stage(Ri, RJ + (q.mat * d.nrinv + q.rbase) * bb, q.sb * q.sb);
  const int64_t per_ch = d.B * d.nkt, self = q.mat * d.nkt + kz;
  if constexpr (kDF)  // the chunks that hold the nodes of J's later rows
    wait_deps(flags, P.bdep, P.bdep_ptr[q.id], P.bdep_ptr[q.id + 1], per_ch, self, timeout,
              ticks);
  {
    const int nr = q.nr;
    const int64_t rb = q.rows;
    // column l of block (a, c) of the panel: stride b down its rows
    const T *Wc = W + (q.mat * d.npanel + q.pbase + int64_t(q.s) * q.s + q.c) * bb + l;
    const Reader<kDF, T> xr(x + q.mat * d.n * b * k, d.n * b * k);  // this matrix's x
    T acc = T(0);
    for (int a0 = 0; a0 < nr; a0 += kIdx) {  // the later rows' labels, staged in LDS
      const int a1 = nr - a0 < kIdx ? nr : a0 + kIdx;
      __syncthreads();  // the previous batch has been read
      stage(idx, P.row_node + rb + a0, a1 - a0);
      __syncthreads();
      if (q.g < q.G) {  // this part's groups take every stride-th row
        const int stride = nparts * q.G;
        int a = part * q.G + q.g;
        if (a < a0) a += (a0 - a + stride - 1) / stride * stride;
#pragma unroll 4
        for (; a < a1; a += stride) {
          const T *Wb = Wc + int64_t(a) * q.s * bb;
          const int64_t xw = int64_t(idx[a - a0]) * b * k + q.koff;
#pragma unroll
          for (int i = 0; i < b; ++i) acc += Wb[i * b] * xr[xw + i * k];
        }
      }
    }
    if (q.g < q.G) part_s[q.g * q.ne + (t - q.g * q.ne)] = acc;
  }
  __syncthreads();
  T sum = T(0);
  if (t < q.ne)
    for (int gg = 0; gg < q.G; ++gg) sum += part_s[gg * q.ne + t];
  if constexpr (kDF) {
    if (nparts > 1) {  // the last part to arrive adds the parts' sums in order
      const int64_t sl = P.split_off[q.id];
      T *my = slots + ((sl + part) * per_ch + self) * kST;
      if (!arrive_last(my, sum, t < q.ne, cnt + q.id * per_ch + self, nparts, idx)) return;
      const df::CoherentReader<T> sr(slots + sl * per_ch * kST,
                                     int64_t(nparts) * per_ch * kST);
      sum = T(0);
      if (t < q.ne)
        for (int pp = 0; pp < nparts; ++pp) sum += sr[(pp * per_ch + self) * kST + t];
    }
  }
  if (t < q.ne) rs[t] = vv - sum;
  __syncthreads();
  if (t < q.ne) {
    T s = T(0);
    for (int K = q.I; K < q.sb; ++K) s += Ri[K * q.sb + q.I] * rs[K * q.kt + q.kc];
    if constexpr (kDF) {
      if (df::timed_out(timeout)) s = static_cast<T>(__builtin_nan(""));
    }
    st<kDF>(x + at, s);
  }
  if constexpr (kDF) df::publish(flags, q.id * per_ch + self, t == 0, 1);
}

// Right-hand sides per tile and tiles (k >= 1)
inline void rhs_tiles(const selinv_junction_plan *plan, int64_t k, int &kt, int64_t &nkt) {
  const int64_t ktl = kST / (plan->smax * plan->b);
  kt = static_cast<int>(k < ktl ? k : ktl);
  nkt = (k + kt - 1) / kt;
}

// Workspace of a solve: the row buffer; the flags and the arrival counters
// of both sweeps ([4][nch][B][nkt]: forward flags, backward flags, forward
// counters, backward counters) and the give-up word; the partial-sum slots of
// the split chunks' parts ([nsplit][B][nkt][kST] values).
struct SolveWs {
  size_t rows, words, slots, total;
  int64_t per;  // B nkt
};

inline SolveWs solve_ws(const selinv_junction_plan *plan, int64_t B, int64_t k) {
  if (B <= 0 || k <= 0) return SolveWs{0, 0, 0, 0, 0};
  int kt;
  int64_t nkt;
  rhs_tiles(plan, k, kt, nkt);
  SolveWs o;
  o.per = B * nkt;
  o.rows = align_up(size_t(B) * plan->rows_ptr[plan->nch] * plan->b * size_t(k) *
                    plan->dtype_bytes);
  o.words = 4 * size_t(plan->nch) * size_t(o.per);
  o.slots = size_t(plan->nsplit) * size_t(o.per) * kST;
  o.total = o.rows + align_up((o.words + 1) * sizeof(int32_t)) +
            align_up(o.slots * plan->dtype_bytes);
  return o;
}

template <typename T, int BC>
hipError_t apply_run(const selinv_junction_plan *plan, int64_t B, const T *factor, int64_t k,
                     bool sample, const T *in, T *out, void *ws, hipStream_t s) {
  const int b = plan->b, sbm = plan->smax * b;
  if (sbm > kST) return hipErrorInvalidValue;
  int kt;
  int64_t nkt;
  rhs_tiles(plan, k, kt, nkt);
  if (nkt > 65535) return hipErrorInvalidValue;
  // Split chunks pay a handshake between their parts, which only the longer
  // sums of several right-hand sides per tile repay.
  const bool split = kt >= kSplitMinCols;
  const SDims d{plan->n,  plan->npanel, plan->nrinv, plan->rows_ptr[plan->nch], k, kt, b,
                plan->nch, B,           nkt,         plan->nparts, split};
  const T *W = factor, *RJ = factor + B * plan->npanel * int64_t(b) * b;
  const size_t lds = sizeof(T) * (size_t(sbm) * sbm + 2 * kST) + sizeof(int32_t) * kIdx;
  const auto &lo = plan->level_off;
  const unsigned By = static_cast<unsigned>(B), Z = static_cast<unsigned>(nkt);
  if (sample) {  // no workspace: one launch per level, levels downward
    for (int32_t l = plan->levels - 1; l >= 0; --l)
      js_backward<T, BC, false><<<dim3(static_cast<unsigned>(lo[l + 1] - lo[l]), By, Z),
                                  dim3(kST), lds, s>>>(plan->dev, d, lo[l], W, RJ, in, out,
                                                       nullptr, nullptr, nullptr, nullptr, 0);
    return hipGetLastError();
  }
  const SolveWs o = solve_ws(plan, B, k);
  const int64_t grid = (split ? plan->nparts : plan->nch) * o.per;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  // a matrix's row buffer and vector, and the slots, are read through 32-bit
  // buffer offsets
  const int64_t span = std::max(d.nrows, d.n) * b * k * int64_t(sizeof(T));
  if (span >= (int64_t(1) << 31) || o.slots * sizeof(T) >= (size_t(1) << 31))
    return hipErrorInvalidValue;
  char *base = static_cast<char *>(ws);
  T *U = reinterpret_cast<T *>(base);
  int32_t *words = reinterpret_cast<int32_t *>(base + o.rows);
  const size_t nw = size_t(plan->nch) * size_t(o.per);
  int32_t *fflags = words, *bflags = words + nw, *fcnt = words + 2 * nw, *bcnt = words + 3 * nw;
  int32_t *timeout = words + o.words;
  T *slots = reinterpret_cast<T *>(base + o.rows + align_up((o.words + 1) * sizeof(int32_t)));
  hipError_t e = df::launch_init(static_cast<int64_t>(o.words), words, nullptr, timeout, s);
  if (e != hipSuccess) return e;
  const uint64_t wt = wait_limit_ticks();
  const unsigned G = static_cast<unsigned>(grid);
  js_forward<T, BC, true><<<dim3(G), dim3(kST), lds, s>>>(plan->dev, d, 0, W, RJ, in, out, U,
                                                          fflags, fcnt, slots, timeout, wt);
  js_backward<T, BC, true><<<dim3(G), dim3(kST), lds, s>>>(plan->dev, d, 0, W, RJ, out, out,
                                                           bflags, bcnt, slots, timeout, wt);
  return hipGetLastError();
}

}  // namespace

size_t junction_solve_workspace_bytes(const selinv_junction_plan *plan, int64_t B, int64_t k) {
  return solve_ws(plan, B, k).total;
}

template <typename T>
hipError_t junction_apply_launch(const selinv_junction_plan *plan, int64_t B, const T *factor,
                                 int64_t k, bool sample, const T *in, T *out, void *ws,
                                 hipStream_t s) {
  switch (plan->b) {
    case 4: return apply_run<T, 4>(plan, B, factor, k, sample, in, out, ws, s);
    case 8: return apply_run<T, 8>(plan, B, factor, k, sample, in, out, ws, s);
    case 16: return apply_run<T, 16>(plan, B, factor, k, sample, in, out, ws, s);
    default: return apply_run<T, 0>(plan, B, factor, k, sample, in, out, ws, s);
  }
}

template hipError_t junction_apply_launch<double>(const selinv_junction_plan *, int64_t,
                                                  const double *, int64_t, bool, const double *,
                                                  double *, void *, hipStream_t);
template hipError_t junction_apply_launch<float>(const selinv_junction_plan *, int64_t,
                                                 const float *, int64_t, bool, const float *,
                                                 float *, void *, hipStream_t);

}  // namespace selinv
