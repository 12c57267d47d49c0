// internal.h -- declarations shared by the HIP sources of libselinv (not part
// of the public ABI; the public header is include/selinv.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "selinv.h"

namespace selinv {

// Workspace carve-up helper: every region starts 256-byte aligned.
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *p) : base(static_cast<char *>(p)) {}
  template <typename U>
  U *take(size_t count) {
    U *p = reinterpret_cast<U *>(base ? base + off : nullptr);
    off = align_up(off + count * sizeof(U));
    return p;
  }
};

// Host-side tree plan: depth level sets in breadth-first order.
//   pos    = breadth-first position (levels contiguous, each node's children
//            contiguous in the next level, in increasing node index)
//   node_at[pos]    original node index
//   parent_pos[pos] position of the parent (-1 for the root, pos 0)
//   child_beg/end[pos]  children positions [beg, end)
//   fail_rank[pos]  rank of the node in the order (depth descending, index
//                   ascending) used to name the first failing pivot
//   rank_node[r]    node index of rank r
//   parent_node[pos] node index of the parent (saves a dependent lookup)
struct TreePlanDev {
  int32_t *node_at = nullptr;
  int32_t *parent_pos = nullptr;
  int32_t *child_beg = nullptr;
  int32_t *child_end = nullptr;
  int32_t *fail_rank = nullptr;
  int32_t *rank_node = nullptr;
  int32_t *parent_node = nullptr;  // node index of the parent of position p (-1 at the root)
  // tiles of kTreeTile consecutive positions within one level, levels from
  // the root down: tile t covers positions [tile_lo[t], tile_hi[t])
  int32_t *tile_lo = nullptr;
  int32_t *tile_hi = nullptr;
};

constexpr int kTreeTile = 8;  // positions per tile (one wavefront of the b <= 8 kernels)

// Device tables of a junction plan (junction_plan.cpp builds them).  Chunks
// (pieces of supernodes, treated as fat nodes) are numbered level by level.
//   order[s]          label eliminated at step s
//   ch_first/s/n[J]   first position, columns and later rows of chunk J
//   ch_pbase[J]       first block of J's panel ((s + n) x s blocks)
//   ch_rbase[J]       first block of J's pivot inverse (s x s blocks, dense)
//   ch_gptr[J]        first entry of J's n x n G_{w,x} read codes in gtab
//   rows_ptr[J]       first flat row of J; row_chunk[row] its chunk
//   ch_cptr[J]        first flat column of J; col_chunk[column] its chunk
//   tiles_ptr[J]      first row tile of J (tiles of 64 / b rows); tile_chunk[tile]
//   tg_chunk/tg_rc/ain  per forward target: chunk, r * 64 + col, input block
//                     (label for a diagonal, edge * 2 + transposed, -1 fill)
//   fptr/fpair        Schur update pairs (panel block of W_{t,u}, of W_{v,u})
//   gtab              -(label + 1) for a diagonal G block, else output
//                     position * 2 + transpose
//   poutenc           output code of every panel block (as gtab, -1 unused)
//   row_node          label of every flat row (the solve sweeps)
//   occ_ptr/occ_row   per flat column, the flat rows of the same node
struct JunctionPlanDev {
  int32_t *order = nullptr;
  int32_t *ch_first = nullptr, *ch_s = nullptr, *ch_n = nullptr;
  int64_t *ch_pbase = nullptr, *ch_rbase = nullptr, *ch_gptr = nullptr, *rows_ptr = nullptr;
  int64_t *ch_cptr = nullptr, *tiles_ptr = nullptr;
  int32_t *row_chunk = nullptr, *col_chunk = nullptr, *tile_chunk = nullptr;
  int32_t *tg_chunk = nullptr, *tg_rc = nullptr, *ain = nullptr;
  int32_t *fptr = nullptr, *fpair = nullptr;
  int32_t *gtab = nullptr, *poutenc = nullptr;
  // Schur-sum work items: target, pair range, partial-sum slot (-1: the
  // target's only item); targets with several items per level; it_ptr[tg]
  int32_t *it_tg = nullptr, *it_lo = nullptr, *it_hi = nullptr, *it_slot = nullptr;
  int32_t *multi_tg = nullptr, *it_ptr = nullptr;
  int32_t *row_node = nullptr, *occ_ptr = nullptr, *occ_row = nullptr;
  int32_t *fdep_ptr = nullptr, *fdep = nullptr, *bdep_ptr = nullptr, *bdep = nullptr;
  int32_t *part_off = nullptr, *split_off = nullptr, *part_chunk = nullptr;
};

}  // namespace selinv

struct selinv_junction_plan {
  int64_t n = 0, m = 0, nnz = 0, nch = 0, npanel = 0, nrinv = 0;
  int32_t b = 0, smax = 0;
  int dtype_bytes = 0;
  int32_t levels = 0, node_levels = 0;
  std::vector<int64_t> level_off;  // chunk-id range of every level (levels + 1)
  std::vector<int64_t> ch_tptr;    // first forward target of every chunk (nch + 1)
  std::vector<int64_t> rows_ptr;   // first flat row of every chunk (nch + 1)
  std::vector<int64_t> ch_cptr;    // first flat column of every chunk (nch + 1)
  std::vector<int64_t> tiles_ptr;  // first row tile of every chunk (nch + 1)
  std::vector<int64_t> it_ptr;     // first Schur work item of every target (ntg + 1)
  std::vector<int64_t> multi_off;  // range of multi-item targets of every level (levels + 1)
  int64_t max_slots = 0;           // partial-sum slots of the busiest level
  int64_t nparts = 0, nsplit = 0;  // solve workgroups per (matrix, tile); parts of split chunks
  std::vector<int32_t> S_index;    // [2][nnz], host copy for the caller
  std::vector<int32_t> order;      // elimination order (labels)
  selinv::JunctionPlanDev dev;
  void *dev_block = nullptr;
};

struct selinv_tree_plan {
  int64_t n = 0;
  int32_t b = 0;
  int dtype_bytes = 0;
  int32_t levels = 0;
  int64_t *level_off = nullptr;   // host, levels+1 entries
  int32_t max_children = 0;
  int64_t tiles = 0;              // number of tiles (see TreePlanDev)
  selinv::TreePlanDev dev;
  void *dev_block = nullptr;      // one device allocation backing `dev`
};

// A tree plan's launch sequence captured for fixed buffers (abi.cpp).
struct selinv_tree_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int64_t nodes = 0;
};

namespace selinv {

// ---------------------------------------------------------------- chain
size_t chain_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
// b <= 8: eight chains per wavefront, one block row per lane (chain_small.hip)
size_t chain_small_workspace_bytes(int dtype_bytes, int64_t B, int64_t L);
template <typename T>
hipError_t chain_small_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                              T *G_diag, T *G_lower, double *logdet, int32_t *info, void *ws,
                              hipStream_t s);
// b = 16: one wavefront per chain on the matrix cores (chain_b16.hip)
size_t chain16_workspace_bytes(int dtype_bytes, int64_t B, int64_t L);
template <typename T>
hipError_t chain16_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                          T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s);
// b = 32: two-sided sweep, one workgroup of two wavefronts per chain (chain_b32.hip)
size_t chain32_workspace_bytes(int dtype_bytes, int64_t B, int64_t L);
template <typename T>
hipError_t chain32_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                          T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s);
// b = 32 with few chains: segment-parallel elimination (chain_b32_seg.hip);
// chain32_segments returns the number of segments per chain, 0 = not used
int chain32_segments(int64_t B, int64_t L);
size_t chain32_seg_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int P);
template <typename T>
hipError_t chain32_seg_launch(int64_t B, int64_t L, int P, const T *diag, const T *lower,
                              T *G_diag, T *G_lower, double *logdet, int32_t *info, void *ws,
                              hipStream_t s);
template <typename T>
hipError_t chain_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *G_diag,
                        T *G_lower, double *logdet, int32_t *info, void *ws, hipStream_t s);

// ----------------------------------------------------------------- star
size_t star_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
// b = 32: wavefront per 16 leaves on the matrix cores (star_b32.hip)
size_t star32_workspace_bytes(int dtype_bytes, int64_t B, int64_t K);
template <typename T>
hipError_t star32_launch(int64_t B, int64_t K, const T *center, const T *leaves, const T *coupling,
                         T *G_center, T *G_leaf, T *G_cross, double *logdet, int32_t *info,
                         void *ws, hipStream_t s);
template <typename T>
hipError_t star_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                       const T *coupling, T *G_center, T *G_leaf, T *G_cross, double *logdet,
                       int32_t *info, void *ws, hipStream_t s);

// ----------------------------------------------------------------- tree
size_t tree_workspace_bytes(const selinv_tree_plan *plan);
// b <= 8: one block row per lane, eight nodes per wavefront (tree_b8.hip)
size_t tree8_workspace_bytes(const selinv_tree_plan *plan);
template <typename T>
hipError_t tree8_launch(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag,
                        T *G_edge, double *logdet, int32_t *info, void *ws, hipStream_t s);
template <typename T>
hipError_t tree_launch(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag,
                       T *G_edge, double *logdet, int32_t *info, void *ws, hipStream_t s);

// ------------------------------------------- reverse mode (vjp_*.hip)
size_t chain_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
// b = 16: one wavefront per chain on the matrix cores (vjp_chain_b16.hip)
size_t chain16_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L);
template <typename T>
hipError_t chain16_vjp_launch(int64_t B, int64_t L, const T *diag, const T *lower, const T *gd,
                              const T *gl, const double *ld_bar, T *d_bar, T *l_bar,
                              int32_t *info, void *ws, hipStream_t s);
// few long chains: parallel over segments of each chain (vjp_chain_seg.hip);
// chain_vjp_segments returns the number of segments, 0 = not used
int chain_vjp_segments(int64_t B, int64_t L, int32_t b);
size_t chain_vjp_seg_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b, int P);
template <typename T>
hipError_t chain_vjp_seg_launch(int64_t B, int64_t L, int32_t b, int P, const T *diag,
                                const T *lower, const T *gd, const T *gl, const double *ld_bar,
                                T *d_bar, T *l_bar, int32_t *info, void *ws, hipStream_t s);
template <typename T>
hipError_t chain_vjp_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                            const T *gd, const T *gl, const double *ld_bar, T *d_bar, T *l_bar,
                            int32_t *info, void *ws, hipStream_t s);
size_t star_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
// b = 32: wavefront per 16 leaves on the matrix cores (vjp_star_b32.hip)
size_t star32_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K);
template <typename T>
hipError_t star32_vjp_launch(int64_t B, int64_t K, const T *center, const T *leaves,
                             const T *coupling, const T *gc, const T *gleaf, const T *gcross,
                             const double *ld_bar, T *center_bar, T *leaves_bar, T *coupling_bar,
                             int32_t *info, void *ws, hipStream_t s);
template <typename T>
hipError_t star_vjp_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                           const T *coupling, const T *gc, const T *gleaf, const T *gcross,
                           const double *ld_bar, T *center_bar, T *leaves_bar, T *coupling_bar,
                           int32_t *info, void *ws, hipStream_t s);
size_t tree_vjp_workspace_bytes(const selinv_tree_plan *plan);
// b <= 8: one block row per lane, eight nodes per wavefront (vjp_tree_b8.hip)
size_t tree8_vjp_workspace_bytes(const selinv_tree_plan *plan);
template <typename T>
hipError_t tree8_vjp_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                            const T *gd, const T *ge, const double *ld_bar, T *d_bar, T *e_bar,
                            int32_t *info, void *ws, hipStream_t s);
template <typename T>
hipError_t tree_vjp_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                           const T *gd, const T *ge, const double *ld_bar, T *d_bar, T *e_bar,
                           int32_t *info, void *ws, hipStream_t s);

// ------------------------- shared-factor siblings (shared_factor.hip)
// factor = packed lower triangles of S_v^{-1} (wg::packed_entries(b) per block)
template <typename T>
hipError_t chain16_factor_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *factor,
                                 double *logdet, int32_t *info, hipStream_t s);
size_t star32_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K);
template <typename T>
hipError_t star32_factor_launch(int64_t B, int64_t K, const T *center, const T *leaves,
                                const T *coupling, T *factor, double *logdet, int32_t *info,
                                void *ws, hipStream_t s);
size_t tree8_factor_workspace_bytes(const selinv_tree_plan *plan);
template <typename T>
hipError_t tree8_factor_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                               T *factor, double *logdet, int32_t *info, void *ws,
                               hipStream_t s);
size_t chain_factor_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
template <typename T>
hipError_t chain_factor_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                               T *factor, double *logdet, int32_t *info, hipStream_t s);
template <typename T>
hipError_t chain_apply_launch(int64_t B, int64_t L, int32_t b, int64_t k, bool sample,
                              const T *lower, const T *factor, const T *in, T *out,
                              hipStream_t s);
size_t star_factor_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
size_t star_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
template <typename T>
hipError_t star_factor_launch(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                              const T *coupling, T *factor, double *logdet, int32_t *info,
                              void *ws, hipStream_t s);
size_t star_apply_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b, int64_t k);
template <typename T>
hipError_t star_apply_launch(int64_t B, int64_t K, int32_t b, int64_t k, bool sample,
                             const T *coupling, const T *factor, const T *in_center,
                             const T *in_leaves, T *x_center, T *x_leaves, void *ws,
                             hipStream_t s);
size_t tree_factor_bytes(const selinv_tree_plan *plan);
size_t tree_factor_workspace_bytes(const selinv_tree_plan *plan);
template <typename T>
hipError_t tree_factor_launch(const selinv_tree_plan *plan, const T *diag, const T *edge,
                              T *factor, double *logdet, int32_t *info, void *ws, hipStream_t s);
size_t tree_apply_workspace_bytes(const selinv_tree_plan *plan, int64_t k);
// b = 16 chain solve, one wavefront per chain and 16 right-hand sides
// (chain_solve_b16.hip)
template <typename T>
hipError_t chain16_solve_launch(int64_t B, int64_t L, int64_t k, const T *lower, const T *factor,
                                const T *y, T *x, hipStream_t s);
// b = 16 chain sampling for k <= 4, one wavefront per chain
template <typename T>
hipError_t chain16_sample_launch(int64_t B, int64_t L, int64_t k, const T *lower,
                                 const T *factor, const T *z, T *x, hipStream_t s);
// b = 32 star solve / sampling for k <= 4 (star_solve_b32.hip)
template <typename T>
hipError_t star32_apply_launch(int64_t B, int64_t K, int64_t k, bool sample, const T *coupling,
                               const T *factor, const T *in_center, const T *in_leaves,
                               T *x_center, T *x_leaves, void *ws, hipStream_t s);
// b <= 8 solve and sampling on the single-launch schedule (tree_b8.hip);
// both take the workspace of tree8_solve_workspace_bytes
size_t tree8_solve_workspace_bytes(const selinv_tree_plan *plan, int64_t k);
template <typename T>
hipError_t tree8_solve_launch(const selinv_tree_plan *plan, int64_t k, const T *edge,
                              const T *factor, const T *y, T *x, void *ws, hipStream_t s);
template <typename T>
hipError_t tree8_sample_launch(const selinv_tree_plan *plan, int64_t k, const T *edge,
                               const T *factor, const T *z, T *x, void *ws, hipStream_t s);
template <typename T>
hipError_t tree_apply_launch(const selinv_tree_plan *plan, int64_t k, bool sample, const T *edge,
                             const T *factor, const T *in, T *out, void *ws, hipStream_t s);

// --------------------------------- general sparse SPD (junction.hip)
size_t junction_workspace_bytes(const selinv_junction_plan *plan, int64_t B);
template <typename T>
hipError_t junction_launch(const selinv_junction_plan *plan, int64_t B, const T *diag,
                           const T *edge_val, T *G_diag, T *G_lower, double *logdet,
                           int32_t *info, void *ws, hipStream_t s);
// the shared-factor siblings: the factorisation into a caller-owned factor
// (junction.hip), then the solve / sample sweeps (junction_solve.hip)
size_t junction_factor_workspace_bytes(const selinv_junction_plan *plan, int64_t B);
size_t junction_factor_bytes(const selinv_junction_plan *plan, int64_t B);
template <typename T>
hipError_t junction_factor_launch(const selinv_junction_plan *plan, int64_t B, const T *diag,
                                  const T *edge_val, T *factor, double *logdet, int32_t *info,
                                  void *ws, hipStream_t s);
size_t junction_solve_workspace_bytes(const selinv_junction_plan *plan, int64_t B, int64_t k);
template <typename T>
hipError_t junction_apply_launch(const selinv_junction_plan *plan, int64_t B, const T *factor,
                                 int64_t k, bool sample, const T *in, T *out, void *ws,
                                 hipStream_t s);

// ------------------------------------ non-symmetric ladder (nonsym.hip)
size_t bidiag_workspace_bytes(int64_t B);
// b = 16: one wavefront per matrix on the matrix cores (bidiag_b16.hip)
template <typename T>
hipError_t bidiag16_launch(int64_t B, int64_t L, const T *diag, const T *lower, T *G_diag,
                           T *G_lower, int32_t *info, hipStream_t s);
template <typename T>
hipError_t bidiag_launch(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower,
                         T *G_diag, T *G_lower, int32_t *info, void *ws, hipStream_t s);
size_t nonsym_tree_workspace_bytes(const selinv_tree_plan *plan);
// b <= 8: one block row per lane, eight nodes per wavefront (nonsym_b8.hip)
size_t nstree8_workspace_bytes(const selinv_tree_plan *plan);
template <typename T>
hipError_t nstree8_launch(const selinv_tree_plan *plan, const T *diag, const T *up, const T *down,
                          T *G_diag, T *G_up, T *G_down, int32_t *info, void *ws, hipStream_t s);
template <typename T>
hipError_t nonsym_tree_launch(const selinv_tree_plan *plan, const T *diag, const T *up,
                              const T *down, T *G_diag, T *G_up, T *G_down, int32_t *info,
                              void *ws, hipStream_t s);

}  // namespace selinv
