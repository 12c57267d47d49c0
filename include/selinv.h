/*
 * selinv.h -- C ABI of the MI355X (gfx950) batched selected inverse of
 * block-structured SPD matrices.
 *
 * What every entry point computes (gabp-sparse-inv 0.3.2 project page,
 * opening paragraphs and section "Implemented and tested kernels", items
 * Chain, Star and Tree): for an SPD matrix A whose block graph is a tree, the
 * blocks of A^-1 that lie on A's own block pattern -- every diagonal block and
 * every pattern edge -- and log det A, without forming the dense inverse.
 * The work is a collect pass (block Cholesky / LDL^T Schur sweep, leaves ->
 * root) followed by a distribute pass (Takahashi back-recursion, root ->
 * leaves); the page identifies this two-pass schedule with Gaussian belief
 * propagation.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - Every array argument is a DEVICE pointer (memory of the current HIP
 *   device), except `parent_host` of selinv_tree_plan_create.  The caller owns
 *   all memory; the library never allocates per call.  Scratch memory comes in
 *   through `workspace` (size from the matching *_workspace_bytes query; NULL
 *   is allowed when that size is 0).  The workspace must not be used by
 *   another call that is still running.
 * - Blocks are b x b, row-major, contiguous; batches are contiguous
 *   ("leading batch dimensions", Quickstart section).  Outputs must not alias
 *   inputs or each other.
 * - Every block array must be 16-byte aligned (allocator pointers are; a view
 *   into a larger array is when its byte offset is a multiple of 16), and the
 *   workspace 256-byte aligned; otherwise the call returns
 *   SELINV_ERR_INVALID_ARG.
 * - Only the lower triangle of each diagonal input block is read (they are
 *   taken to be symmetric).  Diagonal output blocks are written in full and
 *   are symmetric.
 * - `logdet` is always float64 (natural log of det A), also for the f32
 *   entry points, which accumulate it in float64.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *   default stream) and returns; nothing synchronises the device.
 * - `info` (may be NULL): per matrix, 0 if every Schur pivot was positive
 *   definite, else 1 + the index of a block whose pivot was not (NaN
 *   included).  That matrix's outputs are then unspecified and its logdet is
 *   NaN.  With a single bad block the index is that block; numbering is per
 *   entry point below.  This follows the "not positive definite -> error"
 *   convention of the sparsax page (Features list); the Python binding's
 *   check=True turns a nonzero info into an exception.
 * - info = SELINV_INFO_WAIT_TIMEOUT (-1) is not a numerical failure: the
 *   single-launch tree schedules (selinv_tree_*, selinv_nonsym_tree_*, the
 *   tree reverse mode and solve) bound every wait of one workgroup on
 *   another; a wait that expires reports -1, NaN outputs and a NaN log det.
 *   It can happen when other work keeps the GPU's workgroup slots busy for
 *   longer than the bound (selinv_set_wait_limit); calling again on an idle
 *   stream, or with a larger bound, is the remedy.  selinv_strerror(
 *   SELINV_ERR_WAIT_TIMEOUT) gives its text.
 * - Return value: a synchronous status (SELINV_OK or an error below) about
 *   the arguments and the launch, not about the numerics.
 * - Supported block sizes: 1 <= b <= 32.  Distinct calls on distinct streams
 *   with distinct workspaces may run concurrently.
 */
#ifndef SELINV_H
#define SELINV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SELINV_API __attribute__((visibility("default")))
#else
#define SELINV_API
#endif

#define SELINV_OK 0
#define SELINV_ERR_INVALID_ARG 1 /* null pointer, bad size, b unsupported, workspace too small */
#define SELINV_ERR_BAD_TREE 2    /* parent array is not one rooted tree                        */
#define SELINV_ERR_HIP 3         /* HIP runtime or launch error                                 */
#define SELINV_ERR_BAD_PATTERN 4 /* junction pattern or elimination order is invalid            */
#define SELINV_ERR_WAIT_TIMEOUT 5 /* a bounded dataflow wait expired (reported as info = -1)    */

#define SELINV_ERR_SCRATCH_LIMIT 6 /* the call needs more scratch than the static array holds */

/* info value of a call whose bounded dataflow wait expired */
#define SELINV_INFO_WAIT_TIMEOUT (-1)

#define SELINV_MAX_B 32

/* Human-readable text for a status code (static storage). */
SELINV_API const char *selinv_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
SELINV_API int selinv_version(void);

/* ------------------------------------------------------------------ chain
 * Block-tridiagonal SPD chains (item "Chain": block LDL^T factorisation plus
 * Takahashi back-recursion, O(L b^3) time).  Per matrix m of B:
 *   diag    [B][L][b][b]    D_i = A_{i,i}
 *   lower   [B][L-1][b][b]  lower[i] = A_{i+1,i}
 *   G_diag  [B][L][b][b]    (A^-1)_{i,i}
 *   G_lower [B][L-1][b][b]  (A^-1)_{i+1,i}
 *   logdet  [B]             ln det A (float64)
 *   info    [B]             0, or 1 + failing block index i
 * L >= 1; with L == 1, lower and G_lower may be NULL. */
SELINV_API size_t selinv_chain_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
SELINV_API int selinv_chain_f64(int64_t B, int64_t L, int32_t b, const double *diag, const double *lower,
                     double *G_diag, double *G_lower, double *logdet, int32_t *info,
                     void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_chain_f32(int64_t B, int64_t L, int32_t b, const float *diag, const float *lower,
                     float *G_diag, float *G_lower, double *logdet, int32_t *info,
                     void *workspace, size_t workspace_bytes, void *stream);

/* The chain call without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, layouts, info, logdet
 * and stream semantics as selinv_chain_f64 / _f32, minus workspace.  The
 * kernels' scratch is a file-scope device array of
 * selinv_chain_static_scratch_bytes() bytes (256 MiB) on each device the
 * library runs on, held until the process ends; the call itself allocates
 * nothing.  A call that needs more scratch than that
 * (selinv_chain_workspace_bytes > the array) returns SELINV_ERR_SCRATCH_LIMIT
 * and launches nothing.  The array is shared by every call on a device:
 * calls that overlap in time on one device (different streams, or host
 * threads) race and must be serialised by the caller.  The stream's device
 * must be the current device. */
SELINV_API size_t selinv_chain_static_scratch_bytes(void);
SELINV_API int selinv_chain_noalloc_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                                        const double *lower, double *G_diag, double *G_lower,
                                        double *logdet, int32_t *info, void *stream);
SELINV_API int selinv_chain_noalloc_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                                        const float *lower, float *G_diag, float *G_lower,
                                        double *logdet, int32_t *info, void *stream);

/* ------------------------------------------------------------------- star
 * Block-arrowhead SPD matrices (item "Star": one centre block coupled to K
 * leaf blocks, no leaf-leaf coupling; leaves are eliminated in parallel).
 * Block 0 is the centre, leaf j is block j+1.  Per matrix m of B:
 *   center   [B][b][b]      A_{0,0}
 *   leaves   [B][K][b][b]   A_{j,j}
 *   coupling [B][K][b][b]   A_{j,0} (leaf row, centre column)
 *   G_center [B][b][b]      (A^-1)_{0,0}
 *   G_leaf   [B][K][b][b]   (A^-1)_{j,j}
 *   G_cross  [B][K][b][b]   (A^-1)_{j,0}
 *   logdet   [B], info [B]  info: 1 = centre pivot, j+2 = leaf j
 * K >= 0; with K == 0 the leaf arrays may be NULL.  The off-pattern
 * leaf-leaf blocks of A^-1 are never formed. */
SELINV_API size_t selinv_star_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
SELINV_API int selinv_star_f64(int64_t B, int64_t K, int32_t b, const double *center, const double *leaves,
                    const double *coupling, double *G_center, double *G_leaf, double *G_cross,
                    double *logdet, int32_t *info, void *workspace, size_t workspace_bytes,
                    void *stream);
SELINV_API int selinv_star_f32(int64_t B, int64_t K, int32_t b, const float *center, const float *leaves,
                    const float *coupling, float *G_center, float *G_leaf, float *G_cross,
                    double *logdet, int32_t *info, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------------------------- tree
 * Arbitrary rooted tree (item "Tree": a parent array and one edge block per
 * non-root node; collect leaves -> root, then distribute root -> leaves).
 *
 * selinv_tree_plan_create validates `parent_host` (HOST memory, n entries,
 * exactly one -1 = the root, every other entry in [0, n), no cycle; else
 * SELINV_ERR_BAD_TREE) and builds the depth level-set schedule once per
 * pattern: breadth-first relabelling so that each depth level and each
 * node's children are contiguous, level offsets and child ranges, copied to
 * the device on `stream` (the plan owns these device arrays; the call
 * synchronises `stream` before returning).  A plan is immutable after creation
 * and may be shared by concurrent calls; it is specific to (n, b, dtype_bytes).
 *
 * selinv_tree_f64 / _f32, for the plan's tree:
 *   diag   [n][b][b]   A_{v,v}
 *   edge   [n][b][b]   edge[v] = A_{parent(v),v}; the root slot is ignored
 *   G_diag [n][b][b]   (A^-1)_{v,v}
 *   G_edge [n][b][b]   (A^-1)_{parent(v),v}; the root slot is written as 0
 *   logdet [1], info [1]   info: v+1 for node v
 * With several bad pivots, info names the first failure in the order
 * (deepest depth first, increasing node index within a depth).
 * For b <= 8 each pass is one launch in which tiles of a level wait for
 * flags set by the tiles of the level they depend on; every such wait is
 * bounded (selinv_set_wait_limit), and a call in which one gives up ends
 * with info = -1, a NaN log det and unusable blocks (it cannot hang). */
typedef struct selinv_tree_plan selinv_tree_plan;

SELINV_API int selinv_tree_plan_create(const int32_t *parent_host, int64_t n, int32_t b, int dtype_bytes,
                            void *stream, selinv_tree_plan **out);
SELINV_API void selinv_tree_plan_destroy(selinv_tree_plan *plan);
/* number of depth levels (tree height + 1) of a plan, or -1 for NULL */
SELINV_API int32_t selinv_tree_plan_levels(const selinv_tree_plan *plan);

/* The level-set schedule selinv_tree_plan_create builds, computed on the host
 * alone (no device work), for inspection and tests.  Nodes get breadth-first
 * positions p: node_at[p] is the node at position p, so every depth level is
 * the contiguous range [level_off[d], level_off[d + 1]) and the children of
 * the node at p are the contiguous positions [child_beg[p], child_end[p]) in
 * increasing node index; parent_pos[p] is the parent's position (-1 at the
 * root); fail_rank[p] is the node's rank in the oracle's elimination order
 * (depth descending, then node index ascending), used to name the first
 * failing pivot.  Every output is caller-owned host memory and may be NULL:
 * n int32 each, level_off at most n + 1 int64 (levels + 1 are written),
 * *levels = tree height + 1.  Returns SELINV_OK, SELINV_ERR_INVALID_ARG
 * (NULL parent, n < 1) or SELINV_ERR_BAD_TREE (as selinv_tree_plan_create). */
SELINV_API int selinv_tree_schedule(const int32_t *parent_host, int64_t n, int32_t *node_at,
                                    int32_t *parent_pos, int32_t *child_beg, int32_t *child_end,
                                    int32_t *fail_rank, int64_t *level_off, int32_t *levels);
SELINV_API size_t selinv_tree_workspace_bytes(const selinv_tree_plan *plan);
SELINV_API int selinv_tree_f64(const selinv_tree_plan *plan, const double *diag, const double *edge,
                    double *G_diag, double *G_edge, double *logdet, int32_t *info,
                    void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_f32(const selinv_tree_plan *plan, const float *diag, const float *edge,
                    float *G_diag, float *G_edge, double *logdet, int32_t *info,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Tree schedule recorded as one HIP graph.  The batched form on the page
 * (item Tree: collect over depth levels leaves -> root, then distribute root
 * -> leaves) issues one batched step per level; here the whole launch
 * sequence of selinv_tree_f64 / _f32 for fixed buffers -- collect kernels
 * from the deepest level to the root, distribute kernels from depth 1 down,
 * then the log-det reduction -- is captured once and replayed with a single
 * launch.
 *   selinv_tree_graph_create_*: same arguments, layouts and checks as
 *     selinv_tree_* (SELINV_ERR_INVALID_ARG on the same conditions), minus
 *     the stream: capture runs on a private stream.  Nothing is computed at
 *     creation.  Returns SELINV_ERR_HIP if capture or instantiation fails;
 *     *out is set only on success.  The plan and every buffer must outlive
 *     the graph; the graph owns no device memory of its own.
 *   selinv_tree_graph_launch: replays the graph on `stream`: the outputs are
 *     recomputed from the current contents of diag and edge, exactly as a
 *     selinv_tree_* call on that stream would (bitwise the same results).
 *     Replays of one graph on one stream run in order; replays that overlap
 *     on different streams race on the shared workspace.
 *   selinv_tree_graph_nodes: number of kernel launches in the graph, -1 for
 *     NULL.  selinv_tree_graph_destroy: frees the graph (NULL is ignored);
 *     no replay may be pending. */
typedef struct selinv_tree_graph selinv_tree_graph;
/* Bound of each wait inside a single-launch level schedule, in ticks of the
 * GPU's 100 MHz constant clock (default 2^24, about 0.17 s).  Process-wide;
 * read when a call is issued (a tree graph keeps the value it was created
 * with).  A wait that expires makes its call report info = -1.  Meant for
 * diagnostics and tests of that path: 0 gives up on the first unready flag.
 * selinv_wait_limit returns the current value. */
SELINV_API void selinv_set_wait_limit(uint64_t ticks);
SELINV_API uint64_t selinv_wait_limit(void);
SELINV_API int selinv_tree_graph_create_f64(const selinv_tree_plan *plan, const double *diag,
                                 const double *edge, double *G_diag, double *G_edge,
                                 double *logdet, int32_t *info, void *workspace,
                                 size_t workspace_bytes, selinv_tree_graph **out);
SELINV_API int selinv_tree_graph_create_f32(const selinv_tree_plan *plan, const float *diag,
                                 const float *edge, float *G_diag, float *G_edge,
                                 double *logdet, int32_t *info, void *workspace,
                                 size_t workspace_bytes, selinv_tree_graph **out);
SELINV_API int selinv_tree_graph_launch(const selinv_tree_graph *graph, void *stream);
SELINV_API int64_t selinv_tree_graph_nodes(const selinv_tree_graph *graph);
SELINV_API void selinv_tree_graph_destroy(selinv_tree_graph *graph);

/* ---------------------------------------------------- reverse mode (VJP)
 * Vector-Jacobian products of the three computations above: given the
 * cotangents of every output, the cotangents of the inputs (the analytic
 * backward of gabp-sparse-inv 0.3.2, "Implemented and tested kernels", item
 * Differentiable tree: a second collect / distribute pair on the same tree,
 * O((|V| + |E|) b^3) like the forward).  Each call recomputes the forward
 * collect internally; nothing is kept between calls, so a caller passes the
 * same inputs it gave the forward call.
 *
 * Convention (the dense identity d(A^-1) = -A^-1 dA A^-1 restricted to the
 * pattern, d log det A = <A^-1, dA>):
 *   - the loss is L(G_diag, G_edge, logdet); the cotangent arrays have the
 *     shapes of the forward outputs, and `logdet_bar` has one float64 per
 *     matrix (NULL = all zero);
 *   - a diagonal output block is symmetric, so only the symmetric part of its
 *     cotangent matters (the call reads the whole block and uses sym(.) =
 *     (X + X^T) / 2);
 *   - diagonal inputs are symmetric parameters: the returned diagonal
 *     cotangent is the symmetric block sym(dL/dA_vv), the gradient with
 *     respect to symmetric perturbations, written in full;
 *   - an edge input block appears in A twice (as E at (p, v) and E^T at
 *     (v, p)); the returned edge cotangent counts both: dL/dA_{p,v} +
 *     (dL/dA_{v,p})^T, in the orientation of the input array.
 * info, alignment, stream, workspace and return-status conventions are those
 * of the forward entry points; on a failed pivot the matrix's cotangents are
 * NaN.  Outputs must not alias inputs or each other. */

/* chain: diag, lower as for selinv_chain_*; G_diag_bar [B][L][b][b],
 * G_lower_bar [B][L-1][b][b] (may be NULL when L == 1), logdet_bar [B];
 * outputs diag_bar [B][L][b][b], lower_bar [B][L-1][b][b]; info [B]. */
SELINV_API size_t selinv_chain_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
SELINV_API int selinv_chain_vjp_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                         const double *lower, const double *G_diag_bar,
                         const double *G_lower_bar, const double *logdet_bar, double *diag_bar,
                         double *lower_bar, int32_t *info, void *workspace,
                         size_t workspace_bytes, void *stream);
SELINV_API int selinv_chain_vjp_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                         const float *lower, const float *G_diag_bar, const float *G_lower_bar,
                         const double *logdet_bar, float *diag_bar, float *lower_bar,
                         int32_t *info, void *workspace, size_t workspace_bytes, void *stream);

/* star: center, leaves, coupling as for selinv_star_*; cotangents
 * G_center_bar [B][b][b], G_leaf_bar [B][K][b][b], G_cross_bar [B][K][b][b]
 * (on G_cross[j] = (A^-1)_{j,0}), logdet_bar [B]; outputs center_bar,
 * leaves_bar, coupling_bar (on coupling[j] = A_{j,0}, counting A_{0,j} too);
 * info [B].  With K == 0 the leaf arrays may be NULL. */
SELINV_API size_t selinv_star_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
SELINV_API int selinv_star_vjp_f64(int64_t B, int64_t K, int32_t b, const double *center,
                        const double *leaves, const double *coupling,
                        const double *G_center_bar, const double *G_leaf_bar,
                        const double *G_cross_bar, const double *logdet_bar, double *center_bar,
                        double *leaves_bar, double *coupling_bar, int32_t *info,
                        void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_star_vjp_f32(int64_t B, int64_t K, int32_t b, const float *center,
                        const float *leaves, const float *coupling, const float *G_center_bar,
                        const float *G_leaf_bar, const float *G_cross_bar,
                        const double *logdet_bar, float *center_bar, float *leaves_bar,
                        float *coupling_bar, int32_t *info, void *workspace,
                        size_t workspace_bytes, void *stream);

/* tree, for a plan from selinv_tree_plan_create: cotangents G_diag_bar
 * [n][b][b], G_edge_bar [n][b][b] (root slot ignored), logdet_bar [1];
 * outputs diag_bar [n][b][b], edge_bar [n][b][b] (root slot written as 0);
 * info [1] as for selinv_tree_*. */
SELINV_API size_t selinv_tree_vjp_workspace_bytes(const selinv_tree_plan *plan);
SELINV_API int selinv_tree_vjp_f64(const selinv_tree_plan *plan, const double *diag,
                        const double *edge, const double *G_diag_bar, const double *G_edge_bar,
                        const double *logdet_bar, double *diag_bar, double *edge_bar,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_vjp_f32(const selinv_tree_plan *plan, const float *diag,
                        const float *edge, const float *G_diag_bar, const float *G_edge_bar,
                        const double *logdet_bar, float *diag_bar, float *edge_bar,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------- shared-factor siblings
 * "Factor once, do everything" (gabp-sparse-inv 0.3.2 page: tree_logdet /
 * junction_logdet take log det A straight from the LDL^T factorization,
 * junction_solve solves on the same pattern sharing it, and
 * sample_gaussian_tree draws x ~ N(0, A^{-1}) reusing it).  The collect pass
 * is a block LDL^T factorisation A = L D L^T, D = blockdiag(S_v),
 * L_{p,v} = E_v S_v^{-1}; the *factor* calls run it once and keep the S_v^{-1}
 * in a caller-owned buffer, and the *solve* / *sample* calls reuse it:
 *   solve:  x = A^{-1} y (k right-hand sides at once);
 *   sample: x = L^{-T} D^{-1/2} z with D^{-1/2}_v the upper triangular
 *           factor U_v of S_v^{-1} (U_v U_v^T = S_v^{-1}; U_v = R_v^{-T} for
 *           S_v = R_v R_v^T), so x ~ N(0, A^{-1}) when z ~ N(0, I).  The caller
 *           draws z; the map z -> x is deterministic.
 * A factor call with factor == NULL computes log det and info only (the
 * log-det fast path).
 *
 * The factor buffer's layout is private to the library: size it with the
 * matching *_factor_bytes query, keep it 16-byte aligned, and pass it only to
 * solve / sample calls with the same sizes, dtype (and plan) and the same
 * edge blocks as the factor call.  Where that call reported info != 0 for a
 * matrix, that matrix's solve / sample results are unspecified.
 * Vectors (y, z, x) are [..., n_blocks, b, k] row-major (k fastest), with no
 * alignment requirement; x must not alias y / z.  Other conventions (stream,
 * workspace, return status) as above. */

/* chain: factor [B][L] packed blocks; y, z, x [B][L][b][k] */
SELINV_API size_t selinv_chain_factor_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b);
SELINV_API int selinv_chain_factor_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                            const double *lower, double *factor, double *logdet, int32_t *info,
                            void *stream);
SELINV_API int selinv_chain_factor_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                            const float *lower, float *factor, double *logdet, int32_t *info,
                            void *stream);
SELINV_API int selinv_chain_solve_f64(int64_t B, int64_t L, int32_t b, const double *lower,
                           const double *factor, int64_t k, const double *y, double *x,
                           void *stream);
SELINV_API int selinv_chain_solve_f32(int64_t B, int64_t L, int32_t b, const float *lower,
                           const float *factor, int64_t k, const float *y, float *x,
                           void *stream);
SELINV_API int selinv_chain_sample_f64(int64_t B, int64_t L, int32_t b, const double *lower,
                            const double *factor, int64_t k, const double *z, double *x,
                            void *stream);
SELINV_API int selinv_chain_sample_f32(int64_t B, int64_t L, int32_t b, const float *lower,
                            const float *factor, int64_t k, const float *z, float *x,
                            void *stream);

/* star: vectors split as the centre [B][b][k] and the leaves [B][K][b][k] */
SELINV_API size_t selinv_star_factor_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b);
SELINV_API size_t selinv_star_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K,
                                          int32_t b);
SELINV_API size_t selinv_star_solve_workspace_bytes(int dtype_bytes, int64_t B, int64_t K,
                                         int32_t b, int64_t k);
SELINV_API int selinv_star_factor_f64(int64_t B, int64_t K, int32_t b, const double *center,
                           const double *leaves, const double *coupling, double *factor,
                           double *logdet, int32_t *info, void *workspace,
                           size_t workspace_bytes, void *stream);
SELINV_API int selinv_star_factor_f32(int64_t B, int64_t K, int32_t b, const float *center,
                           const float *leaves, const float *coupling, float *factor,
                           double *logdet, int32_t *info, void *workspace,
                           size_t workspace_bytes, void *stream);
SELINV_API int selinv_star_solve_f64(int64_t B, int64_t K, int32_t b, const double *coupling,
                          const double *factor, int64_t k, const double *y_center,
                          const double *y_leaves, double *x_center, double *x_leaves,
                          void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_star_solve_f32(int64_t B, int64_t K, int32_t b, const float *coupling,
                          const float *factor, int64_t k, const float *y_center,
                          const float *y_leaves, float *x_center, float *x_leaves,
                          void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_star_sample_f64(int64_t B, int64_t K, int32_t b, const double *coupling,
                           const double *factor, int64_t k, const double *z_center,
                           const double *z_leaves, double *x_center, double *x_leaves,
                           void *stream);
SELINV_API int selinv_star_sample_f32(int64_t B, int64_t K, int32_t b, const float *coupling,
                           const float *factor, int64_t k, const float *z_center,
                           const float *z_leaves, float *x_center, float *x_leaves,
                           void *stream);

/* tree: vectors [n][b][k] by node index.  For b <= 8 the solve runs both
 * sweeps, and the sampler its one parents-first sweep, as single launches with
 * bounded waits (see selinv_tree_f64); a call whose wait gives up returns NaN
 * in x.  Solve and sample take a workspace of selinv_tree_solve_workspace_bytes
 * (plan, k) bytes (device, caller-owned, 256-byte aligned, contents need not
 * be initialised; none is needed for the sampler when b > 8: pass NULL, 0). */
SELINV_API size_t selinv_tree_factor_bytes(const selinv_tree_plan *plan);
SELINV_API size_t selinv_tree_factor_workspace_bytes(const selinv_tree_plan *plan);
SELINV_API size_t selinv_tree_solve_workspace_bytes(const selinv_tree_plan *plan, int64_t k);
SELINV_API int selinv_tree_factor_f64(const selinv_tree_plan *plan, const double *diag,
                           const double *edge, double *factor, double *logdet, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_factor_f32(const selinv_tree_plan *plan, const float *diag,
                           const float *edge, float *factor, double *logdet, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_solve_f64(const selinv_tree_plan *plan, const double *edge,
                          const double *factor, int64_t k, const double *y, double *x,
                          void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_solve_f32(const selinv_tree_plan *plan, const float *edge,
                          const float *factor, int64_t k, const float *y, float *x,
                          void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_sample_f64(const selinv_tree_plan *plan, const double *edge,
                           const double *factor, int64_t k, const double *z, double *x,
                           void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_tree_sample_f32(const selinv_tree_plan *plan, const float *edge,
                           const float *factor, int64_t k, const float *z, float *x,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------ non-symmetric ladder
 * (gabp-sparse-inv 0.3.2, "Implemented and tested kernels", items
 * Non-symmetric chain and Non-symmetric tree.)  General blocks, no symmetry
 * or definiteness assumed, eliminated without pivoting (safe while the matrix
 * is block-diagonally dominant); info = 1 + the block whose elimination met a
 * zero or non-finite pivot, and that matrix's outputs are NaN.
 *
 * Block lower-bidiagonal M (fully local: G_ii = M_ii^{-1} and
 * G_{i+1,i} = -M_{i+1,i+1}^{-1} M_{i+1,i} M_ii^{-1}), per matrix of B:
 *   diag [B][L][b][b] M_ii, lower [B][L-1][b][b] M_{i+1,i};
 *   G_diag, G_lower likewise; info [B] (1 + smallest failing block index).
 * Workspace: selinv_bidiag_workspace_bytes. */
SELINV_API size_t selinv_bidiag_workspace_bytes(int64_t B);
SELINV_API int selinv_bidiag_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                      const double *lower, double *G_diag, double *G_lower, int32_t *info,
                      void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_bidiag_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                      const float *lower, float *G_diag, float *G_lower, int32_t *info,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Non-symmetric tree with independent directed edge blocks, for a plan of
 * selinv_tree_plan_create (same n, b, dtype):
 *   diag [n][b][b] M_vv, up [n][b][b] up[v] = M_{parent(v),v},
 *   down [n][b][b] down[v] = M_{v,parent(v)} (root slots ignored);
 *   G_diag, G_up [v] = (M^-1)_{parent(v),v}, G_down [v] = (M^-1)_{v,parent(v)}
 *   (root slots written as 0); info [1] as for selinv_tree_*. */
SELINV_API size_t selinv_nonsym_tree_workspace_bytes(const selinv_tree_plan *plan);
SELINV_API int selinv_nonsym_tree_f64(const selinv_tree_plan *plan, const double *diag,
                           const double *up, const double *down, double *G_diag, double *G_up,
                           double *G_down, int32_t *info, void *workspace, size_t workspace_bytes,
                           void *stream);
SELINV_API int selinv_nonsym_tree_f32(const selinv_tree_plan *plan, const float *diag,
                           const float *up, const float *down, float *G_diag, float *G_up,
                           float *G_down, int32_t *info, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ---------------------------------------------------- general sparse SPD
 * Junction tree (gabp-sparse-inv page, junction-tree section): an arbitrary
 * block sparsity pattern, eliminated in an elimination order (default:
 * greedy minimum degree) and thereby completed to its chordal filled
 * pattern S = pattern(L + L^T); the selected inverse is returned on S (a
 * superset of the input pattern wherever elimination creates fill), from a
 * sparse block Cholesky factorisation and the multi-neighbour Takahashi
 * recurrence, run level by level over the elimination tree.  A batch of B
 * matrices shares one pattern (one plan).
 *
 * selinv_junction_plan_create (all arguments HOST memory):
 *   edge_index_host [2][m] int32: row 0 = i, row 1 = j, one entry per pattern
 *       edge {i, j} with 0 <= j < i < n, no repeats (m may be 0 and the
 *       pointer then NULL); else SELINV_ERR_BAD_PATTERN
 *   order_host [n] int32 or NULL: the elimination order (order[s] = the node
 *       eliminated at step s; a permutation, else SELINV_ERR_BAD_PATTERN).
 *       NULL = greedy minimum degree: at every step the remaining node with
 *       the fewest remaining neighbours, the smallest index among ties.
 * It runs the symbolic analysis once per pattern (elimination, S, the
 * elimination-tree level sets and every index table of the kernels) and
 * copies the tables to the device on `stream` (the plan owns them; the call
 * synchronises `stream`).  A plan is immutable and may be shared by
 * concurrent calls; it is specific to (pattern, order, b, dtype_bytes).
 *
 * selinv_junction_plan_nnz: number of lower blocks of S (-1 for NULL);
 * selinv_junction_plan_levels: number of elimination-tree levels;
 * selinv_junction_plan_pattern copies to HOST memory S_index [2][nnz]
 *   (pairs (i, j), i > j, sorted by i then j; may be NULL) and the
 *   elimination order [n] (may be NULL).
 *
 * selinv_junction_f64 / _f32, for B matrices on the plan's pattern:
 *   diag     [B][n][b][b]    A_{v,v}
 *   edge_val [B][m][b][b]    edge_val[e] = A_{i_e, j_e}
 *   G_diag   [B][n][b][b]    (A^-1)_{v,v}
 *   G_lower  [B][nnz][b][b]  G_lower[k] = (A^-1)_{i_k, j_k} for S_index pair k
 *   logdet [B], info [B]     info: 1 + the node index whose Schur pivot is
 *                            not positive definite, the earliest such node
 *                            in the elimination order
 * Workspace: selinv_junction_workspace_bytes(plan, B). */
typedef struct selinv_junction_plan selinv_junction_plan;

SELINV_API int selinv_junction_plan_create(int64_t n, int64_t m, const int32_t *edge_index_host,
                                const int32_t *order_host, int32_t b, int dtype_bytes,
                                void *stream, selinv_junction_plan **out);
SELINV_API void selinv_junction_plan_destroy(selinv_junction_plan *plan);
SELINV_API int64_t selinv_junction_plan_nnz(const selinv_junction_plan *plan);
SELINV_API int32_t selinv_junction_plan_levels(const selinv_junction_plan *plan);
SELINV_API int selinv_junction_plan_pattern(const selinv_junction_plan *plan, int32_t *S_index_host,
                                 int32_t *order_host);
/* The symbolic analysis alone, on the host (no device work): nnz and the
 * number of levels, S_index [2][nnz] when `cap` >= nnz (else not written),
 * and the elimination order [n]; each output may be NULL.  Same validation
 * and statuses as selinv_junction_plan_create. */
SELINV_API int selinv_junction_symbolic(int64_t n, int64_t m, const int32_t *edge_index_host,
                             const int32_t *order_host, int64_t *nnz_out, int32_t *levels_out,
                             int32_t *S_index_host, int64_t cap, int32_t *order_out);
SELINV_API size_t selinv_junction_workspace_bytes(const selinv_junction_plan *plan, int64_t B);
SELINV_API int selinv_junction_f64(const selinv_junction_plan *plan, int64_t B, const double *diag,
                        const double *edge_val, double *G_diag, double *G_lower, double *logdet,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_junction_f32(const selinv_junction_plan *plan, int64_t B, const float *diag,
                        const float *edge_val, float *G_diag, float *G_lower, double *logdet,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream);
/* log det A alone from the same factorisation (the junction_logdet sibling
 * of the same section): the sparse block Cholesky pass of selinv_junction_*
 * without the Takahashi pass; logdet [B], info [B] and the workspace as
 * above (same size query). */
SELINV_API int selinv_junction_logdet_f64(const selinv_junction_plan *plan, int64_t B,
                               const double *diag, const double *edge_val, double *logdet,
                               int32_t *info, void *workspace, size_t workspace_bytes,
                               void *stream);
SELINV_API int selinv_junction_logdet_f32(const selinv_junction_plan *plan, int64_t B,
                               const float *diag, const float *edge_val, double *logdet,
                               int32_t *info, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Solve and Gaussian sampling on the filled pattern (the junction_solve
 * sibling of the junction-tree section, one or several right-hand sides,
 * and Gaussian sampling; both reuse the factorisation of the selected
 * inverse, as in the shared-factor section above):
 *   selinv_junction_factor_*: the factorisation of selinv_junction_logdet_*
 *     (logdet [B], info [B] as there), keeping the factor in `factor`, a
 *     caller-owned device buffer of selinv_junction_factor_bytes(plan, B)
 *     bytes, 16-byte aligned, layout private to the library; factor must not
 *     be NULL (selinv_junction_logdet_* computes log det alone).  Workspace:
 *     selinv_junction_factor_workspace_bytes(plan, B).
 *   selinv_junction_solve_*:  x = A^{-1} y,       y, x [B][n][b][k]
 *   selinv_junction_sample_*: x = L^{-T} D^{-1/2} z, z, x [B][n][b][k]
 *     with A = L D L^T the block LDL^T in the plan's elimination order and
 *     D^{-1/2}_v = R_v^{-T} for D_v = R_v R_v^T, so x ~ N(0, A^{-1}) when
 *     z ~ N(0, I) (the caller draws z; the map z -> x is deterministic).
 *     Vectors by node label, k fastest, no alignment requirement; x must not
 *     alias y / z (x == y is rejected).  The factor must come from a factor
 *     call with the same plan and B; where that call reported info != 0 for
 *     a matrix, that matrix's x is unspecified.  The solve's workspace:
 *     selinv_junction_solve_workspace_bytes(plan, B, k) (per later row of
 *     every chunk a b x k vector, and the flags of its single-launch
 *     sweeps); the sample needs none.  Each solve sweep is one launch whose
 *     workgroups wait for one another (bounded by selinv_set_wait_limit); if
 *     a wait gives up, every x entry computed after that is NaN (there is no
 *     info output): calling again, or raising the limit, is the remedy. */
SELINV_API size_t selinv_junction_factor_bytes(const selinv_junction_plan *plan, int64_t B);
SELINV_API size_t selinv_junction_factor_workspace_bytes(const selinv_junction_plan *plan,
                                                        int64_t B);
SELINV_API int selinv_junction_factor_f64(const selinv_junction_plan *plan, int64_t B,
                               const double *diag, const double *edge_val, double *factor,
                               double *logdet, int32_t *info, void *workspace,
                               size_t workspace_bytes, void *stream);
SELINV_API int selinv_junction_factor_f32(const selinv_junction_plan *plan, int64_t B,
                               const float *diag, const float *edge_val, float *factor,
                               double *logdet, int32_t *info, void *workspace,
                               size_t workspace_bytes, void *stream);
SELINV_API size_t selinv_junction_solve_workspace_bytes(const selinv_junction_plan *plan,
                                                       int64_t B, int64_t k);
SELINV_API int selinv_junction_solve_f64(const selinv_junction_plan *plan, int64_t B,
                              const double *factor, int64_t k, const double *y, double *x,
                              void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_junction_solve_f32(const selinv_junction_plan *plan, int64_t B,
                              const float *factor, int64_t k, const float *y, float *x,
                              void *workspace, size_t workspace_bytes, void *stream);
SELINV_API int selinv_junction_sample_f64(const selinv_junction_plan *plan, int64_t B,
                               const double *factor, int64_t k, const double *z, double *x,
                               void *stream);
SELINV_API int selinv_junction_sample_f32(const selinv_junction_plan *plan, int64_t B,
                               const float *factor, int64_t k, const float *z, float *x,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SELINV_H */
