// abi.cpp -- the extern "C" entry points declared in include/selinv.h:
// argument validation, workspace checks and dispatch to the kernels.  No
// allocation happens here; all device memory is the caller's.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

inline bool bad_b(int32_t b) { return b < 1 || b > SELINV_MAX_B; }

// block arrays: 16-byte aligned (null passes; required pointers are checked
// separately); workspace: 256-byte aligned
inline bool misaligned(const void *p) { return reinterpret_cast<uintptr_t>(p) & 15; }
inline bool misaligned_ws(const void *p) { return reinterpret_cast<uintptr_t>(p) & 255; }

template <typename T>
int chain_entry(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *G_diag,
                T *G_lower, double *logdet, int32_t *info, void *ws, size_t ws_bytes,
                void *stream) {
  if (B < 0 || L < 1 || bad_b(b) || B > 0x7fffffff) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !G_diag || !logdet) return SELINV_ERR_INVALID_ARG;
  if (L > 1 && (!lower || !G_lower)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(G_diag) || (L > 1 && (misaligned(lower) || misaligned(G_lower))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::chain_workspace_bytes(sizeof(T), B, L, b);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::chain_launch<T>(B, L, b, diag, lower, G_diag, G_lower, logdet,
                                               info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int star_entry(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
               const T *coupling, T *G_center, T *G_leaf, T *G_cross, double *logdet,
               int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (B < 0 || K < 0 || bad_b(b) || B > 0x7fffffff || B * K > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!center || !G_center || !logdet) return SELINV_ERR_INVALID_ARG;
  if (K > 0 && (!leaves || !coupling || !G_leaf || !G_cross)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(center) || misaligned(G_center) ||
      (K > 0 && (misaligned(leaves) || misaligned(coupling) || misaligned(G_leaf) ||
                 misaligned(G_cross))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::star_workspace_bytes(sizeof(T), B, K, b);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e =
      selinv::star_launch<T>(B, K, b, center, leaves, coupling, G_center, G_leaf, G_cross,
                             logdet, info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int tree_entry(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag, T *G_edge,
               double *logdet, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (!diag || !edge || !G_diag || !G_edge || !logdet) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge) || misaligned(G_diag) || misaligned(G_edge))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::tree_workspace_bytes(plan);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::tree_launch<T>(plan, diag, edge, G_diag, G_edge, logdet, info, ws,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int chain_vjp_entry(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, const T *gd,
                    const T *gl, const double *ld_bar, T *d_bar, T *l_bar, int32_t *info,
                    void *ws, size_t ws_bytes, void *stream) {
  if (B < 0 || L < 1 || bad_b(b) || B > 0x7fffffff) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !gd || !d_bar) return SELINV_ERR_INVALID_ARG;
  if (L > 1 && (!lower || !gl || !l_bar)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(gd) || misaligned(d_bar) ||
      (L > 1 && (misaligned(lower) || misaligned(gl) || misaligned(l_bar))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::chain_vjp_workspace_bytes(sizeof(T), B, L, b);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::chain_vjp_launch<T>(B, L, b, diag, lower, gd, gl, ld_bar, d_bar,
                                                   l_bar, info, ws,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int star_vjp_entry(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                   const T *coupling, const T *gc, const T *gleaf, const T *gcross,
                   const double *ld_bar, T *center_bar, T *leaves_bar, T *coupling_bar,
                   int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (B < 0 || K < 0 || bad_b(b) || B > 0x7fffffff || B * K > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!center || !gc || !center_bar) return SELINV_ERR_INVALID_ARG;
  if (K > 0 && (!leaves || !coupling || !gleaf || !gcross || !leaves_bar || !coupling_bar))
    return SELINV_ERR_INVALID_ARG;
  if (misaligned(center) || misaligned(gc) || misaligned(center_bar) ||
      (K > 0 && (misaligned(leaves) || misaligned(coupling) || misaligned(gleaf) ||
                 misaligned(gcross) || misaligned(leaves_bar) || misaligned(coupling_bar))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::star_vjp_workspace_bytes(sizeof(T), B, K, b);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::star_vjp_launch<T>(
      B, K, b, center, leaves, coupling, gc, gleaf, gcross, ld_bar, center_bar, leaves_bar,
      coupling_bar, info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int tree_vjp_entry(const selinv_tree_plan *plan, const T *diag, const T *edge, const T *gd,
                   const T *ge, const double *ld_bar, T *d_bar, T *e_bar, int32_t *info, void *ws,
                   size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (!diag || !edge || !gd || !ge || !d_bar || !e_bar) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge) || misaligned(gd) || misaligned(ge) ||
      misaligned(d_bar) || misaligned(e_bar))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::tree_vjp_workspace_bytes(plan);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::tree_vjp_launch<T>(plan, diag, edge, gd, ge, ld_bar, d_bar, e_bar,
                                                  info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

}  // namespace

extern "C" {

const char *selinv_strerror(int status) {
  switch (status) {
    case SELINV_OK: return "ok";
    case SELINV_ERR_INVALID_ARG: return "invalid argument (pointer, size, block size or workspace)";
    case SELINV_ERR_BAD_TREE: return "parent array is not a single rooted tree";
    case SELINV_ERR_HIP: return "HIP runtime or kernel launch error";
    default: return "unknown status";
  }
}

int selinv_version(void) { return 100; }

size_t selinv_chain_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || L < 1 || bad_b(b)) return 0;
  return selinv::chain_workspace_bytes(dtype_bytes, B, L, b);
}

int selinv_chain_f64(int64_t B, int64_t L, int32_t b, const double *diag, const double *lower,
                     double *G_diag, double *G_lower, double *logdet, int32_t *info,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return chain_entry<double>(B, L, b, diag, lower, G_diag, G_lower, logdet, info, workspace,
                             workspace_bytes, stream);
}

int selinv_chain_f32(int64_t B, int64_t L, int32_t b, const float *diag, const float *lower,
                     float *G_diag, float *G_lower, double *logdet, int32_t *info,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return chain_entry<float>(B, L, b, diag, lower, G_diag, G_lower, logdet, info, workspace,
                            workspace_bytes, stream);
}

size_t selinv_star_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || K < 0 || bad_b(b)) return 0;
  return selinv::star_workspace_bytes(dtype_bytes, B, K, b);
}

int selinv_star_f64(int64_t B, int64_t K, int32_t b, const double *center, const double *leaves,
                    const double *coupling, double *G_center, double *G_leaf, double *G_cross,
                    double *logdet, int32_t *info, void *workspace, size_t workspace_bytes,
                    void *stream) {
  return star_entry<double>(B, K, b, center, leaves, coupling, G_center, G_leaf, G_cross, logdet,
                            info, workspace, workspace_bytes, stream);
}

int selinv_star_f32(int64_t B, int64_t K, int32_t b, const float *center, const float *leaves,
                    const float *coupling, float *G_center, float *G_leaf, float *G_cross,
                    double *logdet, int32_t *info, void *workspace, size_t workspace_bytes,
                    void *stream) {
  return star_entry<float>(B, K, b, center, leaves, coupling, G_center, G_leaf, G_cross, logdet,
                           info, workspace, workspace_bytes, stream);
}

size_t selinv_tree_workspace_bytes(const selinv_tree_plan *plan) {
  return plan ? selinv::tree_workspace_bytes(plan) : 0;
}

int selinv_tree_f64(const selinv_tree_plan *plan, const double *diag, const double *edge,
                    double *G_diag, double *G_edge, double *logdet, int32_t *info,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return tree_entry<double>(plan, diag, edge, G_diag, G_edge, logdet, info, workspace,
                            workspace_bytes, stream);
}

int selinv_tree_f32(const selinv_tree_plan *plan, const float *diag, const float *edge,
                    float *G_diag, float *G_edge, double *logdet, int32_t *info,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return tree_entry<float>(plan, diag, edge, G_diag, G_edge, logdet, info, workspace,
                           workspace_bytes, stream);
}

size_t selinv_chain_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || L < 1 || bad_b(b)) return 0;
  return selinv::chain_vjp_workspace_bytes(dtype_bytes, B, L, b);
}

int selinv_chain_vjp_f64(int64_t B, int64_t L, int32_t b, const double *diag, const double *lower,
                         const double *G_diag_bar, const double *G_lower_bar,
                         const double *logdet_bar, double *diag_bar, double *lower_bar,
                         int32_t *info, void *workspace, size_t workspace_bytes, void *stream) {
  return chain_vjp_entry<double>(B, L, b, diag, lower, G_diag_bar, G_lower_bar, logdet_bar,
                                 diag_bar, lower_bar, info, workspace, workspace_bytes, stream);
}

int selinv_chain_vjp_f32(int64_t B, int64_t L, int32_t b, const float *diag, const float *lower,
                         const float *G_diag_bar, const float *G_lower_bar,
                         const double *logdet_bar, float *diag_bar, float *lower_bar,
                         int32_t *info, void *workspace, size_t workspace_bytes, void *stream) {
  return chain_vjp_entry<float>(B, L, b, diag, lower, G_diag_bar, G_lower_bar, logdet_bar,
                                diag_bar, lower_bar, info, workspace, workspace_bytes, stream);
}

size_t selinv_star_vjp_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || K < 0 || bad_b(b)) return 0;
  return selinv::star_vjp_workspace_bytes(dtype_bytes, B, K, b);
}

int selinv_star_vjp_f64(int64_t B, int64_t K, int32_t b, const double *center,
                        const double *leaves, const double *coupling, const double *G_center_bar,
                        const double *G_leaf_bar, const double *G_cross_bar,
                        const double *logdet_bar, double *center_bar, double *leaves_bar,
                        double *coupling_bar, int32_t *info, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return star_vjp_entry<double>(B, K, b, center, leaves, coupling, G_center_bar, G_leaf_bar,
                                G_cross_bar, logdet_bar, center_bar, leaves_bar, coupling_bar,
                                info, workspace, workspace_bytes, stream);
}

int selinv_star_vjp_f32(int64_t B, int64_t K, int32_t b, const float *center, const float *leaves,
                        const float *coupling, const float *G_center_bar,
                        const float *G_leaf_bar, const float *G_cross_bar,
                        const double *logdet_bar, float *center_bar, float *leaves_bar,
                        float *coupling_bar, int32_t *info, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return star_vjp_entry<float>(B, K, b, center, leaves, coupling, G_center_bar, G_leaf_bar,
                               G_cross_bar, logdet_bar, center_bar, leaves_bar, coupling_bar,
                               info, workspace, workspace_bytes, stream);
}

size_t selinv_tree_vjp_workspace_bytes(const selinv_tree_plan *plan) {
  return plan ? selinv::tree_vjp_workspace_bytes(plan) : 0;
}

int selinv_tree_vjp_f64(const selinv_tree_plan *plan, const double *diag, const double *edge,
                        const double *G_diag_bar, const double *G_edge_bar,
                        const double *logdet_bar, double *diag_bar, double *edge_bar,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream) {
  return tree_vjp_entry<double>(plan, diag, edge, G_diag_bar, G_edge_bar, logdet_bar, diag_bar,
                                edge_bar, info, workspace, workspace_bytes, stream);
}

int selinv_tree_vjp_f32(const selinv_tree_plan *plan, const float *diag, const float *edge,
                        const float *G_diag_bar, const float *G_edge_bar,
                        const double *logdet_bar, float *diag_bar, float *edge_bar, int32_t *info,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return tree_vjp_entry<float>(plan, diag, edge, G_diag_bar, G_edge_bar, logdet_bar, diag_bar,
                               edge_bar, info, workspace, workspace_bytes, stream);
}

}  // extern "C"
