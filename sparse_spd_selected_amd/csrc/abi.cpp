// abi.cpp -- the extern "C" entry points declared in include/selinv.h:
// argument validation, workspace checks and dispatch to the kernels.  No
// device memory is allocated here; all of it is the caller's (a tree graph
// holds only its HIP graph objects).
#include <hip/hip_runtime.h>

#include <atomic>
#include <new>

#include "internal.h"

namespace selinv {

namespace {
std::atomic<uint64_t> g_wait_ticks{uint64_t(1) << 24};
}  // namespace

uint64_t wait_limit_ticks() { return g_wait_ticks.load(std::memory_order_relaxed); }

}  // namespace selinv

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
int tree_check(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag, T *G_edge,
               double *logdet, void *ws, size_t ws_bytes) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (!diag || !edge || !G_diag || !G_edge || !logdet) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge) || misaligned(G_diag) || misaligned(G_edge))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::tree_workspace_bytes(plan);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  return SELINV_OK;
}

template <typename T>
int tree_entry(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag, T *G_edge,
               double *logdet, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  const int rc = tree_check(plan, diag, edge, G_diag, G_edge, logdet, ws, ws_bytes);
  if (rc != SELINV_OK) return rc;
  const hipError_t e = selinv::tree_launch<T>(plan, diag, edge, G_diag, G_edge, logdet, info, ws,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

// The tree launch sequence captured on a private stream.  The capture is
// always ended (and the stream destroyed) before returning, also when a
// launch inside it fails.
template <typename T>
int tree_graph_create(const selinv_tree_plan *plan, const T *diag, const T *edge, T *G_diag,
                      T *G_edge, double *logdet, int32_t *info, void *ws, size_t ws_bytes,
                      selinv_tree_graph **out) {
  if (!out) return SELINV_ERR_INVALID_ARG;
  const int rc = tree_check(plan, diag, edge, G_diag, G_edge, logdet, ws, ws_bytes);
  if (rc != SELINV_OK) return rc;
  hipStream_t cap = nullptr;
  if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) return SELINV_ERR_HIP;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    const hipError_t el =
        selinv::tree_launch<T>(plan, diag, edge, G_diag, G_edge, logdet, info, ws, cap);
    e = hipStreamEndCapture(cap, &graph);
    if (el != hipSuccess) e = el;
  }
  (void)hipStreamDestroy(cap);
  size_t nodes = 0;
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess) e = hipGraphGetNodes(graph, nullptr, &nodes);
  if (e == hipSuccess) e = hipGraphInstantiateWithFlags(&exec, graph, 0);
  selinv_tree_graph *g = nullptr;
  if (e == hipSuccess) {
    g = new (std::nothrow) selinv_tree_graph();
    if (!g) e = hipErrorOutOfMemory;
  }
  if (e != hipSuccess) {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    return SELINV_ERR_HIP;
  }
  g->graph = graph;
  g->exec = exec;
  g->nodes = static_cast<int64_t>(nodes);
  *out = g;
  return SELINV_OK;
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

template <typename T>
int chain_factor_entry(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *factor,
                       double *logdet, int32_t *info, void *stream) {
  if (B < 0 || L < 1 || bad_b(b) || B > 0x7fffffff) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !logdet || (L > 1 && !lower)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(factor) || (L > 1 && misaligned(lower)))
    return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::chain_factor_launch<T>(B, L, b, diag, lower, factor, logdet, info,
                                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int chain_apply_entry(int64_t B, int64_t L, int32_t b, const T *lower, const T *factor,
                      int64_t k, const T *in, T *out, bool sample, void *stream) {
  if (B < 0 || L < 1 || bad_b(b) || k < 0 || B > 0x7fffffff || B * ((k + 15) / 16) > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0 || k == 0) return SELINV_OK;
  if (!factor || !in || !out || (L > 1 && !lower)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(factor) || (L > 1 && misaligned(lower))) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::chain_apply_launch<T>(B, L, b, k, sample, lower, factor, in, out,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int star_factor_entry(int64_t B, int64_t K, int32_t b, const T *center, const T *leaves,
                      const T *coupling, T *factor, double *logdet, int32_t *info, void *ws,
                      size_t ws_bytes, void *stream) {
  if (B < 0 || K < 0 || bad_b(b) || B > 0x7fffffff || B * K > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!center || !logdet || (K > 0 && (!leaves || !coupling))) return SELINV_ERR_INVALID_ARG;
  if (misaligned(center) || misaligned(factor) ||
      (K > 0 && (misaligned(leaves) || misaligned(coupling))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::star_factor_workspace_bytes(sizeof(T), B, K, b);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::star_factor_launch<T>(B, K, b, center, leaves, coupling, factor,
                                                     logdet, info, ws,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int star_apply_entry(int64_t B, int64_t K, int32_t b, const T *coupling, const T *factor,
                     int64_t k, const T *in_c, const T *in_l, T *x_c, T *x_l, void *ws,
                     size_t ws_bytes, bool sample, void *stream) {
  const int64_t nch = (k + 15) / 16;
  if (B < 0 || K < 0 || bad_b(b) || k < 0 || B > 0x7fffffff || B * K > 0x7fffffff ||
      B * (K + 1) * nch > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0 || k == 0) return SELINV_OK;
  if (!factor || !in_c || !x_c || (K > 0 && (!coupling || !in_l || !x_l)))
    return SELINV_ERR_INVALID_ARG;
  if (misaligned(factor) || (K > 0 && misaligned(coupling))) return SELINV_ERR_INVALID_ARG;
  const size_t need = sample ? 0 : selinv::star_apply_workspace_bytes(sizeof(T), B, K, b, k);
  if (ws_bytes < need || (need && !ws) || (need && misaligned_ws(ws)))
    return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::star_apply_launch<T>(B, K, b, k, sample, coupling, factor, in_c,
                                                    in_l, x_c, x_l, ws,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int tree_factor_entry(const selinv_tree_plan *plan, const T *diag, const T *edge, T *factor,
                      double *logdet, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (!diag || !edge || !logdet) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge) || misaligned(factor)) return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::tree_factor_workspace_bytes(plan);
  if (ws_bytes < need || (need && !ws) || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::tree_factor_launch<T>(plan, diag, edge, factor, logdet, info, ws,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int tree_apply_entry(const selinv_tree_plan *plan, const T *edge, const T *factor, int64_t k,
                     const T *in, T *out, void *ws, size_t ws_bytes, bool sample, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T)) || k < 0)
    return SELINV_ERR_INVALID_ARG;
  if (plan->n * ((k + 15) / 16) > 0x7fffffff) return SELINV_ERR_INVALID_ARG;
  if (k == 0) return SELINV_OK;
  if (!edge || !factor || !in || !out) return SELINV_ERR_INVALID_ARG;
  if (misaligned(edge) || misaligned(factor)) return SELINV_ERR_INVALID_ARG;
  // the b > 8 sampler runs per-level launches and needs no workspace
  const size_t need = (sample && plan->b > 8) ? 0 : selinv::tree_apply_workspace_bytes(plan, k);
  if (ws_bytes < need || (need && !ws) || (need && misaligned_ws(ws)))
    return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::tree_apply_launch<T>(plan, k, sample, edge, factor, in, out, ws,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int bidiag_entry(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *G_diag,
                 T *G_lower, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (B < 0 || L < 1 || bad_b(b) || B * L > 0x7fffffff) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !G_diag || (L > 1 && (!lower || !G_lower))) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(G_diag) || (L > 1 && (misaligned(lower) || misaligned(G_lower))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::bidiag_workspace_bytes(B);
  if (ws_bytes < need || !ws || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::bidiag_launch<T>(B, L, b, diag, lower, G_diag, G_lower, info, ws,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int nonsym_tree_entry(const selinv_tree_plan *plan, const T *diag, const T *up, const T *down,
                      T *G_diag, T *G_up, T *G_down, int32_t *info, void *ws, size_t ws_bytes,
                      void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (!diag || !up || !down || !G_diag || !G_up || !G_down) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(up) || misaligned(down) || misaligned(G_diag) ||
      misaligned(G_up) || misaligned(G_down))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::nonsym_tree_workspace_bytes(plan);
  if (ws_bytes < need || !ws || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::nonsym_tree_launch<T>(plan, diag, up, down, G_diag, G_up, G_down,
                                                     info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int junction_entry(const selinv_junction_plan *plan, int64_t B, const T *diag, const T *edge_val,
                   T *G_diag, T *G_lower, double *logdet, int32_t *info, void *ws,
                   size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (B < 0 || B > 65535) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !G_diag || !logdet || (plan->m > 0 && !edge_val) || (plan->nnz > 0 && !G_lower))
    return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge_val) || misaligned(G_diag) || misaligned(G_lower))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::junction_workspace_bytes(plan, B);
  if (ws_bytes < need || !ws || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::junction_launch<T>(plan, B, diag, edge_val, G_diag, G_lower, logdet,
                                                  info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int junction_logdet_entry(const selinv_junction_plan *plan, int64_t B, const T *diag,
                          const T *edge_val, double *logdet, int32_t *info, void *ws,
                          size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (B < 0 || B > 65535) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !logdet || (plan->m > 0 && !edge_val)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge_val)) return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::junction_workspace_bytes(plan, B);
  if (ws_bytes < need || !ws || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::junction_launch<T>(plan, B, diag, edge_val, nullptr, nullptr,
                                                  logdet, info, ws,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int junction_factor_entry(const selinv_junction_plan *plan, int64_t B, const T *diag,
                          const T *edge_val, T *factor, double *logdet, int32_t *info, void *ws,
                          size_t ws_bytes, void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (B < 0 || B > 65535) return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !factor || !logdet || (plan->m > 0 && !edge_val)) return SELINV_ERR_INVALID_ARG;
  if (misaligned(diag) || misaligned(edge_val) || misaligned(factor)) return SELINV_ERR_INVALID_ARG;
  const size_t need = selinv::junction_factor_workspace_bytes(plan, B);
  if (ws_bytes < need || !ws || misaligned_ws(ws)) return SELINV_ERR_INVALID_ARG;
  const hipError_t e = selinv::junction_factor_launch<T>(plan, B, diag, edge_val, factor, logdet,
                                                         info, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

template <typename T>
int junction_apply_entry(const selinv_junction_plan *plan, int64_t B, const T *factor, int64_t k,
                         const T *in, T *out, void *ws, size_t ws_bytes, bool sample,
                         void *stream) {
  if (!plan || plan->dtype_bytes != static_cast<int>(sizeof(T))) return SELINV_ERR_INVALID_ARG;
  if (B < 0 || B > 65535 || k < 0) return SELINV_ERR_INVALID_ARG;
  if (B == 0 || k == 0) return SELINV_OK;
  if (!factor || !in || !out || in == out || misaligned(factor)) return SELINV_ERR_INVALID_ARG;
  if (!sample) {
    const size_t need = selinv::junction_solve_workspace_bytes(plan, B, k);
    if (ws_bytes < need || (need && (!ws || misaligned_ws(ws)))) return SELINV_ERR_INVALID_ARG;
  }
  const hipError_t e = selinv::junction_apply_launch<T>(plan, B, factor, k, sample, in, out, ws,
                                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

}  // namespace

extern "C" {

int selinv_junction_logdet_f64(const selinv_junction_plan *plan, int64_t B, const double *diag,
                               const double *edge_val, double *logdet, int32_t *info,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return junction_logdet_entry<double>(plan, B, diag, edge_val, logdet, info, workspace,
                                       workspace_bytes, stream);
}

int selinv_junction_logdet_f32(const selinv_junction_plan *plan, int64_t B, const float *diag,
                               const float *edge_val, double *logdet, int32_t *info,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return junction_logdet_entry<float>(plan, B, diag, edge_val, logdet, info, workspace,
                                      workspace_bytes, stream);
}

size_t selinv_junction_factor_bytes(const selinv_junction_plan *plan, int64_t B) {
  return (plan && B >= 0) ? selinv::junction_factor_bytes(plan, B) : 0;
}

size_t selinv_junction_factor_workspace_bytes(const selinv_junction_plan *plan, int64_t B) {
  return (plan && B >= 0) ? selinv::junction_factor_workspace_bytes(plan, B) : 0;
}

int selinv_junction_factor_f64(const selinv_junction_plan *plan, int64_t B, const double *diag,
                               const double *edge_val, double *factor, double *logdet,
                               int32_t *info, void *workspace, size_t workspace_bytes,
                               void *stream) {
  return junction_factor_entry<double>(plan, B, diag, edge_val, factor, logdet, info, workspace,
                                       workspace_bytes, stream);
}

int selinv_junction_factor_f32(const selinv_junction_plan *plan, int64_t B, const float *diag,
                               const float *edge_val, float *factor, double *logdet,
                               int32_t *info, void *workspace, size_t workspace_bytes,
                               void *stream) {
  return junction_factor_entry<float>(plan, B, diag, edge_val, factor, logdet, info, workspace,
                                      workspace_bytes, stream);
}

size_t selinv_junction_solve_workspace_bytes(const selinv_junction_plan *plan, int64_t B,
                                             int64_t k) {
  return (plan && B >= 0 && k >= 0) ? selinv::junction_solve_workspace_bytes(plan, B, k) : 0;
}

int selinv_junction_solve_f64(const selinv_junction_plan *plan, int64_t B, const double *factor,
                              int64_t k, const double *y, double *x, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return junction_apply_entry<double>(plan, B, factor, k, y, x, workspace, workspace_bytes, false,
                                      stream);
}

int selinv_junction_solve_f32(const selinv_junction_plan *plan, int64_t B, const float *factor,
                              int64_t k, const float *y, float *x, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return junction_apply_entry<float>(plan, B, factor, k, y, x, workspace, workspace_bytes, false,
                                     stream);
}

int selinv_junction_sample_f64(const selinv_junction_plan *plan, int64_t B, const double *factor,
                               int64_t k, const double *z, double *x, void *stream) {
  return junction_apply_entry<double>(plan, B, factor, k, z, x, nullptr, 0, true, stream);
}

int selinv_junction_sample_f32(const selinv_junction_plan *plan, int64_t B, const float *factor,
                               int64_t k, const float *z, float *x, void *stream) {
  return junction_apply_entry<float>(plan, B, factor, k, z, x, nullptr, 0, true, stream);
}

size_t selinv_junction_workspace_bytes(const selinv_junction_plan *plan, int64_t B) {
  if (!plan || B < 0) return 0;
  return selinv::junction_workspace_bytes(plan, B);
}

int selinv_junction_f64(const selinv_junction_plan *plan, int64_t B, const double *diag,
                        const double *edge_val, double *G_diag, double *G_lower, double *logdet,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream) {
  return junction_entry<double>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, workspace,
                                workspace_bytes, stream);
}

int selinv_junction_f32(const selinv_junction_plan *plan, int64_t B, const float *diag,
                        const float *edge_val, float *G_diag, float *G_lower, double *logdet,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream) {
  return junction_entry<float>(plan, B, diag, edge_val, G_diag, G_lower, logdet, info, workspace,
                               workspace_bytes, stream);
}

const char *selinv_strerror(int status) {
  switch (status) {
    case SELINV_OK: return "ok";
    case SELINV_ERR_INVALID_ARG: return "invalid argument (pointer, size, block size or workspace)";
    case SELINV_ERR_BAD_TREE: return "parent array is not a single rooted tree";
    case SELINV_ERR_HIP: return "HIP runtime or kernel launch error";
    case SELINV_ERR_BAD_PATTERN: return "invalid junction pattern or elimination order";
    case SELINV_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the static scratch array holds";
    case SELINV_ERR_WAIT_TIMEOUT:
      return "a bounded wait of the single-launch tree schedule expired (info = -1)";
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

int selinv_tree_graph_create_f64(const selinv_tree_plan *plan, const double *diag,
                                 const double *edge, double *G_diag, double *G_edge,
                                 double *logdet, int32_t *info, void *workspace,
                                 size_t workspace_bytes, selinv_tree_graph **out) {
  return tree_graph_create<double>(plan, diag, edge, G_diag, G_edge, logdet, info, workspace,
                                   workspace_bytes, out);
}

int selinv_tree_graph_create_f32(const selinv_tree_plan *plan, const float *diag,
                                 const float *edge, float *G_diag, float *G_edge,
                                 double *logdet, int32_t *info, void *workspace,
                                 size_t workspace_bytes, selinv_tree_graph **out) {
  return tree_graph_create<float>(plan, diag, edge, G_diag, G_edge, logdet, info, workspace,
                                  workspace_bytes, out);
}

int selinv_tree_graph_launch(const selinv_tree_graph *graph, void *stream) {
  if (!graph) return SELINV_ERR_INVALID_ARG;
  return hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SELINV_OK
             : SELINV_ERR_HIP;
}

void selinv_set_wait_limit(uint64_t ticks) {
  selinv::g_wait_ticks.store(ticks, std::memory_order_relaxed);
}

uint64_t selinv_wait_limit(void) { return selinv::wait_limit_ticks(); }

int64_t selinv_tree_graph_nodes(const selinv_tree_graph *graph) {
  return graph ? graph->nodes : -1;
}

void selinv_tree_graph_destroy(selinv_tree_graph *graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
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

size_t selinv_chain_factor_bytes(int dtype_bytes, int64_t B, int64_t L, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || L < 1 || bad_b(b)) return 0;
  return selinv::chain_factor_bytes(dtype_bytes, B, L, b);
}

size_t selinv_star_factor_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || K < 0 || bad_b(b)) return 0;
  return selinv::star_factor_bytes(dtype_bytes, B, K, b);
}

size_t selinv_star_factor_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || K < 0 || bad_b(b)) return 0;
  return selinv::star_factor_workspace_bytes(dtype_bytes, B, K, b);
}

size_t selinv_star_solve_workspace_bytes(int dtype_bytes, int64_t B, int64_t K, int32_t b,
                                         int64_t k) {
  if ((dtype_bytes != 4 && dtype_bytes != 8) || B < 0 || K < 0 || bad_b(b) || k < 0) return 0;
  return selinv::star_apply_workspace_bytes(dtype_bytes, B, K, b, k);
}

size_t selinv_tree_factor_bytes(const selinv_tree_plan *plan) {
  return plan ? selinv::tree_factor_bytes(plan) : 0;
}

size_t selinv_tree_factor_workspace_bytes(const selinv_tree_plan *plan) {
  return plan ? selinv::tree_factor_workspace_bytes(plan) : 0;
}

size_t selinv_tree_solve_workspace_bytes(const selinv_tree_plan *plan, int64_t k) {
  return (plan && k >= 0) ? selinv::tree_apply_workspace_bytes(plan, k) : 0;
}

int selinv_chain_factor_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                            const double *lower, double *factor, double *logdet, int32_t *info,
                            void *stream) {
  return chain_factor_entry<double>(B, L, b, diag, lower, factor, logdet, info, stream);
}

int selinv_chain_solve_f64(int64_t B, int64_t L, int32_t b, const double *lower, const double *factor,
                           int64_t k, const double *y, double *x, void *stream) {
  return chain_apply_entry<double>(B, L, b, lower, factor, k, y, x, false, stream);
}

int selinv_chain_sample_f64(int64_t B, int64_t L, int32_t b, const double *lower, const double *factor,
                            int64_t k, const double *z, double *x, void *stream) {
  return chain_apply_entry<double>(B, L, b, lower, factor, k, z, x, true, stream);
}

int selinv_star_factor_f64(int64_t B, int64_t K, int32_t b, const double *center, const double *leaves,
                           const double *coupling, double *factor, double *logdet, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return star_factor_entry<double>(B, K, b, center, leaves, coupling, factor, logdet, info,
                                workspace, workspace_bytes, stream);
}

int selinv_star_solve_f64(int64_t B, int64_t K, int32_t b, const double *coupling, const double *factor,
                          int64_t k, const double *y_center, const double *y_leaves, double *x_center,
                          double *x_leaves, void *workspace, size_t workspace_bytes, void *stream) {
  return star_apply_entry<double>(B, K, b, coupling, factor, k, y_center, y_leaves, x_center,
                               x_leaves, workspace, workspace_bytes, false, stream);
}

int selinv_star_sample_f64(int64_t B, int64_t K, int32_t b, const double *coupling,
                           const double *factor, int64_t k, const double *z_center, const double *z_leaves,
                           double *x_center, double *x_leaves, void *stream) {
  return star_apply_entry<double>(B, K, b, coupling, factor, k, z_center, z_leaves, x_center,
                               x_leaves, nullptr, 0, true, stream);
}

int selinv_tree_factor_f64(const selinv_tree_plan *plan, const double *diag, const double *edge,
                           double *factor, double *logdet, int32_t *info, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return tree_factor_entry<double>(plan, diag, edge, factor, logdet, info, workspace,
                                workspace_bytes, stream);
}

int selinv_tree_solve_f64(const selinv_tree_plan *plan, const double *edge, const double *factor,
                          int64_t k, const double *y, double *x, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return tree_apply_entry<double>(plan, edge, factor, k, y, x, workspace, workspace_bytes, false,
                               stream);
}

int selinv_tree_sample_f64(const selinv_tree_plan *plan, const double *edge, const double *factor,
                           int64_t k, const double *z, double *x, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return tree_apply_entry<double>(plan, edge, factor, k, z, x, workspace, workspace_bytes, true,
                              stream);
}

int selinv_chain_factor_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                            const float *lower, float *factor, double *logdet, int32_t *info,
                            void *stream) {
  return chain_factor_entry<float>(B, L, b, diag, lower, factor, logdet, info, stream);
}

int selinv_chain_solve_f32(int64_t B, int64_t L, int32_t b, const float *lower, const float *factor,
                           int64_t k, const float *y, float *x, void *stream) {
  return chain_apply_entry<float>(B, L, b, lower, factor, k, y, x, false, stream);
}

int selinv_chain_sample_f32(int64_t B, int64_t L, int32_t b, const float *lower, const float *factor,
                            int64_t k, const float *z, float *x, void *stream) {
  return chain_apply_entry<float>(B, L, b, lower, factor, k, z, x, true, stream);
}

int selinv_star_factor_f32(int64_t B, int64_t K, int32_t b, const float *center, const float *leaves,
                           const float *coupling, float *factor, double *logdet, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return star_factor_entry<float>(B, K, b, center, leaves, coupling, factor, logdet, info,
                                workspace, workspace_bytes, stream);
}

int selinv_star_solve_f32(int64_t B, int64_t K, int32_t b, const float *coupling, const float *factor,
                          int64_t k, const float *y_center, const float *y_leaves, float *x_center,
                          float *x_leaves, void *workspace, size_t workspace_bytes, void *stream) {
  return star_apply_entry<float>(B, K, b, coupling, factor, k, y_center, y_leaves, x_center,
                               x_leaves, workspace, workspace_bytes, false, stream);
}

int selinv_star_sample_f32(int64_t B, int64_t K, int32_t b, const float *coupling,
                           const float *factor, int64_t k, const float *z_center, const float *z_leaves,
                           float *x_center, float *x_leaves, void *stream) {
  return star_apply_entry<float>(B, K, b, coupling, factor, k, z_center, z_leaves, x_center,
                               x_leaves, nullptr, 0, true, stream);
}

int selinv_tree_factor_f32(const selinv_tree_plan *plan, const float *diag, const float *edge,
                           float *factor, double *logdet, int32_t *info, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return tree_factor_entry<float>(plan, diag, edge, factor, logdet, info, workspace,
                                workspace_bytes, stream);
}

int selinv_tree_solve_f32(const selinv_tree_plan *plan, const float *edge, const float *factor,
                          int64_t k, const float *y, float *x, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return tree_apply_entry<float>(plan, edge, factor, k, y, x, workspace, workspace_bytes, false,
                               stream);
}

int selinv_tree_sample_f32(const selinv_tree_plan *plan, const float *edge, const float *factor,
                           int64_t k, const float *z, float *x, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return tree_apply_entry<float>(plan, edge, factor, k, z, x, workspace, workspace_bytes, true,
                              stream);
}

size_t selinv_bidiag_workspace_bytes(int64_t B) {
  return B < 0 ? 0 : selinv::bidiag_workspace_bytes(B);
}

size_t selinv_nonsym_tree_workspace_bytes(const selinv_tree_plan *plan) {
  return plan ? selinv::nonsym_tree_workspace_bytes(plan) : 0;
}

int selinv_bidiag_f64(int64_t B, int64_t L, int32_t b, const double *diag, const double *lower,
                      double *G_diag, double *G_lower, int32_t *info, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return bidiag_entry<double>(B, L, b, diag, lower, G_diag, G_lower, info, workspace,
                           workspace_bytes, stream);
}

int selinv_nonsym_tree_f64(const selinv_tree_plan *plan, const double *diag, const double *up,
                           const double *down, double *G_diag, double *G_up, double *G_down, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return nonsym_tree_entry<double>(plan, diag, up, down, G_diag, G_up, G_down, info, workspace,
                                workspace_bytes, stream);
}

int selinv_bidiag_f32(int64_t B, int64_t L, int32_t b, const float *diag, const float *lower,
                      float *G_diag, float *G_lower, int32_t *info, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return bidiag_entry<float>(B, L, b, diag, lower, G_diag, G_lower, info, workspace,
                           workspace_bytes, stream);
}

int selinv_nonsym_tree_f32(const selinv_tree_plan *plan, const float *diag, const float *up,
                           const float *down, float *G_diag, float *G_up, float *G_down, int32_t *info,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return nonsym_tree_entry<float>(plan, diag, up, down, G_diag, G_up, G_down, info, workspace,
                                workspace_bytes, stream);
}

}  // extern "C"
