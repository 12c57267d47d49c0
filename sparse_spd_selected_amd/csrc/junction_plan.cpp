// junction_plan.cpp -- host-side symbolic analysis for the general sparse SPD
// selected inverse (the junction-tree section of the gabp-sparse-inv page).
//
// An arbitrary block pattern is eliminated node by node in an elimination
// order (default: greedy minimum degree, the smallest label on ties).
// Eliminating v joins its remaining neighbours into a clique, so the pattern
// grows to its chordal completion S; the later neighbours N(v) of v are the
// row structure of column v of the block factor.  The numeric work then
// runs over the levels of the elimination tree (parent(v) = the earliest
// node of N(v)): a node's level is one more than the highest level among its
// children, so every node of a level depends only on lower levels in the
// factorisation and only on higher levels in the Takahashi pass -- the
// level-set schedule the page describes for the batched path (its height is
// about sqrt(n) on a 2-D grid).
//
// The plan renumbers the nodes level by level (elimination position within
// a level) and precomputes every index the kernels need, so that a kernel
// only follows flat integer tables:
//   * W slots: column v's blocks (w, v), w in N(v), contiguous, rows in
//     elimination order (the canonical orientation: later node first);
//   * forward targets: per node, the diagonal then one per slot; per target
//     the list of (W_{t,u}, W_{v,u}) pairs of its Schur update, u in
//     elimination order, and the input block it starts from;
//   * backward tables: per node, the k x k reads of G_{w,x} (w, x in N(v))
//     as positions in the caller's output arrays with a transpose bit;
//   * the output position of every slot in S_index order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "internal.h"

namespace {

using Vec = std::vector<int32_t>;

// Sorted union of a and b without the entries x and y.
void merge_without(const Vec &a, const Vec &b, int32_t x, int32_t y, Vec &out) {
  out.clear();
  size_t i = 0, j = 0;
  while (i < a.size() || j < b.size()) {
    int32_t t;
    if (j == b.size() || (i < a.size() && a[i] < b[j])) {
      t = a[i++];
    } else if (i == a.size() || b[j] < a[i]) {
      t = b[j++];
    } else {
      t = a[i++];
      ++j;
    }
    if (t != x && t != y) out.push_back(t);
  }
}

// Runs the elimination; fills order (step -> label) and nbr[step] (labels of
// the later neighbours, ascending).  Returns false for a bad order.
bool eliminate(int64_t n, std::vector<Vec> adj, const int32_t *order_in, Vec &order,
               std::vector<Vec> &nbr) {
  order.assign(n, -1);
  nbr.assign(n, Vec());
  std::vector<char> gone(n, 0);
  std::set<std::pair<int64_t, int32_t>> queue;  // (degree, label)
  if (!order_in)
    for (int64_t v = 0; v < n; ++v) queue.insert({static_cast<int64_t>(adj[v].size()), int32_t(v)});
  Vec merged;
  for (int64_t s = 0; s < n; ++s) {
    int32_t v;
    if (order_in) {
      v = order_in[s];
      if (v < 0 || v >= n || gone[v]) return false;
    } else {
      v = queue.begin()->second;
      queue.erase(queue.begin());
    }
    gone[v] = 1;
    order[s] = v;
    const Vec nb = adj[v];
    for (int32_t a : nb) {
      if (!order_in) queue.erase({static_cast<int64_t>(adj[a].size()), a});
      merge_without(adj[a], nb, a, v, merged);
      adj[a].swap(merged);
      if (!order_in) queue.insert({static_cast<int64_t>(adj[a].size()), a});
    }
    nbr[s] = nb;
    Vec().swap(adj[v]);
  }
  return true;
}


// Everything the symbolic analysis produces (host memory).
struct HostTables {
  int64_t n = 0, nnz = 0, npairs = 0, ntg = 0, ng = 0;
  int32_t L = 0;
  Vec order, S_index, node_label, node_pos, slot_node, outenc, tgt_node, ain, fpair, gtab;
  std::vector<int64_t> level_off, colptr, fptr, gptr;
};

// Symbolic analysis; with tables == false only the order, S and the levels.
int analyze(int64_t n, int64_t m, const int32_t *edge_index_host, const int32_t *order_host,
            bool tables, HostTables &h) {
  // ---- pattern: adjacency lists, validated
  std::vector<Vec> adj(n);
  std::unordered_map<int64_t, int32_t> edge_of;
  edge_of.reserve(static_cast<size_t>(m) * 2 + 1);
  for (int64_t e = 0; e < m; ++e) {
    const int64_t i = edge_index_host[e], j = edge_index_host[m + e];
    if (j < 0 || i <= j || i >= n) return SELINV_ERR_BAD_PATTERN;
    if (!edge_of.emplace(i * n + j, static_cast<int32_t>(e)).second) return SELINV_ERR_BAD_PATTERN;
    adj[i].push_back(static_cast<int32_t>(j));
    adj[j].push_back(static_cast<int32_t>(i));
  }
  for (auto &a : adj) std::sort(a.begin(), a.end());

  Vec order;
  std::vector<Vec> nbr;
  if (!eliminate(n, std::move(adj), order_host, order, nbr)) return SELINV_ERR_BAD_PATTERN;
  h.n = n;

  Vec epos(n);  // label -> elimination position
  for (int64_t s = 0; s < n; ++s) epos[order[s]] = static_cast<int32_t>(s);

  // ---- elimination tree levels (children come earlier in the order)
  Vec level(n, 0);  // by position
  int32_t H = 0;
  for (int64_t s = 0; s < n; ++s) {
    int32_t par = -1;
    for (int32_t w : nbr[s]) par = par < 0 ? epos[w] : std::min(par, epos[w]);
    if (par >= 0) level[par] = std::max(level[par], level[s] + 1);
    H = std::max(H, level[s]);
  }
  const int32_t L = H + 1;

  // ---- node ids: by level, then elimination position
  Vec id_of_pos(n), pos_of_id(n);
  std::vector<int64_t> level_off(L + 1, 0);
  for (int64_t s = 0; s < n; ++s) level_off[level[s] + 1]++;
  for (int32_t l = 0; l < L; ++l) level_off[l + 1] += level_off[l];
  {
    std::vector<int64_t> next(level_off.begin(), level_off.end() - 1);
    for (int64_t s = 0; s < n; ++s) {
      const int64_t p = next[level[s]]++;
      id_of_pos[s] = static_cast<int32_t>(p);
      pos_of_id[p] = static_cast<int32_t>(s);
    }
  }

  // ---- W slots by node id; rows (as positions) ascending
  std::vector<int64_t> colptr(n + 1, 0);
  for (int64_t p = 0; p < n; ++p) colptr[p + 1] = colptr[p] + nbr[pos_of_id[p]].size();
  const int64_t nnz = colptr[n];
  if (nnz >= (int64_t(1) << 30)) return SELINV_ERR_INVALID_ARG;
  Vec rowpos(nnz), slot_node(nnz);
  for (int64_t p = 0; p < n; ++p) {
    const Vec &nb = nbr[pos_of_id[p]];
    int64_t k = colptr[p];
    for (int32_t w : nb) rowpos[k++] = epos[w];
    std::sort(rowpos.begin() + colptr[p], rowpos.begin() + colptr[p + 1]);
    for (int64_t t = colptr[p]; t < colptr[p + 1]; ++t) slot_node[t] = static_cast<int32_t>(p);
  }
  // slot of block (w, v) given positions, w later than v
  auto slot_of = [&](int32_t wpos, int32_t vpos) -> int64_t {
    const int64_t p = id_of_pos[vpos];
    const auto b0 = rowpos.begin() + colptr[p], b1 = rowpos.begin() + colptr[p + 1];
    const auto it = std::lower_bound(b0, b1, wpos);
    return (it == b1 || *it != wpos) ? -1 : colptr[p] + (it - rowpos.begin() - colptr[p]);
  };

  // ---- output positions: S_index sorted by (i, j), i > j labels
  std::vector<int64_t> by_out(nnz);
  for (int64_t t = 0; t < nnz; ++t) by_out[t] = t;
  auto lab_pair = [&](int64_t t) {
    const int32_t w = order[rowpos[t]], v = order[pos_of_id[slot_node[t]]];
    return std::make_pair(std::max(w, v), std::min(w, v));
  };
  std::sort(by_out.begin(), by_out.end(),
            [&](int64_t a, int64_t c) { return lab_pair(a) < lab_pair(c); });
  Vec outenc(nnz);        // output position * 2 + (stored transposed)
  Vec S_index(2 * nnz);
  for (int64_t k = 0; k < nnz; ++k) {
    const int64_t t = by_out[k];
    const int32_t w = order[rowpos[t]], v = order[pos_of_id[slot_node[t]]];
    outenc[t] = static_cast<int32_t>(k * 2 + (w < v ? 1 : 0));
    S_index[k] = std::max(w, v);
    S_index[nnz + k] = std::min(w, v);
  }

  h.order = order;
  h.S_index.swap(S_index);
  h.level_off = level_off;
  h.colptr = colptr;
  h.nnz = nnz;
  h.L = L;
  if (!tables) return SELINV_OK;

  // ---- forward targets: per node id the diagonal, then one per slot
  const int64_t ntg = nnz + n;
  Vec tgt_node(ntg), ain(ntg);
  for (int64_t p = 0; p < n; ++p) {
    const int64_t t0 = colptr[p] + p;
    const int32_t v = order[pos_of_id[p]];
    tgt_node[t0] = static_cast<int32_t>(p);
    ain[t0] = v;
    for (int64_t t = colptr[p]; t < colptr[p + 1]; ++t) {
      const int64_t tg = t0 + 1 + (t - colptr[p]);
      tgt_node[tg] = static_cast<int32_t>(p);
      const int32_t w = order[rowpos[t]];
      const auto it = edge_of.find(int64_t(std::max(w, v)) * n + std::min(w, v));
      ain[tg] = it == edge_of.end() ? -1 : it->second * 2 + (w < v ? 1 : 0);
    }
  }
  auto target_of = [&](int32_t tpos, int32_t vpos) -> int64_t {  // t later than or equal to v
    const int64_t p = id_of_pos[vpos];
    if (tpos == vpos) return colptr[p] + p;
    const int64_t s = slot_of(tpos, vpos);
    return s < 0 ? -1 : colptr[p] + p + 1 + (s - colptr[p]);
  };
  // pairs: two passes over u in elimination order (count, then fill)
  std::vector<int64_t> fptr(ntg + 1, 0);
  for (int pass = 0; pass < 2; ++pass) {
    std::vector<int64_t> fillp;
    if (pass == 1) fillp.assign(fptr.begin(), fptr.end() - 1);
    for (int64_t s = 0; s < n; ++s) {
      const int64_t pu = id_of_pos[s];
      for (int64_t i2 = colptr[pu]; i2 < colptr[pu + 1]; ++i2)    // v = rowpos[i2]
        for (int64_t i1 = i2; i1 < colptr[pu + 1]; ++i1) {        // t = rowpos[i1] >= v
          const int64_t tg = target_of(rowpos[i1], rowpos[i2]);
          if (tg < 0) return SELINV_ERR_BAD_PATTERN;               // not chordal: cannot happen
          if (pass == 0)
            fptr[tg + 1]++;
          else
            fillp[tg]++;
        }
    }
    if (pass == 0) {
      for (int64_t tg = 0; tg < ntg; ++tg) fptr[tg + 1] += fptr[tg];
    }
  }
  const int64_t npairs = fptr[ntg];
  if (npairs >= (int64_t(1) << 31)) return SELINV_ERR_INVALID_ARG;
  std::vector<int32_t> fpair(2 * npairs);
  {
    std::vector<int64_t> fillp(fptr.begin(), fptr.end() - 1);
    for (int64_t s = 0; s < n; ++s) {
      const int64_t pu = id_of_pos[s];
      for (int64_t i2 = colptr[pu]; i2 < colptr[pu + 1]; ++i2)
        for (int64_t i1 = i2; i1 < colptr[pu + 1]; ++i1) {
          const int64_t tg = target_of(rowpos[i1], rowpos[i2]);
          const int64_t q = fillp[tg]++;
          fpair[2 * q] = static_cast<int32_t>(i1);      // W_{t,u}
          fpair[2 * q + 1] = static_cast<int32_t>(i2);  // W_{v,u}
        }
    }
  }

  // ---- backward tables: per node id, k x k encoded reads of G_{w,x}
  std::vector<int64_t> gptr(n + 1, 0);
  for (int64_t p = 0; p < n; ++p) {
    const int64_t k = colptr[p + 1] - colptr[p];
    gptr[p + 1] = gptr[p] + k * k;
  }
  const int64_t ng = gptr[n];
  Vec gtab(ng);
  for (int64_t p = 0; p < n; ++p) {
    const int64_t c0 = colptr[p], k = colptr[p + 1] - c0;
    for (int64_t a = 0; a < k; ++a)
      for (int64_t c = 0; c < k; ++c) {
        const int32_t wp = rowpos[c0 + a], xp = rowpos[c0 + c];
        int32_t enc;
        if (a == c) {
          enc = -(order[wp] + 1);                       // G_diag of w
        } else {
          const bool w_later = a > c;
          const int64_t s = w_later ? slot_of(wp, xp) : slot_of(xp, wp);
          if (s < 0) return SELINV_ERR_BAD_PATTERN;
          const int32_t o = outenc[s];
          // the slot's canonical block is G_{w,x} (w later) or G_{x,w};
          // the output holds the canonical block transposed when o & 1
          const int flip = (o & 1) ^ (w_later ? 0 : 1);
          enc = (o & ~1) | flip;
        }
        gtab[gptr[p] + a * k + c] = enc;
      }
  }

  h.ntg = ntg;
  h.npairs = npairs;
  h.ng = ng;
  h.node_label.resize(n);
  h.node_pos.resize(n);
  for (int64_t p = 0; p < n; ++p) {
    h.node_pos[p] = pos_of_id[p];
    h.node_label[p] = order[pos_of_id[p]];
  }
  h.slot_node.swap(slot_node);
  h.outenc.swap(outenc);
  h.tgt_node.swap(tgt_node);
  h.ain.swap(ain);
  h.fpair.swap(fpair);
  h.gtab.swap(gtab);
  h.fptr.swap(fptr);
  h.gptr.swap(gptr);
  return SELINV_OK;
}

}  // namespace

extern "C" int selinv_junction_plan_create(int64_t n, int64_t m, const int32_t *edge_index_host,
                                           const int32_t *order_host, int32_t b, int dtype_bytes,
                                           void *stream, selinv_junction_plan **out) {
  if (!out) return SELINV_ERR_INVALID_ARG;
  *out = nullptr;
  if (n < 1 || n > (int64_t(1) << 24) || m < 0 || (m > 0 && !edge_index_host) || b < 1 ||
      b > SELINV_MAX_B || (dtype_bytes != 4 && dtype_bytes != 8))
    return SELINV_ERR_INVALID_ARG;
  HostTables h;
  const int rc = analyze(n, m, edge_index_host, order_host, true, h);
  if (rc != SELINV_OK) return rc;
  const int64_t nnz = h.nnz, ntg = h.ntg, npairs = h.npairs, ng = h.ng;
  const int32_t L = h.L;

  // ---- plan object and device tables
  selinv_junction_plan *plan = new (std::nothrow) selinv_junction_plan();
  if (!plan) return SELINV_ERR_HIP;
  plan->n = n;
  plan->m = m;
  plan->b = b;
  plan->dtype_bytes = dtype_bytes;
  plan->nnz = nnz;
  plan->levels = L;
  plan->npairs = npairs;
  plan->level_off = h.level_off;
  plan->colptr_host = h.colptr;
  plan->S_index.swap(h.S_index);
  plan->order.swap(h.order);
  int64_t maxk = 0;
  for (int64_t p = 0; p < n; ++p) maxk = std::max(maxk, h.colptr[p + 1] - h.colptr[p]);
  plan->max_k = maxk;

  Vec colptr32(n + 1), fptr32(ntg + 1);
  for (int64_t p = 0; p <= n; ++p) colptr32[p] = static_cast<int32_t>(h.colptr[p]);
  for (int64_t t = 0; t <= ntg; ++t) fptr32[t] = static_cast<int32_t>(h.fptr[t]);

  const size_t i4 = sizeof(int32_t);
  const size_t bytes = selinv::align_up((n + 1) * i4) + 2 * selinv::align_up(n * i4) +
                       selinv::align_up(n * i4) + 2 * selinv::align_up(ntg * i4) +
                       selinv::align_up((ntg + 1) * i4) + selinv::align_up(2 * npairs * i4) +
                       2 * selinv::align_up(nnz * i4) + selinv::align_up((n + 1) * 8) +
                       selinv::align_up(ng * i4) + 4096;
  if (hipMalloc(&plan->dev_block, bytes) != hipSuccess) {
    delete plan;
    return SELINV_ERR_HIP;
  }
  selinv::Carve cv(plan->dev_block);
  selinv::JunctionPlanDev &dv = plan->dev;
  dv.colptr = cv.take<int32_t>(n + 1);
  dv.node_label = cv.take<int32_t>(n);
  dv.node_pos = cv.take<int32_t>(n);
  dv.order = cv.take<int32_t>(n);
  dv.tgt_node = cv.take<int32_t>(ntg);
  dv.ain = cv.take<int32_t>(ntg);
  dv.fptr = cv.take<int32_t>(ntg + 1);
  dv.fpair = cv.take<int32_t>(2 * npairs);
  dv.slot_node = cv.take<int32_t>(nnz);
  dv.outenc = cv.take<int32_t>(nnz);
  dv.gptr = cv.take<int64_t>(n + 1);
  dv.gtab = cv.take<int32_t>(ng);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  auto up = [&](void *dst, const void *src, size_t nbytes) {
    if (e == hipSuccess && nbytes) e = hipMemcpyAsync(dst, src, nbytes, hipMemcpyHostToDevice, st);
  };
  up(dv.colptr, colptr32.data(), (n + 1) * i4);
  up(dv.node_label, h.node_label.data(), n * i4);
  up(dv.node_pos, h.node_pos.data(), n * i4);
  up(dv.order, plan->order.data(), n * i4);
  up(dv.tgt_node, h.tgt_node.data(), ntg * i4);
  up(dv.ain, h.ain.data(), ntg * i4);
  up(dv.fptr, fptr32.data(), (ntg + 1) * i4);
  up(dv.fpair, h.fpair.data(), 2 * npairs * i4);
  up(dv.slot_node, h.slot_node.data(), nnz * i4);
  up(dv.outenc, h.outenc.data(), nnz * i4);
  up(dv.gptr, h.gptr.data(), (n + 1) * 8);
  up(dv.gtab, h.gtab.data(), ng * i4);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    selinv_junction_plan_destroy(plan);
    return SELINV_ERR_HIP;
  }
  *out = plan;
  return SELINV_OK;
}

extern "C" void selinv_junction_plan_destroy(selinv_junction_plan *plan) {
  if (!plan) return;
  if (plan->dev_block) (void)hipFree(plan->dev_block);
  delete plan;
}

extern "C" int64_t selinv_junction_plan_nnz(const selinv_junction_plan *plan) {
  return plan ? plan->nnz : -1;
}

extern "C" int32_t selinv_junction_plan_levels(const selinv_junction_plan *plan) {
  return plan ? plan->levels : -1;
}

extern "C" int selinv_junction_plan_pattern(const selinv_junction_plan *plan,
                                            int32_t *S_index_host, int32_t *order_host) {
  if (!plan) return SELINV_ERR_INVALID_ARG;
  if (S_index_host && plan->nnz)
    std::memcpy(S_index_host, plan->S_index.data(), 2 * plan->nnz * sizeof(int32_t));
  if (order_host) std::memcpy(order_host, plan->order.data(), plan->n * sizeof(int32_t));
  return SELINV_OK;
}

extern "C" int selinv_junction_symbolic(int64_t n, int64_t m, const int32_t *edge_index_host,
                                        const int32_t *order_host, int64_t *nnz_out,
                                        int32_t *levels_out, int32_t *S_index_host, int64_t cap,
                                        int32_t *order_out) {
  if (n < 1 || n > (int64_t(1) << 24) || m < 0 || (m > 0 && !edge_index_host))
    return SELINV_ERR_INVALID_ARG;
  HostTables h;
  const int rc = analyze(n, m, edge_index_host, order_host, false, h);
  if (rc != SELINV_OK) return rc;
  if (nnz_out) *nnz_out = h.nnz;
  if (levels_out) *levels_out = h.L;
  if (S_index_host && cap >= h.nnz && h.nnz)
    std::memcpy(S_index_host, h.S_index.data(), 2 * h.nnz * sizeof(int32_t));
  if (order_out) std::memcpy(order_out, h.order.data(), n * sizeof(int32_t));
  return SELINV_OK;
}
