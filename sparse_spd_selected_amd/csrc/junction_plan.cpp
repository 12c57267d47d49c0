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
// Supernodes.  Consecutive columns j, j+1 of the elimination form a
// supernode when j+1 is j's parent and j's other later neighbours are
// exactly j+1's; the factor's columns there share one dense structure.  The
// plan cuts supernodes into chunks of at most s_max columns (s_max b <= 48,
// so that a chunk's dense pivot fits in LDS) and the numeric work treats a
// chunk as one fat node: its pivot is the dense (s b) x (s b) block, its
// later rows N_J are the later neighbours of its last column.  The schedule
// is the level sets of the chunk tree, much shorter than the node-level one
// where supernodes are long.
//
// Tables (chunk ids level by level, then by position):
//   * panels: chunk J's factor columns as (s + n_J) x s blocks, row-major
//     by block, rows = the chunk's own columns then N_J in elimination
//     order; only blocks on or below the block diagonal are used;
//   * forward targets: every used panel block; per target the list of
//     (W_{t,u}, W_{v,u}) panel blocks of its Schur update over the earlier
//     columns u outside the chunk, u in elimination order, and the input
//     block it starts from; long lists are cut into work items of at most
//     64 pairs whose partial sums are added in order;
//   * backward: per chunk the n_J x n_J reads of G_{w,x} (w, x in N_J) as
//     positions in the caller's output arrays with a transpose bit, and the
//     output code of every panel block.
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
  int64_t n = 0, nnz = 0, nch = 0, ntg = 0, npairs = 0, nrows = 0, npanel = 0, nrinv = 0, ng = 0;
  int32_t node_levels = 0, levels = 0, smax = 0;
  Vec order, S_index;
  std::vector<int64_t> level_off;     // chunk-id range of every level
  // chunk tables (by chunk id)
  Vec ch_first, ch_s, ch_n;
  std::vector<int64_t> ch_pbase, ch_rbase, ch_gptr, ch_tptr, rows_ptr, ch_cptr, tiles_ptr;
  Vec row_chunk, col_chunk, tile_chunk, tg_chunk, tg_rc, ain, fpair, gtab, poutenc;
  // solve sweeps: the label of every flat row, and per flat column the flat
  // rows whose node is that column's node (in flat-row order)
  Vec row_node, occ_ptr, occ_row;
  // single-launch solve: per chunk, the chunks it waits for in the forward
  // sweep (fdep: those whose later rows hold its nodes) and in the backward
  // sweep (bdep: those that hold the nodes of its later rows)
  Vec fdep_ptr, fdep, bdep_ptr, bdep;
  // ... and the workgroups ("parts") each chunk is split over: part_off
  // (prefix over chunks), the chunk of every part, and the prefix over
  // chunks of the parts of split chunks (slots for partial sums)
  Vec part_off, part_chunk, split_off;
  std::vector<int64_t> fptr;
  // Schur-sum work items: each target's pair list cut into runs of at most
  // kItemPairs; targets with several items add partial sums (slots)
  std::vector<int64_t> it_ptr, multi_off;
  Vec it_tg, it_lo, it_hi, it_slot, multi_tg;
  int64_t nitems = 0, max_slots = 0;
};

constexpr int64_t kItemPairs = 64;

// Symbolic analysis.  With tables == false: the order, S and the height of
// the elimination tree only; else also the supernode chunks (at most
// `smax` columns each) and every table of the numeric kernels.
int analyze(int64_t n, int64_t m, const int32_t *edge_index_host, const int32_t *order_host,
            int32_t smax, int32_t tile_rows, bool tables, HostTables &h) {
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
  // later neighbours as positions, ascending
  std::vector<Vec> np(n);
  int64_t nnz = 0;
  for (int64_t s = 0; s < n; ++s) {
    for (int32_t w : nbr[s]) np[s].push_back(epos[w]);
    std::sort(np[s].begin(), np[s].end());
    nnz += np[s].size();
  }
  std::vector<Vec>().swap(nbr);
  if (nnz >= (int64_t(1) << 29)) return SELINV_ERR_INVALID_ARG;

  // ---- height of the elimination tree (children come earlier)
  {
    Vec level(n, 0);
    int32_t H = 0;
    for (int64_t s = 0; s < n; ++s) {
      if (!np[s].empty()) level[np[s][0]] = std::max(level[np[s][0]], level[s] + 1);
      H = std::max(H, level[s]);
    }
    h.node_levels = H + 1;
  }

  // ---- S_index (pairs i > j by label, sorted) and the output code of every
  // block (w, v) of S, w later: position * 2 + (stored transposed)
  std::vector<std::pair<std::pair<int32_t, int32_t>, int64_t>> pairs;
  pairs.reserve(nnz);
  for (int64_t s = 0; s < n; ++s)
    for (int32_t wp : np[s]) {
      const int32_t w = order[wp], v = order[s];
      pairs.push_back({{std::max(w, v), std::min(w, v)}, int64_t(wp) * n + s});
    }
  std::sort(pairs.begin(), pairs.end());
  std::unordered_map<int64_t, int32_t> out_of;  // (wpos * n + vpos) -> code
  out_of.reserve(nnz * 2 + 1);
  Vec S_index(2 * nnz);
  for (int64_t k = 0; k < nnz; ++k) {
    const int64_t key = pairs[k].second;
    const int32_t w = order[key / n], v = order[key % n];
    out_of[key] = static_cast<int32_t>(k * 2 + (w < v ? 1 : 0));
    S_index[k] = pairs[k].first.first;
    S_index[nnz + k] = pairs[k].first.second;
  }
  decltype(pairs)().swap(pairs);
  h.order = order;
  h.S_index.swap(S_index);
  h.nnz = nnz;
  if (!tables) return SELINV_OK;

  // ---- supernodes (column j+1 is j's parent and j's other later
  // neighbours are exactly j+1's), cut into chunks of at most smax columns
  std::vector<std::pair<int32_t, int32_t>> chunks;  // (first position, size)
  for (int64_t j = 0; j < n;) {
    int64_t e = j;
    while (e + 1 < n && e - j + 1 < smax && !np[e].empty() && np[e][0] == e + 1 &&
           np[e].size() == np[e + 1].size() + 1 &&
           std::equal(np[e].begin() + 1, np[e].end(), np[e + 1].begin()))
      ++e;
    chunks.push_back({static_cast<int32_t>(j), static_cast<int32_t>(e - j + 1)});
    j = e + 1;
  }
  const int64_t nch = static_cast<int64_t>(chunks.size());
  Vec chunk_of(n);  // position -> chunk (in position order)
  for (int64_t c = 0; c < nch; ++c)
    for (int32_t j = 0; j < chunks[c].second; ++j) chunk_of[chunks[c].first + j] = int32_t(c);
  // the later rows of a chunk: the later neighbours of its last column
  auto below = [&](int64_t c) -> const Vec & { return np[chunks[c].first + chunks[c].second - 1]; };
  // chunk levels (children come earlier)
  Vec clevel(nch, 0);
  int32_t CH = 0;
  for (int64_t c = 0; c < nch; ++c) {
    const Vec &N = below(c);
    if (!N.empty()) {
      const int32_t p = chunk_of[N[0]];
      clevel[p] = std::max(clevel[p], clevel[c] + 1);
    }
    CH = std::max(CH, clevel[c]);
  }
  const int32_t L = CH + 1;
  // chunk ids: by level, then position
  Vec id_of(nch), chunk_at(nch);
  std::vector<int64_t> level_off(L + 1, 0);
  for (int64_t c = 0; c < nch; ++c) level_off[clevel[c] + 1]++;
  for (int32_t l = 0; l < L; ++l) level_off[l + 1] += level_off[l];
  {
    std::vector<int64_t> next(level_off.begin(), level_off.end() - 1);
    for (int64_t c = 0; c < nch; ++c) {
      const int64_t id = next[clevel[c]]++;
      id_of[c] = static_cast<int32_t>(id);
      chunk_at[id] = static_cast<int32_t>(c);
    }
  }
  // per-id sizes and offsets
  h.ch_first.resize(nch);
  h.ch_s.resize(nch);
  h.ch_n.resize(nch);
  h.ch_pbase.assign(nch + 1, 0);
  h.ch_rbase.assign(nch + 1, 0);
  h.ch_gptr.assign(nch + 1, 0);
  h.ch_tptr.assign(nch + 1, 0);
  h.rows_ptr.assign(nch + 1, 0);
  h.ch_cptr.assign(nch + 1, 0);
  h.tiles_ptr.assign(nch + 1, 0);
  for (int64_t id = 0; id < nch; ++id) {
    const int64_t c = chunk_at[id];
    const int64_t sz = chunks[c].second, nr = static_cast<int64_t>(below(c).size());
    h.ch_first[id] = chunks[c].first;
    h.ch_s[id] = static_cast<int32_t>(sz);
    h.ch_n[id] = static_cast<int32_t>(nr);
    h.ch_pbase[id + 1] = h.ch_pbase[id] + (sz + nr) * sz;
    h.ch_rbase[id + 1] = h.ch_rbase[id] + sz * sz;
    h.ch_gptr[id + 1] = h.ch_gptr[id] + nr * nr;
    h.ch_tptr[id + 1] = h.ch_tptr[id] + sz * (sz + 1) / 2 + nr * sz;
    h.rows_ptr[id + 1] = h.rows_ptr[id] + nr;
    h.ch_cptr[id + 1] = h.ch_cptr[id] + sz;
    h.tiles_ptr[id + 1] = h.tiles_ptr[id] + (nr + tile_rows - 1) / tile_rows;
  }
  const int64_t npanel = h.ch_pbase[nch];
  if (npanel >= (int64_t(1) << 30)) return SELINV_ERR_INVALID_ARG;
  // panel block of (w, v), w at or after v, both positions, (w, v) in S or w == v
  auto panel_row = [&](int64_t id, int32_t wpos) -> int64_t {
    const int64_t c = chunk_at[id];
    const int32_t f = chunks[c].first, sz = chunks[c].second;
    if (wpos >= f && wpos < f + sz) return wpos - f;
    const Vec &N = below(c);
    const auto it = std::lower_bound(N.begin(), N.end(), wpos);
    if (it == N.end() || *it != wpos) return -1;
    return sz + (it - N.begin());
  };
  auto panel_index = [&](int32_t wpos, int32_t vpos) -> int64_t {
    const int64_t id = id_of[chunk_of[vpos]];
    const int64_t r = panel_row(id, wpos);
    if (r < 0) return -1;
    return h.ch_pbase[id] + r * h.ch_s[id] + (vpos - h.ch_first[id]);
  };
  // flat rows (chunk, a): a-th later row of the chunk
  h.row_chunk.resize(h.rows_ptr[nch]);
  for (int64_t id = 0; id < nch; ++id)
    for (int64_t r = h.rows_ptr[id]; r < h.rows_ptr[id + 1]; ++r)
      h.row_chunk[r] = static_cast<int32_t>(id);
  h.tile_chunk.resize(h.tiles_ptr[nch]);
  for (int64_t id = 0; id < nch; ++id)
    for (int64_t c = h.tiles_ptr[id]; c < h.tiles_ptr[id + 1]; ++c) h.tile_chunk[c] = int32_t(id);
  h.col_chunk.resize(n);
  for (int64_t id = 0; id < nch; ++id)
    for (int64_t c = h.ch_cptr[id]; c < h.ch_cptr[id + 1]; ++c) h.col_chunk[c] = int32_t(id);
  // output codes of every panel block: -(label + 1) on the diagonal, the S
  // code below it, -1 above
  h.poutenc.assign(npanel, -1);
  for (int64_t id = 0; id < nch; ++id) {
    const int64_t c = chunk_at[id];
    const int32_t f = chunks[c].first, sz = chunks[c].second;
    const Vec &N = below(c);
    for (int64_t r = 0; r < sz + static_cast<int64_t>(N.size()); ++r)
      for (int32_t col = 0; col < sz && col <= r; ++col) {
        const int32_t wpos = r < sz ? f + int32_t(r) : N[r - sz], vpos = f + col;
        int32_t code;
        if (wpos == vpos) {
          code = -(order[vpos] + 1);
        } else {
          const auto it = out_of.find(int64_t(wpos) * n + vpos);
          if (it == out_of.end()) return SELINV_ERR_BAD_PATTERN;  // cannot happen: S is closed
          code = it->second;
        }
        h.poutenc[h.ch_pbase[id] + r * sz + col] = code;
      }
  }
  // ---- solve sweeps: node of every flat row; flat rows by their node's
  // flat column (chunk id order, then column)
  h.row_node.resize(h.rows_ptr[nch]);
  h.occ_ptr.assign(n + 1, 0);
  auto flat_col = [&](int32_t wpos) -> int64_t {
    const int64_t c = chunk_of[wpos];
    return h.ch_cptr[id_of[c]] + (wpos - chunks[c].first);
  };
  for (int64_t id = 0; id < nch; ++id) {
    const Vec &N = below(chunk_at[id]);
    for (size_t a = 0; a < N.size(); ++a) {
      h.row_node[h.rows_ptr[id] + a] = order[N[a]];
      h.occ_ptr[flat_col(N[a]) + 1]++;
    }
  }
  for (int64_t c = 0; c < n; ++c) h.occ_ptr[c + 1] += h.occ_ptr[c];
  h.occ_row.resize(h.rows_ptr[nch]);
  {
    Vec next(h.occ_ptr.begin(), h.occ_ptr.end() - 1);
    for (int64_t id = 0; id < nch; ++id) {
      const Vec &N = below(chunk_at[id]);
      for (size_t a = 0; a < N.size(); ++a)
        h.occ_row[next[flat_col(N[a])]++] = static_cast<int32_t>(h.rows_ptr[id] + a);
    }
  }
  // ---- dependencies of the single-launch solve.  The nodes of a chunk's
  // later rows belong to its ancestors in the elimination tree, which have
  // higher chunk levels and so larger ids; fdep is the transposed relation.
  h.bdep_ptr.assign(nch + 1, 0);
  for (int64_t id = 0; id < nch; ++id) {
    int32_t last = -1;
    for (const int32_t w : below(chunk_at[id])) {  // positions ascending: chunks ascending
      const int32_t x = id_of[chunk_of[w]];
      if (x == last) continue;
      if (x <= id) return SELINV_ERR_BAD_PATTERN;  // cannot happen: ancestors come later
      h.bdep.push_back(x);
      last = x;
    }
    h.bdep_ptr[id + 1] = static_cast<int32_t>(h.bdep.size());
  }
  h.fdep_ptr.assign(nch + 1, 0);
  for (const int32_t x : h.bdep) h.fdep_ptr[x + 1]++;
  for (int64_t id = 0; id < nch; ++id) h.fdep_ptr[id + 1] += h.fdep_ptr[id];
  h.fdep.resize(h.bdep.size());
  {
    Vec next(h.fdep_ptr.begin(), h.fdep_ptr.end() - 1);
    for (int64_t id = 0; id < nch; ++id)
      for (int32_t e = h.bdep_ptr[id]; e < h.bdep_ptr[id + 1]; ++e)
        h.fdep[next[h.bdep[e]]++] = static_cast<int32_t>(id);
  }
  // Parts: a chunk whose nodes occur in many later rows (forward sum) or
  // that has many later rows (backward sum) is split over up to kMaxParts
  // workgroups, about kOccPerPart occurrences or kRowsPerPart rows each.
  {
    constexpr int64_t kMaxParts = 8, kOccPerPart = 64, kRowsPerPart = 16;
    h.part_off.assign(nch + 1, 0);
    h.split_off.assign(nch + 1, 0);
    for (int64_t id = 0; id < nch; ++id) {
      const int64_t occ = h.occ_ptr[h.ch_cptr[id] + h.ch_s[id]] - h.occ_ptr[h.ch_cptr[id]];
      const int64_t P = std::min<int64_t>(
          kMaxParts, std::max<int64_t>({1, (occ + kOccPerPart - 1) / kOccPerPart,
                                        (h.ch_n[id] + kRowsPerPart - 1) / kRowsPerPart}));
      h.part_off[id + 1] = h.part_off[id] + static_cast<int32_t>(P);
      h.split_off[id + 1] = h.split_off[id] + static_cast<int32_t>(P > 1 ? P : 0);
      for (int64_t q = 0; q < P; ++q) h.part_chunk.push_back(static_cast<int32_t>(id));
    }
  }
  // ---- forward targets: every panel block (r >= col), chunk by chunk
  const int64_t ntg = h.ch_tptr[nch];
  h.tg_chunk.resize(ntg);
  h.tg_rc.resize(ntg);
  h.ain.resize(ntg);
  for (int64_t id = 0; id < nch; ++id) {
    const int64_t c = chunk_at[id];
    const int32_t f = chunks[c].first, sz = chunks[c].second;
    const Vec &N = below(c);
    int64_t tg = h.ch_tptr[id];
    for (int32_t col = 0; col < sz; ++col)
      for (int64_t r = col; r < sz + static_cast<int64_t>(N.size()); ++r, ++tg) {
        h.tg_chunk[tg] = static_cast<int32_t>(id);
        h.tg_rc[tg] = static_cast<int32_t>(r * 64 + col);
        const int32_t wpos = r < sz ? f + int32_t(r) : N[r - sz], vpos = f + col;
        const int32_t w = order[wpos], v = order[vpos];
        if (wpos == vpos) {
          h.ain[tg] = v;
        } else {
          const auto it = edge_of.find(int64_t(std::max(w, v)) * n + std::min(w, v));
          h.ain[tg] = it == edge_of.end() ? -1 : it->second * 2 + (w < v ? 1 : 0);
        }
      }
  }
  auto target_of = [&](int32_t tpos, int32_t vpos) -> int64_t {
    const int64_t id = id_of[chunk_of[vpos]];
    const int64_t r = panel_row(id, tpos);
    if (r < 0) return -1;
    const int64_t sz = h.ch_s[id], nr = h.ch_n[id], col = vpos - h.ch_first[id];
    // targets of column col start after columns 0..col-1 (each sz + nr - col' entries)
    const int64_t before = col * (sz + nr) - col * (col - 1) / 2;
    return h.ch_tptr[id] + before + (r - col);
  };
  // Schur pairs from every column u into the targets of later chunks, u in
  // elimination order (two passes: count, then fill)
  h.fptr.assign(ntg + 1, 0);
  for (int pass = 0; pass < 2; ++pass) {
    std::vector<int64_t> fillp;
    if (pass == 1) fillp.assign(h.fptr.begin(), h.fptr.end() - 1);
    for (int64_t u = 0; u < n; ++u) {
      const Vec &N = np[u];
      for (size_t i2 = 0; i2 < N.size(); ++i2) {
        if (chunk_of[N[i2]] == chunk_of[u]) continue;  // inside the fat pivot
        for (size_t i1 = i2; i1 < N.size(); ++i1) {
          const int64_t tg = target_of(N[i1], N[i2]);
          if (tg < 0) return SELINV_ERR_BAD_PATTERN;
          if (pass == 0) {
            h.fptr[tg + 1]++;
          } else {
            const int64_t q = fillp[tg]++;
            const int64_t p1 = panel_index(N[i1], int32_t(u)), p2 = panel_index(N[i2], int32_t(u));
            if (p1 < 0 || p2 < 0) return SELINV_ERR_BAD_PATTERN;  // cannot happen: S is closed
            h.fpair[2 * q] = static_cast<int32_t>(p1);
            h.fpair[2 * q + 1] = static_cast<int32_t>(p2);
          }
        }
      }
    }
    if (pass == 0) {
      for (int64_t tg = 0; tg < ntg; ++tg) h.fptr[tg + 1] += h.fptr[tg];
      if (h.fptr[ntg] >= (int64_t(1) << 31)) return SELINV_ERR_INVALID_ARG;
      h.fpair.resize(2 * h.fptr[ntg]);
    }
  }
  // ---- backward: per chunk the n x n reads of G_{w,x}, w, x later rows
  h.gtab.resize(h.ch_gptr[nch]);
  for (int64_t id = 0; id < nch; ++id) {
    const Vec &N = below(chunk_at[id]);
    const int64_t nr = static_cast<int64_t>(N.size());
    for (int64_t a = 0; a < nr; ++a)
      for (int64_t q = 0; q < nr; ++q) {
        int32_t enc;
        if (a == q) {
          enc = -(order[N[a]] + 1);
        } else {
          const bool w_later = a > q;
          const int32_t hi = w_later ? N[a] : N[q], lo = w_later ? N[q] : N[a];
          const auto it = out_of.find(int64_t(hi) * n + lo);
          if (it == out_of.end()) return SELINV_ERR_BAD_PATTERN;
          const int32_t o = it->second;
          enc = (o & ~1) | ((o & 1) ^ (w_later ? 0 : 1));
        }
        h.gtab[h.ch_gptr[id] + a * nr + q] = enc;
      }
  }
  // ---- Schur-sum work items, level by level (targets are level-ordered)
  h.it_ptr.assign(ntg + 1, 0);
  for (int64_t tg = 0; tg < ntg; ++tg) {
    const int64_t np = h.fptr[tg + 1] - h.fptr[tg];
    h.it_ptr[tg + 1] = h.it_ptr[tg] + std::max<int64_t>(1, (np + kItemPairs - 1) / kItemPairs);
  }
  h.nitems = h.it_ptr[ntg];
  if (h.nitems >= (int64_t(1) << 31)) return SELINV_ERR_INVALID_ARG;
  h.it_tg.resize(h.nitems);
  h.it_lo.resize(h.nitems);
  h.it_hi.resize(h.nitems);
  h.it_slot.assign(h.nitems, -1);
  h.multi_off.assign(L + 1, 0);
  for (int32_t l = 0; l < L; ++l) {
    int64_t slots = 0;
    for (int64_t tg = h.ch_tptr[level_off[l]]; tg < h.ch_tptr[level_off[l + 1]]; ++tg) {
      const int64_t i0 = h.it_ptr[tg], ni = h.it_ptr[tg + 1] - i0;
      for (int64_t k = 0; k < ni; ++k) {
        h.it_tg[i0 + k] = static_cast<int32_t>(tg);
        h.it_lo[i0 + k] = static_cast<int32_t>(h.fptr[tg] + k * kItemPairs);
        h.it_hi[i0 + k] = static_cast<int32_t>(std::min(h.fptr[tg + 1], h.fptr[tg] + (k + 1) * kItemPairs));
        if (ni > 1) h.it_slot[i0 + k] = static_cast<int32_t>(slots++);
      }
      if (ni > 1) h.multi_tg.push_back(static_cast<int32_t>(tg));
    }
    h.multi_off[l + 1] = static_cast<int64_t>(h.multi_tg.size());
    h.max_slots = std::max(h.max_slots, slots);
  }
  h.nch = nch;
  h.ntg = ntg;
  h.npairs = h.fptr[ntg];
  h.nrows = h.rows_ptr[nch];
  h.npanel = npanel;
  h.nrinv = h.ch_rbase[nch];
  h.ng = h.ch_gptr[nch];
  h.levels = L;
  h.level_off = level_off;
  h.smax = smax;
  return SELINV_OK;
}

// columns per chunk: the chunk's pivot (s b x s b) and its inverse fit LDS
int32_t chunk_columns(int32_t b) { return std::max<int32_t>(1, 48 / b); }

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
  const int rc = analyze(n, m, edge_index_host, order_host, chunk_columns(b),
                         b >= 64 ? 1 : 64 / b, true, h);
  if (rc != SELINV_OK) return rc;

  selinv_junction_plan *plan = new (std::nothrow) selinv_junction_plan();
  if (!plan) return SELINV_ERR_HIP;
  plan->n = n;
  plan->m = m;
  plan->b = b;
  plan->dtype_bytes = dtype_bytes;
  plan->nnz = h.nnz;
  plan->nch = h.nch;
  plan->npanel = h.npanel;
  plan->nrinv = h.nrinv;
  plan->smax = h.smax;
  plan->levels = h.levels;
  plan->node_levels = h.node_levels;
  plan->level_off = h.level_off;
  plan->ch_tptr = h.ch_tptr;
  plan->rows_ptr = h.rows_ptr;
  plan->ch_cptr = h.ch_cptr;
  plan->tiles_ptr = h.tiles_ptr;
  plan->it_ptr = h.it_ptr;
  plan->multi_off = h.multi_off;
  plan->max_slots = h.max_slots;
  plan->nparts = h.part_off[h.nch];
  plan->nsplit = h.split_off[h.nch];
  plan->S_index.swap(h.S_index);
  plan->order.swap(h.order);

  std::vector<int32_t> fptr32(h.ntg + 1);
  for (int64_t t = 0; t <= h.ntg; ++t) fptr32[t] = static_cast<int32_t>(h.fptr[t]);
  const size_t i4 = sizeof(int32_t), i8 = sizeof(int64_t);
  using selinv::align_up;
  const size_t bytes = align_up(n * i4) + 3 * align_up(h.nch * i4) +
                       6 * align_up((h.nch + 1) * i8) + align_up(h.nrows * i4) +
                       align_up(n * i4) + align_up(h.tiles_ptr[h.nch] * i4) +
                       3 * align_up(h.ntg * i4) + align_up((h.ntg + 1) * i4) +
                       align_up(2 * h.npairs * i4) + align_up(h.ng * i4) +
                       align_up(h.npanel * i4) + 4 * align_up(h.nitems * i4) +
                       align_up(h.multi_tg.size() * i4) + align_up((h.ntg + 1) * i4) +
                       2 * align_up(h.nrows * i4) + align_up((n + 1) * i4) +
                       2 * align_up((h.nch + 1) * i4) + 2 * align_up(h.bdep.size() * i4) +
                       2 * align_up((h.nch + 1) * i4) + align_up(h.part_chunk.size() * i4) + 4096;
  if (hipMalloc(&plan->dev_block, bytes) != hipSuccess) {
    delete plan;
    return SELINV_ERR_HIP;
  }
  selinv::Carve cv(plan->dev_block);
  selinv::JunctionPlanDev &dv = plan->dev;
  dv.order = cv.take<int32_t>(n);
  dv.ch_first = cv.take<int32_t>(h.nch);
  dv.ch_s = cv.take<int32_t>(h.nch);
  dv.ch_n = cv.take<int32_t>(h.nch);
  dv.ch_pbase = cv.take<int64_t>(h.nch + 1);
  dv.ch_rbase = cv.take<int64_t>(h.nch + 1);
  dv.ch_gptr = cv.take<int64_t>(h.nch + 1);
  dv.rows_ptr = cv.take<int64_t>(h.nch + 1);
  dv.ch_cptr = cv.take<int64_t>(h.nch + 1);
  dv.row_chunk = cv.take<int32_t>(h.nrows);
  dv.col_chunk = cv.take<int32_t>(n);
  dv.tiles_ptr = cv.take<int64_t>(h.nch + 1);
  dv.tile_chunk = cv.take<int32_t>(h.tiles_ptr[h.nch]);
  dv.tg_chunk = cv.take<int32_t>(h.ntg);
  dv.tg_rc = cv.take<int32_t>(h.ntg);
  dv.ain = cv.take<int32_t>(h.ntg);
  dv.fptr = cv.take<int32_t>(h.ntg + 1);
  dv.fpair = cv.take<int32_t>(2 * h.npairs);
  dv.gtab = cv.take<int32_t>(h.ng);
  dv.poutenc = cv.take<int32_t>(h.npanel);
  dv.it_tg = cv.take<int32_t>(h.nitems);
  dv.it_lo = cv.take<int32_t>(h.nitems);
  dv.it_hi = cv.take<int32_t>(h.nitems);
  dv.it_slot = cv.take<int32_t>(h.nitems);
  dv.multi_tg = cv.take<int32_t>(h.multi_tg.size());
  dv.it_ptr = cv.take<int32_t>(h.ntg + 1);
  dv.row_node = cv.take<int32_t>(h.nrows);
  dv.occ_ptr = cv.take<int32_t>(n + 1);
  dv.occ_row = cv.take<int32_t>(h.nrows);
  dv.fdep_ptr = cv.take<int32_t>(h.nch + 1);
  dv.fdep = cv.take<int32_t>(h.fdep.size());
  dv.bdep_ptr = cv.take<int32_t>(h.nch + 1);
  dv.bdep = cv.take<int32_t>(h.bdep.size());
  dv.part_off = cv.take<int32_t>(h.nch + 1);
  dv.split_off = cv.take<int32_t>(h.nch + 1);
  dv.part_chunk = cv.take<int32_t>(h.part_chunk.size());
  std::vector<int32_t> itptr32(h.ntg + 1);
  for (int64_t t = 0; t <= h.ntg; ++t) itptr32[t] = static_cast<int32_t>(h.it_ptr[t]);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  auto up = [&](void *dst, const void *src, size_t nbytes) {
    if (e == hipSuccess && nbytes) e = hipMemcpyAsync(dst, src, nbytes, hipMemcpyHostToDevice, st);
  };
  up(dv.order, plan->order.data(), n * i4);
  up(dv.ch_first, h.ch_first.data(), h.nch * i4);
  up(dv.ch_s, h.ch_s.data(), h.nch * i4);
  up(dv.ch_n, h.ch_n.data(), h.nch * i4);
  up(dv.ch_pbase, h.ch_pbase.data(), (h.nch + 1) * i8);
  up(dv.ch_rbase, h.ch_rbase.data(), (h.nch + 1) * i8);
  up(dv.ch_gptr, h.ch_gptr.data(), (h.nch + 1) * i8);
  up(dv.rows_ptr, h.rows_ptr.data(), (h.nch + 1) * i8);
  up(dv.ch_cptr, h.ch_cptr.data(), (h.nch + 1) * i8);
  up(dv.row_chunk, h.row_chunk.data(), h.nrows * i4);
  up(dv.col_chunk, h.col_chunk.data(), n * i4);
  up(dv.tiles_ptr, h.tiles_ptr.data(), (h.nch + 1) * i8);
  up(dv.tile_chunk, h.tile_chunk.data(), h.tiles_ptr[h.nch] * i4);
  up(dv.tg_chunk, h.tg_chunk.data(), h.ntg * i4);
  up(dv.tg_rc, h.tg_rc.data(), h.ntg * i4);
  up(dv.ain, h.ain.data(), h.ntg * i4);
  up(dv.fptr, fptr32.data(), (h.ntg + 1) * i4);
  up(dv.fpair, h.fpair.data(), 2 * h.npairs * i4);
  up(dv.gtab, h.gtab.data(), h.ng * i4);
  up(dv.poutenc, h.poutenc.data(), h.npanel * i4);
  up(dv.it_tg, h.it_tg.data(), h.nitems * i4);
  up(dv.it_lo, h.it_lo.data(), h.nitems * i4);
  up(dv.it_hi, h.it_hi.data(), h.nitems * i4);
  up(dv.it_slot, h.it_slot.data(), h.nitems * i4);
  up(dv.multi_tg, h.multi_tg.data(), h.multi_tg.size() * i4);
  up(dv.it_ptr, itptr32.data(), (h.ntg + 1) * i4);
  up(dv.row_node, h.row_node.data(), h.nrows * i4);
  up(dv.occ_ptr, h.occ_ptr.data(), (n + 1) * i4);
  up(dv.occ_row, h.occ_row.data(), h.nrows * i4);
  up(dv.fdep_ptr, h.fdep_ptr.data(), (h.nch + 1) * i4);
  up(dv.fdep, h.fdep.data(), h.fdep.size() * i4);
  up(dv.bdep_ptr, h.bdep_ptr.data(), (h.nch + 1) * i4);
  up(dv.bdep, h.bdep.data(), h.bdep.size() * i4);
  up(dv.part_off, h.part_off.data(), (h.nch + 1) * i4);
  up(dv.split_off, h.split_off.data(), (h.nch + 1) * i4);
  up(dv.part_chunk, h.part_chunk.data(), h.part_chunk.size() * i4);
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
  const int rc = analyze(n, m, edge_index_host, order_host, 1, 1, false, h);
  if (rc != SELINV_OK) return rc;
  if (nnz_out) *nnz_out = h.nnz;
  if (levels_out) *levels_out = h.node_levels;
  if (S_index_host && cap >= h.nnz && h.nnz)
    std::memcpy(S_index_host, h.S_index.data(), 2 * h.nnz * sizeof(int32_t));
  if (order_out) std::memcpy(order_out, h.order.data(), n * sizeof(int32_t));
  return SELINV_OK;
}
