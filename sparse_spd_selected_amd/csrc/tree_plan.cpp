// tree_plan.cpp -- host-side level-set schedule for the tree selected inverse.
//
// The tree kernel of the gabp-sparse-inv 0.3.2 page ("Implemented and tested
// kernels", item Tree) collects leaves -> root and distributes root -> leaves;
// its batched variant loops over levels rather than nodes, each level being a
// few batched block operations ("Differentiable selected inverse" and the
// junction-tree section's batched=True remark).  The plan below makes that
// schedule concrete once per parent array: nodes are relabelled breadth-first
// so that every depth level is a contiguous range and every node's children
// are contiguous (in increasing node index) in the next level.  Message sums
// then read a contiguous child range in a fixed order, with no atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"

namespace {

// Returns SELINV_OK and fills depth/root, or SELINV_ERR_BAD_TREE.
int validate(const int32_t *parent, int64_t n, std::vector<int32_t> &depth, int64_t &root) {
  root = -1;
  for (int64_t v = 0; v < n; ++v) {
    const int32_t p = parent[v];
    if (p == -1) {
      if (root >= 0) return SELINV_ERR_BAD_TREE;
      root = v;
    } else if (p < 0 || p >= n || p == v) {
      return SELINV_ERR_BAD_TREE;
    }
  }
  if (root < 0) return SELINV_ERR_BAD_TREE;
  depth.assign(n, -1);
  depth[root] = 0;
  std::vector<int64_t> path;
  for (int64_t v = 0; v < n; ++v) {
    path.clear();
    int64_t u = v;
    while (depth[u] < 0) {
      if (static_cast<int64_t>(path.size()) > n) return SELINV_ERR_BAD_TREE;  // cycle
      path.push_back(u);
      u = parent[u];
    }
    int32_t d = depth[u];
    for (auto it = path.rbegin(); it != path.rend(); ++it) depth[*it] = ++d;
  }
  return SELINV_OK;
}

// The host-side schedule of one parent array (no device work).
struct Schedule {
  int64_t root = -1;
  int32_t levels = 0, max_children = 0;
  std::vector<int64_t> level_off;  // levels + 1
  std::vector<int32_t> node_at, parent_pos, child_beg, child_end, fail_rank, rank_node,
      parent_node;
};

int build_schedule(const int32_t *parent_host, int64_t n, Schedule &sc) {
  std::vector<int32_t> depth;
  int64_t root;
  int rc = validate(parent_host, n, depth, root);
  if (rc != SELINV_OK) return rc;
  sc.root = root;

  // children lists, increasing index (counting sort by parent)
  std::vector<int64_t> cstart(n + 1, 0);
  for (int64_t v = 0; v < n; ++v)
    if (parent_host[v] >= 0) cstart[parent_host[v] + 1]++;
  for (int64_t v = 0; v < n; ++v) cstart[v + 1] += cstart[v];
  std::vector<int32_t> clist(n > 0 ? n - 1 : 0);
  {
    std::vector<int64_t> fillp(cstart.begin(), cstart.end() - 1);
    for (int64_t v = 0; v < n; ++v)
      if (parent_host[v] >= 0) clist[fillp[parent_host[v]]++] = static_cast<int32_t>(v);
  }
  // breadth-first order
  std::vector<int32_t> pos(n);
  sc.node_at.assign(n, 0);
  sc.parent_pos.assign(n, 0);
  sc.child_beg.assign(n, 0);
  sc.child_end.assign(n, 0);
  int64_t head = 0, tail = 0;
  sc.node_at[tail++] = static_cast<int32_t>(root);
  sc.max_children = 0;
  while (head < tail) {
    const int32_t v = sc.node_at[head];
    pos[v] = static_cast<int32_t>(head);
    sc.child_beg[head] = static_cast<int32_t>(tail);
    for (int64_t k = cstart[v]; k < cstart[v + 1]; ++k) sc.node_at[tail++] = clist[k];
    sc.child_end[head] = static_cast<int32_t>(tail);
    sc.max_children = std::max<int32_t>(sc.max_children, sc.child_end[head] - sc.child_beg[head]);
    ++head;
  }
  for (int64_t p = 0; p < n; ++p) {
    const int32_t par = parent_host[sc.node_at[p]];
    sc.parent_pos[p] = par < 0 ? -1 : pos[par];
  }
  const int32_t H = *std::max_element(depth.begin(), depth.end());
  std::vector<int64_t> level_count(H + 1, 0);
  for (int64_t v = 0; v < n; ++v) level_count[depth[v]]++;
  // rank in the order (depth descending, index ascending)
  std::vector<int64_t> rank_start(H + 1, 0);  // rank of the first node of each depth
  {
    int64_t acc = 0;
    for (int32_t d = H; d >= 0; --d) {
      rank_start[d] = acc;
      acc += level_count[d];
    }
  }
  std::vector<int32_t> rank_of(n);
  sc.rank_node.assign(n, 0);
  {
    std::vector<int64_t> next(rank_start.begin(), rank_start.end());
    for (int64_t v = 0; v < n; ++v) {  // increasing index within each depth
      const int64_t r = next[depth[v]]++;
      rank_of[v] = static_cast<int32_t>(r);
      sc.rank_node[r] = static_cast<int32_t>(v);
    }
  }
  sc.fail_rank.assign(n, 0);
  sc.parent_node.assign(n, 0);
  for (int64_t p = 0; p < n; ++p) {
    sc.fail_rank[p] = rank_of[sc.node_at[p]];
    sc.parent_node[p] = parent_host[sc.node_at[p]];
  }
  sc.levels = H + 1;
  sc.level_off.assign(H + 2, 0);
  for (int32_t d = 0; d <= H; ++d) sc.level_off[d + 1] = sc.level_off[d] + level_count[d];
  return SELINV_OK;
}

}  // namespace

extern "C" int selinv_tree_schedule(const int32_t *parent_host, int64_t n, int32_t *node_at,
                                    int32_t *parent_pos, int32_t *child_beg, int32_t *child_end,
                                    int32_t *fail_rank, int64_t *level_off, int32_t *levels) {
  if (!parent_host || n < 1 || n > (int64_t(1) << 30)) return SELINV_ERR_INVALID_ARG;
  Schedule sc;
  const int rc = build_schedule(parent_host, n, sc);
  if (rc != SELINV_OK) return rc;
  const size_t nb = static_cast<size_t>(n) * sizeof(int32_t);
  if (node_at) std::memcpy(node_at, sc.node_at.data(), nb);
  if (parent_pos) std::memcpy(parent_pos, sc.parent_pos.data(), nb);
  if (child_beg) std::memcpy(child_beg, sc.child_beg.data(), nb);
  if (child_end) std::memcpy(child_end, sc.child_end.data(), nb);
  if (fail_rank) std::memcpy(fail_rank, sc.fail_rank.data(), nb);
  if (level_off)
    std::memcpy(level_off, sc.level_off.data(), sc.level_off.size() * sizeof(int64_t));
  if (levels) *levels = sc.levels;
  return SELINV_OK;
}

extern "C" int selinv_tree_plan_create(const int32_t *parent_host, int64_t n, int32_t b,
                                       int dtype_bytes, void *stream, selinv_tree_plan **out) {
  if (!out) return SELINV_ERR_INVALID_ARG;
  *out = nullptr;
  if (!parent_host || n < 1 || n > (int64_t(1) << 30) || b < 1 || b > SELINV_MAX_B ||
      (dtype_bytes != 4 && dtype_bytes != 8))
    return SELINV_ERR_INVALID_ARG;
  Schedule sc;
  int rc = build_schedule(parent_host, n, sc);
  if (rc != SELINV_OK) return rc;
  const int32_t H = sc.levels - 1;
  std::vector<int32_t> &node_at = sc.node_at, &parent_pos = sc.parent_pos,
                       &child_beg = sc.child_beg, &child_end = sc.child_end,
                       &fail_rank = sc.fail_rank, &rank_node = sc.rank_node,
                       &parent_node = sc.parent_node;
  const int32_t max_children = sc.max_children;

  selinv_tree_plan *plan = new (std::nothrow) selinv_tree_plan();
  if (!plan) return SELINV_ERR_HIP;
  plan->n = n;
  plan->b = b;
  plan->dtype_bytes = dtype_bytes;
  plan->levels = H + 1;
  plan->max_children = max_children;
  plan->level_off = new (std::nothrow) int64_t[H + 2];
  if (!plan->level_off) {
    delete plan;
    return SELINV_ERR_HIP;
  }
  for (int32_t d = 0; d <= H + 1; ++d) plan->level_off[d] = sc.level_off[d];

  // tiles of kTreeTile positions, level by level from the root
  std::vector<int32_t> tile_lo, tile_hi;
  for (int32_t d = 0; d <= H; ++d)
    for (int64_t q = plan->level_off[d]; q < plan->level_off[d + 1]; q += selinv::kTreeTile) {
      tile_lo.push_back(static_cast<int32_t>(q));
      tile_hi.push_back(static_cast<int32_t>(std::min<int64_t>(q + selinv::kTreeTile,
                                                               plan->level_off[d + 1])));
    }
  const int64_t T = static_cast<int64_t>(tile_lo.size());
  plan->tiles = T;

  const size_t bytes =
      7 * selinv::align_up(n * sizeof(int32_t)) + 2 * selinv::align_up(T * sizeof(int32_t));
  if (hipMalloc(&plan->dev_block, bytes) != hipSuccess) {
    delete[] plan->level_off;
    delete plan;
    return SELINV_ERR_HIP;
  }
  selinv::Carve cv(plan->dev_block);
  selinv::TreePlanDev &dv = plan->dev;
  dv.node_at = cv.take<int32_t>(n);
  dv.parent_pos = cv.take<int32_t>(n);
  dv.child_beg = cv.take<int32_t>(n);
  dv.child_end = cv.take<int32_t>(n);
  dv.fail_rank = cv.take<int32_t>(n);
  dv.rank_node = cv.take<int32_t>(n);
  dv.parent_node = cv.take<int32_t>(n);
  dv.tile_lo = cv.take<int32_t>(T);
  dv.tile_hi = cv.take<int32_t>(T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t nb = n * sizeof(int32_t);
  hipError_t e = hipSuccess;
  const std::pair<int32_t *, const int32_t *> copies[] = {
      {dv.node_at, node_at.data()},     {dv.parent_pos, parent_pos.data()},
      {dv.child_beg, child_beg.data()}, {dv.child_end, child_end.data()},
      {dv.fail_rank, fail_rank.data()}, {dv.rank_node, rank_node.data()},
      {dv.parent_node, parent_node.data()}};
  for (const auto &c : copies)
    if (e == hipSuccess) e = hipMemcpyAsync(c.first, c.second, nb, hipMemcpyHostToDevice, s);
  const size_t tb = T * sizeof(int32_t);
  if (e == hipSuccess) e = hipMemcpyAsync(dv.tile_lo, tile_lo.data(), tb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(dv.tile_hi, tile_hi.data(), tb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    selinv_tree_plan_destroy(plan);
    return SELINV_ERR_HIP;
  }
  *out = plan;
  return SELINV_OK;
}

extern "C" void selinv_tree_plan_destroy(selinv_tree_plan *plan) {
  if (!plan) return;
  if (plan->dev_block) (void)hipFree(plan->dev_block);
  delete[] plan->level_off;
  delete plan;
}

extern "C" int32_t selinv_tree_plan_levels(const selinv_tree_plan *plan) {
  return plan ? plan->levels : -1;
}
