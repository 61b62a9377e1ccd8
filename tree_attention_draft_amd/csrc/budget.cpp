// Host tree-budget policy: what a draft tree is worth, how many nodes a batch can afford,
// and the static tree of a given size that is worth the most.
//
// Method ("Tree attention mask for draft-tree verification", sections "What it buys" and
// "What it costs"; "Tree Verification", section "The Cost Side"): under greedy
// verification the chance of reaching a node is the product, over the drafter ranks on
// its path, of each rank's acceptance probability, and the expected tokens per step are one (the target's own
// token) plus the sum of those products.  A step verifies B x N tokens; below the ridge of
// a bandwidth-bound decode step that costs about one pass, past it every extra node is
// paid-for compute, so the tree shrinks as the batch grows.  A node's worth is its path
// product, and a product never exceeds its parent's, so the N - 1 most probable rank paths
// always form a tree: a best-first search over the rank tree finds them in order.
//
// Readings: ranks without a listed probability have probability 0; siblings carry
// distinct ranks; ties between equal products go to the shorter, then the
// lexicographically smaller rank path; paths of probability 0 are never added.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <queue>
#include <set>
#include <utility>
#include <vector>

#include "tree_verify.h"
#include "tv_internal.h"

namespace {

constexpr int32_t kMaxRanks = 4096;
constexpr int32_t kMaxDepth = TV_MAX_NODES - 1;

tv_status check_probs(const double* rank_prob, int32_t num_ranks) {
  if (!rank_prob || num_ranks < 1 || num_ranks > kMaxRanks)
    return tv::fail(TV_ERR_INVALID_ARG, "rank_prob must hold 1..4096 probabilities");
  double sum = 0.0;
  for (int32_t r = 0; r < num_ranks; ++r) {
    const double p = rank_prob[r];
    if (!(p >= 0.0 && p <= 1.0))
      return tv::fail(TV_ERR_INVALID_ARG, "rank probabilities must lie in [0, 1]");
    sum += p;
  }
  if (sum > 1.0 + 1e-9)
    return tv::fail(TV_ERR_INVALID_ARG, "rank probabilities must sum to at most 1");
  return TV_OK;
}

inline double prob_of(const double* rank_prob, int32_t num_ranks, int32_t r) {
  return r < num_ranks ? rank_prob[r] : 0.0;
}

// One candidate of the best-first search: a rank path and its product.
struct Cand {
  double p;
  std::vector<int32_t> path;
};

// Priority: larger product first, then shorter path, then lexicographically smaller.
struct CandWorse {
  bool operator()(const Cand& a, const Cand& b) const {
    if (a.p != b.p) return a.p < b.p;
    if (a.path.size() != b.path.size()) return a.path.size() > b.path.size();
    return b.path < a.path;
  }
};

}  // namespace

extern "C" tv_status tree_ridge_tokens(double peak_flops, double hbm_bytes_per_s,
                                       double bytes_per_weight, double* ridge) {
  if (!ridge) return tv::fail(TV_ERR_INVALID_ARG, "ridge is NULL");
  if (!(peak_flops > 0.0) || !(hbm_bytes_per_s > 0.0) || !(bytes_per_weight > 0.0) ||
      !std::isfinite(peak_flops) || !std::isfinite(hbm_bytes_per_s) ||
      !std::isfinite(bytes_per_weight))
    return tv::fail(TV_ERR_INVALID_ARG, "flops, bandwidth and bytes per weight must be > 0");
  *ridge = peak_flops * bytes_per_weight / (2.0 * hbm_bytes_per_s);
  return TV_OK;
}

extern "C" tv_status tree_budget_nodes(int32_t batch, double ridge_tokens, int32_t max_nodes,
                                       int32_t* nodes) {
  if (!nodes) return tv::fail(TV_ERR_INVALID_ARG, "nodes is NULL");
  if (batch < 1 || max_nodes < 1 || !(ridge_tokens >= 0.0) || !std::isfinite(ridge_tokens))
    return tv::fail(TV_ERR_INVALID_ARG, "batch >= 1, max_nodes >= 1, finite ridge >= 0");
  const double fit = std::floor(ridge_tokens / static_cast<double>(batch));
  *nodes = fit >= static_cast<double>(max_nodes) ? max_nodes
                                                 : std::max<int32_t>(1, static_cast<int32_t>(fit));
  return TV_OK;
}

extern "C" tv_status tree_expected_tokens(const int32_t* parent, const int32_t* rank, int32_t n,
                                          const double* rank_prob, int32_t num_ranks,
                                          double* reach, double* expected) {
  if (!parent || !rank || !expected || n < 1)
    return tv::fail(TV_ERR_INVALID_ARG, "parent, rank, expected non-NULL and n >= 1");
  if (tv_status s = check_probs(rank_prob, num_ranks); s != TV_OK) return s;
  if (parent[0] != -1) return tv::fail(TV_ERR_INVALID_ARG, "parent[0] must be -1");
  std::vector<double> own(static_cast<size_t>(n));
  std::set<std::pair<int32_t, int32_t>> sibling_ranks;
  own[0] = 1.0;
  double sum = 0.0;
  for (int32_t i = 1; i < n; ++i) {
    if (parent[i] < 0 || parent[i] >= i)
      return tv::fail(TV_ERR_INVALID_ARG, "parent[i] must lie in [0, i)");
    if (rank[i] < 0) return tv::fail(TV_ERR_INVALID_ARG, "ranks must be >= 0");
    if (!sibling_ranks.insert({parent[i], rank[i]}).second)
      return tv::fail(TV_ERR_INVALID_ARG, "two siblings carry the same rank");
    own[i] = own[parent[i]] * prob_of(rank_prob, num_ranks, rank[i]);
    sum += own[i];
  }
  if (reach)
    for (int32_t i = 0; i < n; ++i) reach[i] = own[i];
  *expected = 1.0 + sum;
  return TV_OK;
}

extern "C" tv_status tree_best_static(const double* rank_prob, int32_t num_ranks,
                                      int32_t nodes, int32_t max_depth, int32_t* ranks,
                                      int64_t ranks_cap, int64_t* path_off,
                                      int32_t* num_paths, double* expected) {
  if (!ranks || !path_off || !num_paths)
    return tv::fail(TV_ERR_INVALID_ARG, "ranks, path_off and num_paths must be non-NULL");
  if (tv_status s = check_probs(rank_prob, num_ranks); s != TV_OK) return s;
  if (nodes < 1 || nodes > TV_MAX_NODES)
    return tv::fail(TV_ERR_CAPACITY, "nodes must lie in 1..64");
  if (max_depth < 1 || max_depth > kMaxDepth)
    return tv::fail(TV_ERR_INVALID_ARG, "max_depth must lie in 1..63");
  if (ranks_cap < 0) return tv::fail(TV_ERR_INVALID_ARG, "ranks_cap < 0");

  std::priority_queue<Cand, std::vector<Cand>, CandWorse> heap;
  auto push_children = [&](const Cand& c) {
    if (static_cast<int32_t>(c.path.size()) >= max_depth) return;
    for (int32_t r = 0; r < num_ranks; ++r) {
      const double p = c.p * rank_prob[r];
      if (!(p > 0.0)) continue;
      Cand k{p, c.path};
      k.path.push_back(r);
      heap.push(std::move(k));
    }
  };
  push_children(Cand{1.0, {}});
  std::vector<Cand> chosen;
  while (static_cast<int32_t>(chosen.size()) < nodes - 1 && !heap.empty()) {
    Cand c = heap.top();
    heap.pop();
    push_children(c);
    chosen.push_back(std::move(c));
  }
  // node order of the builder: (length, lexicographic)
  std::sort(chosen.begin(), chosen.end(), [](const Cand& a, const Cand& b) {
    if (a.path.size() != b.path.size()) return a.path.size() < b.path.size();
    return a.path < b.path;
  });
  int64_t total = 0;
  for (const Cand& c : chosen) total += static_cast<int64_t>(c.path.size());
  if (total > ranks_cap)
    return tv::fail(TV_ERR_CAPACITY, "ranks array too small for the chosen paths");
  int64_t off = 0;
  double sum = 0.0;
  path_off[0] = 0;
  for (size_t i = 0; i < chosen.size(); ++i) {
    for (int32_t r : chosen[i].path) ranks[off++] = r;
    path_off[i + 1] = off;
    sum += chosen[i].p;
  }
  *num_paths = static_cast<int32_t>(chosen.size());
  if (expected) {
    // the same sum the expected-tokens entry point forms: in node order
    *expected = 1.0 + sum;
  }
  return TV_OK;
}

extern "C" tv_status tree_budget_plan(int32_t batch, double ridge_tokens, int32_t max_nodes,
                                      const double* rank_prob, int32_t num_ranks,
                                      int32_t max_depth, int32_t* nodes, int32_t* ranks,
                                      int64_t ranks_cap, int64_t* path_off,
                                      int32_t* num_paths, double* expected) {
  int32_t n = 0;
  if (tv_status s = tree_budget_nodes(batch, ridge_tokens, std::min(max_nodes, TV_MAX_NODES), &n);
      s != TV_OK)
    return s;
  if (tv_status s = tree_best_static(rank_prob, num_ranks, n, max_depth, ranks, ranks_cap,
                                     path_off, num_paths, expected);
      s != TV_OK)
    return s;
  if (nodes) *nodes = n;
  return TV_OK;
}
