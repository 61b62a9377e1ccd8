// Host tree-metadata builder: drafter-rank paths -> parent, depth, ancestor bitmask, pos.
//
// Method ("Tree attention mask for draft-tree verification", section "A strong answer"):
// candidates are tuples of drafter ranks under an implicit root (node 0, the last accepted
// token); distinct candidates become nodes 1.. in (length, lexicographic) order; a node's
// parent is the node of its one-shorter prefix and a candidate without one is rejected;
// depth is the tuple length; position id is prefix length + depth; node i may see node j
// iff j is i or an ancestor.  Because parents precede children in this order, the
// ancestor bitmask of node i is its parent's bitmask plus bit i -- one pass, O(N).
//
// Implementation: sort references into the CSR rank arrays (no copies of the paths;
// thread-local scratch, so a batch allocates nothing per tree), drop adjacent duplicates, and resolve each parent by binary
// search for the one-shorter prefix among the already-placed nodes of the previous
// length (they are contiguous and sorted in the node order).  When every rank fits b bits
// and the longest candidate has at most 56/b ranks (drafter trees: a few bits, depth
// ~10), each candidate is first packed into one 64-bit key -- length in the top byte,
// ranks below it most significant first at fixed field positions -- so integer order is
// the (length, lexicographic) order, and a parent's key is the child's with its length
// decremented and its last field cleared.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tree_verify.h"
#include "tv_internal.h"

namespace {

struct PathRef {
  const int32_t* r;
  int32_t len;
  int32_t input_index;
};

// (length, lexicographic) order of the node numbering.
inline bool path_less(const PathRef& a, const PathRef& b) {
  if (a.len != b.len) return a.len < b.len;
  for (int32_t t = 0; t < a.len; ++t)
    if (a.r[t] != b.r[t]) return a.r[t] < b.r[t];
  return false;
}

inline bool same_path(const PathRef& a, const PathRef& b) {
  return a.len == b.len && std::memcmp(a.r, b.r, sizeof(int32_t) * a.len) == 0;
}

// Compare the first `len` ranks of `full` with the whole of `node` (node.len == len).
inline int prefix_cmp(const PathRef& node, const int32_t* full, int32_t len) {
  for (int32_t t = 0; t < len; ++t) {
    if (node.r[t] != full[t]) return node.r[t] < full[t] ? -1 : 1;
  }
  return 0;
}

}  // namespace

namespace {

struct Scratch {
  std::vector<PathRef> refs, nodes;
  struct Group { int32_t len; int64_t begin, end; };
  std::vector<Group> groups;
  struct Keyed { uint64_t key; int32_t input_index; };
  std::vector<Keyed> keyed;
  std::vector<uint64_t> node_keys;
};

// The packed-key form of build_one (see the file comment); refs validated, b bits per rank.
tv_status build_keyed(Scratch& sc, int32_t max_len, int32_t b, int32_t prefix_len,
                      int32_t cap, int32_t* parent, int32_t* depth, uint64_t* bitmask,
                      int32_t* pos, int32_t* num_nodes, int32_t* bad) {
  auto& keyed = sc.keyed;
  auto& keys = sc.node_keys;
  keyed.clear();
  keys.clear();
  for (const PathRef& r : sc.refs) {
    uint64_t k = static_cast<uint64_t>(r.len) << 56;
    for (int32_t t = 0; t < r.len; ++t)
      k |= static_cast<uint64_t>(r.r[t]) << (b * (max_len - 1 - t));
    keyed.push_back(Scratch::Keyed{k, r.input_index});
  }
  std::sort(keyed.begin(), keyed.end(), [](const Scratch::Keyed& x, const Scratch::Keyed& y) {
    return x.key != y.key ? x.key < y.key : x.input_index < y.input_index;
  });
  keys.push_back(0);  // the root: length 0, no ranks
  for (size_t i = 0; i < keyed.size(); ++i)
    if (i == 0 || keyed[i].key != keyed[i - 1].key) keys.push_back(keyed[i].key);
  const int64_t n = static_cast<int64_t>(keys.size());
  if (n > cap || n > TV_MAX_NODES)
    return tv::fail(TV_ERR_CAPACITY, "tree has more nodes than the output capacity");
  parent[0] = -1;
  depth[0] = 0;
  bitmask[0] = 1ull;
  const uint64_t field = (1ull << b) - 1;
  size_t first = 0;  // first keyed entry of the current node (its first input occurrence)
  for (int64_t i = 1; i < n; ++i) {
    while (keyed[first].key != keys[i]) ++first;
    const uint64_t k = keys[i];
    const int32_t len = static_cast<int32_t>(k >> 56);
    const uint64_t pk = (static_cast<uint64_t>(len - 1) << 56) |
                        (k & ((1ull << 56) - 1) & ~(field << (b * (max_len - len))));
    const auto it = std::lower_bound(keys.begin(), keys.begin() + i, pk);
    if (it == keys.begin() + i || *it != pk) {
      *bad = keyed[first].input_index;
      return tv::fail(TV_ERR_MISSING_PARENT, "a path's one-shorter prefix is not a node");
    }
    const int64_t found = it - keys.begin();
    parent[i] = static_cast<int32_t>(found);
    depth[i] = len;
    bitmask[i] = bitmask[found] | (1ull << i);
  }
  for (int64_t i = 0; i < n; ++i) pos[i] = prefix_len + depth[i];
  *num_nodes = static_cast<int32_t>(n);
  return TV_OK;
}

// One tree from candidates [p0, p1) of a CSR list with absolute offsets path_off[].
// Writes up to `cap` nodes; *bad gets the offending candidate's index relative to p0.
tv_status build_one(const int32_t* ranks, const int64_t* path_off, int64_t p0, int64_t p1,
                    int32_t prefix_len, int32_t cap, int32_t* parent, int32_t* depth,
                    uint64_t* bitmask, int32_t* pos, int32_t* num_nodes, int32_t* bad) {
  thread_local Scratch sc;
  std::vector<PathRef>& refs = sc.refs;
  std::vector<PathRef>& nodes = sc.nodes;
  refs.clear();
  nodes.clear();
  sc.groups.clear();
  int32_t max_len = 0, max_rank = 0;
  for (int64_t p = p0; p < p1; ++p) {
    const int64_t a = path_off[p], b = path_off[p + 1];
    const int32_t rel = static_cast<int32_t>(p - p0);
    if (b < a) return tv::fail(TV_ERR_INVALID_ARG, "path_off is not non-decreasing");
    if (b - a > INT32_MAX) return tv::fail(TV_ERR_INVALID_ARG, "path too long");
    if (b == a) {
      *bad = rel;
      return tv::fail(TV_ERR_INVALID_PATH, "empty path (the root is implicit)");
    }
    for (int64_t t = a; t < b; ++t) {
      if (ranks[t] < 0) {
        *bad = rel;
        return tv::fail(TV_ERR_INVALID_PATH, "negative rank");
      }
      max_rank = std::max(max_rank, ranks[t]);
    }
    max_len = std::max(max_len, static_cast<int32_t>(b - a));
    refs.push_back(PathRef{ranks + a, static_cast<int32_t>(b - a), rel});
  }
  int32_t bits = 1;
  while (bits < 31 && (max_rank >> bits) != 0) ++bits;
  if (static_cast<int64_t>(max_len) * bits <= 56)
    return build_keyed(sc, max_len, bits, prefix_len, cap, parent, depth, bitmask, pos,
                       num_nodes, bad);
  // (length, lexicographic) order; among duplicates the first input occurrence first
  std::sort(refs.begin(), refs.end(), [](const PathRef& x, const PathRef& y) {
    if (path_less(x, y)) return true;
    if (path_less(y, x)) return false;
    return x.input_index < y.input_index;
  });
  nodes.push_back(PathRef{nullptr, 0, -1});  // root
  for (const PathRef& r : refs)
    if (nodes.size() == 1 || !same_path(nodes.back(), r)) nodes.push_back(r);

  const int64_t n = static_cast<int64_t>(nodes.size());
  if (n > cap || n > TV_MAX_NODES)
    return tv::fail(TV_ERR_CAPACITY, "tree has more nodes than the output capacity");

  // nodes are grouped by length; a parent lives in the group one shorter
  auto& groups = sc.groups;
  for (int64_t i = 1; i < n; ++i) {
    if (groups.empty() || groups.back().len != nodes[i].len)
      groups.push_back(Scratch::Group{nodes[i].len, i, i + 1});
    else
      groups.back().end = i + 1;
  }
  parent[0] = -1;
  depth[0] = 0;
  bitmask[0] = 1ull;
  size_t g = 0;
  for (int64_t i = 1; i < n; ++i) {
    const PathRef& me = nodes[i];
    while (groups[g].end <= i) ++g;  // groups[g] holds node i
    int64_t found = -1;
    if (me.len == 1) {
      found = 0;
    } else if (g > 0 && groups[g - 1].len == me.len - 1) {
      int64_t lo = groups[g - 1].begin, hi = groups[g - 1].end;  // binary search [lo, hi)
      while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        const int c = prefix_cmp(nodes[mid], me.r, me.len - 1);
        if (c == 0) { found = mid; break; }
        if (c < 0) lo = mid + 1; else hi = mid;
      }
    }
    if (found < 0) {
      *bad = me.input_index;
      return tv::fail(TV_ERR_MISSING_PARENT, "a path's one-shorter prefix is not a node");
    }
    parent[i] = static_cast<int32_t>(found);
    depth[i] = me.len;
    bitmask[i] = bitmask[found] | (1ull << i);
  }
  for (int64_t i = 0; i < n; ++i) pos[i] = prefix_len + depth[i];
  *num_nodes = static_cast<int32_t>(n);
  return TV_OK;
}

bool prefix_ok(int32_t L) { return L >= 0 && L <= INT32_MAX - 2 * TV_MAX_NODES; }

}  // namespace

extern "C" tv_status tree_meta_build(const int32_t* ranks, const int64_t* path_off,
                                     int32_t num_paths, int32_t prefix_len, int32_t max_nodes,
                                     int32_t* parent, int32_t* depth, uint64_t* bitmask,
                                     int32_t* pos, int32_t* num_nodes, int32_t* bad_path) {
  if (bad_path) *bad_path = -1;
  if (num_paths < 0) return tv::fail(TV_ERR_INVALID_ARG, "num_paths < 0");
  if (!path_off || !parent || !depth || !bitmask || !pos || !num_nodes)
    return tv::fail(TV_ERR_INVALID_ARG, "null output or path_off pointer");
  if (path_off[0] != 0) return tv::fail(TV_ERR_INVALID_ARG, "path_off[0] != 0");
  if (num_paths > 0 && !ranks && path_off[num_paths] > 0)
    return tv::fail(TV_ERR_INVALID_ARG, "ranks is null");
  if (!prefix_ok(prefix_len)) return tv::fail(TV_ERR_INVALID_ARG, "prefix_len out of range");
  if (max_nodes < 1) return tv::fail(TV_ERR_INVALID_ARG, "max_nodes < 1");
  int32_t bad = -1;
  const tv_status st = build_one(ranks, path_off, 0, num_paths, prefix_len, max_nodes, parent,
                                 depth, bitmask, pos, num_nodes, &bad);
  if (bad_path) *bad_path = bad;
  return st;
}

extern "C" tv_status tree_meta_build_batch(const int32_t* ranks, const int64_t* path_off,
                                           const int64_t* tree_off, int32_t B,
                                           const int32_t* prefix_len, int32_t N,
                                           int32_t* parent, int32_t* depth, uint64_t* bitmask,
                                           int32_t* pos, int32_t* num_nodes, int32_t* bad_tree,
                                           int32_t* bad_path) {
  if (bad_tree) *bad_tree = -1;
  if (bad_path) *bad_path = -1;
  if (B < 0) return tv::fail(TV_ERR_INVALID_ARG, "B < 0");
  if (N < 1) return tv::fail(TV_ERR_INVALID_ARG, "N < 1");
  if (N > TV_MAX_NODES) return tv::fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (B == 0) return TV_OK;
  if (!path_off || !tree_off || !prefix_len || !parent || !depth || !bitmask || !pos ||
      !num_nodes)
    return tv::fail(TV_ERR_INVALID_ARG, "null pointer");
  // Every argument check covers the whole batch before anything is written: tree and
  // path offsets (so no offset is dereferenced before it is known to be in order), the
  // ranks pointer, and every prefix length.
  if (tree_off[0] != 0 || path_off[0] != 0)
    return tv::fail(TV_ERR_INVALID_ARG, "tree_off[0] and path_off[0] must be 0");
  for (int32_t b = 0; b < B; ++b) {
    if (tree_off[b + 1] < tree_off[b]) {
      if (bad_tree) *bad_tree = b;
      return tv::fail(TV_ERR_INVALID_ARG, "tree_off is not non-decreasing");
    }
  }
  const int64_t num_paths = tree_off[B];
  for (int64_t p = 0; p < num_paths; ++p) {
    if (path_off[p + 1] < path_off[p])
      return tv::fail(TV_ERR_INVALID_ARG, "path_off is not non-decreasing");
  }
  if (!ranks && path_off[num_paths] > 0) return tv::fail(TV_ERR_INVALID_ARG, "ranks is null");
  for (int32_t b = 0; b < B; ++b) {
    if (!prefix_ok(prefix_len[b])) {
      if (bad_tree) *bad_tree = b;
      return tv::fail(TV_ERR_INVALID_ARG, "prefix_len out of range");
    }
  }
  for (int32_t b = 0; b < B; ++b) {
    const size_t row = static_cast<size_t>(b) * N;
    int32_t n = 0, bad = -1;
    const tv_status st = build_one(ranks, path_off, tree_off[b], tree_off[b + 1], prefix_len[b],
                                   N, parent + row, depth + row, bitmask + row, pos + row, &n,
                                   &bad);
    if (st != TV_OK) {
      if (bad_tree) *bad_tree = b;
      if (bad_path) *bad_path = bad;
      return st;
    }
    num_nodes[b] = n;
    for (int32_t i = n; i < N; ++i) {  // padding leaves under the root
      parent[row + i] = 0;
      depth[row + i] = 1;
      bitmask[row + i] = 1ull | (1ull << i);
      pos[row + i] = prefix_len[b] + 1;
    }
  }
  return TV_OK;
}
