// Prefix compression (host): rollouts that share a prefix are stored once.
//
// Trajectories of one rollout group share their prompt and often longer
// prefixes; AReaL-DTA (abstract) and HARTS (abstract) process the resulting
// prefix tree so that every shared token is one unique row.  This file turns
// per-trajectory token lists into that tree: a token trie whose chains of
// single-child tokens are merged into segments (a radix tree), numbered and
// packed in depth-first preorder with children in order of first
// appearance, plus the index of every trajectory position into the packed
// unique tokens and, per unique token, the trajectory positions that map to
// it (for deterministic gradient sums).
#include "prefix_tree.h"

#include <sstream>
#include <unordered_map>
#include <vector>

namespace tree_attn {
namespace {

struct TrieNode {
  int32_t token = -1;
  int32_t parent = -1;
  std::vector<int32_t> children;  // in order of first appearance
  std::unordered_map<int32_t, int32_t> child_of;
};

Status fail(std::string* err, Status s, const std::string& msg) {
  if (err) *err = msg;
  return s;
}

}  // namespace

Status build_prefix_tree(const int32_t* tokens, const int64_t* traj_offsets, int32_t num_traj,
                         int32_t* parent, int32_t* seg_start, int32_t* seg_len,
                         int32_t* unique_tokens, int32_t* traj_index, int32_t* mult,
                         int32_t* inv_offsets, int32_t* inv_positions, int32_t* num_nodes,
                         int32_t* num_tokens, std::string* err) {
  if (num_traj < 0 || !traj_offsets || !num_nodes || !num_tokens)
    return fail(err, Status::kInvalidArg, "null argument or negative trajectory count");
  const int64_t total = num_traj > 0 ? traj_offsets[num_traj] : 0;
  if (num_traj > 0 && traj_offsets[0] != 0)
    return fail(err, Status::kInvalidArg, "traj_offsets[0] must be 0");
  for (int32_t b = 0; b < num_traj; ++b)
    if (traj_offsets[b + 1] < traj_offsets[b])
      return fail(err, Status::kInvalidArg, "traj_offsets must be non-decreasing");
  if (total > INT32_MAX - 1) return fail(err, Status::kUnsupported, "more than 2^31 - 2 tokens");
  if (total > 0 && (!tokens || !parent || !seg_start || !seg_len || !unique_tokens ||
                    !traj_index))
    return fail(err, Status::kInvalidArg, "null array");
  for (int64_t i = 0; i < total; ++i)
    if (tokens[i] < 0) return fail(err, Status::kInvalidArg, "token ids must be >= 0");

  // ---- token trie (one trie node per distinct prefix); trie node 0 is a
  // virtual root above the first tokens
  std::vector<TrieNode> trie(1);
  std::vector<int32_t> pos_trie(total);  // trie node of each trajectory position
  for (int32_t b = 0; b < num_traj; ++b) {
    int32_t cur = 0;
    for (int64_t i = traj_offsets[b]; i < traj_offsets[b + 1]; ++i) {
      const int32_t tok = tokens[i];
      auto it = trie[cur].child_of.find(tok);
      int32_t nxt;
      if (it == trie[cur].child_of.end()) {
        nxt = static_cast<int32_t>(trie.size());
        trie.emplace_back();
        trie[nxt].token = tok;
        trie[nxt].parent = cur;
        trie[cur].child_of.emplace(tok, nxt);
        trie[cur].children.push_back(nxt);
      } else {
        nxt = it->second;
      }
      pos_trie[i] = nxt;
      cur = nxt;
    }
  }
  const int64_t n = static_cast<int64_t>(trie.size()) - 1;  // unique tokens

  // ---- depth-first preorder of trie tokens; a tree node starts at a token
  // whose parent is the virtual root or has more than one child, and runs
  // down the chain of single children
  std::vector<int32_t> packed(trie.size(), -1);  // trie node -> packed row
  int32_t m = 0, row = 0;
  std::vector<int32_t> stack;  // trie nodes that start a tree node
  std::vector<int32_t> start_parent_node;  // tree node of the parent for each start
  for (auto it = trie[0].children.rbegin(); it != trie[0].children.rend(); ++it) {
    stack.push_back(*it);
    start_parent_node.push_back(-1);
  }
  while (!stack.empty()) {
    int32_t t = stack.back();
    const int32_t pnode = start_parent_node.back();
    stack.pop_back();
    start_parent_node.pop_back();
    const int32_t node = m++;
    parent[node] = pnode;
    seg_start[node] = row;
    int32_t len = 0;
    while (true) {
      packed[t] = row;
      unique_tokens[row] = trie[t].token;
      ++row;
      ++len;
      if (trie[t].children.size() != 1) break;
      t = trie[t].children[0];
    }
    seg_len[node] = len;
    for (auto it = trie[t].children.rbegin(); it != trie[t].children.rend(); ++it) {
      stack.push_back(*it);
      start_parent_node.push_back(node);
    }
  }
  for (int64_t i = 0; i < total; ++i) traj_index[i] = packed[pos_trie[i]];

  // ---- multiplicities and the inverse map (positions per unique token,
  // ascending)
  if (mult || inv_offsets || inv_positions) {
    std::vector<int32_t> cnt(n + 1, 0);
    for (int64_t i = 0; i < total; ++i) ++cnt[traj_index[i] + 1];
    if (mult)
      for (int64_t u = 0; u < n; ++u) mult[u] = cnt[u + 1];
    for (int64_t u = 0; u < n; ++u) cnt[u + 1] += cnt[u];
    if (inv_offsets)
      for (int64_t u = 0; u <= n; ++u) inv_offsets[u] = cnt[u];
    if (inv_positions) {
      std::vector<int32_t> fill(cnt.begin(), cnt.end() - 1);
      for (int64_t i = 0; i < total; ++i) inv_positions[fill[traj_index[i]]++] = static_cast<int32_t>(i);
    }
  }
  *num_nodes = m;
  *num_tokens = static_cast<int32_t>(n);
  return Status::kOk;
}

}  // namespace tree_attn
