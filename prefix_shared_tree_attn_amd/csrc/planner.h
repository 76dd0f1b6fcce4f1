// Host planner for prefix-shared tree attention.
//
// Turns a node table (parent, segment start, segment length) into the work
// items of the forward and backward kernels.  The forward pass works per
// query tile: a tile of rows inside one node, with the list of key ranges it
// sees (its ancestors' segments, root first, then its own node up to the
// tile's last row).  The backward pass works per key tile: a tile of rows
// inside one node, with the list of query ranges that see it (the rest of its
// own node and every descendant node's segment).  Work is counted in
// (query row, key row, head) units -- the compact-token work left after
// prefix compression, on which HARTS (abstract) plans its batches -- and
// items are ordered longest first.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tree_attn {

enum class Status : int {
  kOk = 0,
  kInvalidArg = 1,
  kBadTree = 2,
  kLayout = 3,
  kUnsupported = 4,
  kWorkspace = 5,
  kHip = 6,
  kNoDevicePlan = 7,
};

// Tile shapes shared by the planner and the kernels.
constexpr int kFwdRows = 128;  // query rows per forward workgroup (4 waves x 32)
constexpr int kFwdKeys = 64;   // keys per forward step
constexpr int kBwdKeys = 128;  // keys per backward workgroup (4 waves x 32)
constexpr int kBwdRows = 32;   // query rows per backward step
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, 8 L2s
constexpr int kLinChunk = 64;  // chunk of chunkwise linear attention (trajectory depth)
constexpr int kFwdFill = 1;      // forward workgroups per CU a split launch may reach
constexpr int kFwdMaxParts = 16; // most parts one query tile's keys are split into
constexpr int kFwdMinPartSteps = 16;  // fewest key steps a part of a split tile keeps
constexpr int kFwdSplitSteps = 48;    // a plan splits only if a tile has this many key steps
// Most key-range entries a plan may hold (forward ranges, backward entries).
// A tree stored depth first needs a few per tile; one whose children are
// not stored after their parents needs as many as its depth per tile.
constexpr int64_t kMaxRangeEntries = int64_t{1} << 27;

struct I4 {
  int32_t x, y, z, w;
};
struct I8 {
  int32_t v[8];
};

struct HostPlan {
  int64_t num_tokens = 0, num_nodes = 0, hq = 0, hkv = 0, head_dim = 0;
  int dtype = 0;  // 0 bf16, 1 fp32
  int num_cus = 256;
  // Query-subset plan: only the rows of the listed nodes are queries (their
  // keys are still every ancestor row).  The forward pass writes those rows
  // only, and every backward key tile writes fp32 slots that the reduction
  // adds into caller-owned fp32 dK / dV accumulators.
  bool subset = false;
  int64_t query_rows = 0;  // rows of the query nodes
  int64_t pairs = 0;

  // forward: tiles (q0, q1, range_begin, range_end) longest first;
  // ranges (k0, k1, causal, 0)
  std::vector<I4> fwd_tiles;
  std::vector<I4> fwd_ranges;
  int64_t fwd_groups = 0;  // tiles * hkv
  int64_t fwd_blocks = 0;  // launch size (padded to whole XCD rounds) * group size
  // A launch with too few (tile, head) workgroups to fill the chip splits the
  // keys of its query tiles into parts: fwd_part[tile] is the part's slot
  // (-1: the tile holds all of its rows' keys and writes the outputs), and
  // fwd_combine holds (q0, q1, slot_begin, num_slots) per split query tile,
  // whose parts' partial results a combine pass merges.  The same tiles
  // drive the dQ pass, whose parts' partial sums are added the same way.
  std::vector<int32_t> fwd_part;
  std::vector<I4> fwd_combine;
  int64_t fwd_slots = 0;
  // every query tile once, (q0, q1, 0, 0): the rows a query-subset plan's
  // backward preprocess covers
  std::vector<I4> fwd_qtiles;

  // backward: items (k0, k1, kv_head, entry_begin, entry_end, slot, xcd, 0)
  // in launch order (item b runs on XCD b % 8; empty items pad the per-XCD
  // queues); entries (q_head, q0, q1, causal); reductions of split key tiles
  // (k0, k1, kv_head, slot_begin, num_slots, 0, 0, 0)
  std::vector<I8> bwd_items;
  std::vector<I4> bwd_entries;
  std::vector<I8> bwd_reduce;
  int64_t bwd_slots = 0;
  int64_t bwd_split_tiles = 0;
  bool bwd_has_limit = false;  // some entry carries a key limit

  // segments sorted by start: (seg_start, seg_len, depth offset = ancestor
  // tokens of the node, node index), for the per-token position pass
  std::vector<I4> segments;

  // linear attention: pieces (token0, len, pred, succ_begin, succ_end, node,
  // flags: 1 first / 2 last piece of its node, 0) in root-first order,
  // pred = -1 at a root; successor piece indices
  std::vector<I8> lin_pieces;
  std::vector<int32_t> lin_succ;
  // nodes in the same root-first order: (first piece, pieces, parent node or
  // -1, node)
  std::vector<I4> lin_nodes;
  // the state scans' order: heavy paths (each node followed by its child with
  // the most pieces below it) as runs of lin_nodes indices, lin_chains
  // (begin, end, phase, 0) into lin_chain_nodes; phase p holds the chains
  // whose head hangs off a chain of phase p - 1 (roots: phase 0), and
  // lin_phases (chain_begin, chain_end, 0, 0) lists them phase by phase
  std::vector<int32_t> lin_chain_nodes;
  std::vector<I4> lin_chains;
  std::vector<I4> lin_phases;
};

// Validates the table and fills `out`.  `query_nodes` (num_query_nodes
// entries, repeats allowed) makes a query-subset plan; null plans the whole
// tree.  On error returns the status and a message in *err; `out` is then
// unspecified.
Status build_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                  int32_t num_nodes, int32_t num_tokens, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int dtype, int num_cus,
                  HostPlan* out, std::string* err, const int32_t* query_nodes = nullptr,
                  int32_t num_query_nodes = 0);

// The calls of a memory-bounded depth-first walk: the nodes in preorder
// (roots, and each node's children, in index order) in order[num_nodes], cut
// into runs of consecutive nodes, run r = order[run_start[r] ..
// run_start[r + 1]), *num_runs of them.  A run takes the next node while the
// union of its nodes' root paths holds at most `budget` tokens; a node whose
// own root path is longer starts a run and closes it.  budget <= 0: the
// longest root-to-leaf path's token count.  Checks parents (kBadTree) and
// segment lengths (kLayout) only.
Status walk_runs(const int32_t* parent, const int32_t* seg_len, int32_t num_nodes,
                 int64_t budget, int32_t* order, int32_t* run_start, int32_t* num_runs,
                 std::string* err);

}  // namespace tree_attn
