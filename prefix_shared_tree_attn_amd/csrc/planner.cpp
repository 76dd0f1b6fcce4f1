// Host planner: node-table validation and work-item construction.
// The prefix tree (AReaL-DTA, abstract) is turned into forward query tiles
// with ancestor key ranges and backward key tiles with descendant query
// ranges; work is balanced on compact-token work (HARTS, abstract).
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <map>
#include <numeric>
#include <sstream>
#include <tuple>

namespace tree_attn {
namespace {

struct Range {
  int64_t b, e;  // [b, e)
};

// Appends [b, e) to a list of ranges, merging with the last range when the
// two are contiguous in memory.
void push_range(std::vector<Range>& v, int64_t b, int64_t e) {
  if (!v.empty() && v.back().e == b) {
    v.back().e = e;
  } else {
    v.push_back({b, e});
  }
}

Status fail(std::string* err, Status s, const std::string& msg) {
  if (err) *err = msg;
  return s;
}

// Pieces of chunkwise linear attention.  A node's tokens are cut where
// their trajectory depth is a multiple of kLinChunk, so every state a piece
// starts from is either a trajectory chunk boundary or a branch point.
// Pieces are listed in the root-first node order, so a piece's predecessor
// (the previous piece of its node, else its parent's last piece) comes
// before it and its successors (the next piece of its node, else the first
// pieces of the child nodes) after it.
void build_lin_pieces(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                      const std::vector<int32_t>& order,
                      const std::vector<std::vector<int32_t>>& children,
                      const std::vector<int64_t>& depth, HostPlan* out) {
  const size_t m = order.size();
  std::vector<int32_t> first(m, -1), last(m, -1);
  std::vector<I8>& pc = out->lin_pieces;
  for (int32_t i : order) {
    const int64_t s = seg_start[i], e = s + seg_len[i];
    int64_t t = s, d = depth[i];
    int32_t pred = parent[i] >= 0 ? last[parent[i]] : -1;
    while (t < e) {
      const int64_t len = std::min<int64_t>(e - t, kLinChunk - d % kLinChunk);
      const int32_t id = static_cast<int32_t>(pc.size());
      pc.push_back({{static_cast<int32_t>(t), static_cast<int32_t>(len), pred, 0, 0, i, 0, 0}});
      if (first[i] < 0) first[i] = id;
      pred = id;
      t += len;
      d += len;
    }
    last[i] = pred;
    out->lin_nodes.push_back({first[i], pred - first[i] + 1,
                              parent[i] >= 0 ? parent[i] : -1, i});
  }
  // heavy paths for the state scans: chains of nodes run one after another
  // in one thread, while the chains of a phase run side by side
  {
    std::vector<int64_t> below(m, 0);  // pieces in a node's subtree, indexed by node
    for (size_t k = m; k-- > 0;) {
      const int32_t i = order[k];
      below[i] += last[i] - first[i] + 1;
      if (parent[i] >= 0) below[parent[i]] += below[i];
    }
    std::vector<int32_t> pos(m, -1), heavy(m, -1), phase(m, 0);
    for (size_t k = 0; k < m; ++k) pos[order[k]] = static_cast<int32_t>(k);
    for (int32_t i : order) {
      int64_t best = -1;
      for (int32_t c : children[i])
        if (below[c] > best) {
          best = below[c];
          heavy[i] = c;
        }
    }
    struct Chain {
      int32_t phase;
      std::vector<int32_t> nodes;
    };
    std::vector<Chain> chains;
    for (int32_t i : order) {  // chain heads in root-first order
      const int32_t pa = parent[i];
      if (pa >= 0 && heavy[pa] == i) continue;
      Chain c;
      c.phase = pa >= 0 ? phase[pa] + 1 : 0;
      for (int32_t j = i; j >= 0; j = heavy[j]) {
        phase[j] = c.phase;
        c.nodes.push_back(pos[j]);
      }
      chains.push_back(std::move(c));
    }
    std::stable_sort(chains.begin(), chains.end(),
                     [](const Chain& x, const Chain& y) { return x.phase < y.phase; });
    for (const Chain& c : chains) {
      const int32_t b = static_cast<int32_t>(out->lin_chain_nodes.size());
      out->lin_chain_nodes.insert(out->lin_chain_nodes.end(), c.nodes.begin(), c.nodes.end());
      out->lin_chains.push_back(
          {b, static_cast<int32_t>(out->lin_chain_nodes.size()), c.phase, 0});
      const int32_t ci = static_cast<int32_t>(out->lin_chains.size()) - 1;
      if (out->lin_phases.empty() || c.phase != static_cast<int32_t>(out->lin_phases.size()) - 1)
        out->lin_phases.push_back({ci, ci + 1, 0, 0});
      else
        out->lin_phases.back().y = ci + 1;
    }
  }
  std::vector<int32_t>& sc = out->lin_succ;
  for (size_t j = 0; j < pc.size(); ++j) {
    const int32_t node = pc[j].v[5];
    pc[j].v[3] = static_cast<int32_t>(sc.size());
    if (static_cast<int32_t>(j) != last[node])
      sc.push_back(static_cast<int32_t>(j + 1));
    else
      for (int32_t c : children[node]) sc.push_back(first[c]);
    pc[j].v[4] = static_cast<int32_t>(sc.size());
    pc[j].v[6] = (static_cast<int32_t>(j) == first[node] ? 1 : 0) |
                 (static_cast<int32_t>(j) == last[node] ? 2 : 0);
  }
}

}  // namespace

Status build_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                  int32_t num_nodes, int32_t num_tokens, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int dtype, int num_cus,
                  HostPlan* out, std::string* err, const int32_t* query_nodes,
                  int32_t num_query_nodes) {
  if (!out) return fail(err, Status::kInvalidArg, "null output plan");
  if (num_nodes < 0 || num_tokens < 0)
    return fail(err, Status::kInvalidArg, "negative num_nodes or num_tokens");
  if (num_nodes > 0 && (!parent || !seg_start || !seg_len))
    return fail(err, Status::kInvalidArg, "null node-table pointer");
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(err, Status::kUnsupported,
                "num_q_heads must be a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(err, Status::kUnsupported, "head_dim must be 64 or 128");
  if (dtype != 0 && dtype != 1) return fail(err, Status::kUnsupported, "unknown dtype");
  if (num_nodes == 0 && num_tokens != 0)
    return fail(err, Status::kLayout, "tokens given but no nodes");
  if (num_query_nodes < 0 || (num_query_nodes > 0 && !query_nodes))
    return fail(err, Status::kInvalidArg, "bad query-node list");
  for (int32_t j = 0; j < num_query_nodes; ++j)
    if (query_nodes[j] < 0 || query_nodes[j] >= num_nodes) {
      std::ostringstream os;
      os << "query node " << query_nodes[j] << " is not a node index";
      return fail(err, Status::kInvalidArg, os.str());
    }

  const int64_t m = num_nodes, n = num_tokens;
  HostPlan& p = *out;
  p = HostPlan();
  p.num_tokens = n;
  p.num_nodes = m;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.head_dim = head_dim;
  p.dtype = dtype;
  p.num_cus = num_cus > 0 ? num_cus : 256;
  p.subset = query_nodes != nullptr;
  if (m == 0) return Status::kOk;
  // queries: every node, or the listed ones
  std::vector<char> active(m, p.subset ? 0 : 1);
  for (int32_t j = 0; j < num_query_nodes; ++j) active[query_nodes[j]] = 1;

  // ---- validation: parents, segment lengths, exact partition of [0, N)
  for (int64_t i = 0; i < m; ++i) {
    const int32_t pa = parent[i];
    if (pa < -1 || pa >= m || pa == i) {
      std::ostringstream os;
      os << "node " << i << " has invalid parent " << pa;
      return fail(err, Status::kBadTree, os.str());
    }
    if (seg_len[i] < 1 || seg_start[i] < 0 ||
        static_cast<int64_t>(seg_start[i]) + seg_len[i] > n) {
      std::ostringstream os;
      os << "node " << i << " has segment [" << seg_start[i] << ", +" << seg_len[i]
         << ") outside [0, " << n << ") or empty";
      return fail(err, Status::kLayout, os.str());
    }
  }
  std::vector<int32_t> by_start(m);
  std::iota(by_start.begin(), by_start.end(), 0);
  std::sort(by_start.begin(), by_start.end(),
            [&](int32_t a, int32_t b) { return seg_start[a] < seg_start[b]; });
  int64_t pos = 0;
  for (int32_t i : by_start) {
    if (seg_start[i] != pos) {
      std::ostringstream os;
      os << "segments do not tile [0, N): expected a segment at row " << pos
         << ", found node " << i << " at " << seg_start[i];
      return fail(err, Status::kLayout, os.str());
    }
    pos += seg_len[i];
  }
  if (pos != n) return fail(err, Status::kLayout, "segments do not cover [0, N)");

  // ---- children and a root-first order; nodes unreachable from a root lie
  // on a cycle
  std::vector<std::vector<int32_t>> children(m);
  std::vector<int32_t> order;
  order.reserve(m);
  for (int64_t i = 0; i < m; ++i) {
    if (parent[i] >= 0) children[parent[i]].push_back(static_cast<int32_t>(i));
    else order.push_back(static_cast<int32_t>(i));
  }
  for (size_t h = 0; h < order.size(); ++h)
    for (int32_t c : children[order[h]]) order.push_back(c);
  if (static_cast<int64_t>(order.size()) != m)
    return fail(err, Status::kBadTree, "parent pointers contain a cycle");

  // ---- size guard.  Ancestor ranges merge only where a parent's segment
  // ends where the next ancestor's begins, and a node's side subtrees (all
  // children but the one stored right after it) each add a query range to
  // the key tiles of its run.  Stored depth first, a tree needs a few
  // entries per tile; stored in another order, a deep tree needs its depth
  // per tile, quadratic in the node count.  Count the entries (O(M)) before
  // building anything and refuse plans beyond kMaxRangeEntries.
  {
    std::vector<int64_t> nanc(m, 0), anc_end(m, -1), act_sub(m, 0);
    for (int32_t i : order) {  // root first: ancestor range counts
      const int32_t pa = parent[i];
      if (pa < 0) continue;
      const bool merged = nanc[pa] > 0 && anc_end[pa] == seg_start[pa];
      nanc[i] = nanc[pa] + (merged ? 0 : 1);
      anc_end[i] = static_cast<int64_t>(seg_start[pa]) + seg_len[pa];
    }
    for (size_t h = order.size(); h-- > 0;) {  // leaves first: query nodes below
      const int32_t i = order[h];
      act_sub[i] += active[i] ? 1 : 0;
      if (parent[i] >= 0) act_sub[parent[i]] += act_sub[i];
    }
    int64_t fwd_entries = 0, bwd_ranges = 0;
    std::vector<int64_t> side_cnt(m, 0);
    for (int64_t i = 0; i < m; ++i) {
      const int64_t end = static_cast<int64_t>(seg_start[i]) + seg_len[i];
      for (int32_t c : children[i])
        if (p.subset || seg_start[c] != end) side_cnt[i] += act_sub[c];
      if (active[i])
        fwd_entries += ((static_cast<int64_t>(seg_len[i]) + kFwdRows - 1) / kFwdRows) * (nanc[i] + 1);
    }
    // a key tile of a run collects the side ranges of the run's nodes from
    // its own on: bounded by the run's tiles times the run's side ranges
    for (int32_t r : order) {
      const int32_t pa = parent[r];
      const bool cont = !p.subset && pa >= 0 &&
                        static_cast<int64_t>(seg_start[pa]) + seg_len[pa] == seg_start[r];
      if (cont) continue;  // not the start of a run
      int64_t len = 0, sides = 0;
      for (int32_t c = r; c >= 0;) {
        len += seg_len[c];
        sides += side_cnt[c];
        const int64_t end = static_cast<int64_t>(seg_start[c]) + seg_len[c];
        int32_t nx = -1;
        if (!p.subset)
          for (int32_t cc : children[c])
            if (seg_start[cc] == end) nx = cc;
        c = nx;
      }
      bwd_ranges += ((len + kBwdKeys - 1) / kBwdKeys) * (sides + 1);
      if (bwd_ranges > kMaxRangeEntries) break;
    }
    if (fwd_entries > kMaxRangeEntries || bwd_ranges * num_q_heads > kMaxRangeEntries) {
      std::ostringstream os;
      os << "the plan would hold " << std::max(fwd_entries, bwd_ranges * num_q_heads)
         << " key-range entries (limit " << kMaxRangeEntries
         << "): store each node's segment after its parent's (depth-first preorder)";
      return fail(err, Status::kUnsupported, os.str());
    }
  }

  // ---- ancestor key ranges (root first, merged when contiguous) and depth
  // offsets, in root-first order so a parent is done before its children
  std::vector<std::vector<Range>> anc(m);
  std::vector<int64_t> depth(m, 0);
  for (int32_t i : order) {
    const int32_t pa = parent[i];
    if (pa < 0) continue;
    anc[i] = anc[pa];
    push_range(anc[i], seg_start[pa], static_cast<int64_t>(seg_start[pa]) + seg_len[pa]);
    depth[i] = depth[pa] + seg_len[pa];
  }
  p.segments.reserve(m);
  for (int32_t i : by_start)
    p.segments.push_back({seg_start[i], seg_len[i], static_cast<int32_t>(depth[i]), i});
  build_lin_pieces(parent, seg_start, seg_len, order, children, depth, &p);
  p.pairs = 0;
  p.query_rows = 0;
  for (int64_t i = 0; i < m; ++i) {
    if (!active[i]) continue;
    const int64_t L = seg_len[i];
    p.pairs += L * depth[i] + L * (L + 1) / 2;
    p.query_rows += L;
  }

  // ---- forward query tiles, over runs: a node whose segment starts where
  // its parent's ends (depth-first packing puts a first child there)
  // continues its parent's run.  Every row of a run sees the run's first
  // node's ancestors and the run's earlier rows, so query tiles may cross
  // node boundaries inside a run, and the last tile of a short node is not
  // left ragged.
  std::vector<int64_t> run_end(m, -1);  // run start node -> end row of its run
  std::vector<int32_t> run_of(m);       // node -> start node of its run
  for (int32_t i : order) {
    const int32_t pa = parent[i];
    const bool cont = pa >= 0 && active[i] && active[pa] &&
                      static_cast<int64_t>(seg_start[pa]) + seg_len[pa] == seg_start[i];
    run_of[i] = cont ? run_of[pa] : i;
    run_end[run_of[i]] = static_cast<int64_t>(seg_start[i]) + seg_len[i];
  }
  struct FTile {
    I4 t;
    int64_t cost;
    int32_t part;
  };
  std::vector<FTile> ftiles;
  std::vector<I4> franges;
  for (int64_t i = 0; i < m; ++i) {
    if (!active[i] || run_of[i] != i) continue;
    const int64_t s = seg_start[i], e = run_end[i];
    for (int64_t r0 = s; r0 < e; r0 += kFwdRows) {
      const int64_t r1 = std::min<int64_t>(e, r0 + kFwdRows);
      const int32_t rb = static_cast<int32_t>(franges.size());
      int64_t keys = 0;
      const auto& a = anc[i];
      for (size_t j = 0; j < a.size(); ++j) {
        const bool last = j + 1 == a.size();
        if (last && a[j].e == s) break;  // merged into the causal range below
        franges.push_back({static_cast<int32_t>(a[j].b), static_cast<int32_t>(a[j].e), 0, 0});
        keys += a[j].e - a[j].b;
      }
      const int64_t cb = (!a.empty() && a.back().e == s) ? a.back().b : s;
      franges.push_back({static_cast<int32_t>(cb), static_cast<int32_t>(r1), 1, 0});
      keys += r1 - cb;
      ftiles.push_back({{static_cast<int32_t>(r0), static_cast<int32_t>(r1), rb,
                         static_cast<int32_t>(franges.size())},
                        (r1 - r0) * keys, -1});
    }
  }
  p.fwd_qtiles.reserve(ftiles.size());
  for (auto& t : ftiles) p.fwd_qtiles.push_back({t.t.x, t.t.y, 0, 0});
  // ---- forward key splitting.  When (tile, head) workgroups would leave
  // CUs idle (small trees, and the one-node calls of a depth-first walk,
  // whose few query tiles each see a long ancestor path), a tile's keys are
  // cut into parts, with parts in proportion to the tile's cost and at most
  // kFwdFill workgroups per CU in all: a part then runs alone on its CU at
  // full speed, where two workgroups sharing one would each run slower and
  // a launch past one round would add a second.  Each part keeps at least
  // kFwdMinPartSteps steps (a
  // shorter part would save less time than the merge costs).  The merge
  // passes (forward and dQ) are two more launches of fixed cost, about as
  // long as 15 key steps of one workgroup, so a plan splits only when its
  // longest tile has at least kFwdSplitSteps steps.  A part keeps
  // the tile's rows and a contiguous run of its key steps (cuts fall on
  // kFwdKeys boundaries of a range, so no part adds a ragged step); the
  // parts' partial softmax results are merged after the launch.  Every
  // (query, key) pair stays in exactly one item.
  {
    const int64_t items = static_cast<int64_t>(ftiles.size()) * num_q_heads;
    const int64_t target = static_cast<int64_t>(kFwdFill) * num_cus;
    auto tile_steps = [&](const FTile& t) {
      int64_t steps = 0;
      for (int32_t r = t.t.z; r < t.t.w; ++r)
        steps += (static_cast<int64_t>(franges[r].y) - franges[r].x + kFwdKeys - 1) / kFwdKeys;
      return steps;
    };
    int64_t longest = 0;
    for (const FTile& t : ftiles) longest = std::max(longest, tile_steps(t));
    if (items > 0 && items < target && longest >= kFwdSplitSteps) {
      const double want = static_cast<double>(target) / static_cast<double>(num_q_heads);
      double total = 0;
      for (const FTile& t : ftiles) total += static_cast<double>(t.cost);
      std::vector<FTile> out;
      out.reserve(ftiles.size() * 2);
      for (const FTile& t : ftiles) {
        const int64_t steps = tile_steps(t);
        int64_t parts =
            total > 0 ? static_cast<int64_t>(want * static_cast<double>(t.cost) / total) : 1;
        parts = std::max<int64_t>(
            1, std::min<int64_t>({parts, steps / kFwdMinPartSteps, kFwdMaxParts}));
        if (parts == 1) {
          out.push_back(t);
          continue;
        }
        const int32_t slot0 = static_cast<int32_t>(p.fwd_slots);
        p.fwd_combine.push_back({t.t.x, t.t.y, slot0, static_cast<int32_t>(parts)});
        p.fwd_slots += parts;
        int32_t r = t.t.z;
        int64_t pos = franges[r].x;
        for (int64_t i = 0; i < parts; ++i) {
          int64_t need = steps / parts + (i < steps % parts ? 1 : 0);
          const int32_t rb = static_cast<int32_t>(franges.size());
          int64_t keys = 0;
          while (need > 0) {
            const I4 rg = franges[r];  // copy: franges grows below
            const int64_t left = (static_cast<int64_t>(rg.y) - pos + kFwdKeys - 1) / kFwdKeys;
            if (left <= 0) {  // an empty range (none are built; kept safe)
              if (r + 1 >= t.t.w) break;
              ++r;
              pos = franges[r].x;
              continue;
            }
            const int64_t take = std::min(need, left);
            const int64_t end = std::min<int64_t>(rg.y, pos + take * kFwdKeys);
            franges.push_back({static_cast<int32_t>(pos), static_cast<int32_t>(end), rg.z, 0});
            keys += end - pos;
            need -= take;
            pos = end;
            if (pos == rg.y && r + 1 < t.t.w) {
              ++r;
              pos = franges[r].x;
            }
          }
          out.push_back({{t.t.x, t.t.y, rb, static_cast<int32_t>(franges.size())},
                         (t.t.y - t.t.x) * keys, slot0 + static_cast<int32_t>(i)});
        }
      }
      ftiles = std::move(out);
    }
  }
  std::stable_sort(ftiles.begin(), ftiles.end(),
                   [](const FTile& a, const FTile& b) { return a.cost > b.cost; });
  p.fwd_tiles.reserve(ftiles.size());
  p.fwd_part.reserve(ftiles.size());
  for (auto& t : ftiles) {
    p.fwd_tiles.push_back(t.t);
    p.fwd_part.push_back(t.part);
  }
  p.fwd_ranges = std::move(franges);
  const int64_t gsize = num_q_heads / num_kv_heads;
  p.fwd_groups = static_cast<int64_t>(p.fwd_tiles.size()) * num_kv_heads;
  p.fwd_blocks = ((p.fwd_groups + kXcds - 1) / kXcds) * kXcds * gsize;

  // ---- backward key tiles over runs.  With a run n_1 .. n_k (each node the
  // contiguous child of the previous), a key of n_c is seen by the run's
  // later rows (causal) and by the side subtrees -- subtrees of the
  // children that do not continue the run -- of n_c .. n_k.  A key tile
  // that starts in n_a and ends in n_b is therefore seen in full by the side
  // subtrees of n_b .. n_k, and by those of n_j (a <= j < b) only up to the
  // end of n_j: a key-limit entry.  Key tiles then cross node boundaries
  // inside a run, so a short node does not leave a ragged tile that its
  // whole descendant set would walk.  Query-subset plans keep one node per
  // run (only their query nodes' rows are queries).
  std::vector<int32_t> next_in_run(m, -1);
  std::vector<char> continues(m, 0);
  if (!p.subset)
    for (int64_t i = 0; i < m; ++i) {
      const int32_t pa = parent[i];
      if (pa >= 0 && static_cast<int64_t>(seg_start[pa]) + seg_len[pa] == seg_start[i]) {
        next_in_run[pa] = static_cast<int32_t>(i);
        continues[i] = 1;
      }
    }
  // side-subtree segments of each node that hold queries, sorted by start
  // and merged
  std::vector<std::vector<Range>> side(m);
  {
    std::vector<int32_t> stack;
    for (int64_t i = 0; i < m; ++i) {
      std::vector<Range> segs;
      stack.clear();
      for (int32_t c : children[i])
        if (c != next_in_run[i]) stack.push_back(c);
      while (!stack.empty()) {
        const int32_t c = stack.back();
        stack.pop_back();
        if (active[c])
          segs.push_back({seg_start[c], static_cast<int64_t>(seg_start[c]) + seg_len[c]});
        for (int32_t cc : children[c]) stack.push_back(cc);
      }
      std::sort(segs.begin(), segs.end(), [](const Range& a, const Range& b) { return a.b < b.b; });
      for (auto& r : segs) push_range(side[i], r.b, r.e);
    }
  }
  struct BItem {
    int64_t k0, k1, g, slot;
    std::vector<I4> entries;
    int64_t cost;
    int64_t node, chunk;  // node of the key tile's last key, chunk of a split tile
  };
  std::vector<BItem> items;
  int64_t total_cost = 0;
  struct KTile {
    int64_t k0, k1, node;
    std::vector<Range> causal, full;  // query ranges
    std::vector<std::pair<Range, int64_t>> limited;  // query range, keys < limit
    int64_t rows;
  };
  std::vector<KTile> ktiles;
  auto seg_end = [&](int32_t i) { return static_cast<int64_t>(seg_start[i]) + seg_len[i]; };
  for (int64_t r = 0; r < m; ++r) {
    if (continues[r]) continue;
    std::vector<int32_t> run;
    for (int32_t c = static_cast<int32_t>(r); c >= 0; c = next_in_run[c]) run.push_back(c);
    const int64_t s = seg_start[r], e = seg_end(run.back());
    size_t a = 0;
    for (int64_t k0 = s; k0 < e; k0 += kBwdKeys) {
      KTile kt;
      kt.k0 = k0;
      kt.k1 = std::min<int64_t>(e, k0 + kBwdKeys);
      while (seg_end(run[a]) <= k0) ++a;  // node of the first key
      size_t b = a;
      while (seg_end(run[b]) < kt.k1) ++b;  // node of the last key
      // placement groups tiles by the node of their last key: the tiles of
      // one node read the same rows, those of another node of the run fewer
      kt.node = run[b];
      // rows that see every key: side subtrees of n_b .. n_k
      std::vector<Range> segs, full;
      for (size_t j = b; j < run.size(); ++j)
        segs.insert(segs.end(), side[run[j]].begin(), side[run[j]].end());
      std::sort(segs.begin(), segs.end(), [](const Range& x, const Range& y) { return x.b < y.b; });
      for (auto& rg : segs) push_range(full, rg.b, rg.e);
      // the run from the tile's first row on (causal) when its rows are
      // queries, merged with the full ranges that follow it contiguously
      kt.rows = 0;
      if (active[run[a]]) {
        Range own{k0, e};
        for (const Range& f : full) {
          if (f.b == own.e) own.e = f.e;
          else kt.full.push_back(f);
        }
        kt.causal.push_back(own);
        kt.rows = own.e - own.b;
      } else {
        kt.full = full;
      }
      for (auto& rg : kt.full) kt.rows += rg.e - rg.b;
      // side subtrees of n_a .. n_(b-1): only the keys before their node's end
      for (size_t j = a; j < b; ++j)
        for (const Range& rg : side[run[j]]) {
          p.bwd_has_limit = true;
          kt.limited.push_back({rg, seg_end(run[j])});
          kt.rows += rg.e - rg.b;
        }
      if (kt.rows == 0) continue;  // no query sees this tile
      total_cost += kt.rows * (kt.k1 - kt.k0) * gsize;
      ktiles.push_back(std::move(kt));
    }
  }
  total_cost *= num_kv_heads;
  // Split heavy key tiles along their query rows so that no item exceeds
  // about 1/(8 * num_cus) of the total; split chunks write fp32 partial dK/dV
  // slots that a fixed-order reduction sums afterwards.
  const int64_t cap = std::max<int64_t>(total_cost / (8 * static_cast<int64_t>(p.num_cus)),
                                        static_cast<int64_t>(kBwdKeys) * kBwdRows * 64);
  int64_t slots = 0;
  for (const KTile& kt : ktiles) {
    const int64_t nk = kt.k1 - kt.k0;
    for (int64_t g = 0; g < num_kv_heads; ++g) {
      std::vector<I4> all;
      for (int64_t h = g * gsize; h < (g + 1) * gsize; ++h) {
        for (auto& r : kt.causal)
          all.push_back({static_cast<int32_t>(h), static_cast<int32_t>(r.b),
                         static_cast<int32_t>(r.e), 1});
        for (auto& r : kt.full)
          all.push_back({static_cast<int32_t>(h), static_cast<int32_t>(r.b),
                         static_cast<int32_t>(r.e), 0});
        for (auto& rl : kt.limited)  // keys >= limit hidden: w = -(limit + 1)
          all.push_back({static_cast<int32_t>(h), static_cast<int32_t>(rl.first.b),
                         static_cast<int32_t>(rl.first.e),
                         static_cast<int32_t>(-(rl.second + 1))});
      }
      const int64_t cost = kt.rows * gsize * nk;
      if (cost <= cap && !p.subset) {
        items.push_back({kt.k0, kt.k1, g, -1, std::move(all), cost, kt.node, 0});
        continue;
      }
      // chunk the entries (rows cut at kBwdRows boundaries of each entry)
      const int64_t slot_begin = slots;
      int64_t chunk = 0;
      BItem cur{kt.k0, kt.k1, g, slots, {}, 0, kt.node, chunk};
      for (const I4& en : all) {
        int64_t q0 = en.y;
        while (q0 < en.z) {
          const int64_t room_rows = std::max<int64_t>(
              kBwdRows, ((cap - cur.cost) / nk + kBwdRows - 1) / kBwdRows * kBwdRows);
          const int64_t q1 = std::min<int64_t>(en.z, q0 + room_rows);
          cur.entries.push_back({en.x, static_cast<int32_t>(q0), static_cast<int32_t>(q1), en.w});
          cur.cost += (q1 - q0) * nk;
          q0 = q1;
          if (cur.cost >= cap) {
            items.push_back(std::move(cur));
            ++slots;
            cur = BItem{kt.k0, kt.k1, g, slots, {}, 0, kt.node, ++chunk};
          }
        }
      }
      if (!cur.entries.empty()) {
        items.push_back(std::move(cur));
        ++slots;
      }
      p.bwd_reduce.push_back({{static_cast<int32_t>(kt.k0), static_cast<int32_t>(kt.k1),
                               static_cast<int32_t>(g), static_cast<int32_t>(slot_begin),
                               static_cast<int32_t>(slots - slot_begin), 0, 0, 0}});
      ++p.bwd_split_tiles;
    }
  }
  p.bwd_slots = slots;

  // Placement.  The key tiles of one node (and, for split tiles, the same
  // chunk of each) read the same query rows of the same heads: a group.
  // Workgroup b is dispatched to XCD b % 8 and each XCD takes its workgroups
  // in order, so
  //  * each group goes whole to one XCD, groups longest first onto the XCD
  //    with the least work so far, and its re-reads of the rows can hit
  //    that XCD's L2;
  //  * an XCD takes its groups eight at a time and interleaves them by rank
  //    (the largest item of each, then the second largest, ...): a few items
  //    of a group run side by side, not all at once on the same rows;
  //  * the last 40% of an XCD's work is ordered longest first, so that it
  //    ends on short items;
  // and the queues are interleaved into the launch order, with empty items
  // (no entries) filling the ends of the shorter queues.
  std::map<std::tuple<int64_t, int64_t, int64_t>, std::vector<int64_t>> groups;
  for (int64_t ii = 0; ii < static_cast<int64_t>(items.size()); ++ii) {
    const BItem& it = items[ii];
    groups[{it.node, it.g, it.chunk}].push_back(ii);
  }
  struct Group {
    int64_t cost;
    std::vector<int64_t> members;
  };
  std::vector<Group> glist;
  for (auto& kv : groups) {
    Group gr{0, std::move(kv.second)};
    for (int64_t ii : gr.members) gr.cost += items[ii].cost;
    std::stable_sort(gr.members.begin(), gr.members.end(),
                     [&](int64_t a, int64_t b) { return items[a].cost > items[b].cost; });
    glist.push_back(std::move(gr));
  }
  std::stable_sort(glist.begin(), glist.end(),
                   [](const Group& a, const Group& b) { return a.cost > b.cost; });
  constexpr size_t kBatch = 8;          // groups interleaved together on an XCD
  constexpr int64_t kTailPercent = 40;  // share of an XCD's work sorted longest first
  std::vector<int64_t> qg[kXcds];
  int64_t load[kXcds] = {};
  for (int64_t gi = 0; gi < static_cast<int64_t>(glist.size()); ++gi) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    load[x] += glist[gi].cost;
    qg[x].push_back(gi);
  }
  std::vector<int64_t> queue[kXcds];
  for (int x = 0; x < kXcds; ++x) {
    for (size_t b0 = 0; b0 < qg[x].size(); b0 += kBatch) {
      const size_t b1 = std::min(qg[x].size(), b0 + kBatch);
      for (size_t r = 0;; ++r) {
        bool any = false;
        for (size_t b = b0; b < b1; ++b) {
          const auto& mem = glist[qg[x][b]].members;
          if (r < mem.size()) {
            queue[x].push_back(mem[r]);
            any = true;
          }
        }
        if (!any) break;
      }
    }
    int64_t acc = 0;
    size_t cut = queue[x].size();
    for (size_t q = 0; q < queue[x].size(); ++q) {
      acc += items[queue[x][q]].cost;
      if (acc * 100 >= load[x] * (100 - kTailPercent)) {
        cut = q + 1;
        break;
      }
    }
    std::stable_sort(queue[x].begin() + cut, queue[x].end(),
                     [&](int64_t a, int64_t b) { return items[a].cost > items[b].cost; });
  }
  size_t qlen = 0;
  for (int x = 0; x < kXcds; ++x) qlen = std::max(qlen, queue[x].size());
  for (size_t q = 0; q < qlen; ++q) {
    for (int x = 0; x < kXcds; ++x) {
      const int32_t eb = static_cast<int32_t>(p.bwd_entries.size());
      if (q >= queue[x].size()) {
        p.bwd_items.push_back({{0, 0, 0, eb, eb, -1, -1, 0}});
        continue;
      }
      const BItem& it = items[queue[x][q]];
      p.bwd_entries.insert(p.bwd_entries.end(), it.entries.begin(), it.entries.end());
      p.bwd_items.push_back({{static_cast<int32_t>(it.k0), static_cast<int32_t>(it.k1),
                              static_cast<int32_t>(it.g), eb,
                              static_cast<int32_t>(p.bwd_entries.size()),
                              static_cast<int32_t>(it.slot), x, 0}});
    }
  }
  return Status::kOk;
}

// AReaL-DTA (abstract) walks the tree depth first with one root-to-leaf path
// resident at a time.  Nodes that follow one another in preorder share most
// of their root paths, so several of them fit in the rows one deep path
// needs; each run is one query-subset call of the walk.
Status walk_runs(const int32_t* parent, const int32_t* seg_len, int32_t num_nodes,
                 int64_t budget, int32_t* order, int32_t* run_start, int32_t* num_runs,
                 std::string* err) {
  if (num_nodes < 0 || !num_runs || !run_start ||
      (num_nodes > 0 && (!parent || !seg_len || !order)))
    return fail(err, Status::kInvalidArg, "null pointer or negative node count");
  const int64_t m = num_nodes;
  for (int64_t i = 0; i < m; ++i) {
    if (parent[i] < -1 || parent[i] >= m || parent[i] == i) {
      std::ostringstream os;
      os << "node " << i << " has invalid parent " << parent[i];
      return fail(err, Status::kBadTree, os.str());
    }
    if (seg_len[i] < 1) {
      std::ostringstream os;
      os << "node " << i << " has segment length " << seg_len[i];
      return fail(err, Status::kLayout, os.str());
    }
  }
  // children in index order; preorder by an explicit stack
  std::vector<int32_t> first(m + 1, 0), kids(m);
  for (int64_t i = 0; i < m; ++i)
    if (parent[i] >= 0) ++first[parent[i] + 1];
  for (int64_t i = 0; i < m; ++i) first[i + 1] += first[i];
  {
    std::vector<int32_t> fill(first.begin(), first.end() - 1);
    for (int64_t i = 0; i < m; ++i)
      if (parent[i] >= 0) kids[fill[parent[i]]++] = static_cast<int32_t>(i);
  }
  std::vector<int32_t> stack;
  for (int64_t i = m - 1; i >= 0; --i)
    if (parent[i] < 0) stack.push_back(static_cast<int32_t>(i));
  std::vector<int64_t> path(m, 0);  // tokens on the root path, the node's own included
  int64_t n_order = 0, longest = 0;
  while (!stack.empty()) {
    const int32_t v = stack.back();
    stack.pop_back();
    order[n_order++] = v;
    path[v] = (parent[v] >= 0 ? path[parent[v]] : 0) + seg_len[v];
    longest = std::max(longest, path[v]);
    for (int32_t c = first[v + 1] - 1; c >= first[v]; --c) stack.push_back(kids[c]);
  }
  if (n_order != m) return fail(err, Status::kBadTree, "parent pointers contain a cycle");
  if (budget <= 0) budget = longest;

  // greedy cut.  The nodes of a run are consecutive in preorder, so the
  // part of a new node's root path that the run already holds is the root
  // path of its lowest common ancestor with the previous node: no earlier
  // node shares a deeper ancestor with it.  Walking up from the new node to
  // that ancestor visits only nodes that preorder enters there, O(M) in all.
  std::vector<int32_t> tin(m), sub(m, 0);
  for (int64_t j = 0; j < m; ++j) tin[order[j]] = static_cast<int32_t>(j);
  for (int64_t j = m - 1; j >= 0; --j) {
    const int32_t v = order[j];
    sub[v] += 1;
    if (parent[v] >= 0) sub[parent[v]] += sub[v];
  }
  auto holds = [&](int32_t a, int32_t v) { return tin[a] <= tin[v] && tin[v] < tin[a] + sub[a]; };
  int32_t runs = 0;
  int64_t resident = 0;
  run_start[0] = 0;
  for (int64_t j = 0; j < m; ++j) {
    const int32_t v = order[j];
    int64_t add = path[v];
    if (runs > 0) {
      const int32_t prev = order[j - 1];
      int32_t u = parent[v];
      while (u >= 0 && !holds(u, prev)) u = parent[u];
      add = path[v] - (u >= 0 ? path[u] : 0);
    }
    if (runs == 0 || resident + add > budget) {
      // close the current run (if any) and open one at v
      if (runs > 0) run_start[runs] = static_cast<int32_t>(j);
      ++runs;
      resident = 0;
      add = path[v];
    }
    resident += add;
  }
  run_start[runs] = static_cast<int32_t>(m);
  *num_runs = runs;
  return Status::kOk;
}

}  // namespace tree_attn
