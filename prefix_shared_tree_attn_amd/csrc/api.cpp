// C ABI of libtree_attn.so: plan objects, argument checks and launches.
// The operations are defined in include/tree_attn.h.
#include "tree_attn.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "planner.h"
#include "prefix_tree.h"

using tree_attn::HostPlan;
using tree_attn::I4;
using tree_attn::I8;
using tree_attn::Status;

struct tree_attn_plan_s {
  HostPlan hp;
  bool has_device = false;
  int device = -1;
  char* dev_buf = nullptr;
  const I4* d_fwd_tiles = nullptr;
  const I4* d_fwd_ranges = nullptr;
  const int32_t* d_fwd_part = nullptr;
  const I4* d_fwd_combine = nullptr;
  const I4* d_fwd_qtiles = nullptr;
  const I8* d_bwd_items = nullptr;
  const I4* d_bwd_entries = nullptr;
  const I8* d_bwd_reduce = nullptr;
  const I4* d_segments = nullptr;
  const I8* d_lin_pieces = nullptr;
  const int32_t* d_lin_succ = nullptr;
  const I4* d_lin_nodes = nullptr;
  const int32_t* d_lin_chain_nodes = nullptr;
  const I4* d_lin_chains = nullptr;
};

namespace {

thread_local std::string g_last_error;

tree_attn_status_t report(Status s, const std::string& msg) {
  g_last_error = msg;
  return static_cast<tree_attn_status_t>(s);
}

tree_attn_status_t report_hip(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return TREE_ATTN_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The kernels move tensor rows in 16-byte pieces (vector loads and
// buffer-to-LDS transfers), so every tensor pointer must be 16-byte aligned.
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
  return true;
}

// Softmax attention masks scores with -inf and scales them afterwards, and
// the forward pass takes row maxima on unscaled scores: the scale must be a
// positive finite number.
bool valid_softmax_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Key parts of split forward tiles: fp32 [slots, Hq, kFwdRows, D] partial O
// (forward) or partial dQ (backward), and [slots, Hq, kFwdRows, 2] reference
// and row sum (forward).
size_t part_rows(const HostPlan& p) {
  return static_cast<size_t>(p.fwd_slots) * p.hq * tree_attn::kFwdRows;
}

struct FwdLayout {
  size_t o_part = 0, ml_part = 0, total = 0;
};

FwdLayout fwd_layout(const HostPlan& p) {
  FwdLayout l;
  if (p.fwd_slots == 0 || p.num_tokens == 0) return l;
  l.ml_part = align256(part_rows(p) * p.head_dim * 4);
  l.total = l.ml_part + align256(part_rows(p) * 2 * 4);
  return l;
}

struct BwdLayout {
  size_t neg_d = 0, neg_lse2 = 0, dk_slots = 0, dv_slots = 0, dq_part = 0, total = 0;
};

BwdLayout bwd_layout(const HostPlan& p) {
  BwdLayout l;
  const size_t dv = static_cast<size_t>(p.num_tokens) * p.hq * 4;
  const size_t slot =
      static_cast<size_t>(p.bwd_slots) * tree_attn::kBwdKeys * p.head_dim * 4;
  l.neg_d = 0;
  l.neg_lse2 = align256(dv);
  l.dk_slots = l.neg_lse2 + align256(dv);
  l.dv_slots = l.dk_slots + align256(slot);
  l.dq_part = l.dv_slots + align256(slot);
  l.total = l.dq_part + align256(part_rows(p) * p.head_dim * 4);
  if (p.num_tokens == 0) l.total = 0;
  return l;
}

// Linear attention workspace: bf16 piece states and per-piece deltas, each
// [pieces, Hkv, D, D], and fp32 node-end states [nodes, Hkv, D, D]; the
// backward pass adds the bf16 state gradients.
size_t lin_block(const HostPlan& p) {
  return align256(p.lin_pieces.size() * static_cast<size_t>(p.hkv) * p.head_dim * p.head_dim * 2);
}
size_t lin_ends(const HostPlan& p) {
  return align256(static_cast<size_t>(p.num_nodes) * p.hkv * p.head_dim * p.head_dim * 4);
}

tree_attn_status_t make_host_plan(const int32_t* parent, const int32_t* seg_start,
                                  const int32_t* seg_len, int32_t num_nodes, int32_t num_tokens,
                                  int32_t hq, int32_t hkv, int32_t head_dim,
                                  tree_attn_dtype_t dtype, int num_cus, tree_attn_plan_s** out,
                                  const int32_t* query_nodes = nullptr,
                                  int32_t num_query_nodes = 0) {
  if (!out) return report(Status::kInvalidArg, "null output plan pointer");
  tree_attn_plan_s* p = new (std::nothrow) tree_attn_plan_s();
  if (!p) return report(Status::kInvalidArg, "out of host memory");
  std::string err;
  const Status s = tree_attn::build_plan(parent, seg_start, seg_len, num_nodes, num_tokens, hq,
                                         hkv, head_dim, static_cast<int>(dtype), num_cus,
                                         &p->hp, &err, query_nodes, num_query_nodes);
  if (s != Status::kOk) {
    delete p;
    return report(s, err);
  }
  *out = p;
  return TREE_ATTN_OK;
}

template <typename V>
size_t bytes_of(const V& v) {
  return v.size() * sizeof(typename V::value_type);
}

// Optional per-kernel timing: HIP events around each launch, read later.
constexpr int kTimingKinds = 16;
struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  struct Rec {
    int kind;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  int64_t launches[kTimingKinds] = {};
  double total_ms[kTimingKinds] = {};
};

Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event(Timing& t) {
  hipEvent_t e = nullptr;
  if (!t.pool.empty()) {
    e = t.pool.back();
    t.pool.pop_back();
  } else if (hipEventCreate(&e) != hipSuccess) {
    e = nullptr;
  }
  return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  Timing& t = timing();
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> g(t.mu);
    if (t.enabled) {
      a = take_event(t);
      b = take_event(t);
    }
  }
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  const hipError_t e2 = hipEventRecord(b, s);
  std::lock_guard<std::mutex> g(t.mu);
  t.recs.push_back({kind, a, b});
  return e != hipSuccess ? e : e2;
}

tree_attn_status_t check_device(const tree_attn_plan_s* p) {
  if (!p) return report(Status::kInvalidArg, "null plan");
  if (!p->has_device)
    return report(Status::kNoDevicePlan, "plan was built with tree_attn_plan_host");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report_hip(e, "hipGetDevice");
  if (dev != p->device)
    return report(Status::kInvalidArg, "plan belongs to device " + std::to_string(p->device) +
                                           ", current device is " + std::to_string(dev));
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

tree_attn_status_t tree_attn_plan_host(const int32_t* parent, const int32_t* seg_start,
                                       const int32_t* seg_len, int32_t num_nodes,
                                       int32_t num_tokens, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       tree_attn_dtype_t dtype, int32_t num_cus,
                                       tree_attn_plan_t* out) {
  return make_host_plan(parent, seg_start, seg_len, num_nodes, num_tokens, num_q_heads,
                        num_kv_heads, head_dim, dtype, num_cus, out);
}

tree_attn_status_t tree_attn_plan_host_subset(const int32_t* parent, const int32_t* seg_start,
                                              const int32_t* seg_len, int32_t num_nodes,
                                              int32_t num_tokens, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              tree_attn_dtype_t dtype,
                                              const int32_t* query_nodes,
                                              int32_t num_query_nodes, int32_t num_cus,
                                              tree_attn_plan_t* out) {
  if (!query_nodes && num_query_nodes != 0)
    return report(Status::kInvalidArg, "null query-node list");
  static const int32_t kNone = 0;
  return make_host_plan(parent, seg_start, seg_len, num_nodes, num_tokens, num_q_heads,
                        num_kv_heads, head_dim, dtype, num_cus, out,
                        query_nodes ? query_nodes : &kNone, num_query_nodes);
}

}  // extern "C"

namespace {

tree_attn_status_t device_plan(const int32_t* parent, const int32_t* seg_start,
                               const int32_t* seg_len, int32_t num_nodes, int32_t num_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               tree_attn_dtype_t dtype, const int32_t* query_nodes,
                               int32_t num_query_nodes, hipStream_t stream,
                               tree_attn_plan_t* out) {
  if (!out) return report(Status::kInvalidArg, "null output plan pointer");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report_hip(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return report_hip(e, "hipDeviceGetAttribute");
  tree_attn_plan_s* p = nullptr;
  tree_attn_status_t st =
      make_host_plan(parent, seg_start, seg_len, num_nodes, num_tokens, num_q_heads,
                     num_kv_heads, head_dim, dtype, cus, &p, query_nodes, num_query_nodes);
  if (st != TREE_ATTN_OK) return st;
  const HostPlan& hp = p->hp;
  const size_t o_ft = 0;
  const size_t o_fr = o_ft + align256(bytes_of(hp.fwd_tiles));
  const size_t o_fp = o_fr + align256(bytes_of(hp.fwd_ranges));
  const size_t o_fc = o_fp + align256(bytes_of(hp.fwd_part));
  const size_t o_fq = o_fc + align256(bytes_of(hp.fwd_combine));
  const size_t o_bi = o_fq + align256(bytes_of(hp.fwd_qtiles));
  const size_t o_be = o_bi + align256(bytes_of(hp.bwd_items));
  const size_t o_br = o_be + align256(bytes_of(hp.bwd_entries));
  const size_t o_sg = o_br + align256(bytes_of(hp.bwd_reduce));
  const size_t o_lp = o_sg + align256(bytes_of(hp.segments));
  const size_t o_ls = o_lp + align256(bytes_of(hp.lin_pieces));
  const size_t o_ln = o_ls + align256(bytes_of(hp.lin_succ));
  const size_t o_lcn = o_ln + align256(bytes_of(hp.lin_nodes));
  const size_t o_lc = o_lcn + align256(bytes_of(hp.lin_chain_nodes));
  const size_t total = o_lc + align256(bytes_of(hp.lin_chains));
  if (total > 0) {
    e = hipMalloc(reinterpret_cast<void**>(&p->dev_buf), total);
    if (e != hipSuccess) {
      delete p;
      return report_hip(e, "hipMalloc(plan arrays)");
    }
    struct Part {
      size_t off;
      const void* src;
      size_t n;
    } parts[] = {{o_ft, hp.fwd_tiles.data(), bytes_of(hp.fwd_tiles)},
                 {o_fr, hp.fwd_ranges.data(), bytes_of(hp.fwd_ranges)},
                 {o_fp, hp.fwd_part.data(), bytes_of(hp.fwd_part)},
                 {o_fc, hp.fwd_combine.data(), bytes_of(hp.fwd_combine)},
                 {o_fq, hp.fwd_qtiles.data(), bytes_of(hp.fwd_qtiles)},
                 {o_bi, hp.bwd_items.data(), bytes_of(hp.bwd_items)},
                 {o_be, hp.bwd_entries.data(), bytes_of(hp.bwd_entries)},
                 {o_br, hp.bwd_reduce.data(), bytes_of(hp.bwd_reduce)},
                 {o_sg, hp.segments.data(), bytes_of(hp.segments)},
                 {o_lp, hp.lin_pieces.data(), bytes_of(hp.lin_pieces)},
                 {o_ls, hp.lin_succ.data(), bytes_of(hp.lin_succ)},
                 {o_ln, hp.lin_nodes.data(), bytes_of(hp.lin_nodes)},
                 {o_lcn, hp.lin_chain_nodes.data(), bytes_of(hp.lin_chain_nodes)},
                 {o_lc, hp.lin_chains.data(), bytes_of(hp.lin_chains)}};
    for (const Part& part : parts) {
      if (part.n == 0) continue;
      e = hipMemcpyAsync(p->dev_buf + part.off, part.src, part.n, hipMemcpyHostToDevice, stream);
      if (e != hipSuccess) {
        (void)hipFree(p->dev_buf);
        delete p;
        return report_hip(e, "hipMemcpyAsync(plan arrays)");
      }
    }
  }
  p->d_fwd_tiles = reinterpret_cast<const I4*>(p->dev_buf + o_ft);
  p->d_fwd_ranges = reinterpret_cast<const I4*>(p->dev_buf + o_fr);
  p->d_fwd_part = reinterpret_cast<const int32_t*>(p->dev_buf + o_fp);
  p->d_fwd_combine = reinterpret_cast<const I4*>(p->dev_buf + o_fc);
  p->d_fwd_qtiles = reinterpret_cast<const I4*>(p->dev_buf + o_fq);
  p->d_bwd_items = reinterpret_cast<const I8*>(p->dev_buf + o_bi);
  p->d_bwd_entries = reinterpret_cast<const I4*>(p->dev_buf + o_be);
  p->d_bwd_reduce = reinterpret_cast<const I8*>(p->dev_buf + o_br);
  p->d_segments = reinterpret_cast<const I4*>(p->dev_buf + o_sg);
  p->d_lin_pieces = reinterpret_cast<const I8*>(p->dev_buf + o_lp);
  p->d_lin_succ = reinterpret_cast<const int32_t*>(p->dev_buf + o_ls);
  p->d_lin_nodes = reinterpret_cast<const I4*>(p->dev_buf + o_ln);
  p->d_lin_chain_nodes = reinterpret_cast<const int32_t*>(p->dev_buf + o_lcn);
  p->d_lin_chains = reinterpret_cast<const I4*>(p->dev_buf + o_lc);
  p->has_device = true;
  p->device = dev;
  *out = p;
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

tree_attn_status_t tree_attn_plan(const int32_t* parent, const int32_t* seg_start,
                                  const int32_t* seg_len, int32_t num_nodes,
                                  int32_t num_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  tree_attn_dtype_t dtype, hipStream_t stream,
                                  tree_attn_plan_t* out) {
  return device_plan(parent, seg_start, seg_len, num_nodes, num_tokens, num_q_heads,
                     num_kv_heads, head_dim, dtype, nullptr, 0, stream, out);
}

tree_attn_status_t tree_attn_plan_subset(const int32_t* parent, const int32_t* seg_start,
                                         const int32_t* seg_len, int32_t num_nodes,
                                         int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         tree_attn_dtype_t dtype, const int32_t* query_nodes,
                                         int32_t num_query_nodes, hipStream_t stream,
                                         tree_attn_plan_t* out) {
  if (!query_nodes && num_query_nodes != 0)
    return report(Status::kInvalidArg, "null query-node list");
  static const int32_t kNone = 0;
  return device_plan(parent, seg_start, seg_len, num_nodes, num_tokens, num_q_heads,
                     num_kv_heads, head_dim, dtype, query_nodes ? query_nodes : &kNone,
                     num_query_nodes, stream, out);
}

void tree_attn_plan_destroy(tree_attn_plan_t plan) {
  if (!plan) return;
  if (plan->dev_buf) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != plan->device) (void)hipSetDevice(plan->device);
    (void)hipFree(plan->dev_buf);
    if (cur != plan->device && cur >= 0) (void)hipSetDevice(cur);
  }
  delete plan;
}

tree_attn_status_t tree_attn_workspace_size(tree_attn_plan_t plan, size_t* fwd_bytes,
                                            size_t* bwd_bytes) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  if (fwd_bytes) *fwd_bytes = fwd_layout(plan->hp).total;
  if (bwd_bytes) *bwd_bytes = bwd_layout(plan->hp).total;
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_fwd(tree_attn_plan_t plan, const void* q, const void* k,
                                 const void* v, float softmax_scale, void* o, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (hp.num_tokens == 0 || hp.query_rows == 0) return check_device(plan);
  // argument checks come first, so that a bad call is rejected the same way
  // on any plan
  if (!q || !k || !v || !o || !lse) return report(Status::kInvalidArg, "null tensor pointer");
  if (!aligned16({q, k, v, o, lse}))
    return report(Status::kInvalidArg, "tensor pointers must be 16-byte aligned");
  if (!valid_softmax_scale(softmax_scale))
    return report(Status::kInvalidArg, "softmax_scale must be finite and > 0");
  const FwdLayout l = fwd_layout(hp);
  if (l.total > 0) {
    if (!ws || ws_bytes < l.total)
      return report(Status::kWorkspace, "forward workspace needs " + std::to_string(l.total) +
                                            " bytes, got " + std::to_string(ws_bytes));
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
      return report(Status::kWorkspace, "workspace must be 256-byte aligned");
  }
  tree_attn_status_t st = check_device(plan);
  if (st != TREE_ATTN_OK) return st;
  tree_attn::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.tiles = plan->d_fwd_tiles;
  a.ranges = plan->d_fwd_ranges;
  a.part = plan->d_fwd_part;
  if (l.total > 0) {
    a.o_part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.o_part);
    a.ml_part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.ml_part);
  }
  a.combine = plan->d_fwd_combine;
  a.n_combine = static_cast<int64_t>(hp.fwd_combine.size());
  a.n_tokens = hp.num_tokens;
  a.n_groups = hp.fwd_groups;
  a.hq = static_cast<int>(hp.hq);
  a.hkv = static_cast<int>(hp.hkv);
  a.gsize = static_cast<int>(hp.hq / hp.hkv);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  const int hd = static_cast<int>(hp.head_dim);
  const hipError_t e = timed(0, stream, [&] {
    hipError_t r = tree_attn::launch_fwd(a, hp.dtype, hd, hp.fwd_blocks, stream);
    if (r == hipSuccess) r = tree_attn::launch_fwd_combine(a, hp.dtype, hd, stream);
    return r;
  });
  if (e != hipSuccess) return report_hip(e, "forward launch");
  return TREE_ATTN_OK;
}

}  // extern "C"

namespace {

// dk / dv are the outputs (whole-tree plans) or, with acc != 0, fp32
// accumulators (query-subset plans).
tree_attn_status_t bwd_common(tree_attn_plan_t plan, const void* q, const void* k,
                              const void* v, const void* o, const float* lse, const void* dout,
                              float softmax_scale, void* dq, void* dk, void* dv, void* ws,
                              size_t ws_bytes, hipStream_t stream, bool acc) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (acc && !hp.subset)
    return report(Status::kInvalidArg,
                  "tree_attn_bwd_accum takes a query-subset plan (tree_attn_plan_subset)");
  if (!acc && hp.subset)
    return report(Status::kInvalidArg,
                  "a query-subset plan's backward is tree_attn_bwd_accum");
  if (hp.num_tokens == 0 || hp.query_rows == 0) return check_device(plan);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return report(Status::kInvalidArg, "null tensor pointer");
  if (!aligned16({q, k, v, o, lse, dout, dq, dk, dv}))
    return report(Status::kInvalidArg, "tensor pointers must be 16-byte aligned");
  if (!valid_softmax_scale(softmax_scale))
    return report(Status::kInvalidArg, "softmax_scale must be finite and > 0");
  const BwdLayout l = bwd_layout(hp);
  if (!ws || ws_bytes < l.total)
    return report(Status::kWorkspace, "backward workspace needs " + std::to_string(l.total) +
                                          " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return report(Status::kWorkspace, "workspace must be 256-byte aligned");
  tree_attn_status_t st = check_device(plan);
  if (st != TREE_ATTN_OK) return st;
  char* w = static_cast<char*>(ws);
  tree_attn::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  if (acc) {
    a.acc_dk = static_cast<float*>(dk);
    a.acc_dv = static_cast<float*>(dv);
    a.pre_tiles = plan->d_fwd_qtiles;
    a.n_pre_tiles = static_cast<int64_t>(hp.fwd_qtiles.size());
  } else {
    a.dk = dk;
    a.dv = dv;
  }
  a.neg_d = reinterpret_cast<float*>(w + l.neg_d);
  a.neg_lse2 = reinterpret_cast<float*>(w + l.neg_lse2);
  a.dk_slots = reinterpret_cast<float*>(w + l.dk_slots);
  a.dv_slots = reinterpret_cast<float*>(w + l.dv_slots);
  a.items = plan->d_bwd_items;
  a.entries = plan->d_bwd_entries;
  a.reduce = plan->d_bwd_reduce;
  a.tiles = plan->d_fwd_tiles;
  a.ranges = plan->d_fwd_ranges;
  a.part = plan->d_fwd_part;
  a.dq_part = reinterpret_cast<float*>(w + l.dq_part);
  a.combine = plan->d_fwd_combine;
  a.n_combine = static_cast<int64_t>(hp.fwd_combine.size());
  a.n_tokens = hp.num_tokens;
  a.n_items = static_cast<int64_t>(hp.bwd_items.size());
  a.n_reduce = static_cast<int64_t>(hp.bwd_reduce.size());
  a.has_limit = hp.bwd_has_limit ? 1 : 0;
  a.n_groups = hp.fwd_groups;
  a.dq_blocks = hp.fwd_blocks;
  a.hq = static_cast<int>(hp.hq);
  a.hkv = static_cast<int>(hp.hkv);
  a.gsize = static_cast<int>(hp.hq / hp.hkv);
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  const int hd = static_cast<int>(hp.head_dim);
  hipError_t e = timed(1, stream, [&] { return tree_attn::launch_bwd_pre(a, hp.dtype, hd, stream); });
  if (e != hipSuccess) return report_hip(e, "backward preprocess launch");
  e = timed(2, stream, [&] { return tree_attn::launch_bwd_dkdv(a, hp.dtype, hd, stream); });
  if (e != hipSuccess) return report_hip(e, "backward dK/dV launch");
  e = timed(3, stream, [&] { return tree_attn::launch_bwd_post(a, hp.dtype, hd, stream); });
  if (e != hipSuccess) return report_hip(e, "backward reduction launch");
  e = timed(4, stream, [&] {
    hipError_t r = tree_attn::launch_bwd_dq(a, hp.dtype, hd, stream);
    if (r == hipSuccess) r = tree_attn::launch_bwd_dq_sum(a, hp.dtype, hd, stream);
    return r;
  });
  if (e != hipSuccess) return report_hip(e, "backward dQ launch");
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

tree_attn_status_t tree_attn_bwd(tree_attn_plan_t plan, const void* q, const void* k,
                                 const void* v, const void* o, const float* lse,
                                 const void* dout, float softmax_scale, void* dq, void* dk,
                                 void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_common(plan, q, k, v, o, lse, dout, softmax_scale, dq, dk, dv, ws, ws_bytes, stream,
                    false);
}

tree_attn_status_t tree_attn_bwd_noalloc(tree_attn_plan_t plan, const void* q, const void* k,
                                         const void* v, const void* o, const float* lse,
                                         const void* dout, float softmax_scale, void* dq,
                                         void* dk, void* dv, hipStream_t stream) {
  static_assert(tree_attn::kStaticScratchBytes == TREE_ATTN_STATIC_SCRATCH_BYTES,
                "library scratch size and its documented value differ");
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (hp.subset)
    return report(Status::kInvalidArg,
                  "a query-subset plan's backward is tree_attn_bwd_accum");
  const size_t need = bwd_layout(hp).total;
  if (need > tree_attn::kStaticScratchBytes)
    return report(Status::kWorkspace,
                  "backward scratch needs " + std::to_string(need) +
                      " bytes, more than the library's fixed " +
                      std::to_string(tree_attn::kStaticScratchBytes) +
                      "; use tree_attn_bwd with a caller workspace");
  if (hp.num_tokens == 0 || hp.query_rows == 0) return check_device(plan);
  tree_attn_status_t st = check_device(plan);
  if (st != TREE_ATTN_OK) return st;
  void* ws = nullptr;
  const hipError_t e = tree_attn::static_scratch(&ws);
  if (e != hipSuccess) return report_hip(e, "hipGetSymbolAddress(library scratch)");
  return bwd_common(plan, q, k, v, o, lse, dout, softmax_scale, dq, dk, dv, ws,
                    tree_attn::kStaticScratchBytes, stream, false);
}

tree_attn_status_t tree_attn_bwd_accum(tree_attn_plan_t plan, const void* q, const void* k,
                                       const void* v, const void* o, const float* lse,
                                       const void* dout, float softmax_scale, void* dq,
                                       float* dk_acc, float* dv_acc, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  return bwd_common(plan, q, k, v, o, lse, dout, softmax_scale, dq, dk_acc, dv_acc, ws, ws_bytes,
                    stream, true);
}

tree_attn_status_t tree_attn_accum_cast(const float* acc, void* out, int64_t count,
                                        tree_attn_dtype_t dtype, hipStream_t stream) {
  if (count < 0) return report(Status::kInvalidArg, "negative count");
  if (count == 0) return TREE_ATTN_OK;
  if (!acc || !out) return report(Status::kInvalidArg, "null pointer");
  if (dtype != TREE_ATTN_BF16 && dtype != TREE_ATTN_FP32)
    return report(Status::kUnsupported, "unknown dtype");
  if (reinterpret_cast<uintptr_t>(acc) % 16 != 0)
    return report(Status::kInvalidArg, "acc must be 16-byte aligned");
  const hipError_t e = tree_attn::launch_cast(acc, out, count, static_cast<int>(dtype), stream);
  if (e != hipSuccess) return report_hip(e, "accumulator cast launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_lin_workspace_size(tree_attn_plan_t plan, size_t* fwd_bytes,
                                                size_t* bwd_bytes) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const bool any = plan->hp.num_tokens > 0;
  const size_t b = any ? lin_block(plan->hp) : 0, e = any ? lin_ends(plan->hp) : 0;
  if (fwd_bytes) *fwd_bytes = 2 * b + e;
  if (bwd_bytes) *bwd_bytes = 3 * b + e;
  return TREE_ATTN_OK;
}

namespace {

tree_attn_status_t lin_common(tree_attn_plan_t plan, float scale, void* ws, size_t ws_bytes,
                              size_t need) {
  tree_attn_status_t st = check_device(plan);
  if (st != TREE_ATTN_OK) return st;
  const HostPlan& hp = plan->hp;
  if (hp.subset) return report(Status::kUnsupported, "linear attention takes a whole-tree plan");
  if (hp.dtype != 0) return report(Status::kUnsupported, "linear attention takes bf16 tensors");
  if (!std::isfinite(scale)) return report(Status::kInvalidArg, "scale must be finite");
  if (hp.num_tokens == 0) return TREE_ATTN_OK;
  if (!ws || ws_bytes < need)
    return report(Status::kWorkspace, "linear attention workspace needs " +
                                          std::to_string(need) + " bytes, got " +
                                          std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return report(Status::kWorkspace, "workspace must be 256-byte aligned");
  return TREE_ATTN_OK;
}

tree_attn::LinArgs lin_args(tree_attn_plan_t plan, float scale) {
  const HostPlan& hp = plan->hp;
  tree_attn::LinArgs a{};
  a.pieces = plan->d_lin_pieces;
  a.succ = plan->d_lin_succ;
  a.lnodes = plan->d_lin_nodes;
  a.chains = plan->d_lin_chains;
  a.chain_nodes = plan->d_lin_chain_nodes;
  a.phases = hp.lin_phases.data();
  a.n_phases = static_cast<int>(hp.lin_phases.size());
  a.n_pieces = static_cast<int64_t>(hp.lin_pieces.size());
  a.n_nodes = static_cast<int64_t>(hp.lin_nodes.size());
  a.hq = static_cast<int>(hp.hq);
  a.hkv = static_cast<int>(hp.hkv);
  a.gsize = static_cast<int>(hp.hq / hp.hkv);
  a.scale = scale;
  return a;
}

}  // namespace

tree_attn_status_t tree_attn_lin_fwd(tree_attn_plan_t plan, const void* q, const void* k,
                                     const void* v, float scale, void* o, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const size_t blk = lin_block(plan->hp);
  tree_attn_status_t st = lin_common(plan, scale, ws, ws_bytes, 2 * blk + lin_ends(plan->hp));
  if (st != TREE_ATTN_OK || plan->hp.num_tokens == 0) return st;
  if (!q || !k || !v || !o) return report(Status::kInvalidArg, "null tensor pointer");
  if (!aligned16({q, k, v, o}))
    return report(Status::kInvalidArg, "tensor pointers must be 16-byte aligned");
  tree_attn::LinArgs a = lin_args(plan, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = o;
  a.state = ws;
  a.delta = static_cast<char*>(ws) + blk;
  a.ends = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * blk);
  const int hd = static_cast<int>(plan->hp.head_dim);
  hipError_t e = timed(9, stream, [&] { return tree_attn::launch_lin_outer(a, 0, hd, stream); });
  if (e == hipSuccess)
    e = timed(10, stream, [&] { return tree_attn::launch_lin_scan(a, 0, hd, stream); });
  if (e == hipSuccess)
    e = timed(11, stream, [&] { return tree_attn::launch_lin_chunk(a, 0, hd, stream); });
  if (e != hipSuccess) return report_hip(e, "linear attention forward launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_lin_bwd(tree_attn_plan_t plan, const void* q, const void* k,
                                     const void* v, const void* dout, float scale, void* dq,
                                     void* dk, void* dv, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const size_t blk = lin_block(plan->hp);
  tree_attn_status_t st = lin_common(plan, scale, ws, ws_bytes, 3 * blk + lin_ends(plan->hp));
  if (st != TREE_ATTN_OK || plan->hp.num_tokens == 0) return st;
  if (!q || !k || !v || !dout || !dq || !dk || !dv)
    return report(Status::kInvalidArg, "null tensor pointer");
  if (!aligned16({q, k, v, dout, dq, dk, dv}))
    return report(Status::kInvalidArg, "tensor pointers must be 16-byte aligned");
  char* w = static_cast<char*>(ws);
  tree_attn::LinArgs a = lin_args(plan, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  const int hd = static_cast<int>(plan->hp.head_dim);
  // states S recomputed (block 0, deltas in block 1), then the state
  // gradients R (block 2, deltas again in block 1); node ends after them
  void* s_state = w;
  void* r_state = w + 2 * blk;
  a.delta = w + blk;
  a.ends = reinterpret_cast<float*>(w + 3 * blk);
  a.state = s_state;
  hipError_t e = timed(9, stream, [&] { return tree_attn::launch_lin_outer(a, 0, hd, stream); });
  if (e == hipSuccess)
    e = timed(10, stream, [&] { return tree_attn::launch_lin_scan(a, 0, hd, stream); });
  if (e == hipSuccess) {
    a.out = dq;
    e = timed(14, stream, [&] { return tree_attn::launch_lin_chunk(a, 1, hd, stream); });
  }
  a.state = r_state;
  if (e == hipSuccess)
    e = timed(12, stream, [&] { return tree_attn::launch_lin_outer(a, 1, hd, stream); });
  if (e == hipSuccess)
    e = timed(13, stream, [&] { return tree_attn::launch_lin_scan(a, 1, hd, stream); });
  if (e == hipSuccess) {
    a.out = dk;
    a.out2 = dv;
    e = timed(15, stream, [&] { return tree_attn::launch_lin_chunk(a, 4, hd, stream); });
  }
  if (e != hipSuccess) return report_hip(e, "linear attention backward launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_positions(tree_attn_plan_t plan, int32_t* node_id,
                                       int32_t* pos_id, hipStream_t stream) {
  tree_attn_status_t st = check_device(plan);
  if (st != TREE_ATTN_OK) return st;
  const HostPlan& hp = plan->hp;
  if (hp.num_tokens == 0 || (!node_id && !pos_id)) return TREE_ATTN_OK;
  tree_attn::PosArgs a{};
  a.segments = plan->d_segments;
  a.n_segments = static_cast<int32_t>(hp.segments.size());
  a.n_tokens = hp.num_tokens;
  a.node_id = node_id;
  a.pos_id = pos_id;
  const hipError_t e = timed(5, stream, [&] { return tree_attn::launch_positions(a, stream); });
  if (e != hipSuccess) return report_hip(e, "positions launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_walk_runs(const int32_t* parent, const int32_t* seg_len,
                                       int32_t num_nodes, int64_t budget, int32_t* order,
                                       int32_t* run_start, int32_t* num_runs) {
  std::string err;
  const Status s =
      tree_attn::walk_runs(parent, seg_len, num_nodes, budget, order, run_start, num_runs, &err);
  if (s != Status::kOk) return report(s, err);
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_build_tree(const int32_t* tokens, const int64_t* traj_offsets,
                                        int32_t num_traj, int32_t* parent, int32_t* seg_start,
                                        int32_t* seg_len, int32_t* unique_tokens,
                                        int32_t* traj_index, int32_t* mult, int32_t* inv_offsets,
                                        int32_t* inv_positions, int32_t* num_nodes,
                                        int32_t* num_tokens) {
  std::string err;
  const Status s = tree_attn::build_prefix_tree(tokens, traj_offsets, num_traj, parent, seg_start,
                                                seg_len, unique_tokens, traj_index, mult,
                                                inv_offsets, inv_positions, num_nodes, num_tokens,
                                                &err);
  if (s != Status::kOk) return report(s, err);
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_gather_rows(const void* src, void* dst, const int32_t* index,
                                         int64_t num_rows, int64_t row_bytes,
                                         hipStream_t stream) {
  if (num_rows < 0 || row_bytes < 0)
    return report(Status::kInvalidArg, "negative row count or row size");
  if (num_rows == 0 || row_bytes == 0) return TREE_ATTN_OK;
  if (!src || !dst || !index) return report(Status::kInvalidArg, "null pointer");
  const hipError_t e = timed(6, stream, [&] {
    return tree_attn::launch_gather(src, dst, index, num_rows, row_bytes, stream);
  });
  if (e != hipSuccess) return report_hip(e, "gather launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_scatter_sum_rows(const void* src, void* dst,
                                              const int32_t* inv_offsets,
                                              const int32_t* inv_positions, int64_t num_rows,
                                              int64_t row_elems, tree_attn_dtype_t dtype,
                                              hipStream_t stream) {
  if (num_rows < 0 || row_elems < 0)
    return report(Status::kInvalidArg, "negative row count or row size");
  if (dtype != TREE_ATTN_BF16 && dtype != TREE_ATTN_FP32)
    return report(Status::kUnsupported, "unknown dtype");
  if (num_rows == 0 || row_elems == 0) return TREE_ATTN_OK;
  if (!src || !dst || !inv_offsets || !inv_positions)
    return report(Status::kInvalidArg, "null pointer");
  const hipError_t e = timed(7, stream, [&] {
    return tree_attn::launch_scatter_sum(src, dst, inv_offsets, inv_positions, num_rows, row_elems,
                                         static_cast<int>(dtype), stream);
  });
  if (e != hipSuccess) return report_hip(e, "scatter-sum launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_rope(void* x, const int32_t* pos_id, int64_t num_tokens,
                                  int32_t num_heads, int32_t head_dim, float theta,
                                  int32_t inverse, tree_attn_dtype_t dtype, hipStream_t stream) {
  if (num_tokens < 0 || num_heads < 0)
    return report(Status::kInvalidArg, "negative token or head count");
  if (head_dim <= 0 || head_dim % 2 != 0)
    return report(Status::kUnsupported, "head_dim must be positive and even");
  if (!(theta > 1.f) || !std::isfinite(theta))
    return report(Status::kInvalidArg, "theta must be finite and > 1");
  if (dtype != TREE_ATTN_BF16 && dtype != TREE_ATTN_FP32)
    return report(Status::kUnsupported, "unknown dtype");
  if (num_tokens == 0 || num_heads == 0) return TREE_ATTN_OK;
  if (!x || !pos_id) return report(Status::kInvalidArg, "null pointer");
  const hipError_t e = timed(8, stream, [&] {
    return tree_attn::launch_rope(x, pos_id, num_tokens, num_heads, head_dim,
                                  std::log2(static_cast<double>(theta)), inverse ? 1 : 0,
                                  static_cast<int>(dtype), stream);
  });
  if (e != hipSuccess) return report_hip(e, "rope launch");
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_plan_stats(tree_attn_plan_t plan, tree_attn_plan_stats_t* out) {
  if (!plan || !out) return report(Status::kInvalidArg, "null argument");
  const HostPlan& hp = plan->hp;
  std::memset(out, 0, sizeof(*out));
  out->num_tokens = hp.num_tokens;
  out->num_nodes = hp.num_nodes;
  out->num_q_heads = hp.hq;
  out->num_kv_heads = hp.hkv;
  out->head_dim = hp.head_dim;
  out->pairs = hp.pairs;
  out->fwd_tiles = static_cast<int64_t>(hp.fwd_tiles.size());
  out->fwd_ranges = static_cast<int64_t>(hp.fwd_ranges.size());
  out->fwd_blocks = hp.fwd_blocks;
  out->bwd_items = static_cast<int64_t>(hp.bwd_items.size());
  out->bwd_entries = static_cast<int64_t>(hp.bwd_entries.size());
  out->bwd_split_tiles = hp.bwd_split_tiles;
  out->bwd_slots = hp.bwd_slots;
  out->fwd_tile_rows = tree_attn::kFwdRows;
  out->fwd_tile_keys = tree_attn::kFwdKeys;
  out->bwd_tile_keys = tree_attn::kBwdKeys;
  out->bwd_block_rows = tree_attn::kBwdRows;
  out->lin_pieces = static_cast<int64_t>(hp.lin_pieces.size());
  out->lin_succ = static_cast<int64_t>(hp.lin_succ.size());
  out->lin_chunk = tree_attn::kLinChunk;
  out->subset = hp.subset ? 1 : 0;
  out->query_rows = hp.query_rows;
  out->fwd_split_tiles = static_cast<int64_t>(hp.fwd_combine.size());
  out->fwd_slots = hp.fwd_slots;
  out->lin_chains = static_cast<int64_t>(hp.lin_chains.size());
  out->lin_phases = static_cast<int64_t>(hp.lin_phases.size());
  out->lin_nodes = static_cast<int64_t>(hp.lin_nodes.size());
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_lin_plan_export_chains(tree_attn_plan_t plan, int32_t* chains,
                                                    int32_t* chain_nodes, int32_t* phases) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (chains && !hp.lin_chains.empty())
    std::memcpy(chains, hp.lin_chains.data(), bytes_of(hp.lin_chains));
  if (chain_nodes && !hp.lin_chain_nodes.empty())
    std::memcpy(chain_nodes, hp.lin_chain_nodes.data(), bytes_of(hp.lin_chain_nodes));
  if (phases && !hp.lin_phases.empty())
    std::memcpy(phases, hp.lin_phases.data(), bytes_of(hp.lin_phases));
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_plan_export_split(tree_attn_plan_t plan, int32_t* fwd_part,
                                               int32_t* fwd_combine) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (fwd_part && !hp.fwd_part.empty())
    std::memcpy(fwd_part, hp.fwd_part.data(), bytes_of(hp.fwd_part));
  if (fwd_combine && !hp.fwd_combine.empty())
    std::memcpy(fwd_combine, hp.fwd_combine.data(), bytes_of(hp.fwd_combine));
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_lin_plan_export(tree_attn_plan_t plan, int32_t* pieces,
                                             int32_t* successors) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  if (pieces && !hp.lin_pieces.empty())
    std::memcpy(pieces, hp.lin_pieces.data(), bytes_of(hp.lin_pieces));
  if (successors && !hp.lin_succ.empty())
    std::memcpy(successors, hp.lin_succ.data(), bytes_of(hp.lin_succ));
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_plan_export(tree_attn_plan_t plan, int32_t* fwd_tiles,
                                         int32_t* fwd_ranges, int32_t* bwd_items,
                                         int32_t* bwd_entries) {
  if (!plan) return report(Status::kInvalidArg, "null plan");
  const HostPlan& hp = plan->hp;
  // (memcpy from the null data() of an empty vector is undefined even for 0 bytes)
  if (fwd_tiles && !hp.fwd_tiles.empty())
    std::memcpy(fwd_tiles, hp.fwd_tiles.data(), bytes_of(hp.fwd_tiles));
  if (fwd_ranges && !hp.fwd_ranges.empty())
    std::memcpy(fwd_ranges, hp.fwd_ranges.data(), bytes_of(hp.fwd_ranges));
  if (bwd_items && !hp.bwd_items.empty())
    std::memcpy(bwd_items, hp.bwd_items.data(), bytes_of(hp.bwd_items));
  if (bwd_entries && !hp.bwd_entries.empty())
    std::memcpy(bwd_entries, hp.bwd_entries.data(), bytes_of(hp.bwd_entries));
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.enabled = enable != 0;
  return TREE_ATTN_OK;
}

tree_attn_status_t tree_attn_timing_read(tree_attn_timing_t* out, int reset) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  tree_attn_status_t st = TREE_ATTN_OK;
  for (const Timing::Rec& r : t.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == TREE_ATTN_OK) st = report_hip(e, "timing events");
    t.launches[r.kind] += 1;
    t.total_ms[r.kind] += ms;
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.recs.clear();
  if (out) {
    for (int i = 0; i < kTimingKinds; ++i) {
      out->launches[i] = t.launches[i];
      out->total_ms[i] = t.total_ms[i];
    }
  }
  if (reset) {
    for (int i = 0; i < kTimingKinds; ++i) {
      t.launches[i] = 0;
      t.total_ms[i] = 0;
    }
  }
  return st;
}

const char* tree_attn_status_string(tree_attn_status_t s) {
  switch (s) {
    case TREE_ATTN_OK: return "ok";
    case TREE_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case TREE_ATTN_ERR_BAD_TREE: return "invalid tree (parent index or cycle)";
    case TREE_ATTN_ERR_LAYOUT: return "invalid segment layout";
    case TREE_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case TREE_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case TREE_ATTN_ERR_HIP: return "HIP runtime error";
    case TREE_ATTN_ERR_NO_DEVICE_PLAN: return "plan has no device data";
    default: break;
  }
  return "unknown status";
}

const char* tree_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
