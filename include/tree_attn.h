/*
 * tree_attn.h -- C ABI of libtree_attn.so: causal attention forward and
 * backward over a rollout prefix tree on AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  Rollouts that share prefixes form a tree whose
 * root-to-leaf paths are the trajectories (AReaL-DTA, abstract; HARTS,
 * abstract).  Every unique token is stored once.  A token attends to itself
 * and to every token before it on its root-to-leaf path: all tokens of its
 * node's proper ancestors and the earlier tokens of its own node.  The
 * results equal those of running each trajectory separately through ordinary
 * causal attention, while each shared prefix is computed once in the forward
 * and once in the backward pass (Tree Training, listed on the HARTS page:
 * compute each shared prefix once and reuse it in both passes).  In the
 * backward pass the gradients of a shared token's K and V are the sums over
 * every descendant branch.  All branches go through one packed call per
 * pass (HARTS, abstract: one packed call per round over all branches), and
 * the loss sees only per-unique-token outputs, so an RL objective keeps its
 * interface (HARTS, abstract).
 *
 * Conventions used by every entry point:
 *   N    number of unique (packed) tokens      M    number of tree nodes
 *   Hq   query heads   Hkv  key/value heads    G = Hq / Hkv (GQA group size)
 *   D    head dimension (64 or 128)
 *   Q, O, dO, dQ : [N, Hq, D]   row-major, contiguous, element type `dtype`
 *   K, V, dK, dV : [N, Hkv, D]  row-major, contiguous, element type `dtype`
 *   LSE          : [Hq, N] fp32, natural log of sum_j exp(scale * q . k_j)
 *   query head h reads key/value head h / G.
 *   Pointers to tensors are device pointers owned by the caller; the library
 *   never frees or retains them past the call.  Calls enqueue work on the
 *   given HIP stream and return without synchronising; kernel faults surface
 *   at the caller's next synchronisation.
 *   Graph capture: with timing off (tree_attn_timing_enable), the passes on
 *   an existing plan -- tree_attn_fwd, tree_attn_bwd, tree_attn_bwd_accum,
 *   tree_attn_accum_cast and their linear-attention counterparts -- enqueue
 *   only kernel launches on `stream`: no allocation, copy, memset or host
 *   synchronisation.  They may therefore be recorded into a HIP graph while
 *   `stream` is capturing, and each replay reruns the same kernels on the
 *   same buffers.  Creating or destroying a plan allocates, copies and
 *   frees, and stays outside any capture.
 *
 * Errors: every entry point returns a tree_attn_status_t.  Invalid arguments
 * are rejected before any device work is enqueued; the reason is available
 * from tree_attn_last_error() on the calling thread.  No C++ exception or
 * abort crosses this interface.
 */
#ifndef TREE_ATTN_H_
#define TREE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TREE_ATTN_OK = 0,
  TREE_ATTN_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad plan  */
  TREE_ATTN_ERR_BAD_TREE = 2,     /* parent out of range, self loop, cycle  */
  TREE_ATTN_ERR_LAYOUT = 3,       /* segments overlap, leave gaps, len < 1  */
  TREE_ATTN_ERR_UNSUPPORTED = 4,  /* head_dim, dtype, head counts, plan size */
  TREE_ATTN_ERR_WORKSPACE = 5,    /* workspace missing or too small         */
  TREE_ATTN_ERR_HIP = 6,          /* a HIP runtime call failed              */
  TREE_ATTN_ERR_NO_DEVICE_PLAN = 7, /* host-only plan passed to fwd/bwd     */
  /* Not statuses: these two make every int32 value a valid value of the
   * type, so that a C caller's unknown value reaches the library as a
   * number it can reject instead of undefined behaviour. */
  TREE_ATTN_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  TREE_ATTN_STATUS_RANGE_MAX_ = 0x7fffffff
} tree_attn_status_t;

typedef enum {
  TREE_ATTN_BF16 = 0,
  TREE_ATTN_FP32 = 1,
  /* not dtypes (see tree_attn_status_t): any other value is rejected with
   * TREE_ATTN_ERR_UNSUPPORTED */
  TREE_ATTN_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  TREE_ATTN_DTYPE_RANGE_MAX_ = 0x7fffffff
} tree_attn_dtype_t;

typedef struct tree_attn_plan_s* tree_attn_plan_t; /* opaque, immutable */

/*
 * tree_attn_plan -- validate a node table and build the work plan.
 *
 * The node table describes the rollout prefix tree (AReaL-DTA, abstract:
 * prefix sharing induces a tree over rollouts; HARTS, abstract: planning on
 * the compact-token work left after prefix compression).  It is read on the
 * host during this call only:
 *   parent[i]     parent node of node i, or -1 for a root (a forest of
 *                 independent trees is allowed);
 *   seg_start[i]  first packed row of node i's tokens;
 *   seg_len[i]    number of tokens of node i, >= 1.
 * The segments must partition [0, num_tokens) exactly; node order and
 * packing order are otherwise free.  num_nodes == 0 requires
 * num_tokens == 0 (an empty batch; fwd/bwd then enqueue nothing).
 *
 * The plan holds the work items of the forward pass (query tiles with the
 * key ranges of their ancestors) and of the backward pass (key tiles with
 * the query ranges of their descendants), ordered longest first.  A node
 * stored right after its parent continues the parent's run, and tiles are
 * cut over runs rather than single nodes, so packing the nodes in
 * depth-first preorder (as tree_attn_build_tree does) leaves fewer
 * part-filled tiles; any packing order gives the same results.  Another
 * order costs plan size, though: a node's ancestor ranges merge only where
 * they are stored back to back, and each side subtree adds a range to the
 * key tiles above it, so a deep tree stored out of order needs about its
 * depth in entries per tile.  Its small
 * device arrays are copied asynchronously on `stream`; the plan may be used
 * on any stream once `stream` has passed this point, and reused by any
 * number of fwd/bwd calls (e.g. every layer of a model).
 *
 * Returns BAD_TREE or LAYOUT for an invalid table, UNSUPPORTED when
 * head_dim is not 64 or 128, dtype is unknown, or num_q_heads is not a
 * positive multiple of num_kv_heads, and when the plan would hold more
 * than 2^27 key-range entries (counted before anything is built: a deep
 * tree stored out of depth-first order); INVALID_ARG for null pointers or
 * negative sizes; HIP when device allocation or copy fails.  *out is set
 * only on success.
 */
tree_attn_status_t tree_attn_plan(const int32_t* parent, const int32_t* seg_start,
                                  const int32_t* seg_len, int32_t num_nodes,
                                  int32_t num_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  tree_attn_dtype_t dtype, hipStream_t stream,
                                  tree_attn_plan_t* out);

/*
 * tree_attn_plan_host -- the same validation and planning as tree_attn_plan
 * without touching any GPU.  The resulting plan can be inspected
 * (tree_attn_plan_stats, tree_attn_plan_export) and sized
 * (tree_attn_workspace_size) but fwd/bwd reject it with NO_DEVICE_PLAN.
 * `num_cus` is the compute-unit count the load balancer plans for (256 on
 * MI355X; values < 1 mean 256).
 */
tree_attn_status_t tree_attn_plan_host(const int32_t* parent, const int32_t* seg_start,
                                       const int32_t* seg_len, int32_t num_nodes,
                                       int32_t num_tokens, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       tree_attn_dtype_t dtype, int32_t num_cus,
                                       tree_attn_plan_t* out);

/* Release a plan and its device arrays.  Null is ignored.  The caller must
 * ensure no enqueued fwd/bwd still uses the plan (synchronise first). */
void tree_attn_plan_destroy(tree_attn_plan_t plan);

/*
 * tree_attn_workspace_size -- bytes of device workspace fwd and bwd need.
 * The backward workspace holds two fp32 row-term arrays [Hq, N] (-D_t with
 * D_t = dO_t . O_t, and -LSE_t * log2 e), each padded to 256 bytes, and fp32
 * partial dK/dV slots of key tiles whose descendant work was split
 * for load balance, and fp32 partial dQ of the key parts below.  A plan
 * whose (query tile, head) workgroups would not fill the GPU twice over
 * (small trees, one-node calls of a depth-first walk) splits the keys of
 * its query tiles into parts (tree_attn_plan_export_split); the forward
 * workspace then holds their fp32 partial outputs (unnormalised O, the
 * running maximum and the row sum per row and head), and fwd_bytes is 0
 * for a plan without such parts.  Either pointer may be null.
 */
tree_attn_status_t tree_attn_workspace_size(tree_attn_plan_t plan, size_t* fwd_bytes,
                                            size_t* bwd_bytes);

/*
 * tree_attn_fwd -- forward pass.  For every unique token t and query head h:
 *   s_j = scale * q_{t,h} . k_{j,h/G} over the tokens j that t attends to,
 *   O_{t,h} = sum_j softmax(s)_j v_{j,h/G},   LSE_{h,t} = log sum_j exp(s_j).
 * q, k, v: device inputs in the plan's dtype; o: device output [N,Hq,D]
 * (same dtype, overwritten); lse: device output [Hq,N] fp32 (overwritten).
 * ws/ws_bytes: device workspace of at least fwd_bytes, 256-byte aligned
 * (may be null when fwd_bytes is 0), else WORKSPACE; a plan with split
 * query tiles merges their key parts in a second launch on the same stream.
 * The softmax scale is typically 1/sqrt(D); it must be finite and > 0
 * (masked scores are -inf before scaling), else INVALID_ARG.  Every tensor
 * pointer (q, k, v, o, lse) must be 16-byte aligned (rows move in 16-byte
 * pieces), else INVALID_ARG; torch allocations and whole-row views are.
 * Both checks happen before any launch.  Accumulation is fp32; bf16 outputs
 * are rounded to nearest even.
 */
tree_attn_status_t tree_attn_fwd(tree_attn_plan_t plan, const void* q, const void* k,
                                 const void* v, float softmax_scale, void* o, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * tree_attn_bwd -- backward pass of tree_attn_fwd.
 * dout [N,Hq,D] is the total upstream gradient of each unique output row (a
 * caller that holds per-trajectory gradients sums them per unique token
 * first).  o and lse are the forward outputs.  dq [N,Hq,D], dk and dv
 * [N,Hkv,D] receive the exact gradients with respect to the unique q, k, v:
 * dK and dV of a shared token are summed over every branch below it and over
 * the G query heads of its group.  Outputs are overwritten, not accumulated.
 * ws must hold at least bwd_bytes (256-byte aligned).  No atomics are used:
 * dQ, dK and dV are bitwise reproducible from run to run.  softmax_scale
 * and tensor-pointer alignment (16 bytes, all of q, k, v, o, lse, dout, dq,
 * dk, dv) are checked as in tree_attn_fwd, before any launch.
 */
tree_attn_status_t tree_attn_bwd(tree_attn_plan_t plan, const void* q, const void* k,
                                 const void* v, const void* o, const float* lse,
                                 const void* dout, float softmax_scale, void* dq, void* dk,
                                 void* dv, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * tree_attn_bwd_noalloc -- tree_attn_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and checks as
 * tree_attn_bwd, without ws/ws_bytes: the backward scratch (row terms and
 * split slots) comes from a fixed array of TREE_ATTN_STATIC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the plan's own device arrays were allocated by tree_attn_plan.
 * A plan whose bwd_bytes (tree_attn_workspace_size) exceed
 * TREE_ATTN_STATIC_SCRATCH_BYTES is rejected with WORKSPACE before any
 * launch; a query-subset plan with INVALID_ARG.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind; nothing in it has
 * to start at zero.  Calls that overlap on one GPU (other streams, other
 * threads, other plans) race on it: the caller orders them, e.g. on one
 * stream.  The first call on a device looks up that device's address of
 * the array (hipGetSymbolAddress).
 */
#define TREE_ATTN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
tree_attn_status_t tree_attn_bwd_noalloc(tree_attn_plan_t plan, const void* q, const void* k,
                                         const void* v, const void* o, const float* lse,
                                         const void* dout, float softmax_scale, void* dq,
                                         void* dk, void* dv, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Depth-first schedule.  AReaL-DTA (abstract) walks the prefix tree depth
 * first so that only one root-to-leaf path is resident at a time, while
 * every shared prefix is still computed once.  The entry points below run
 * the same kernels on a plan restricted to some query nodes: visiting the
 * nodes in depth-first preorder, one (or a few) per call, the forward pass
 * needs only the K/V rows of the current path and writes only the current
 * node's rows; the backward pass, in reverse order, adds each node's
 * contribution to the K/V gradients of its path into fp32 accumulators.
 * Summed over a partition of the nodes, the accumulated gradients equal
 * tree_attn_bwd's (up to fp32 summation order).
 */

/*
 * tree_attn_walk_runs -- the calls of a memory-bounded depth-first walk.
 * The walk visits the nodes in depth-first preorder (roots, and the
 * children of each node, in index order); what it must keep resident for a
 * call is the rows of the root paths of the call's query nodes.  This cuts
 * the preorder into runs of consecutive nodes, one query-subset call each:
 * a run takes the next node while the union of its nodes' root paths holds
 * at most `budget` tokens, and a node whose own root path is longer runs
 * alone.  budget <= 0 means the longest root-to-leaf path's token count:
 * then no call keeps more rows resident than the deepest call of a walk
 * with one node per call.
 *   parent, seg_len [num_nodes]: the node table (host memory, as in
 *                   tree_attn_plan; segment starts play no part);
 *   order     [num_nodes] (out): the preorder;
 *   run_start [num_nodes + 1] (out): run r is order[run_start[r] ..
 *                   run_start[r + 1]); run_start[num_runs] = num_nodes;
 *   num_runs  (out): 0 for an empty table.
 * Host memory only, owned by the caller; no GPU call.  Errors: INVALID_ARG
 * (negative num_nodes, null pointer), BAD_TREE (a parent outside
 * [-1, num_nodes), a node its own parent, a cycle), LAYOUT (a segment
 * length below 1).  On error the outputs are unspecified.
 */
tree_attn_status_t tree_attn_walk_runs(const int32_t* parent, const int32_t* seg_len,
                                       int32_t num_nodes, int64_t budget, int32_t* order,
                                       int32_t* run_start, int32_t* num_runs);

/*
 * tree_attn_plan_subset -- a plan whose queries are the tokens of
 * query_nodes[0 .. num_query_nodes) (node indices of the table; repeats are
 * ignored; an empty list gives a plan that does nothing).  Keys are unchanged:
 * a query still attends to every ancestor row and the earlier rows of its
 * node.  Validation, errors and device upload are those of tree_attn_plan;
 * INVALID_ARG also for a node index outside [0, num_nodes) or a null list
 * with num_query_nodes > 0.
 * On such a plan:
 *   tree_attn_fwd  writes O and LSE of the query rows only (other rows are
 *                  untouched) and reads Q of the query rows and K/V of the
 *                  rows they attend to -- nothing else of q, k, v;
 *   tree_attn_bwd  is rejected (INVALID_ARG): use tree_attn_bwd_accum;
 *   linear attention entry points are rejected (UNSUPPORTED).
 */
tree_attn_status_t tree_attn_plan_subset(const int32_t* parent, const int32_t* seg_start,
                                         const int32_t* seg_len, int32_t num_nodes,
                                         int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         tree_attn_dtype_t dtype, const int32_t* query_nodes,
                                         int32_t num_query_nodes, hipStream_t stream,
                                         tree_attn_plan_t* out);

/* tree_attn_plan_host_subset -- tree_attn_plan_subset without a GPU (see
 * tree_attn_plan_host). */
tree_attn_status_t tree_attn_plan_host_subset(const int32_t* parent, const int32_t* seg_start,
                                              const int32_t* seg_len, int32_t num_nodes,
                                              int32_t num_tokens, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              tree_attn_dtype_t dtype,
                                              const int32_t* query_nodes,
                                              int32_t num_query_nodes, int32_t num_cus,
                                              tree_attn_plan_t* out);

/*
 * tree_attn_bwd_accum -- backward pass of a query-subset plan: the
 * gradients of sum over query rows t of <dout_t, O_t>.
 *   dq      [N,Hq,D] in the plan's dtype: rows of the query nodes are
 *           overwritten with their gradient, other rows untouched;
 *   dk_acc, dv_acc  [N,Hkv,D] fp32 device accumulators (16-byte aligned):
 *           the gradient with respect to every key/value row that a query
 *           row attends to is ADDED (fp32); rows no query row sees are
 *           untouched.  The caller zeroes them before the first call of a
 *           schedule and converts them with tree_attn_accum_cast after the
 *           last.
 * Reads o, lse and dout of the query rows only.  Calls on the same
 * accumulators must be ordered (one stream, or synchronised): each adds with
 * plain loads and stores, no atomics, so the result is bitwise reproducible
 * for a fixed call order.  ws: tree_attn_workspace_size's bwd_bytes of this
 * plan.  Errors as tree_attn_bwd; INVALID_ARG for a whole-tree plan.
 */
tree_attn_status_t tree_attn_bwd_accum(tree_attn_plan_t plan, const void* q, const void* k,
                                       const void* v, const void* o, const float* lse,
                                       const void* dout, float softmax_scale, void* dq,
                                       float* dk_acc, float* dv_acc, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * tree_attn_accum_cast -- out[i] = acc[i] rounded to `dtype` (bf16: nearest
 * even; fp32: copy) for i < count.  acc: device fp32, 16-byte aligned; out:
 * device, `dtype`.  Enqueued on `stream`.  Errors: INVALID_ARG (negative
 * count, null or misaligned pointer), UNSUPPORTED (unknown dtype).
 */
tree_attn_status_t tree_attn_accum_cast(const float* acc, void* out, int64_t count,
                                        tree_attn_dtype_t dtype, hipStream_t stream);

/*
 * tree_attn_positions -- per-token node index and position id.
 * Every root-to-leaf path through a unique token t places it after the
 * tokens of its ancestor nodes and the earlier tokens of its own node, so t
 * has one position on all of them (AReaL-DTA, abstract: each shared prefix
 * is computed once for all trajectories through it).  For every t in
 * [0, N): node_id[t] = the node whose segment holds t, and
 * pos_id[t] = d(t) = the number of tokens t attends to besides itself --
 * the 0-based position a trajectory-wise run gives t (for example the
 * position id of rotary embeddings).
 * node_id, pos_id: device int32 [N], overwritten; either may be null (not
 * written).  Enqueued on `stream`; no host synchronisation.  Errors:
 * NO_DEVICE_PLAN for host plans, INVALID_ARG for a plan of another device,
 * HIP for a launch failure.
 */
tree_attn_status_t tree_attn_positions(tree_attn_plan_t plan, int32_t* node_id, int32_t* pos_id,
                                       hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Either side of the attention call.  Rollouts that share prefixes are
 * stored once (AReaL-DTA, abstract; HARTS, abstract: prefix-shared
 * trajectories processed in one packed call, per-trajectory objectives keep
 * their interface).  These entry points build the prefix tree from token
 * lists, hand per-token results back to trajectory positions, sum
 * per-trajectory gradients onto unique tokens, and apply rotary embeddings
 * at tree depth.
 */

/*
 * tree_attn_build_tree -- prefix compression on the host (no device work).
 * tokens[traj_offsets[num_traj]]: the concatenated token ids (>= 0) of
 * num_traj trajectories; trajectory b is tokens[traj_offsets[b] ..
 * traj_offsets[b+1]) (traj_offsets[0] = 0, non-decreasing; empty
 * trajectories are allowed).  Builds the trie of all trajectories and merges
 * its chains of single-child tokens into segments; nodes are numbered and
 * packed in depth-first preorder with children in order of first appearance,
 * so every segment is contiguous and the result is a valid node table for
 * tree_attn_plan.  A trajectory that is a prefix of another adds no node.
 * Outputs (host, caller-owned; T = traj_offsets[num_traj]):
 *   parent, seg_start, seg_len  capacity 2 * num_traj (a node table)
 *   unique_tokens               capacity T: token id of each unique row
 *   traj_index [T]              unique row of every trajectory position
 *   mult (optional)             capacity T: trajectories through each unique row
 *   inv_offsets (optional)      capacity T + 1, and
 *   inv_positions (optional)    [T]: positions mapping to unique row u are
 *       inv_positions[inv_offsets[u] .. inv_offsets[u+1]), ascending
 *   *num_nodes, *num_tokens     the sizes written
 * Errors: INVALID_ARG (null pointer, bad offsets, negative token id),
 * UNSUPPORTED (T >= 2^31 - 1).
 */
tree_attn_status_t tree_attn_build_tree(const int32_t* tokens, const int64_t* traj_offsets,
                                        int32_t num_traj, int32_t* parent, int32_t* seg_start,
                                        int32_t* seg_len, int32_t* unique_tokens,
                                        int32_t* traj_index, int32_t* mult, int32_t* inv_offsets,
                                        int32_t* inv_positions, int32_t* num_nodes,
                                        int32_t* num_tokens);

/*
 * tree_attn_gather_rows -- dst[i, :] = src[index[i], :] for i < num_rows.
 * The inverse of prefix compression: with index = traj_index it unpacks
 * per-unique-token rows (log-probabilities, hidden states, ...) to every
 * trajectory position.  src, dst: device rows of row_bytes bytes each,
 * contiguous; index: device int32 [num_rows], every entry a valid src row
 * (not checked).  Bit-exact copy; 16-byte transfers when row_bytes and the
 * pointers allow.  Enqueued on `stream`.
 */
tree_attn_status_t tree_attn_gather_rows(const void* src, void* dst, const int32_t* index,
                                         int64_t num_rows, int64_t row_bytes, hipStream_t stream);

/*
 * tree_attn_scatter_sum_rows -- the adjoint of the gather:
 *   dst[u, :] = sum over j in [inv_offsets[u], inv_offsets[u+1]) of
 *               src[inv_positions[j], :]      for u < num_rows,
 * accumulated in fp32 in the order of inv_positions (no atomics: bitwise
 * reproducible).  With the inverse map of tree_attn_build_tree it sums
 * per-trajectory gradients (e.g. dO of every trajectory position) onto the
 * unique tokens, which is the dO tree_attn_bwd expects.  src, dst: device
 * [*, row_elems] in `dtype` (bf16 or fp32; dst is overwritten); inv_offsets
 * [num_rows + 1] and inv_positions: device int32.  Enqueued on `stream`.
 */
tree_attn_status_t tree_attn_scatter_sum_rows(const void* src, void* dst,
                                              const int32_t* inv_offsets,
                                              const int32_t* inv_positions, int64_t num_rows,
                                              int64_t row_elems, tree_attn_dtype_t dtype,
                                              hipStream_t stream);

/*
 * tree_attn_rope -- rotary position embedding at tree depth, in place.
 * x: device [num_tokens, num_heads, head_dim] in `dtype`; pos_id: device
 * int32 [num_tokens] (e.g. from tree_attn_positions).  For every token t,
 * head h and i < head_dim/2, the pair (x_i, x_{i + head_dim/2}) is rotated
 * by the angle pos_id[t] * theta^(-2i/head_dim) (rotate-half pairing); with
 * inverse != 0 by minus that angle, which is the backward of the forward
 * rotation.  The angle is reduced in double precision and its sine and
 * cosine taken in single precision.  Since a unique token has one position on
 * every path through it, this equals rotating every trajectory copy at its
 * trajectory position.  Errors: UNSUPPORTED (odd head_dim, unknown dtype),
 * INVALID_ARG (theta <= 1 or not finite, null pointers).
 */
tree_attn_status_t tree_attn_rope(void* x, const int32_t* pos_id, int64_t num_tokens,
                                  int32_t num_heads, int32_t head_dim, float theta,
                                  int32_t inverse, tree_attn_dtype_t dtype, hipStream_t stream);

/* Plan statistics for reports and tests (host values, no device access). */
typedef struct {
  int64_t num_tokens, num_nodes, num_q_heads, num_kv_heads, head_dim;
  int64_t pairs;            /* sum over tokens of (ancestor tokens + 1)     */
  int64_t fwd_tiles;        /* query tiles (per head)                       */
  int64_t fwd_ranges;       /* key ranges over all query tiles              */
  int64_t fwd_blocks;       /* workgroups of one forward launch             */
  int64_t bwd_items;        /* key-tile work items (incl. split chunks and
                               empty items that pad the launch order)     */
  int64_t bwd_entries;      /* (head, query range) entries over all items   */
  int64_t bwd_split_tiles;  /* key tiles whose work was split               */
  int64_t bwd_slots;        /* fp32 partial dK/dV slots                     */
  int64_t fwd_tile_rows;    /* query rows per forward tile                  */
  int64_t fwd_tile_keys;    /* keys per forward key step                    */
  int64_t bwd_tile_keys;    /* keys per backward key tile                   */
  int64_t bwd_block_rows;   /* query rows per backward step                 */
  int64_t lin_pieces;       /* linear attention: pieces                     */
  int64_t lin_succ;         /* linear attention: successor entries          */
  int64_t lin_chunk;        /* linear attention: chunk (trajectory depth)   */
  int64_t subset;           /* 1 for a query-subset plan, else 0            */
  int64_t query_rows;       /* tokens that are queries (N for whole trees)  */
  int64_t fwd_split_tiles;  /* query tiles whose keys were split into parts */
  int64_t fwd_slots;        /* key parts of those tiles (forward / dQ slots) */
  int64_t lin_chains;       /* linear attention: heavy paths of the scans   */
  int64_t lin_phases;       /* linear attention: scan launches per pass     */
  int64_t lin_nodes;        /* linear attention: nodes in the scan order    */
} tree_attn_plan_stats_t;

tree_attn_status_t tree_attn_plan_stats(tree_attn_plan_t plan, tree_attn_plan_stats_t* out);

/*
 * tree_attn_plan_export -- copy the plan's host work arrays (for tests and
 * debugging).  Each array is int32, row-major with the given number of
 * columns; pass null to skip one, and the *_count outputs to size buffers:
 *   fwd_tiles  [fwd_tiles, 4]  : q0, q1, range_begin, range_end
 *   fwd_ranges [fwd_ranges, 4] : k0, k1, causal, 0
 *   bwd_items  [bwd_items, 8]  : k0, k1, kv_head, entry_begin, entry_end,
 *                                slot (-1 = writes dK/dV directly), XCD the
 *                                item is placed on (-1 for an empty item),
 *                                0.  Item b is launched as workgroup b, which
 *                                the hardware sends to XCD b % 8; items that
 *                                read the same query rows share an XCD, and
 *                                empty items (entry_begin == entry_end) fill
 *                                out the per-XCD queues.
 *   bwd_entries[bwd_entries, 4]: q_head, q0, q1, mask
 * A causal range (fwd causal = 1, bwd mask = 1) applies the mask
 * key <= query; a query sees a key in a non-causal range (0)
 * unconditionally (range rows are ancestors/descendants).  A backward key
 * tile may span a parent's last rows and the first rows of the child stored
 * right after it; the rows below the parent's other children then see only
 * the parent's keys: mask = -(limit + 1) hides keys >= limit from them.
 */
tree_attn_status_t tree_attn_plan_export(tree_attn_plan_t plan, int32_t* fwd_tiles,
                                         int32_t* fwd_ranges, int32_t* bwd_items,
                                         int32_t* bwd_entries);

/*
 * tree_attn_plan_export_split -- the key parts of split forward tiles (for
 * tests and debugging); pass null to skip one:
 *   fwd_part    [fwd_tiles]          : slot of the tile's key part, or -1 for
 *                                      a tile that holds all of its rows'
 *                                      keys and writes O / LSE and dQ itself
 *   fwd_combine [fwd_split_tiles, 4] : q0, q1, slot_begin, num_slots of every
 *                                      split query tile; its parts are the
 *                                      tiles with those rows and slots, and
 *                                      together they hold every key of the
 *                                      rows exactly once
 */
tree_attn_status_t tree_attn_plan_export_split(tree_attn_plan_t plan, int32_t* fwd_part,
                                               int32_t* fwd_combine);

/*
 * Chunkwise causal linear attention over the same tree (HARTS, abstract:
 * the chunkwise linear-attention layers of hybrid models run over arbitrary
 * rollout trees in one packed call, with state handed from each prefix to its
 * branches and gradients propagated back through those handoffs).  The pages
 * name no gate or normaliser; the library computes the plain recurrence
 *
 *   O_t = scale * S_t^T q_t,   S_t = sum over s <= t on t's root-to-leaf
 *                              path of k_s v_s^T     (D x D per kv head),
 *
 * i.e. O_t = scale * sum_s (q_t . k_s) v_s, query head h reading kv head
 * h / G, with the results of running each trajectory separately and each
 * shared prefix computed once.  The loss is sum_t <dO_t, O_t> over unique
 * tokens: dQ, dK, dV are its gradients, dK / dV of a shared token summed over
 * every branch that sees it.
 *
 * Chunking: each node is cut where the trajectory depth (ancestor tokens +
 * offset) is a multiple of 64, so every state the kernels materialise is a
 * trajectory chunk-boundary state or a branch-point state; a chunk that
 * straddles a branch point is computed as its parent part once and its child
 * parts once each (no replay).  The states live in the caller's workspace:
 * the scans accumulate in fp32 and store each piece's entering state as bf16
 * [pieces, Hkv, D, D] (the matrix cores' operand type), with fp32 copies at
 * branch points [nodes, Hkv, D, D]; products run in bf16 on the matrix cores.
 *
 * Tensors: Q, O, dO, dQ [N, Hq, D] and K, V, dK, dV [N, Hkv, D], bf16 only
 * (a plan built for fp32 gives TREE_ATTN_ERR_UNSUPPORTED); D 64 or 128.
 * Workspace: device memory, 256-byte aligned, at least the size
 * tree_attn_lin_workspace_size reports (2 piece arrays and the node array
 * forward, 3 piece arrays and the node array backward);
 * it holds no result between calls.  The backward pass recomputes the
 * forward states itself, so it does not need the forward's workspace or O.
 * Errors as for tree_attn_fwd: invalid arguments (null or not 16-byte
 * aligned tensor pointers, a scale that is not finite; any finite scale,
 * including negative, is valid here) are rejected before any launch;
 * TREE_ATTN_ERR_WORKSPACE for a missing or short workspace.
 */
tree_attn_status_t tree_attn_lin_workspace_size(tree_attn_plan_t plan, size_t* fwd_bytes,
                                                size_t* bwd_bytes);
tree_attn_status_t tree_attn_lin_fwd(tree_attn_plan_t plan, const void* q, const void* k,
                                     const void* v, float scale, void* o, void* ws,
                                     size_t ws_bytes, hipStream_t stream);
tree_attn_status_t tree_attn_lin_bwd(tree_attn_plan_t plan, const void* q, const void* k,
                                     const void* v, const void* dout, float scale, void* dq,
                                     void* dk, void* dv, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * Copies the linear-attention piece table to host arrays: pieces [lin_pieces
 * x 8] = (first token, length, predecessor piece or -1, successor begin,
 * successor end, node, 0, 0) in root-first order, and successors [lin_succ].
 * Either pointer may be null.
 */
/*
 * Copies the order of the linear-attention state scans to host arrays (for
 * tests): chains [lin_chains x 4] = (begin, end, phase, 0) into chain_nodes
 * [lin_nodes], which lists positions in the root-first node order, each
 * chain a heavy path from its head (every node followed by its child with
 * the most pieces below it); phases [lin_phases x 4] = (chain begin, chain
 * end, 0, 0).  A pass scans the phases in order (forward) or in reverse
 * (backward), the chains of one phase side by side.  Any pointer may be
 * null.
 */
tree_attn_status_t tree_attn_lin_plan_export_chains(tree_attn_plan_t plan, int32_t* chains,
                                                    int32_t* chain_nodes, int32_t* phases);

tree_attn_status_t tree_attn_lin_plan_export(tree_attn_plan_t plan, int32_t* pieces,
                                             int32_t* successors);

/*
 * Kernel timing for benchmarks and reports.  While enabled, every kernel
 * that the device entry points launch is bracketed by HIP events on the call's stream (no
 * host synchronisation).  tree_attn_timing_read waits for the recorded
 * events, and returns per kernel kind the number of launches and their summed
 * duration in milliseconds since the last reset (reset != 0 clears them).
 * Kinds: 0 forward, 1 backward preprocess, 2 backward dK/dV, 3 backward
 * partial-slot reduction, 4 backward dQ, 5 positions, 6 gather, 7 scatter-sum,
 * 8 rotary embedding, 9 linear-attention piece sums K^T V (forward and
 * the backward's recomputation), 10 its state scan, 11 linear-attention
 * output, 12 piece sums Q^T dO, 13 state-gradient scan, 14 linear-attention
 * dQ, 15 linear-attention dK and dV.  Timing is
 * process-wide and not meant for concurrent callers.
 */
typedef struct {
  int64_t launches[16];
  double total_ms[16];
} tree_attn_timing_t;

tree_attn_status_t tree_attn_timing_enable(int enable);
tree_attn_status_t tree_attn_timing_read(tree_attn_timing_t* out, int reset);

const char* tree_attn_status_string(tree_attn_status_t status);
const char* tree_attn_last_error(void); /* thread-local detail of the last error */

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H_ */
