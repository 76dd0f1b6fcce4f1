// Launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "planner.h"

namespace tree_attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const I4* tiles;   // (q0, q1, range_begin, range_end)
  const I4* ranges;  // (k0, k1, causal, 0)
  const int32_t* part;  // per tile: slot of a key part, or -1 (writes O and LSE)
  float* o_part;     // [slots, Hq, kFwdRows, D] fp32 partial O (unnormalised)
  float* ml_part;    // [slots, Hq, kFwdRows, 2] fp32 (base-2 running max, row sum)
  const I4* combine; // (q0, q1, slot_begin, n_slots) per split query tile
  int64_t n_combine;
  int64_t n_tokens;
  int64_t n_groups;  // tiles * hkv
  int hq, hkv, gsize;
  float scale_log2;  // softmax scale * log2(e)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dk;
  void* dv;
  void* dq;
  float* neg_d;      // [Hq, N] fp32: -(sum_d dO * O), written by the preprocess
  float* neg_lse2;   // [Hq, N] fp32: -LSE * log2(e), written by the preprocess
  float* dk_slots;   // [slots, kBwdKeys, D] fp32
  float* dv_slots;   // [slots, kBwdKeys, D] fp32
  const I8* items;   // dK/dV: (k0, k1, g, entry_begin, entry_end, slot, 0, 0)
  const I4* entries; // dK/dV: (h, q0, q1, causal)
  const I8* reduce;  // (k0, k1, g, slot_begin, n_slots, 0, 0, 0)
  float* acc_dk;     // null, or [N, Hkv, D] fp32 accumulators the reduction adds into
  float* acc_dv;
  const I4* pre_tiles;  // null: the preprocess covers every row; else only these tiles' rows
  int64_t n_pre_tiles;
  const I4* tiles;   // dQ: forward query tiles (q0, q1, range_begin, range_end)
  const I4* ranges;  // dQ: forward key ranges (k0, k1, causal, 0)
  const int32_t* part;  // dQ: per tile, slot of a key part or -1 (writes dQ)
  float* dq_part;    // [slots, Hq, kFwdRows, D] fp32 partial dQ (scaled)
  const I4* combine; // (q0, q1, slot_begin, n_slots) per split query tile
  int64_t n_combine;
  int64_t n_tokens;
  int64_t n_items;
  int64_t n_reduce;
  int has_limit;     // some entry carries a key limit (mask < 0)
  int64_t n_groups;  // dQ: tiles * hkv
  int64_t dq_blocks; // dQ launch size
  int hq, hkv, gsize;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
};

struct PosArgs {
  const I4* segments;  // (seg_start, seg_len, depth offset, node) sorted by start
  int32_t n_segments;
  int64_t n_tokens;
  int32_t* node_id;    // [N] or null
  int32_t* pos_id;     // [N] or null
};

// Chunkwise linear attention over the tree (linear.hip), bf16 tensors.
struct LinArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* out;             // chunk products: O, dQ or dK
  void* out2;            // dV (the fused dK / dV kernel)
  void* state;           // bf16 [pieces, Hkv, D, D] S (forward) or R (backward)
  void* delta;           // bf16 [pieces, Hkv, D, D] K^T V or sum_h Q_h^T dO_h per piece
  float* ends;           // [nodes, Hkv, D, D] fp32 state at a node's end (forward)
                         // or with its first piece's delta added (backward)
  const I8* pieces;      // (token0, len, pred, succ_begin, succ_end, node, flags, 0)
  const int32_t* succ;   // successor piece indices
  const I4* lnodes;      // (first piece, pieces, parent node, node) root first
  const I4* chains;      // scans: heavy paths (begin, end, phase, 0) into chain_nodes
  const int32_t* chain_nodes;  // lnodes indices, each chain's nodes from its head
  const I4* phases;      // host array: (chain_begin, chain_end, 0, 0) per phase
  int n_phases;
  int64_t n_pieces;
  int64_t n_nodes;
  int hq, hkv, gsize;
  float scale;
};

// dtype: 0 bf16, 1 fp32.  Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t n_blocks,
                      hipStream_t stream);
// merges the key parts of split query tiles into O and LSE
hipError_t launch_fwd_combine(const FwdArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int head_dim, hipStream_t stream);
// adds the key parts' partial dQ of split query tiles into dQ
hipError_t launch_bwd_dq_sum(const BwdArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_bwd_post(const BwdArgs& a, int dtype, int head_dim, hipStream_t stream);
// dst[i] = src[i] rounded to the dtype, i < n (src 16-byte aligned)
hipError_t launch_cast(const float* src, void* dst, int64_t n, int dtype, hipStream_t stream);
hipError_t launch_positions(const PosArgs& a, hipStream_t stream);
// backward = 0: delta = K^T V, state scan root first; backward = 1: delta =
// sum_h Q_h^T dO_h, state scan leaves first.  mode: 0 O, 1 dQ, 4 dK and dV.
hipError_t launch_lin_outer(const LinArgs& a, int backward, int head_dim, hipStream_t stream);
hipError_t launch_lin_scan(const LinArgs& a, int backward, int head_dim, hipStream_t stream);
hipError_t launch_lin_chunk(const LinArgs& a, int mode, int head_dim, hipStream_t stream);

// Passes either side of the attention call (prefix_ops.hip).
hipError_t launch_gather(const void* src, void* dst, const int32_t* index, int64_t rows,
                         int64_t row_bytes, hipStream_t stream);
hipError_t launch_scatter_sum(const void* src, void* dst, const int32_t* offsets,
                              const int32_t* positions, int64_t rows, int64_t row_elems, int dtype,
                              hipStream_t stream);
hipError_t launch_rope(void* x, const int32_t* pos, int64_t n_tokens, int heads, int head_dim,
                       double log2_theta, int inverse, int dtype, hipStream_t stream);

// Library-owned backward scratch (scratch.hip): kStaticScratchBytes of
// device memory per GPU, 256-byte aligned.  *out receives the current
// device's address of it (looked up once per device).
constexpr size_t kStaticScratchBytes = static_cast<size_t>(64) << 20;
hipError_t static_scratch(void** out);

}  // namespace tree_attn
