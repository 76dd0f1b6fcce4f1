// Prefix compression: per-trajectory token lists -> prefix tree.
#pragma once

#include <cstdint>
#include <string>

#include "planner.h"

namespace tree_attn {

// Builds the compressed prefix tree (radix tree) of num_traj token
// sequences.  Output arrays are caller-owned with the capacities documented
// in include/tree_attn.h; see tree_attn_build_tree.
Status build_prefix_tree(const int32_t* tokens, const int64_t* traj_offsets, int32_t num_traj,
                         int32_t* parent, int32_t* seg_start, int32_t* seg_len,
                         int32_t* unique_tokens, int32_t* traj_index, int32_t* mult,
                         int32_t* inv_offsets, int32_t* inv_positions, int32_t* num_nodes,
                         int32_t* num_tokens, std::string* err);

}  // namespace tree_attn
