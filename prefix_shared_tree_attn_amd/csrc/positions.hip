// Per-token node index and position id of a prefix tree (gfx950).
//
// A unique token sits at the same position on every root-to-leaf path
// through it: the tokens of its ancestor nodes come first, then the earlier
// tokens of its own node (AReaL-DTA, abstract: a shared prefix is one
// computation for all trajectories through it).  That position -- the
// token's depth -- is the position id a trajectory-wise run would give it,
// e.g. for rotary embeddings.  One thread per token finds its segment by a
// binary search over the segments sorted by start (the node table is small
// and stays in cache) and writes node index and depth; the pass is bound by
// the 8 bytes per token it writes.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace tree_attn {

__global__ __launch_bounds__(256) void tree_attn_positions_kernel(PosArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= a.n_tokens) return;
  // largest segment start <= t
  int lo = 0, hi = a.n_segments - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.segments[mid].x <= t) lo = mid;
    else hi = mid - 1;
  }
  const I4 s = a.segments[lo];
  if (a.node_id) a.node_id[t] = s.w;
  if (a.pos_id) a.pos_id[t] = s.z + static_cast<int32_t>(t - s.x);
}

hipError_t launch_positions(const PosArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 0) return hipSuccess;
  const int64_t blocks = (a.n_tokens + 255) / 256;
  hipLaunchKernelGGL(tree_attn_positions_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace tree_attn
