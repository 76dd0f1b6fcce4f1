// Forward pass of prefix-shared tree attention (gfx950).
//
// Each unique token is computed once and attends to itself and its
// ancestors on its root-to-leaf path (AReaL-DTA, abstract; Tree Training in
// the HARTS page's related list).  One workgroup handles one query tile (up
// to 128 rows of one tree node) for one query head and walks the key ranges
// the planner listed for the tile: its ancestors' segments root first, then
// its own node up to the tile's last row with the causal mask.
//
// Wave w owns query rows 32w .. 32w+31 of the tile.  Scores are formed
// transposed, S^T = K Q^T, so that lane l holds one query row (l % 32) and the
// 32 scores of a 64-key step sit in that lane's registers: the online-softmax
// row max needs one exchange between the two lane halves and the row sum
// none until the end.  The probabilities then feed O^T += V^T P^T as the B
// operand without leaving registers, and V^T is read from the row-major LDS
// tile with transpose loads.  K and V tiles are staged through LDS once per
// step and shared by the four waves.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void tree_attn_fwd_kernel(FwdArgs a) {
  constexpr bool SPLIT = IsSplit<T>::value;
  constexpr int NP = SPLIT ? 2 : 1;
  constexpr int KC = D / 16;  // 16-wide reduction chunks of q.k
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int PLANE = kFwdKeys * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * NP * PLANE];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem);
  LDS_PTR(char) k_hi = lds;
  LDS_PTR(char) k_lo = lds + PLANE;
  LDS_PTR(char) v_hi = lds + NP * PLANE;
  LDS_PTR(char) v_lo = lds + NP * PLANE + PLANE;

  // Workgroup -> (query tile, kv head, query head).  Workgroup b runs on XCD
  // b % 8; the query heads of one kv group get consecutive slots on the same
  // XCD so that their shared K/V tiles meet in one L2, and groups are dealt
  // to XCDs round robin in longest-first order.
  const int b = blockIdx.x;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int64_t gi = static_cast<int64_t>(slot / a.gsize) * kXcds + xcd;
  if (gi >= a.n_groups) return;
  const int tile = static_cast<int>(gi / a.hkv);
  const int g = static_cast<int>(gi % a.hkv);
  const int h = g * a.gsize + slot % a.gsize;
  const I4 t = a.tiles[tile];
  const int q0 = t.x, q1 = t.y;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t last = a.n_tokens - 1;
  const int64_t qs = static_cast<int64_t>(a.hq) * D;   // row stride of Q / O
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;  // row stride of K / V
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k) + static_cast<int64_t>(g) * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<int64_t>(g) * D;

  const int qrow = q0 + 32 * wave + l32;  // this lane's query row
  const int wave_q0 = q0 + 32 * wave;
  Frag<SPLIT> qf[KC];
  {
    const int64_t r = qrow < last ? qrow : last;
    const T* qp = Q + r * qs + static_cast<int64_t>(h) * D + 8 * half;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = load_frag8(qp + 16 * kc);
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  float m = -INFINITY;  // running max of base-2 scaled scores of row qrow
  float lsum = 0.f;     // running sum over this lane's keys

  for (int ri = t.z; ri < t.w; ++ri) {
    const I4 rg = a.ranges[ri];
    const int k0 = rg.x, k1 = rg.y;
    const bool causal = rg.z != 0;
    for (int kt = k0; kt < k1; kt += kFwdKeys) {
      __syncthreads();  // all waves are done reading the previous tile
      load_tile<T, D, kFwdKeys, 256>(k_hi, k_lo, K, ks, kt, last, tid);
      load_tile<T, D, kFwdKeys, 256>(v_hi, v_lo, V, ks, kt, last, tid);
      __syncthreads();

      // S^T for keys kt + 32 kb + (0..31); A row r holds key swap23(r) so
      // that register v of this lane is key 16 (v / 8) + 8 half + v % 8.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
        const int krow = 32 * kb + swap23(l32);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          Frag<SPLIT> af;
          af.h = row_operand<D>(k_hi, krow, 2 * kc + half);
          if constexpr (SPLIT) af.l = row_operand<D>(k_lo, krow, 2 * kc + half);
          mma<SPLIT>(sacc[kb], af, qf[kc]);
        }
      }

      // scale, mask, online softmax
      const bool need_mask = (kt + kFwdKeys > k1) || (causal && kt + kFwdKeys - 1 > wave_q0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float s = sacc[kb][v] * a.scale_log2;
          if (need_mask) {
            const int key = kt + 32 * kb + 16 * (v >> 3) + 8 * half + (v & 7);
            const bool ok = key < k1 && (!causal || key <= qrow);
            s = ok ? s : -INFINITY;
          }
          sacc[kb][v] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][v] - m_use);
          sacc[kb][v] = p;
          psum += p;
        }
      }
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

      // O^T += V^T P^T over four 16-key chunks
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float pv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) pv[s] = sacc[c >> 1][8 * (c & 1) + s];
        const Frag<SPLIT> pf = pack8<SPLIT>(pv);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          Frag<SPLIT> vf;
          vf.h = tr_operand<D>(v_hi, 16 * c, 32 * db, lane);
          if constexpr (SPLIT) vf.l = tr_operand<D>(v_lo, 16 * c, 32 * db, lane);
          mma<SPLIT>(oacc[db], vf, pf);
        }
      }
    }
  }

  // finalize: O = O^T / l, LSE = ln 2 * (m + log2 l)
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (qrow < q1) {
    const float inv = 1.f / ltot;
    T* op = static_cast<T*>(a.o) + static_cast<int64_t>(qrow) * qs + static_cast<int64_t>(h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4(op + 32 * db + 8 * j + 4 * half, oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
               oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
    if (half == 0)
      a.lse[static_cast<int64_t>(h) * a.n_tokens + qrow] =
          kLn2 * (m + __builtin_amdgcn_logf(ltot));
  }
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t n_blocks,
                      hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_blocks)), block(256);
  if (dtype == 0 && head_dim == 128)
    hipLaunchKernelGGL((tree_attn_fwd_kernel<__bf16, 128>), grid, block, 0, stream, a);
  else if (dtype == 0 && head_dim == 64)
    hipLaunchKernelGGL((tree_attn_fwd_kernel<__bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((tree_attn_fwd_kernel<float, 128>), grid, block, 0, stream, a);
  else if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((tree_attn_fwd_kernel<float, 64>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tree_attn
