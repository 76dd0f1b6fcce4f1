// Chunkwise causal linear attention over a prefix tree (gfx950).
//
// HARTS (abstract) runs the chunkwise linear-attention layers of hybrid
// models over arbitrary rollout trees in one packed call: state is handed
// from a prefix to every branch in the forward pass, and gradients flow back
// through those handoffs in the backward pass, while each trajectory keeps the
// chunk partition it has in trajectory-wise training.  The recurrence is the
// plain one (no gate, no normaliser):
//
//   o_t = scale * S_t^T q_t,   S_t = sum over s <= t on t's path of k_s v_s^T.
//
// Pieces.  The planner cuts every node where the trajectory depth is a
// multiple of the chunk (64), so each piece starts from a trajectory chunk
// boundary or from a branch point, and every state a piece needs is the sum
// of whole pieces on its path.  A chunk that straddles a branch point is
// computed as its parent part (once) and one part per child, so no prefix
// token is recomputed.
//
// Forward:  (1) dS_p = K_p^T V_p per piece and kv head;  (2) a scan in
// root-first order, S_p = S_pred + dS_pred;  (3) per piece and kv head,
// O = scale (Q S_p + tril(Q K^T) V) for each query head of the group.
// Backward: (1) dR_p = sum_h Q_h^T dO_h;  (2) a reverse scan, R_p = sum over
// successors c of (R_c + dR_c), the handoff of the state gradient from every
// branch to its prefix;  (3) dQ = scale (dO S_p^T + tril(dO V^T) K),
// dK = scale (V R_p^T + sum_h triu(V dO_h^T) Q_h),
// dV = scale (K R_p + sum_h triu(K Q_h^T) dO_h).
// All products run on the matrix cores in bf16 with fp32 accumulation; the
// states stay fp32 in HBM and are rounded to bf16 as MFMA operands.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {
namespace {

constexpr int CH = kLinChunk;

// LDS operand with R rows of K contiguous bf16 (padded by 8 elements so that
// 16-byte fragment reads of consecutive rows spread over the banks).
template <int R, int K>
struct LOp {
  static constexpr int P = K + 8;
  static constexpr int BYTES = R * P * 2;
};

// acc += A[m0 + 0..31, 0..K) . B[n0 + 0..31, 0..K)^T, with A and B in LDS,
// rows PA / PB elements apart: lane l reads row l % 32, elements
// 8 (l / 32) .. + 7 of each 16-wide chunk (the 32x32x16 operand layout).
template <int PA, int PB, int K>
__device__ __forceinline__ void mma_rows(f32x16& acc, const LDS_PTR(__bf16) a, int m0,
                                         const LDS_PTR(__bf16) b, int n0, int lane) {
  const LDS_PTR(__bf16) pa = a + (m0 + (lane & 31)) * PA + 8 * (lane >> 5);
  const LDS_PTR(__bf16) pb = b + (n0 + (lane & 31)) * PB + 8 * (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < K / 16; ++kk) {
    const bf16x8 fa = *reinterpret_cast<const LDS_PTR(bf16x8)>(pa + 16 * kk);
    const bf16x8 fb = *reinterpret_cast<const LDS_PTR(bf16x8)>(pb + 16 * kk);
    acc = mfma32(fa, fb, acc);
  }
}

// Rows 0 .. CH-1 of a token-major tensor (rows `stride` elements apart, D
// columns from `src`) into x[r][c]; rows at or past n are zero.
template <int D, int P>
__device__ __forceinline__ void stage_rows(LDS_PTR(__bf16) x, const __bf16* src, int64_t stride,
                                           int n, int tid) {
  constexpr int CPR = D / 8;
  for (int c = tid; c < CH * CPR; c += 256) {
    const int r = c / CPR, cc = c % CPR;
    i32x4 v = {0, 0, 0, 0};
    if (r < n) v = gload16(src + r * stride + 8 * cc);
    *reinterpret_cast<LDS_PTR(i32x4)>(x + r * P + 8 * cc) = v;
  }
}

// The same rows transposed: x[c][r] (D rows of CH tokens).
template <int D, int P>
__device__ __forceinline__ void stage_cols(LDS_PTR(__bf16) x, const __bf16* src, int64_t stride,
                                           int n, int tid) {
  constexpr int CPR = D / 8;
  for (int c = tid; c < CH * CPR; c += 256) {
    const int r = c / CPR, cc = c % CPR;
    bf16x8 v;
    if (r < n) {
      v = *reinterpret_cast<const bf16x8*>(src + r * stride + 8 * cc);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = to_bf16(0.f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[(8 * cc + e) * P + r] = v[e];
  }
}

// A D x D fp32 state (row-major) as bf16: x[i][j] = s[i][j], or x[j][i] when
// transposed.
template <int D, int P, bool TR>
__device__ __forceinline__ void stage_state(LDS_PTR(__bf16) x, const float* s, int tid) {
  for (int c = tid; c < D * D / 4; c += 256) {
    const int i = c / (D / 4), j = 4 * (c % (D / 4));
    const f32x4 v = *reinterpret_cast<const f32x4*>(s + i * D + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (TR) x[(j + e) * P + i] = to_bf16(v[e]);
      else x[i * P + j + e] = to_bf16(v[e]);
    }
  }
}

// Row and column of accumulator register v of lane l in a 32x32 block.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

}  // namespace

// (1) Per-piece outer-product sums, one workgroup per (piece, kv head g):
// out[p, g] = sum over heads j < nh of A_j^T B_j over the piece's tokens, a
// D x D fp32 matrix.  Forward: A = K, B = V of head g (nh = 1).  Backward:
// A = Q, B = dO of the group's query heads.
template <int D>
__global__ __launch_bounds__(256) void lin_outer_kernel(LinArgs a, int backward) {
  using OP = LOp<D, CH>;
  constexpr int NBD = D / 32, NB = NBD * NBD, PER = (NB + 3) / 4;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(__bf16) xa = (LDS_PTR(__bf16))(smem_dyn);
  LDS_PTR(__bf16) xb = (LDS_PTR(__bf16))(smem_dyn + OP::BYTES);
  const int p = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const I8 pc = load_plan8(a.pieces, p);
  const int tok0 = pc.v[0], len = pc.v[1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qs = static_cast<int64_t>(a.hq) * D, ks = static_cast<int64_t>(a.hkv) * D;
  f32x16 acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  const int nh = backward ? a.gsize : 1;
  for (int j = 0; j < nh; ++j) {
    if (backward) {
      const int h = g * a.gsize + j;
      const int64_t off = static_cast<int64_t>(tok0) * qs + static_cast<int64_t>(h) * D;
      stage_cols<D, OP::P>(xa, static_cast<const __bf16*>(a.q) + off, qs, len, tid);
      stage_cols<D, OP::P>(xb, static_cast<const __bf16*>(a.dout) + off, qs, len, tid);
    } else {
      const int64_t off = static_cast<int64_t>(tok0) * ks + static_cast<int64_t>(g) * D;
      stage_cols<D, OP::P>(xa, static_cast<const __bf16*>(a.k) + off, ks, len, tid);
      stage_cols<D, OP::P>(xb, static_cast<const __bf16*>(a.v) + off, ks, len, tid);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = wave + 4 * i;
      if (blk < NB) mma_rows<OP::P, OP::P, CH>(acc[i], xa, 32 * (blk / NBD), xb, 32 * (blk % NBD), lane);
    }
    __syncthreads();
  }
  float* out = a.delta + (static_cast<int64_t>(p) * a.hkv + g) * D * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave + 4 * i;
    if (blk >= NB) continue;
    const int r0 = 32 * (blk / NBD), c = 32 * (blk % NBD) + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[(r0 + acc_row(v, lane)) * D + c] = acc[i][v];
  }
}

// (2) State scan over the pieces, one thread per (kv head, state element):
// forward, in root-first order, state[p] = state[pred] + delta[pred] (zero at
// a root); backward, in reverse, state[p] = sum over successors c of
// (state[c] + delta[c]) (zero at a leaf).  The running value of the piece
// just done stays in a register, which covers the usual case of a piece
// followed by the next piece of its node; the deltas of eight pieces are
// loaded ahead of their turn.
template <int D>
__global__ __launch_bounds__(256) void lin_scan_kernel(LinArgs a, int backward) {
  const int64_t per = static_cast<int64_t>(a.hkv) * D * D;  // one piece's states
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= per) return;
  const int64_t np = a.n_pieces;
  constexpr int LA = 8;
  int cached = -1;
  float run = 0.f;  // state + delta of piece `cached`
  for (int64_t b = 0; b < np; b += LA) {
    float dl[LA];
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int64_t i = b + u;
      const int64_t p = backward ? np - 1 - i : i;
      dl[u] = i < np ? a.delta[p * per + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int64_t i = b + u;
      if (i >= np) break;
      const int p = static_cast<int>(backward ? np - 1 - i : i);
      const I8 pc = load_plan8(a.pieces, p);
      float s = 0.f;
      if (!backward) {
        const int pr = pc.v[2];
        if (pr >= 0) s = pr == cached ? run : a.state[pr * per + e] + a.delta[pr * per + e];
      } else {
        for (int j = pc.v[3]; j < pc.v[4]; ++j) {
          const int c = a.succ[j];
          s += c == cached ? run : a.state[c * per + e] + a.delta[c * per + e];
        }
      }
      a.state[p * per + e] = s;
      cached = p;
      run = s + dl[u];
    }
  }
}

// (3) Chunk products, one workgroup per (piece, kv head g), a loop over the
// query heads of the group.  With X the piece's rows of one operand, W a D x D
// state, Z and U the piece's rows of two more, and M the causal mask,
//   out = scale (X W^T + (M o X Z^T) U)
// with W^T, U read as "B^T" operands (row n holds column n):
//   OUT: X = Q_h, W = S^T, Z = K, U = V^T, M: key <= query, out = O_h
//   DQ : X = dO_h, W = S,  Z = V, U = K^T, M: key <= query, out = dQ_h
//   DK : X = V,  W = R,    Z = dO_h, U = Q_h^T, M: query >= key, out = dK
//   DV : X = K,  W = R^T,  Z = Q_h, U = dO_h^T, M: query >= key, out = dV
// (summed over the group's heads for DK and DV).
template <int D, int MODE>
__global__ __launch_bounds__(256) void lin_chunk_kernel(LinArgs a) {
  constexpr bool PER_HEAD_X = MODE < 2;  // OUT, DQ: X changes with the head
  using OX = LOp<CH, D>;   // X, Z: CH rows of D
  using OW = LOp<D, D>;    // W: D rows of D
  using OU = LOp<D, CH>;   // U: D rows of CH
  using OA = LOp<CH, CH>;  // masked X Z^T
  constexpr int NBN = D / 32, NB = 2 * NBN, PER = NB / 4;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(__bf16) xs = (LDS_PTR(__bf16))(smem_dyn);
  LDS_PTR(__bf16) ws = (LDS_PTR(__bf16))(smem_dyn + OX::BYTES);
  LDS_PTR(__bf16) zs = (LDS_PTR(__bf16))(smem_dyn + OX::BYTES + OW::BYTES);
  LDS_PTR(__bf16) us = (LDS_PTR(__bf16))(smem_dyn + 2 * OX::BYTES + OW::BYTES);
  LDS_PTR(__bf16) as = (LDS_PTR(__bf16))(smem_dyn + 2 * OX::BYTES + OW::BYTES + OU::BYTES);

  const int p = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const I8 pc = load_plan8(a.pieces, p);
  const int tok0 = pc.v[0], len = pc.v[1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qs = static_cast<int64_t>(a.hq) * D, ks = static_cast<int64_t>(a.hkv) * D;
  const __bf16* Q = static_cast<const __bf16*>(a.q) + static_cast<int64_t>(tok0) * qs;
  const __bf16* dO = static_cast<const __bf16*>(a.dout) + static_cast<int64_t>(tok0) * qs;
  const __bf16* K = static_cast<const __bf16*>(a.k) + static_cast<int64_t>(tok0) * ks + g * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + static_cast<int64_t>(tok0) * ks + g * D;
  const float* st = a.state + (static_cast<int64_t>(p) * a.hkv + g) * D * D;

  // head-independent operands
  if constexpr (MODE == 0) {
    stage_state<D, OW::P, true>(ws, st, tid);
    stage_rows<D, OX::P>(zs, K, ks, len, tid);
    stage_cols<D, OU::P>(us, V, ks, len, tid);
  } else if constexpr (MODE == 1) {
    stage_state<D, OW::P, false>(ws, st, tid);
    stage_rows<D, OX::P>(zs, V, ks, len, tid);
    stage_cols<D, OU::P>(us, K, ks, len, tid);
  } else if constexpr (MODE == 2) {
    stage_state<D, OW::P, false>(ws, st, tid);
    stage_rows<D, OX::P>(xs, V, ks, len, tid);
  } else {
    stage_state<D, OW::P, true>(ws, st, tid);
    stage_rows<D, OX::P>(xs, K, ks, len, tid);
  }

  f32x16 acc[PER];
  auto inter = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
      const int blk = wave + 4 * i;
      mma_rows<OX::P, OW::P, D>(acc[i], xs, 32 * (blk / NBN), ws, 32 * (blk % NBN), lane);
    }
  };
  auto store = [&](__bf16* out, int64_t stride) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = wave + 4 * i;
      const int r0 = 32 * (blk / NBN), c = 32 * (blk % NBN) + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = r0 + acc_row(v, lane);
        if (r < len) out[r * stride + c] = to_bf16(a.scale * acc[i][v]);
      }
    }
  };

  if constexpr (!PER_HEAD_X) {
    __syncthreads();
    inter();
  }
  for (int j = 0; j < a.gsize; ++j) {
    const int h = g * a.gsize + j;
    if constexpr (MODE == 0) stage_rows<D, OX::P>(xs, Q + h * D, qs, len, tid);
    if constexpr (MODE == 1) stage_rows<D, OX::P>(xs, dO + h * D, qs, len, tid);
    if constexpr (MODE == 2) {
      stage_rows<D, OX::P>(zs, dO + h * D, qs, len, tid);
      stage_cols<D, OU::P>(us, Q + h * D, qs, len, tid);
    }
    if constexpr (MODE == 3) {
      stage_rows<D, OX::P>(zs, Q + h * D, qs, len, tid);
      stage_cols<D, OU::P>(us, dO + h * D, qs, len, tid);
    }
    __syncthreads();
    if constexpr (PER_HEAD_X) inter();
    {
      // one 32x32 block of X Z^T per wave, masked, to LDS as bf16
      const int bi = wave >> 1, bj = wave & 1;
      f32x16 t;
#pragma unroll
      for (int v = 0; v < 16; ++v) t[v] = 0.f;
      mma_rows<OX::P, OX::P, D>(t, xs, 32 * bi, zs, 32 * bj, lane);
      const int c = 32 * bj + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * bi + acc_row(v, lane);
        const bool keep = PER_HEAD_X ? c <= r : c >= r;
        as[r * OA::P + c] = to_bf16(keep ? t[v] : 0.f);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = wave + 4 * i;
      mma_rows<OA::P, OU::P, CH>(acc[i], as, 32 * (blk / NBN), us, 32 * (blk % NBN), lane);
    }
    if constexpr (PER_HEAD_X) {
      __bf16* out = static_cast<__bf16*>(a.out) + static_cast<int64_t>(tok0) * qs + h * D;
      store(out, qs);
    }
    __syncthreads();  // before the next head overwrites the staged operands
  }
  if constexpr (!PER_HEAD_X) {
    __bf16* out = static_cast<__bf16*>(a.out) + static_cast<int64_t>(tok0) * ks + g * D;
    store(out, ks);
  }
}

template __global__ void lin_outer_kernel<128>(LinArgs, int);
template __global__ void lin_outer_kernel<64>(LinArgs, int);
template __global__ void lin_scan_kernel<128>(LinArgs, int);
template __global__ void lin_scan_kernel<64>(LinArgs, int);
template __global__ void lin_chunk_kernel<128, 0>(LinArgs);
template __global__ void lin_chunk_kernel<128, 1>(LinArgs);
template __global__ void lin_chunk_kernel<128, 2>(LinArgs);
template __global__ void lin_chunk_kernel<128, 3>(LinArgs);
template __global__ void lin_chunk_kernel<64, 0>(LinArgs);
template __global__ void lin_chunk_kernel<64, 1>(LinArgs);
template __global__ void lin_chunk_kernel<64, 2>(LinArgs);
template __global__ void lin_chunk_kernel<64, 3>(LinArgs);

namespace {

template <class Kern>
hipError_t launch_dyn(Kern kern, int64_t blocks, int bytes, hipStream_t s, const LinArgs& a) {
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), bytes, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t lin_outer_t(const LinArgs& a, int backward, hipStream_t s) {
  const int bytes = 2 * LOp<D, CH>::BYTES;
  auto kern = lin_outer_kernel<D>;
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_pieces * a.hkv)), dim3(256), bytes, s,
                     a, backward);
  return hipGetLastError();
}

template <int D>
hipError_t lin_scan_t(const LinArgs& a, int backward, hipStream_t s) {
  const int64_t per = static_cast<int64_t>(a.hkv) * D * D;
  hipLaunchKernelGGL(lin_scan_kernel<D>, dim3(static_cast<unsigned>((per + 255) / 256)), dim3(256),
                     0, s, a, backward);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t lin_chunk_t(const LinArgs& a, hipStream_t s) {
  const int bytes = 2 * LOp<CH, D>::BYTES + LOp<D, D>::BYTES + LOp<D, CH>::BYTES +
                    LOp<CH, CH>::BYTES;
  return launch_dyn(lin_chunk_kernel<D, MODE>, a.n_pieces * a.hkv, bytes, s, a);
}

}  // namespace

hipError_t launch_lin_outer(const LinArgs& a, int backward, int head_dim, hipStream_t stream) {
  if (a.n_pieces <= 0) return hipSuccess;
  if (head_dim == 128) return lin_outer_t<128>(a, backward, stream);
  if (head_dim == 64) return lin_outer_t<64>(a, backward, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_lin_scan(const LinArgs& a, int backward, int head_dim, hipStream_t stream) {
  if (a.n_pieces <= 0) return hipSuccess;
  if (head_dim == 128) return lin_scan_t<128>(a, backward, stream);
  if (head_dim == 64) return lin_scan_t<64>(a, backward, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_lin_chunk(const LinArgs& a, int mode, int head_dim, hipStream_t stream) {
  if (a.n_pieces <= 0) return hipSuccess;
  if (head_dim == 128) {
    switch (mode) {
      case 0: return lin_chunk_t<128, 0>(a, stream);
      case 1: return lin_chunk_t<128, 1>(a, stream);
      case 2: return lin_chunk_t<128, 2>(a, stream);
      case 3: return lin_chunk_t<128, 3>(a, stream);
    }
  } else if (head_dim == 64) {
    switch (mode) {
      case 0: return lin_chunk_t<64, 0>(a, stream);
      case 1: return lin_chunk_t<64, 1>(a, stream);
      case 2: return lin_chunk_t<64, 2>(a, stream);
      case 3: return lin_chunk_t<64, 3>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tree_attn
