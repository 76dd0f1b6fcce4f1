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
// All products run on the matrix cores in bf16 with fp32 accumulation.  The
// scans accumulate in fp32 and hand the per-piece states to the chunk kernels
// in bf16 (their MFMA operand type); per-piece deltas are stored in bf16 too.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {
namespace {

constexpr int CH = kLinChunk;

// Rows 0 .. CH-1 of a token-major tensor (rows `stride` elements apart, D
// columns from `src`), 16 bytes per thread and step, into registers (rows at
// or past n read as zero) and from there into a swizzled LDS tile (see
// Tile).  The two halves are separate so that a tile can be fetched while
// the previous one is in use.
template <int D>
struct TileRegs {
  static constexpr int CPR = D / 8, PER = CH * CPR / 256;
  i32x4 v[PER];
  __device__ __forceinline__ void load(const __bf16* src, int64_t stride, int n, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
      v[i] = i32x4{0, 0, 0, 0};
      if (r < n) v[i] = gload16(src + r * stride + 8 * cc);
    }
  }
  __device__ __forceinline__ void store(LDS_PTR(char) t, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
      lds_write16(t, Tile<D, CH>::chunk_off(r, cc), v[i]);
    }
  }
};

template <int D>
__device__ __forceinline__ void stage_tile(LDS_PTR(char) t, const __bf16* src, int64_t stride,
                                           int n, int tid) {
  TileRegs<D> r;
  r.load(src, stride, n, tid);
  r.store(t, tid);
}

// B operand fragments of a D x D bf16 state W read straight from global
// memory (L2): f[kk] holds W[n][16 kk + 8 (lane / 32) + s] for
// n = n0 + lane % 32.  W is the state s itself (TR = false: one 16-byte load
// per fragment) or its transpose (TR = true: eight 2-byte loads, each reading
// 32 consecutive values across the lane half).
template <int D, bool TR>
__device__ __forceinline__ void state_frags(bf16x8 (&f)[D / 16], const __bf16* s, int n0,
                                            int lane) {
  const int n = n0 + (lane & 31), h = 8 * (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int k0 = 16 * kk + h;
    if constexpr (!TR) {
      f[kk] = *reinterpret_cast<const bf16x8*>(s + n * D + k0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[kk][e] = s[(k0 + e) * D + n];
    }
  }
}

// Row and column of accumulator register v of lane l in a 32x32 block.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

}  // namespace

// (1) Per-piece outer-product sums, one workgroup per (piece, kv head g):
// out[p, g] = sum over heads j < nh of A_j^T B_j over the piece's tokens, a
// D x D matrix accumulated in fp32 and stored as bf16.  Forward: A = K, B = V of head g (nh = 1).  Backward:
// A = Q, B = dO of the group's query heads.  Both are staged row-major and
// read as transposed operands (the reduction runs over the tokens).  The
// staging is not overlapped inside a workgroup; three resident workgroups
// per CU (at most 170 registers a lane, with the accumulators kept in
// ordinary VGPRs; the launch's LDS request keeps it from four) overlap one
// another's loads instead.
template <int D>
__global__ __launch_bounds__(256, 3) void lin_outer_kernel(LinArgs a, int backward) {
  using T = Tile<D, CH>;
  constexpr int NBD = D / 32, NB = NBD * NBD, PER = (NB + 3) / 4;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) ta = (LDS_PTR(char))(smem_dyn);
  LDS_PTR(char) tb = (LDS_PTR(char))(smem_dyn + T::BYTES);
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
      stage_tile<D>(ta, static_cast<const __bf16*>(a.q) + off, qs, len, tid);
      stage_tile<D>(tb, static_cast<const __bf16*>(a.dout) + off, qs, len, tid);
    } else {
      const int64_t off = static_cast<int64_t>(tok0) * ks + static_cast<int64_t>(g) * D;
      stage_tile<D>(ta, static_cast<const __bf16*>(a.k) + off, ks, len, tid);
      stage_tile<D>(tb, static_cast<const __bf16*>(a.v) + off, ks, len, tid);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = wave + 4 * i;
      if (blk >= NB) continue;
      const int bi = blk / NBD, bj = blk % NBD;
#pragma unroll
      for (int kk = 0; kk < CH / 16; ++kk)
        acc[i] = mfma32(tr_operand<T>(ta, 16 * kk, 32 * bi, lane),
                        tr_operand<T>(tb, 16 * kk, 32 * bj, lane), acc[i]);
    }
    __syncthreads();
  }
  __bf16* out = static_cast<__bf16*>(a.delta) + (static_cast<int64_t>(p) * a.hkv + g) * D * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave + 4 * i;
    if (blk >= NB) continue;
    const int r0 = 32 * (blk / NBD), c = 32 * (blk % NBD) + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[(r0 + acc_row(v, lane)) * D + c] = to_bf16(acc[i][v]);
  }
}

// (2) State scan, one thread per two neighbouring (kv head, state element)
// pairs, accumulating in fp32, and one workgroup row (blockIdx.y) per heavy
// path of the launch's phase: the path's nodes go head first (forward) or
// tail first (backward), while the paths of one phase, which share no node,
// run side by side; phases are launched in order (forward) or in reverse
// (backward), so that a path's head finds its parent's end state, and a
// node its light children's handed-up gradients, already written.  Inside a
// node the pieces form a chain, streamed with their sums fetched LA pieces
// ahead.
//   Forward: the state entering a node's first piece is the state at its
//   parent's end (zero at a root); each piece's entering state is stored,
//   then its sum added; the node's end state goes to `ends`.
//   Backward: the gradient leaving a node's last piece is the sum of what
//   its children hand up (zero at a leaf); walking the chain backwards, each
//   piece's leaving gradient is stored, then its sum added; what is left is
//   handed to the parent through `ends`.
// The chunk kernels read the stored states as bf16.
template <int D>
__global__ __launch_bounds__(256) void lin_scan_kernel(LinArgs a, int backward, int chain0) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
  const int64_t per = static_cast<int64_t>(a.hkv) * D * D;  // one piece's states
  // two neighbouring elements per thread: 4-byte bf16 accesses
  const int64_t e = 2 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (e >= per) return;
  const __bf16* delta = static_cast<const __bf16*>(a.delta);
  __bf16* state = static_cast<__bf16*>(a.state);
  constexpr int LA = 16;
  const I4 ch = load_plan4(a.chains, chain0 + static_cast<int>(blockIdx.y));
  const int nn = ch.y - ch.x;
  for (int k = 0; k < nn; ++k) {
    const I4 nd =
        load_plan4(a.lnodes, load_plan1(a.chain_nodes, backward ? ch.y - 1 - k : ch.x + k));
    const int first = nd.x, count = nd.y;
    float s0 = 0.f, s1 = 0.f;
    if (!backward) {
      if (nd.z >= 0) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(a.ends + nd.z * per + e);
        s0 = x[0];
        s1 = x[1];
      }
    } else {
      const I8 lp = load_plan8(a.pieces, first + count - 1);
      for (int j = lp.v[3]; j < lp.v[4]; ++j) {  // the children's first pieces
        const int child = load_plan8(a.pieces, load_plan1(a.succ, j)).v[5];
        const f32x2 x = *reinterpret_cast<const f32x2*>(a.ends + child * per + e);
        s0 += x[0];
        s1 += x[1];
      }
    }
    // the chain: i-th piece visited is first + i (forward) or last - i
    auto piece = [&](int i) { return backward ? first + count - 1 - i : first + i; };
    bf16x2 dl[LA], dn[LA];
#pragma unroll
    for (int u = 0; u < LA; ++u)
      dl[u] = u < count ? *reinterpret_cast<const bf16x2*>(delta + piece(u) * per + e)
                        : bf16x2{};
    for (int i0 = 0; i0 < count; i0 += LA) {
#pragma unroll
      for (int u = 0; u < LA; ++u) {
        const int i = i0 + LA + u;
        dn[u] = i < count ? *reinterpret_cast<const bf16x2*>(delta + piece(i) * per + e)
                          : bf16x2{};
      }
#pragma unroll
      for (int u = 0; u < LA; ++u) {
        if (i0 + u >= count) break;
        bf16x2 out;
        out[0] = to_bf16(s0);
        out[1] = to_bf16(s1);
        *reinterpret_cast<bf16x2*>(state + piece(i0 + u) * per + e) = out;
        s0 += static_cast<float>(dl[u][0]);
        s1 += static_cast<float>(dl[u][1]);
      }
#pragma unroll
      for (int u = 0; u < LA; ++u) dl[u] = dn[u];
    }
    f32x2 w;
    w[0] = s0;
    w[1] = s1;
    *reinterpret_cast<f32x2*>(a.ends + nd.w * per + e) = w;
  }
}

// (3) Chunk products for O and dQ, one workgroup per (piece, kv head g), a
// loop over the query heads of the group.  With X, Z, Y the piece's rows of
// three operands, W a D x D state and M the causal mask (key <= query),
//   out = scale (X W^T + (M o X Z^T) Y)          (W^T: W read as B^T)
//   OUT: X = Q_h,  W = S^T, Z = K, Y = V, out = O_h
//   DQ : X = dO_h, W = S,   Z = V, Y = K, out = dQ_h
// X, Z, Y sit row-major in swizzled LDS tiles: X and Z feed X Z^T as row
// operands, Y feeds the second product as transposed operands.  The state
// fragments (bf16) come from global memory once per workgroup and stay in
// registers.  Wave w owns output blocks w and w + 4 (rows 0 and 32 of
// column block w) at D = 128, block w at D = 64, and one 32 x 32 block of
// M o X Z^T, which goes to LDS as bf16.
template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void lin_chunk_kernel(LinArgs a) {
  static_assert(MODE == 0 || MODE == 1, "O or dQ");
  using T = Tile<D, CH>;    // CH tokens x D
  using TA = Tile<CH, CH>;  // masked X Z^T
  constexpr int NBN = D / 32, NB = 2 * NBN, PER = NB / 4, KD = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) xs = (LDS_PTR(char))(smem_dyn);
  LDS_PTR(char) zs = (LDS_PTR(char))(smem_dyn + T::BYTES);
  LDS_PTR(char) ys = (LDS_PTR(char))(smem_dyn + 2 * T::BYTES);
  LDS_PTR(char) as = (LDS_PTR(char))(smem_dyn + 3 * T::BYTES);

  const int p = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const I8 pc = load_plan8(a.pieces, p);
  const int tok0 = pc.v[0], len = pc.v[1];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qs = static_cast<int64_t>(a.hq) * D, ks = static_cast<int64_t>(a.hkv) * D;
  // X rows of the group's heads, Z and Y rows of kv head g
  const __bf16* X = static_cast<const __bf16*>(MODE == 0 ? a.q : a.dout) +
                    static_cast<int64_t>(tok0) * qs;
  const __bf16* K = static_cast<const __bf16*>(a.k) + static_cast<int64_t>(tok0) * ks + g * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + static_cast<int64_t>(tok0) * ks + g * D;
  const __bf16* st =
      static_cast<const __bf16*>(a.state) + (static_cast<int64_t>(p) * a.hkv + g) * D * D;

  stage_tile<D>(zs, MODE == 0 ? K : V, ks, len, tid);
  stage_tile<D>(ys, MODE == 0 ? V : K, ks, len, tid);
  // this wave's output column block and its state fragments
  const int n0 = 32 * (wave % NBN);
  bf16x8 wf[KD];
  state_frags<D, MODE == 0>(wf, st, n0, lane);

  // head j + 1's rows are fetched into registers while head j is computed
  TileRegs<D> rx;
  rx.load(X + g * a.gsize * D, qs, len, tid);
  f32x16 acc[PER];
  for (int j = 0; j < a.gsize; ++j) {
    const int h = g * a.gsize + j;
    rx.store(xs, tid);
    if (j + 1 < a.gsize) rx.load(X + (h + 1) * D, qs, len, tid);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int m0 = 32 * ((wave + 4 * i) / NBN);
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        acc[i] = mfma32(row_operand<T>(xs, m0 + l32, 2 * kk + half), wf[kk], acc[i]);
    }
    {
      // one 32x32 block of M o X Z^T per wave, to LDS as bf16
      const int bi = wave >> 1, bj = wave & 1;
      f32x16 t;
#pragma unroll
      for (int v = 0; v < 16; ++v) t[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        t = mfma32(row_operand<T>(xs, 32 * bi + l32, 2 * kk + half),
                   row_operand<T>(zs, 32 * bj + l32, 2 * kk + half), t);
      const int c = 32 * bj + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * bi + acc_row(v, lane);
        *reinterpret_cast<LDS_PTR(__bf16)>(as + TA::elem_off(r, c)) = to_bf16(c <= r ? t[v] : 0.f);
      }
    }
    __syncthreads();
    __bf16* out = static_cast<__bf16*>(a.out) + static_cast<int64_t>(tok0) * qs + h * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int m0 = 32 * ((wave + 4 * i) / NBN);
#pragma unroll
      for (int kk = 0; kk < CH / 16; ++kk)
        acc[i] = mfma32(row_operand<TA>(as, m0 + l32, 2 * kk + half),
                        tr_operand<T>(ys, 16 * kk, n0, lane), acc[i]);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + acc_row(v, lane);
        if (r < len) out[r * qs + n0 + l32] = to_bf16(a.scale * acc[i][v]);
      }
    }
    __syncthreads();  // before the next head overwrites the staged operands
  }
}

// (3') dK and dV in one pass, one workgroup per (piece, kv head g):
//   dK = scale (V R^T + sum_h (M o V dO_h^T) Q_h)
//   dV = scale (K R   + sum_h (M o K Q_h^T) dO_h),   M: query >= key,
// which share the per-head rows Q_h and dO_h, fetched once.  Tiles: V, K (fixed), dO_h, Q_h, and the two
// masked blocks V dO_h^T and K Q_h^T (80 KiB at D = 128, two workgroups per
// CU).  Each wave holds its dK and dV output blocks and the R fragments of
// both orientations.
template <int D>
__global__ __launch_bounds__(256, 2) void lin_dkdv_kernel(LinArgs a) {
  using T = Tile<D, CH>;
  using TA = Tile<CH, CH>;
  constexpr int NBN = D / 32, NB = 2 * NBN, PER = NB / 4, KD = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) vs = (LDS_PTR(char))(smem_dyn);
  LDS_PTR(char) kt = (LDS_PTR(char))(smem_dyn + T::BYTES);
  LDS_PTR(char) dos = (LDS_PTR(char))(smem_dyn + 2 * T::BYTES);
  LDS_PTR(char) qs_t = (LDS_PTR(char))(smem_dyn + 3 * T::BYTES);
  LDS_PTR(char) ak = (LDS_PTR(char))(smem_dyn + 4 * T::BYTES);
  LDS_PTR(char) av = (LDS_PTR(char))(smem_dyn + 4 * T::BYTES + TA::BYTES);

  const int p = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const I8 pc = load_plan8(a.pieces, p);
  const int tok0 = pc.v[0], len = pc.v[1];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qs = static_cast<int64_t>(a.hq) * D, ks = static_cast<int64_t>(a.hkv) * D;
  const __bf16* Q = static_cast<const __bf16*>(a.q) + static_cast<int64_t>(tok0) * qs;
  const __bf16* dO = static_cast<const __bf16*>(a.dout) + static_cast<int64_t>(tok0) * qs;
  const __bf16* K = static_cast<const __bf16*>(a.k) + static_cast<int64_t>(tok0) * ks + g * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + static_cast<int64_t>(tok0) * ks + g * D;
  const __bf16* st =
      static_cast<const __bf16*>(a.state) + (static_cast<int64_t>(p) * a.hkv + g) * D * D;

  stage_tile<D>(vs, V, ks, len, tid);
  stage_tile<D>(kt, K, ks, len, tid);
  const int n0 = 32 * (wave % NBN);
  f32x16 acc_k[PER], acc_v[PER];
  {
    bf16x8 wk[KD], wv[KD];
    state_frags<D, false>(wk, st, n0, lane);  // dK: W = R
    state_frags<D, true>(wv, st, n0, lane);   // dV: W = R^T
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int m0 = 32 * ((wave + 4 * i) / NBN);
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_k[i][v] = acc_v[i][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        acc_k[i] = mfma32(row_operand<T>(vs, m0 + l32, 2 * kk + half), wk[kk], acc_k[i]);
        acc_v[i] = mfma32(row_operand<T>(kt, m0 + l32, 2 * kk + half), wv[kk], acc_v[i]);
      }
    }
  }
  TileRegs<D> rd, rq;
  auto fetch = [&](int h) __attribute__((always_inline)) {
    rd.load(dO + h * D, qs, len, tid);
    rq.load(Q + h * D, qs, len, tid);
  };
  fetch(g * a.gsize);
  for (int j = 0; j < a.gsize; ++j) {
    const int h = g * a.gsize + j;
    rd.store(dos, tid);
    rq.store(qs_t, tid);
    if (j + 1 < a.gsize) fetch(h + 1);
    __syncthreads();
    {
      // one 32x32 block of each masked product per wave (key row r, query
      // column c, kept for c >= r)
      const int bi = wave >> 1, bj = wave & 1;
      f32x16 tk, tv;
#pragma unroll
      for (int v = 0; v < 16; ++v) tk[v] = tv[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        tk = mfma32(row_operand<T>(vs, 32 * bi + l32, 2 * kk + half),
                    row_operand<T>(dos, 32 * bj + l32, 2 * kk + half), tk);
        tv = mfma32(row_operand<T>(kt, 32 * bi + l32, 2 * kk + half),
                    row_operand<T>(qs_t, 32 * bj + l32, 2 * kk + half), tv);
      }
      const int c = 32 * bj + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * bi + acc_row(v, lane);
        const bool keep = c >= r;
        *reinterpret_cast<LDS_PTR(__bf16)>(ak + TA::elem_off(r, c)) = to_bf16(keep ? tk[v] : 0.f);
        *reinterpret_cast<LDS_PTR(__bf16)>(av + TA::elem_off(r, c)) = to_bf16(keep ? tv[v] : 0.f);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int m0 = 32 * ((wave + 4 * i) / NBN);
#pragma unroll
      for (int kk = 0; kk < CH / 16; ++kk) {
        acc_k[i] = mfma32(row_operand<TA>(ak, m0 + l32, 2 * kk + half),
                          tr_operand<T>(qs_t, 16 * kk, n0, lane), acc_k[i]);
        acc_v[i] = mfma32(row_operand<TA>(av, m0 + l32, 2 * kk + half),
                          tr_operand<T>(dos, 16 * kk, n0, lane), acc_v[i]);
      }
    }
    __syncthreads();  // before the next head overwrites the staged operands
  }
  __bf16* dk = static_cast<__bf16*>(a.out) + static_cast<int64_t>(tok0) * ks + g * D;
  __bf16* dv = static_cast<__bf16*>(a.out2) + static_cast<int64_t>(tok0) * ks + g * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int m0 = 32 * ((wave + 4 * i) / NBN);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m0 + acc_row(v, lane);
      if (r < len) {
        dk[r * ks + n0 + l32] = to_bf16(a.scale * acc_k[i][v]);
        dv[r * ks + n0 + l32] = to_bf16(a.scale * acc_v[i][v]);
      }
    }
  }
}

template __global__ void lin_dkdv_kernel<128>(LinArgs);
template __global__ void lin_dkdv_kernel<64>(LinArgs);
template __global__ void lin_outer_kernel<128>(LinArgs, int);
template __global__ void lin_outer_kernel<64>(LinArgs, int);
template __global__ void lin_scan_kernel<128>(LinArgs, int, int);
template __global__ void lin_scan_kernel<64>(LinArgs, int, int);
template __global__ void lin_chunk_kernel<128, 0>(LinArgs);
template __global__ void lin_chunk_kernel<128, 1>(LinArgs);
template __global__ void lin_chunk_kernel<64, 0>(LinArgs);
template __global__ void lin_chunk_kernel<64, 1>(LinArgs);

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
  // at D = 128 the kernel's registers would admit four workgroups per CU,
  // which measured slower than three: the LDS request holds it to three
  // (3 x 48 KiB fits the CU's 160 KiB, 4 x 48 KiB does not)
  constexpr int kThreePerCu = 48 * 1024;
  const int bytes = D == 128 ? kThreePerCu : 2 * Tile<D, CH>::BYTES;
  static_assert(2 * Tile<128, CH>::BYTES <= kThreePerCu, "tiles fit the request");
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
  constexpr int kMaxRows = 65535;  // grid y limit
  for (int k = 0; k < a.n_phases; ++k) {
    const I4 ph = a.phases[backward ? a.n_phases - 1 - k : k];
    for (int c0 = ph.x; c0 < ph.y; c0 += kMaxRows) {
      const int rows = ph.y - c0 < kMaxRows ? ph.y - c0 : kMaxRows;
      hipLaunchKernelGGL(lin_scan_kernel<D>,
                         dim3(static_cast<unsigned>((per / 2 + 255) / 256),
                              static_cast<unsigned>(rows)),
                         dim3(256), 0, s, a, backward, c0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

template <int D, int MODE>
hipError_t lin_chunk_t(const LinArgs& a, hipStream_t s) {
  const int bytes = 3 * Tile<D, CH>::BYTES + Tile<CH, CH>::BYTES;
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

template <int D>
hipError_t lin_dkdv_t(const LinArgs& a, hipStream_t s) {
  const int bytes = 4 * Tile<D, CH>::BYTES + 2 * Tile<CH, CH>::BYTES;
  return launch_dyn(lin_dkdv_kernel<D>, a.n_pieces * a.hkv, bytes, s, a);
}

hipError_t launch_lin_chunk(const LinArgs& a, int mode, int head_dim, hipStream_t stream) {
  if (a.n_pieces <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (mode == 0) return lin_chunk_t<128, 0>(a, stream);
    if (mode == 1) return lin_chunk_t<128, 1>(a, stream);
    if (mode == 4) return lin_dkdv_t<128>(a, stream);
  } else if (head_dim == 64) {
    if (mode == 0) return lin_chunk_t<64, 0>(a, stream);
    if (mode == 1) return lin_chunk_t<64, 1>(a, stream);
    if (mode == 4) return lin_dkdv_t<64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tree_attn
