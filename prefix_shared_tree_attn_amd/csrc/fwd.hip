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
//
// In a launch with too few (tile, head) workgroups to occupy the chip, the
// planner may cut a tile's keys into parts; a part writes its unnormalised
// partial result and tree_attn_fwd_combine_kernel merges the parts.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {

template <typename T, int D>
struct FwdCfg {
  static constexpr bool SPLIT = IsSplit<T>::value;
  static constexpr int NP = SPLIT ? 2 : 1;
  // K / V buffers: two (the next key tile streams in while the current one
  // is used) unless fp32 tiles (two 16-bit planes) at D = 128 would not fit.
  static constexpr int NBUF = (SPLIT && D == 128) ? 1 : 2;
  static constexpr int PLANE = kFwdKeys * D * 2;
  static constexpr int BYTES = NBUF * 2 * NP * PLANE;
};

// Max of x over lanes l and l ^ 32: v_permlane32_swap exchanges the two
// 32-lane halves between its operands, so with x in both, the pair it returns
// holds x and its partner lane's x in every lane.
__device__ __forceinline__ float max_across_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void tree_attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D>;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int NP = C::NP, NBUF = C::NBUF;
  constexpr int KC = D / 16;  // 16-wide reduction chunks of q.k
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int PLANE = C::PLANE;
  using KT = Tile<D, kFwdKeys>;  // K and V tiles of a key step
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);
  auto k_tile = [&](int buf, int plane) { return lds + ((buf * 2 + 0) * NP + plane) * PLANE; };
  auto v_tile = [&](int buf, int plane) { return lds + ((buf * 2 + 1) * NP + plane) * PLANE; };

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
  const I4 t = load_plan4(a.tiles, tile);
  const int q0 = t.x, q1 = t.y;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Key-tile prefetch: buffer loads straight to LDS for bf16, through
  // registers (split into 16-bit planes) for fp32.
  constexpr int SPLIT_PER = SPLIT ? kFwdKeys * D / 4 / 256 : 1;
  i32x4 kreg[SPLIT_PER], vreg[SPLIT_PER];
  TileLoader<D, kFwdKeys, 4> tl;
  if constexpr (!SPLIT) tl.init(static_cast<int>(ks * sizeof(T)), wave, lane);
  auto issue = [&](int kt, int buf) {
    if constexpr (!SPLIT) {
      const int64_t left = a.n_tokens - kt;
      const int rows = left < kFwdKeys ? static_cast<int>(left) : kFwdKeys;
      const uint32_t rb = static_cast<uint32_t>(ks * sizeof(T));
      tl.issue(k_tile(buf, 0), tile_rsrc(K + static_cast<int64_t>(kt) * ks, rows, rb));
      tl.issue(v_tile(buf, 0), tile_rsrc(V + static_cast<int64_t>(kt) * ks, rows, rb));
    } else {
      constexpr int CPR = D / 4;
#pragma unroll
      for (int i = 0; i < SPLIT_PER; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
        const int64_t row = kt + r < last ? kt + r : last;
        kreg[i] = gload16(K + row * ks + cc * 4);
        vreg[i] = gload16(V + row * ks + cc * 4);
      }
    }
  };
  auto commit = [&](int buf) {
    if constexpr (SPLIT) {
      constexpr int CPR = D / 4;
#pragma unroll
      for (int i = 0; i < SPLIT_PER; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
#pragma unroll
        for (int tv = 0; tv < 2; ++tv) {
          const f32x4 f = __builtin_bit_cast(f32x4, tv ? vreg[i] : kreg[i]);
          bf16x4 hi, lo;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            __bf16 hs, ls;
            split_bits(f[s2], hs, ls);
            hi[s2] = hs;
            lo[s2] = ls;
          }
          const int off = KT::elem_off(r, cc * 4);
          *reinterpret_cast<LDS_PTR(bf16x4)>((tv ? v_tile(buf, 0) : k_tile(buf, 0)) + off) = hi;
          *reinterpret_cast<LDS_PTR(bf16x4)>((tv ? v_tile(buf, 1) : k_tile(buf, 1)) + off) = lo;
        }
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  float m = -INFINITY;                // running max of base-2 scaled scores of row qrow
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // running sum over this lane's keys, four parts

  // Key tiles in order: the tile's ranges (ancestors root first, then the
  // causal range of its own node), kFwdKeys keys at a time.
  int ri = t.z;
  I4 rg = load_plan4(a.ranges, ri);
  int kt = rg.x;
  issue(kt, 0);
  commit(0);
  int step = 0;
  while (true) {
    // the following key tile, if any
    int nri = ri, nkt = kt + kFwdKeys;
    I4 nrg = rg;
    bool has_next = true;
    if (nkt >= rg.y) {
      nri = ri + 1;
      has_next = nri < t.w;
      if (has_next) {
        nrg = load_plan4(a.ranges, nri);
        nkt = nrg.x;
      }
    }
    const int buf = NBUF == 2 ? (step & 1) : 0;
    wait_vm();
    __syncthreads();  // this tile is in LDS; everyone is done with the other buffer
    if (NBUF == 2 && has_next) issue(nkt, buf ^ 1);

    const int k1 = rg.y;
    const bool causal = rg.z != 0;
    // every key of the tile lies past every row of this wave, or the wave
    // has no rows (the last tile of a node): nothing to do, and the SIMD's
    // other wave runs alone meanwhile
    const bool skip = (causal && kt > wave_q0 + 31) || wave_q0 >= q1;
    if (!skip) {
    // S^T for keys kt + 32 kb + (0..31); A row r holds key swap23(r) so
    // that register v of this lane is key 16 (v / 8) + 8 half + v % 8.
    // K fragments are read KLA products ahead of their MFMA; the fences keep
    // the scheduler from folding the reads back next to their use, where
    // each product would wait out a full LDS round trip.
    f32x16 sacc[2];
    {
      constexpr int NSL = 2 * KC, KLA = 4;
      auto kfetch = [&](int i) {
        const int krow = 32 * (i / KC) + swap23(l32);
        Frag<SPLIT> f;
        f.h = row_operand<KT>(k_tile(buf, 0), krow, 2 * (i % KC) + half);
        if constexpr (SPLIT) f.l = row_operand<KT>(k_tile(buf, 1), krow, 2 * (i % KC) + half);
        return f;
      };
      Frag<SPLIT> kop[NSL];
#pragma unroll
      for (int i = 0; i < KLA; ++i) kop[i] = kfetch(i);
      // The two waves of a SIMD come from different workgroups and drift in
      // and out of step.  A wave raises its issue priority over its MFMA
      // runs (here and over O += V^T P^T) and drops it for the element-wise
      // softmax, so that the other wave's MFMAs go first while this one does
      // vector work: the matrix core idles less when both want it at once.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + KLA < NSL) kop[i + KLA] = kfetch(i + KLA);
        const int kb = i / KC;
        if (i % KC == 0) {
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
        }
        mma<SPLIT>(sacc[kb], kop[i], qf[i % KC]);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }

    // Mask only on tiles that reach past the range or cross the diagonal of
    // this wave's rows (wave-uniform test): key inside the range, and key <=
    // query in the causal range.
    const bool need_mask = (kt + kFwdKeys > k1) || (causal && kt + kFwdKeys - 1 > wave_q0);
    if (need_mask) {
      const int klim = (causal ? (k1 < qrow + 1 ? k1 : qrow + 1) : k1) - kt;  // local keys < klim
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kl = 32 * kb + 16 * (v >> 3) + 8 * half + (v & 7);
          sacc[kb][v] = kl < klim ? sacc[kb][v] : -INFINITY;
        }
    }
    // Online softmax in base 2 against a running reference m: p = 2^(c s - m),
    // with O and l always sharing the same m, so the result is exact
    // whichever m is used.  The common step does not look at the block's
    // maximum at all: it forms p with the current m and keeps it unless some
    // lane's partial sum of this block reaches 2^64 (or is not a number: the
    // first block, where m = -inf).  Only then is the row max taken (on raw
    // scores, the scale being positive; four chains, the lane halves joined
    // by a lane swap), m moved to it if it grew by more than 8, O and l
    // rescaled, and p formed again.  p < 2^64 keeps P, O and l far inside the
    // fp32 and bf16 range.
    float pr[2][16], blk[4];
    auto soft = [&](float neg_m) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          pr[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], a.scale_log2, neg_m));
          // the four chains start from their first term, not from 0 + term
          if (kb == 0 && v < 4) blk[v] = pr[kb][v];
          else blk[v & 3] += pr[kb][v];
        }
    };
    soft(-m);
    constexpr float kBig = 18446744073709551616.f;  // 2^64
    const bool ok = (blk[0] < kBig) && (blk[1] < kBig) && (blk[2] < kBig) && (blk[3] < kBig);
    if (__any(!ok)) {
      float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx4[v & 3] = fmaxf(mx4[v & 3], sacc[kb][v]);
      float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
      mx = max_across_halves(mx) * a.scale_log2;
      if (__any(mx > m + 8.f)) {
        const float m_new = fmaxf(m, mx);
        // a row that has seen no key yet (in a key part of a split tile,
        // keys may all lie past some rows) keeps m = -inf and zero sums
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[i] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
      }
      soft(m == -INFINITY ? 0.f : -m);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum[i] += blk[i];

    // O^T += V^T P^T over four 16-key chunks
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float pv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) pv[s] = pr[c >> 1][8 * (c & 1) + s];
      const Frag<SPLIT> pf = pack8<SPLIT>(pv);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        Frag<SPLIT> vf;
        vf.h = tr_operand<KT>(v_tile(buf, 0), 16 * c, 32 * db, lane);
        if constexpr (SPLIT) vf.l = tr_operand<KT>(v_tile(buf, 1), 16 * c, 32 * db, lane);
        mma<SPLIT>(oacc[db], vf, pf);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    }  // !skip

    if (!has_next) break;
    if (NBUF == 1) {
      __syncthreads();  // everyone is done with the single K / V buffer
      issue(nkt, 0);
    }
    commit(NBUF == 2 ? buf ^ 1 : 0);
    ri = nri;
    rg = nrg;
    kt = nkt;
    ++step;
  }

  // finalize: O = O^T / l, LSE = ln 2 * (m + log2 l)
  const float lpart = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  const float ltot = lpart + __shfl_xor(lpart, 32);
  const int part = load_plan1(a.part, tile);
  if (part >= 0) {
    // a key part of a split tile: unnormalised O, the running reference and
    // the row sum, merged by tree_attn_fwd_combine_kernel
    if (qrow < q1) {
      const int64_t row = (static_cast<int64_t>(part) * a.hq + h) * kFwdRows + (qrow - q0);
      float* op = a.o_part + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4(op + 32 * db + 8 * j + 4 * half, oacc[db][4 * j], oacc[db][4 * j + 1],
                 oacc[db][4 * j + 2], oacc[db][4 * j + 3]);
      if (half == 0) {
        a.ml_part[2 * row] = m;
        a.ml_part[2 * row + 1] = ltot;
      }
    }
    return;
  }
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

// Every kernel variant is instantiated explicitly so that the host pass
// always emits its launch stub.
template __global__ void tree_attn_fwd_kernel<__bf16, 128>(FwdArgs);
template __global__ void tree_attn_fwd_kernel<__bf16, 64>(FwdArgs);
template __global__ void tree_attn_fwd_kernel<float, 128>(FwdArgs);
template __global__ void tree_attn_fwd_kernel<float, 64>(FwdArgs);

template <typename T, int D>
static hipError_t fwd_t(const FwdArgs& a, int64_t n_blocks, hipStream_t s) {
  constexpr int bytes = FwdCfg<T, D>::BYTES;
  auto kern = tree_attn_fwd_kernel<T, D>;
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(n_blocks)), dim3(256), bytes, s, a);
  return hipGetLastError();
}

// Merges the key parts of a split query tile: with m_c the reference and
// l_c the row sum of part c and M = max_c m_c, O = sum_c 2^(m_c - M) O_c / L
// and LSE = ln 2 (M + log2 L), L = sum_c 2^(m_c - M) l_c -- the online
// softmax's own rescaling, across parts.  A part without keys for a row
// (m_c = -inf) weighs 0.  One workgroup per (split tile, query head); D / 8
// threads per row, 8 columns each.
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_fwd_combine_kernel(FwdArgs a) {
  const I4 c = load_plan4(a.combine, blockIdx.x);
  const int q0 = c.x, q1 = c.y, s0 = c.z, ns = c.w;
  const int h = blockIdx.y;
  constexpr int TPR = D / 8, RPP = 256 / TPR;
  const int col = (threadIdx.x % TPR) * 8;
  for (int r = q0 + static_cast<int>(threadIdx.x) / TPR; r < q1; r += RPP) {
    auto slot_row = [&](int s) {
      return (static_cast<int64_t>(s0 + s) * a.hq + h) * kFwdRows + (r - q0);
    };
    float mref = -INFINITY;
    for (int s = 0; s < ns; ++s) mref = fmaxf(mref, a.ml_part[2 * slot_row(s)]);
    float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const int64_t row = slot_row(s);
      const float w = __builtin_amdgcn_exp2f(a.ml_part[2 * row] - mref);
      l += w * a.ml_part[2 * row + 1];
      const f32x4* po = reinterpret_cast<const f32x4*>(a.o_part + row * D + col);
      const f32x4 x0 = po[0], x1 = po[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * x0[e];
        acc[e + 4] += w * x1[e];
      }
    }
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.o) + static_cast<int64_t>(r) * a.hq * D +
            static_cast<int64_t>(h) * D + col;
    store4(op, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    store4(op + 4, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (col == 0)
      a.lse[static_cast<int64_t>(h) * a.n_tokens + r] =
          kLn2 * (mref + __builtin_amdgcn_logf(l));
  }
}

template __global__ void tree_attn_fwd_combine_kernel<__bf16, 128>(FwdArgs);
template __global__ void tree_attn_fwd_combine_kernel<__bf16, 64>(FwdArgs);
template __global__ void tree_attn_fwd_combine_kernel<float, 128>(FwdArgs);
template __global__ void tree_attn_fwd_combine_kernel<float, 64>(FwdArgs);

template <typename T, int D>
static hipError_t combine_t(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((tree_attn_fwd_combine_kernel<T, D>),
                     dim3(static_cast<unsigned>(a.n_combine), static_cast<unsigned>(a.hq)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (a.n_combine <= 0) return hipSuccess;
  if (dtype == 0 && head_dim == 128) return combine_t<__bf16, 128>(a, stream);
  if (dtype == 0 && head_dim == 64) return combine_t<__bf16, 64>(a, stream);
  if (dtype == 1 && head_dim == 128) return combine_t<float, 128>(a, stream);
  if (dtype == 1 && head_dim == 64) return combine_t<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t n_blocks,
                      hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  if (dtype == 0 && head_dim == 128) return fwd_t<__bf16, 128>(a, n_blocks, stream);
  if (dtype == 0 && head_dim == 64) return fwd_t<__bf16, 64>(a, n_blocks, stream);
  if (dtype == 1 && head_dim == 128) return fwd_t<float, 128>(a, n_blocks, stream);
  if (dtype == 1 && head_dim == 64) return fwd_t<float, 64>(a, n_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace tree_attn
