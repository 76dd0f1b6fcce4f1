// Backward pass of prefix-shared tree attention (gfx950).
//
// The backward pass of trajectory-wise training recomputes every shared
// prefix once per trajectory (AReaL-DTA, abstract; HARTS, abstract); here a
// shared key is visited once per pass and its dK / dV are summed over every
// descendant branch in registers (Tree Training in the HARTS page's related
// list: reuse shared-prefix work in forward and backward).
//
// Three launches:
//  1. preprocess: D_t = sum_d dO_t O_t per (token, head) and a zeroed fp32
//     dQ accumulator;
//  2. main, one workgroup per key tile (up to 128 keys of one node) and kv
//     head, looping over every query block that sees the tile (the rest of
//     its node with the causal mask, then every descendant node) for each
//     query head of the GQA group.  Wave w owns keys 32w .. 32w+31 and keeps
//     their K and V operands and dK / dV accumulators in registers.  Per
//     32-row query block it recomputes P = exp(S - LSE) from the saved LSE,
//     forms dP = dO V^T and dS = P (dP - D), and accumulates dV += P^T dO and
//     dK += dS^T Q with dO and Q read as transposed operands.  dS goes to LDS
//     so that dQ = dS K sums all 128 keys of the tile before one fp32 atomic
//     add per element.  Key tiles whose descendant work was split for load
//     balance write fp32 partial dK / dV slots instead of the outputs;
//  3. post: a fixed-order sum of partial slots (deterministic dK / dV) and
//     the dQ accumulator converted to the output type.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {

namespace {

// dS tile: [kBwdKeys keys][kBwdRows queries] bf16, rows of 64 bytes, no
// swizzle (transpose reads of 4 rows x 32 bytes are conflict free).
constexpr int kDsRowBytes = kBwdRows * 2;

__device__ __forceinline__ bf16x8 ds_tr_operand(const LDS_PTR(char) base, int row0, int lane) {
  const int grp = lane >> 4, L = lane & 15;
  const int r = row0 + 8 * (grp >> 1) + (L >> 2);
  const int c = 16 * (grp & 1) + 4 * (L & 3);
  const bf16x4 lo = lds_read_tr(base, r * kDsRowBytes + 2 * c);
  const bf16x4 hi = lds_read_tr(base, (r + 4) * kDsRowBytes + 2 * c);
  bf16x8 out;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    out[s] = lo[s];
    out[s + 4] = hi[s];
  }
  return out;
}

template <typename T, int D>
struct BwdSmem {
  static constexpr bool SPLIT = IsSplit<T>::value;
  static constexpr int NP = SPLIT ? 2 : 1;
  static constexpr int K_PLANE = kBwdKeys * D * 2;
  static constexpr int Q_PLANE = kBwdRows * D * 2;
  static constexpr int DS_PLANE = kBwdKeys * kDsRowBytes;
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + NP * K_PLANE;
  static constexpr int DO_OFF = Q_OFF + NP * Q_PLANE;
  static constexpr int DS_OFF = DO_OFF + NP * Q_PLANE;
  static constexpr int LSE_OFF = DS_OFF + NP * DS_PLANE;
  static constexpr int DV_OFF = LSE_OFF + kBwdRows * 4;
  static constexpr int BYTES = DV_OFF + kBwdRows * 4;
};

}  // namespace

// --------------------------------------------------------------------------
// 1. preprocess
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;  // threads per (token, head) row, 8 elements each
  const int64_t rows = a.n_tokens * a.hq;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t off = row * D + 8 * part;
    const T* o = static_cast<const T*>(a.o) + off;
    const T* d = static_cast<const T*>(a.dout) + off;
    float ov[8], dv[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(o);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(d);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        ov[s] = static_cast<float>(x[s]);
        dv[s] = static_cast<float>(y[s]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        ov[s] = o[s];
        dv[s] = d[s];
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc += ov[s] * dv[s];
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.dq_acc + off) = z;
    *reinterpret_cast<f32x4*>(a.dq_acc + off + 4) = z;
  }
#pragma unroll
  for (int w = TPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
  if (row < rows && part == 0) {
    const int64_t t = row / a.hq, h = row % a.hq;
    a.dvec[h * a.n_tokens + t] = acc;
  }
}

// --------------------------------------------------------------------------
// 2. main
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void tree_attn_bwd_kernel(BwdArgs a) {
  using L = BwdSmem<T, D>;
  constexpr bool SPLIT = L::SPLIT;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  constexpr int WPD = 4 / DB;                      // waves per dQ column block
  constexpr int DQ_CHUNKS = kBwdKeys / 16 / WPD;   // 16-key chunks per wave in dQ
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);
  LDS_PTR(char) k_hi = lds + L::K_OFF;
  LDS_PTR(char) k_lo = k_hi + L::K_PLANE;
  LDS_PTR(char) q_hi = lds + L::Q_OFF;
  LDS_PTR(char) q_lo = q_hi + L::Q_PLANE;
  LDS_PTR(char) do_hi = lds + L::DO_OFF;
  LDS_PTR(char) do_lo = do_hi + L::Q_PLANE;
  LDS_PTR(char) ds_hi = lds + L::DS_OFF;
  LDS_PTR(char) ds_lo = ds_hi + L::DS_PLANE;
  LDS_PTR(float) lse_s = (LDS_PTR(float))(lds + L::LSE_OFF);
  LDS_PTR(float) dvec_s = (LDS_PTR(float))(lds + L::DV_OFF);

  const I8 it = a.items[blockIdx.x];
  const int k0 = it.v[0], k1 = it.v[1], g = it.v[2], eb = it.v[3], ee = it.v[4];
  const int slot = it.v[5];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t last = a.n_tokens - 1;
  const int64_t qs = static_cast<int64_t>(a.hq) * D;
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  const T* Kg = static_cast<const T*>(a.k) + static_cast<int64_t>(g) * D;
  const T* Vg = static_cast<const T*>(a.v) + static_cast<int64_t>(g) * D;
  const int key = k0 + 32 * wave + l32;  // this lane's key (column of S)
  const int kmax = (k1 < k0 + kBwdKeys ? k1 : k0 + kBwdKeys) - 1;

  // K tile for dQ (transposed reads) and this wave's K / V operands
  load_tile<T, D, kBwdKeys, 256>(k_hi, k_lo, Kg, ks, k0, last, tid);
  Frag<SPLIT> kf[KC], vf[KC];
  {
    const int64_t r = key < last ? key : last;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = load_frag8(Kg + r * ks + 16 * kc + 8 * half);
      vf[kc] = load_frag8(Vg + r * ks + 16 * kc + 8 * half);
    }
  }
  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dk_acc[db][v] = 0.f;
      dv_acc[db][v] = 0.f;
    }
  const int dq_db = wave / WPD;                 // dQ column block of this wave
  const int dq_kc0 = (wave % WPD) * DQ_CHUNKS;  // first 16-key chunk of this wave
  const int qrow_a = swap23(l32);               // A-operand row of S / dP

  for (int e = eb; e < ee; ++e) {
    const I4 en = a.entries[e];
    const int h = en.x, qa = en.y, qe = en.z;
    const bool causal = en.w != 0;
    const T* Qh = static_cast<const T*>(a.q) + static_cast<int64_t>(h) * D;
    const T* dOh = static_cast<const T*>(a.dout) + static_cast<int64_t>(h) * D;
    const float* lse_h = a.lse + static_cast<int64_t>(h) * a.n_tokens;
    const float* dvec_h = a.dvec + static_cast<int64_t>(h) * a.n_tokens;
    float* dq_h = a.dq_acc + static_cast<int64_t>(h) * D;
    for (int qb = qa; qb < qe; qb += kBwdRows) {
      __syncthreads();  // previous block's LDS readers are done
      load_tile<T, D, kBwdRows, 256>(q_hi, q_lo, Qh, qs, qb, last, tid);
      load_tile<T, D, kBwdRows, 256>(do_hi, do_lo, dOh, qs, qb, last, tid);
      if (tid < kBwdRows) {
        const int64_t r = qb + tid < last ? qb + tid : last;
        lse_s[tid] = lse_h[r] * kLog2e;
        dvec_s[tid] = dvec_h[r];
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for this wave's 32 keys.  Register v of
      // this lane is query row 16 (v / 8) + 8 half + v % 8 of the block.
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[v] = 0.f;
        pacc[v] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        Frag<SPLIT> qa_f, da_f;
        qa_f.h = row_operand<D>(q_hi, qrow_a, 2 * kc + half);
        da_f.h = row_operand<D>(do_hi, qrow_a, 2 * kc + half);
        if constexpr (SPLIT) {
          qa_f.l = row_operand<D>(q_lo, qrow_a, 2 * kc + half);
          da_f.l = row_operand<D>(do_lo, qrow_a, 2 * kc + half);
        }
        mma<SPLIT>(sacc, qa_f, kf[kc]);
        mma<SPLIT>(pacc, da_f, vf[kc]);
      }
      const bool need_mask = (qb + kBwdRows > qe) || (kmax >= k1) || (k1 - k0 < kBwdKeys) ||
                             (causal && kmax > qb);
      float p[16], ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ql = 16 * (v >> 3) + 8 * half + (v & 7);
        float pv = __builtin_amdgcn_exp2f(sacc[v] * a.scale_log2 - lse_s[ql]);
        if (need_mask) {
          const int q = qb + ql;
          const bool ok = q < qe && key < k1 && (!causal || key <= q);
          pv = ok ? pv : 0.f;
        }
        p[v] = pv;
        ds[v] = pv * (pacc[v] - dvec_s[ql]);
      }
      const Frag<SPLIT> pf0 = pack8<SPLIT>(p), pf1 = pack8<SPLIT>(p + 8);
      const Frag<SPLIT> sf0 = pack8<SPLIT>(ds), sf1 = pack8<SPLIT>(ds + 8);

      // dV += P^T dO, dK += dS^T Q (operands dO, Q transposed from LDS)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
          Frag<SPLIT> bo, bq;
          bo.h = tr_operand<D>(do_hi, 16 * qc, 32 * db, lane);
          bq.h = tr_operand<D>(q_hi, 16 * qc, 32 * db, lane);
          if constexpr (SPLIT) {
            bo.l = tr_operand<D>(do_lo, 16 * qc, 32 * db, lane);
            bq.l = tr_operand<D>(q_lo, 16 * qc, 32 * db, lane);
          }
          mma<SPLIT>(dv_acc[db], qc ? pf1 : pf0, bo);
          mma<SPLIT>(dk_acc[db], qc ? sf1 : sf0, bq);
        }
      }

      // dS -> LDS as [key][query]
      {
        const int r = 32 * wave + l32;
        *reinterpret_cast<LDS_PTR(bf16x8)>(ds_hi + r * kDsRowBytes + 16 * half) = sf0.h;
        *reinterpret_cast<LDS_PTR(bf16x8)>(ds_hi + r * kDsRowBytes + 32 + 16 * half) = sf1.h;
        if constexpr (SPLIT) {
          *reinterpret_cast<LDS_PTR(bf16x8)>(ds_lo + r * kDsRowBytes + 16 * half) = sf0.l;
          *reinterpret_cast<LDS_PTR(bf16x8)>(ds_lo + r * kDsRowBytes + 32 + 16 * half) = sf1.l;
        }
      }
      __syncthreads();

      // dQ[q][d] += scale * sum_key dS[q][key] K[key][d] for this wave's
      // column block and key chunks; lane holds column d, rows in registers
      f32x16 qacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) qacc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < DQ_CHUNKS; ++c) {
        const int kc = dq_kc0 + c;
        Frag<SPLIT> af, bf;
        af.h = ds_tr_operand(ds_hi, 16 * kc, lane);
        bf.h = tr_operand<D>(k_hi, 16 * kc, 32 * dq_db, lane);
        if constexpr (SPLIT) {
          af.l = ds_tr_operand(ds_lo, 16 * kc, lane);
          bf.l = tr_operand<D>(k_lo, 16 * kc, 32 * dq_db, lane);
        }
        mma<SPLIT>(qacc, af, bf);
      }
      const int d = 32 * dq_db + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int q = qb + 8 * (v >> 2) + 4 * half + (v & 3);
        if (q < qe) atomicAdd(dq_h + static_cast<int64_t>(q) * qs + d, a.scale * qacc[v]);
      }
    }
  }

  // dK, dV of this wave's keys: lane holds column d, key rows in registers
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int d = 32 * db + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kl = 32 * wave + 8 * (v >> 2) + 4 * half + (v & 3);
      const int kr = k0 + kl;
      if (kr >= k1) continue;
      const float dkv = a.scale * dk_acc[db][v];
      const float dvv = dv_acc[db][v];
      if (slot < 0) {
        T* dk = static_cast<T*>(a.dk) + static_cast<int64_t>(kr) * ks + static_cast<int64_t>(g) * D;
        T* dv = static_cast<T*>(a.dv) + static_cast<int64_t>(kr) * ks + static_cast<int64_t>(g) * D;
        dk[d] = static_cast<T>(dkv);
        dv[d] = static_cast<T>(dvv);
      } else {
        const int64_t so = (static_cast<int64_t>(slot) * kBwdKeys + kl) * D + d;
        a.dk_slots[so] = dkv;
        a.dv_slots[so] = dvv;
      }
    }
  }
}

// --------------------------------------------------------------------------
// 3. post: partial-slot reduction and dQ conversion
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_bwd_reduce_kernel(BwdArgs a) {
  const I8 r = a.reduce[blockIdx.x];
  const int k0 = r.v[0], k1 = r.v[1], g = r.v[2], sb = r.v[3], ns = r.v[4];
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  const int n = (k1 - k0) * D;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int kl = i / D, d = i % D;
    float sk = 0.f, sv = 0.f;
    for (int s = 0; s < ns; ++s) {  // fixed order: deterministic sums
      const int64_t so = (static_cast<int64_t>(sb + s) * kBwdKeys + kl) * D + d;
      sk += a.dk_slots[so];
      sv += a.dv_slots[so];
    }
    const int64_t o = static_cast<int64_t>(k0 + kl) * ks + static_cast<int64_t>(g) * D + d;
    static_cast<T*>(a.dk)[o] = static_cast<T>(sk);
    static_cast<T*>(a.dv)[o] = static_cast<T>(sv);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void tree_attn_dq_convert_kernel(const float* acc, T* out,
                                                                   int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(acc + i);
    store4(out + i, x[0], x[1], x[2], x[3]);
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = static_cast<T>(acc[j]);
  }
}

// --------------------------------------------------------------------------
// launchers

template <typename T, int D>
static hipError_t pre_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.n_tokens * a.hq;
  const int64_t per = 256 / (D / 8);
  const int64_t blocks = (rows + per - 1) / per;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((tree_attn_bwd_pre_kernel<T, D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t main_t(const BwdArgs& a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  constexpr int bytes = BwdSmem<T, D>::BYTES;
  auto kern = tree_attn_bwd_kernel<T, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_items)), dim3(256), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t post_t(const BwdArgs& a, hipStream_t s) {
  if (a.n_reduce > 0) {
    hipLaunchKernelGGL((tree_attn_bwd_reduce_kernel<T, D>),
                       dim3(static_cast<unsigned>(a.n_reduce)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = a.n_tokens * a.hq * D;
  const int64_t blocks = (n + 1023) / 1024;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((tree_attn_dq_convert_kernel<T>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, a.dq_acc, static_cast<T*>(a.dq), n);
  return hipGetLastError();
}

#define TREE_ATTN_DISPATCH(FN)                                       \
  if (dtype == 0 && head_dim == 128) return FN<__bf16, 128>(a, s);   \
  if (dtype == 0 && head_dim == 64) return FN<__bf16, 64>(a, s);     \
  if (dtype == 1 && head_dim == 128) return FN<float, 128>(a, s);    \
  if (dtype == 1 && head_dim == 64) return FN<float, 64>(a, s);      \
  return hipErrorInvalidValue;

hipError_t launch_bwd_pre(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(pre_t)
}
hipError_t launch_bwd_main(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(main_t)
}
hipError_t launch_bwd_post(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(post_t)
}

}  // namespace tree_attn
