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

// Shared-memory layout of the main kernel.  QB query rows per step (two
// 32-row sub-blocks for bf16; one for fp32 inputs, whose hi/lo planes double
// every tile).  Q / dO / (LSE, D) have NBUF buffers: with two, the next
// step's rows stream in while the current step computes.  dS always has two
// buffers: step i writes dS(i) and step i + 1 forms dQ(i) from it.
template <typename T, int D>
struct BwdCfg {
  static constexpr bool SPLIT = IsSplit<T>::value;
  static constexpr int NP = SPLIT ? 2 : 1;
  static constexpr int QB = SPLIT ? 32 : 64;
  static constexpr int NSUB = QB / 32;
  static constexpr int NBUF = (SPLIT && D == 128) ? 1 : 2;
  static constexpr int KC = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int K_PLANE = kBwdKeys * D * 2;
  static constexpr int Q_PLANE = QB * D * 2;
  static constexpr int DS_PLANE = kBwdKeys * QB * 2;
  static constexpr int LD_BYTES = QB * 8;  // LSE * log2(e), then D
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + NP * K_PLANE;
  static constexpr int DO_OFF = Q_OFF + NBUF * NP * Q_PLANE;
  static constexpr int DS_OFF = DO_OFF + NBUF * NP * Q_PLANE;
  static constexpr int LD_OFF = DS_OFF + 2 * NP * DS_PLANE;
  static constexpr int BYTES = LD_OFF + NBUF * LD_BYTES;
};

// One step of work: rows [qb, min(qb + QB, qe)) of query head h.
struct Blk {
  int h, qb, qe, causal, e;
};

__device__ __forceinline__ bool load_entry(Blk& b, int e, int ee, const I4* entries) {
  if (e >= ee) return false;
  const I4 en = entries[e];
  b.h = en.x;
  b.qb = en.y;
  b.qe = en.z;
  b.causal = en.w;
  b.e = e;
  return true;
}

template <int QB>
__device__ __forceinline__ bool advance(Blk& b, int ee, const I4* entries) {
  b.qb += QB;
  if (b.qb < b.qe) return true;
  return load_entry(b, b.e + 1, ee, entries);
}

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
  using C = BwdCfg<T, D>;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int QB = C::QB, NSUB = C::NSUB, NBUF = C::NBUF, KC = C::KC, DB = C::DB;
  constexpr int WPD = 4 / DB;                     // waves per dQ column block
  constexpr int DQ_CHUNKS = kBwdKeys / 16 / WPD;  // 16-key chunks per wave in dQ
  using KT = Tile<D, kBwdKeys>;   // K tile (dQ operand)
  using QT = Tile<D, QB>;         // Q / dO tiles of a step
  using ST = Tile<QB, kBwdKeys>;  // dS tile [key][query]
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);
  LDS_PTR(char) k_hi = lds + C::K_OFF;
  LDS_PTR(char) k_lo = k_hi + C::K_PLANE;

  const I8 it = a.items[blockIdx.x];
  const int k0 = it.v[0], k1 = it.v[1], g = it.v[2], eb = it.v[3], ee = it.v[4];
  const int slot = it.v[5];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t last = a.n_tokens - 1;
  const int64_t qs = static_cast<int64_t>(a.hq) * D;
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  const T* Kg = static_cast<const T*>(a.k) + static_cast<int64_t>(g) * D;
  const T* Vg = static_cast<const T*>(a.v) + static_cast<int64_t>(g) * D;
  const T* Qall = static_cast<const T*>(a.q);
  const T* dOall = static_cast<const T*>(a.dout);
  const int key = k0 + 32 * wave + l32;  // this lane's key (column of S)

  auto q_tile = [&](int buf, int plane) {
    return lds + C::Q_OFF + (buf * C::NP + plane) * C::Q_PLANE;
  };
  auto do_tile = [&](int buf, int plane) {
    return lds + C::DO_OFF + (buf * C::NP + plane) * C::Q_PLANE;
  };
  auto ds_tile = [&](int buf, int plane) {
    return lds + C::DS_OFF + (buf * C::NP + plane) * C::DS_PLANE;
  };
  auto ld_tile = [&](int buf) { return (LDS_PTR(float))(lds + C::LD_OFF + buf * C::LD_BYTES); };

  // Prefetch state for the next step: Q / dO rows (buffer loads straight to
  // LDS for bf16, through registers for fp32) and one LSE or D value per
  // thread.
  constexpr int SPLIT_PER = SPLIT ? QB * D / 4 / 256 : 1;
  i32x4 qreg[SPLIT_PER], dreg[SPLIT_PER];
  float ld_reg = 0.f;
  TileLoader<D, QB, 4> tl;
  if constexpr (!SPLIT) tl.init(static_cast<int>(qs * sizeof(T)), wave, lane);
  const T* Qend = Qall + a.n_tokens * qs;
  const T* dOend = dOall + a.n_tokens * qs;
  auto issue = [&](const Blk& b, int buf) {
    const int64_t r0 = b.qb;
    const T* Qh = Qall + static_cast<int64_t>(b.h) * D;
    const T* dOh = dOall + static_cast<int64_t>(b.h) * D;
    if constexpr (!SPLIT) {
      tl.issue(q_tile(buf, 0), make_rsrc(Qh + r0 * qs, Qend));
      tl.issue(do_tile(buf, 0), make_rsrc(dOh + r0 * qs, dOend));
    } else {
      constexpr int CPR = D / 4;
#pragma unroll
      for (int i = 0; i < SPLIT_PER; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
        const int64_t row = r0 + r < last ? r0 + r : last;
        qreg[i] = gload16(Qh + row * qs + cc * 4);
        dreg[i] = gload16(dOh + row * qs + cc * 4);
      }
    }
    if (tid < 2 * QB) {
      const int r = tid % QB;
      const int64_t row = r0 + r < last ? r0 + r : last;
      const float* src = tid < QB ? a.lse : a.dvec;
      ld_reg = src[static_cast<int64_t>(b.h) * a.n_tokens + row];
    }
  };
  auto commit = [&](int buf) {
    if constexpr (SPLIT) {
      constexpr int CPR = D / 4;
#pragma unroll
      for (int i = 0; i < SPLIT_PER; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 f = __builtin_bit_cast(f32x4, t ? dreg[i] : qreg[i]);
          bf16x4 h, l;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            h[s2] = to_bf16(f[s2]);
            l[s2] = to_bf16(f[s2] - static_cast<float>(h[s2]));
          }
          LDS_PTR(char) hi = t ? do_tile(buf, 0) : q_tile(buf, 0);
          LDS_PTR(char) lo = t ? do_tile(buf, 1) : q_tile(buf, 1);
          *reinterpret_cast<LDS_PTR(bf16x4)>(hi + QT::elem_off(r, cc * 4)) = h;
          *reinterpret_cast<LDS_PTR(bf16x4)>(lo + QT::elem_off(r, cc * 4)) = l;
        }
      }
    }
    if (tid < 2 * QB) ld_tile(buf)[tid] = tid < QB ? ld_reg * kLog2e : ld_reg;
  };

  // K tile (for dQ) and this wave's K / V operands
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

  // dQ[q][d] += scale * sum_key dS[q][key] K[key][d] for a finished step,
  // from its dS buffer; lane holds column d, query rows in registers.  The
  // fp32 adds go through a buffer resource based at the step's first row:
  // rows past the last token fall outside its range and are dropped, rows
  // past the step's range add exact zeros (their dS is zero).
  const int dq_voff = (4 * half * static_cast<int>(qs) + 32 * dq_db + l32) * 4;
  const float* dq_end = a.dq_acc + a.n_tokens * qs;
  auto dq_step = [&](const Blk& b, int dbuf) {
    const rsrc_t rs = make_rsrc(a.dq_acc + static_cast<int64_t>(b.qb) * qs +
                                    static_cast<int64_t>(b.h) * D, dq_end);
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      f32x16 qacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) qacc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < DQ_CHUNKS; ++c) {
        const int kc = dq_kc0 + c;
        Frag<SPLIT> af, bf;
        af.h = tr_operand<ST>(ds_tile(dbuf, 0), 16 * kc, 32 * sb, lane);
        bf.h = tr_operand<KT>(k_hi, 16 * kc, 32 * dq_db, lane);
        if constexpr (SPLIT) {
          af.l = tr_operand<ST>(ds_tile(dbuf, 1), 16 * kc, 32 * sb, lane);
          bf.l = tr_operand<KT>(k_lo, 16 * kc, 32 * dq_db, lane);
        }
        mma<SPLIT>(qacc, af, bf);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * sb + 8 * (v >> 2) + (v & 3);  // plus 4 half (in dq_voff)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
            a.scale * qacc[v], rs, dq_voff, row * static_cast<int>(qs) * 4, 0);
      }
    }
  };

  Blk cur;
  load_entry(cur, eb, ee, a.entries);
  Blk prev = cur;
  bool has_prev = false;
  issue(cur, 0);
  commit(0);
  int step = 0;
  while (true) {
    Blk nxt = cur;
    const bool has_next = advance<QB>(nxt, ee, a.entries);
    const int buf = NBUF == 2 ? (step & 1) : 0;
    wait_vm();
    __syncthreads();  // step's rows are in LDS; dS of the previous step is complete
    if (NBUF == 2 && has_next) issue(nxt, buf ^ 1);
    if (has_prev) dq_step(prev, (step - 1) & 1);

    LDS_PTR(float) ldv = ld_tile(buf);
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const int qs0 = cur.qb + 32 * sb;           // first row of the sub-block
      const int wk0 = k0 + 32 * wave;             // first key of this wave
      // wave-uniform: no row of the sub-block sees any key of this wave
      const bool skip = qs0 >= cur.qe || wk0 >= k1 || (cur.causal && wk0 > qs0 + 31);
      const int r_ds = 32 * wave + l32;           // this lane's row of the dS tile
      if (skip) {
        const bf16x8 z = {};
#pragma unroll
        for (int pl = 0; pl < C::NP; ++pl) {
          LDS_PTR(char) t = ds_tile(step & 1, pl);
          *reinterpret_cast<LDS_PTR(bf16x8)>(t + ST::chunk_off(r_ds, 4 * sb + half)) = z;
          *reinterpret_cast<LDS_PTR(bf16x8)>(t + ST::chunk_off(r_ds, 4 * sb + 2 + half)) = z;
        }
        continue;
      }
      // S = Q K^T and dP = dO V^T for this wave's 32 keys and 32 query rows;
      // register v of this lane is query row 32 sb + 16 (v / 8) + 8 half + v % 8.
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[v] = 0.f;
        pacc[v] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        Frag<SPLIT> qa_f, da_f;
        qa_f.h = row_operand<QT>(q_tile(buf, 0), 32 * sb + qrow_a, 2 * kc + half);
        da_f.h = row_operand<QT>(do_tile(buf, 0), 32 * sb + qrow_a, 2 * kc + half);
        if constexpr (SPLIT) {
          qa_f.l = row_operand<QT>(q_tile(buf, 1), 32 * sb + qrow_a, 2 * kc + half);
          da_f.l = row_operand<QT>(do_tile(buf, 1), 32 * sb + qrow_a, 2 * kc + half);
        }
        mma<SPLIT>(sacc, qa_f, kf[kc]);
        mma<SPLIT>(pacc, da_f, vf[kc]);
      }
      // P = 2^(c s - LSE log2 e) recomputed from the saved LSE; masked where
      // a row is past the range, a key past the tile, or (causal) key > row.
      const bool need_mask = qs0 + 32 > cur.qe || wk0 + 32 > k1 || (cur.causal && wk0 + 31 > qs0);
      float p[16], ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ql = 32 * sb + 16 * (v >> 3) + 8 * half + (v & 7);
        p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], a.scale_log2, -ldv[ql]));
      }
      if (need_mask) {
        const int qlim = cur.qe - cur.qb;                       // local rows < qlim
        const int kq = cur.causal ? key - cur.qb : -(1 << 30);  // local rows >= kq
        const bool kok = key < k1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ql = 32 * sb + 16 * (v >> 3) + 8 * half + (v & 7);
          p[v] = (kok && ql < qlim && ql >= kq) ? p[v] : 0.f;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ql = 32 * sb + 16 * (v >> 3) + 8 * half + (v & 7);
        ds[v] = p[v] * (pacc[v] - ldv[QB + ql]);
      }
      const Frag<SPLIT> pf0 = pack8<SPLIT>(p), pf1 = pack8<SPLIT>(p + 8);
      const Frag<SPLIT> sf0 = pack8<SPLIT>(ds), sf1 = pack8<SPLIT>(ds + 8);

      // dV += P^T dO, dK += dS^T Q (dO, Q read transposed from LDS)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
          Frag<SPLIT> bo, bq;
          bo.h = tr_operand<QT>(do_tile(buf, 0), 32 * sb + 16 * qc, 32 * db, lane);
          bq.h = tr_operand<QT>(q_tile(buf, 0), 32 * sb + 16 * qc, 32 * db, lane);
          if constexpr (SPLIT) {
            bo.l = tr_operand<QT>(do_tile(buf, 1), 32 * sb + 16 * qc, 32 * db, lane);
            bq.l = tr_operand<QT>(q_tile(buf, 1), 32 * sb + 16 * qc, 32 * db, lane);
          }
          mma<SPLIT>(dv_acc[db], qc ? pf1 : pf0, bo);
          mma<SPLIT>(dk_acc[db], qc ? sf1 : sf0, bq);
        }
      }

      // dS -> LDS as [key][query] for the next step's dQ
#pragma unroll
      for (int pl = 0; pl < C::NP; ++pl) {
        LDS_PTR(char) t = ds_tile(step & 1, pl);
        bf16x8 x0, x1;
        if constexpr (SPLIT) {
          x0 = pl ? sf0.l : sf0.h;
          x1 = pl ? sf1.l : sf1.h;
        } else {
          x0 = sf0.h;
          x1 = sf1.h;
        }
        *reinterpret_cast<LDS_PTR(bf16x8)>(t + ST::chunk_off(r_ds, 4 * sb + half)) = x0;
        *reinterpret_cast<LDS_PTR(bf16x8)>(t + ST::chunk_off(r_ds, 4 * sb + 2 + half)) = x1;
      }
    }

    if (!has_next) break;
    if (NBUF == 1) {
      __syncthreads();  // everyone is done with the single Q / dO buffer
      issue(nxt, 0);
    }
    commit(NBUF == 2 ? buf ^ 1 : 0);
    prev = cur;
    has_prev = true;
    cur = nxt;
    ++step;
  }
  __syncthreads();  // dS of the last step is complete
  dq_step(cur, step & 1);

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
  constexpr int bytes = BwdCfg<T, D>::BYTES;
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
