// Backward pass of prefix-shared tree attention (gfx950).
//
// The backward pass of trajectory-wise training recomputes every shared
// prefix once per trajectory (AReaL-DTA, abstract; HARTS, abstract); here a
// shared key is visited once per pass and its dK / dV are summed over every
// descendant branch in registers (Tree Training in the HARTS page's related
// list: reuse shared-prefix work in forward and backward).
//
// Four launches (five with split query tiles), no atomics anywhere:
//  1. preprocess: D_t = sum_d dO_t O_t per (token, head);
//  2. dK / dV, one workgroup per key tile (up to 128 keys of one node) and kv
//     head.  It walks every query step that sees the tile -- the rest of its
//     node under the causal mask, then every descendant node -- for each
//     query head of the GQA group.  Wave w owns keys 32w .. 32w+31 and keeps
//     their K and V operands and their dK / dV accumulators in registers;
//     per 32-row sub-block it recomputes P = exp(S - LSE) from the saved LSE,
//     forms dP = dO V^T and dS = P (dP - D), and accumulates dV += P^T dO and
//     dK += dS^T Q with dO and Q read as transposed operands.  Query rows of
//     the following steps stream into LDS buffers meanwhile.  Key tiles
//     whose descendant work was split for load balance write fp32 partial
//     slots instead of the outputs;
//  3. dQ, one workgroup per query tile and head, walking the tile's ancestor
//     key ranges like the forward pass: S^T = K Q^T and dP^T = V dO^T, then
//     dS^T = P^T (dP^T - D) and dQ^T += K^T dS^T in registers, written once.
//     Recomputing S and dP here costs MFMA work but replaces a per-key-tile
//     fp32 atomic reduction of dQ whose memory traffic would dominate the pass.
//     The key parts of a split query tile write fp32 partial dQ instead;
//  4. a fixed-order sum of the partial slots (deterministic dK / dV), and of
//     the key parts' partial dQ where the plan split query tiles.
#include "device_common.h"
#include "kernels.h"

namespace tree_attn {

namespace {

// Shared memory of the dK / dV kernel: QB query rows per step (two 32-row
// sub-blocks for bf16; one for fp32 inputs, whose two 16-bit planes double every
// tile), Q / dO / (LSE, D) double-buffered.
template <typename T, int D>
struct DkdvCfg {
  static constexpr bool SPLIT = IsSplit<T>::value;
  static constexpr int NP = SPLIT ? 2 : 1;
  static constexpr int QB = SPLIT ? 32 : 64;
  static constexpr int NSUB = QB / 32;
  static constexpr int KC = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int Q_PLANE = QB * D * 2;
  static constexpr int LD_BYTES = QB * 8;  // -LSE * log2(e), then -D
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = Q_OFF + 2 * NP * Q_PLANE;
  static constexpr int LD_OFF = DO_OFF + 2 * NP * Q_PLANE;
  static constexpr int BYTES = LD_OFF + 2 * LD_BYTES;
};

// One step of work: rows [qb, min(qb + QB, qe)) of query head h.
struct Blk {
  int h, qb, qe, causal, e;
};

__device__ __forceinline__ bool load_entry(Blk& b, int e, int ee, const I4* entries) {
  if (e >= ee) return false;
  const I4 en = load_plan4(entries, e);
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
// 1. preprocess: D_t = dO_t . O_t, over every row or (query-subset plans)
// over the rows of the query tiles: grid (tiles, blocks per tile)
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;  // threads per (token, head) row, 8 elements each
  int64_t rows = a.n_tokens * a.hq;  // end of this block's (token, head) row range
  int64_t row;
  if (a.pre_tiles) {
    const I4 t = load_plan4(a.pre_tiles, blockIdx.x);
    row = static_cast<int64_t>(t.x) * a.hq +
          static_cast<int64_t>(blockIdx.y) * (256 / TPR) + threadIdx.x / TPR;
    rows = static_cast<int64_t>(t.y) * a.hq;
  } else {
    row = static_cast<int64_t>(blockIdx.x) * (256 / TPR) + threadIdx.x / TPR;
  }
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t off = row * D + 8 * part;
    const T* o = static_cast<const T*>(a.o) + off;
    const T* d = static_cast<const T*>(a.dout) + off;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(o);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(d);
#pragma unroll
      for (int s = 0; s < 8; ++s) acc += static_cast<float>(x[s]) * static_cast<float>(y[s]);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) acc += o[s] * d[s];
    }
  }
#pragma unroll
  for (int w = TPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
  if (row < rows && part == 0) {
    const int64_t t = row / a.hq, h = row % a.hq;
    const int64_t o = h * a.n_tokens + t;
    a.neg_d[o] = -acc;
    a.neg_lse2[o] = -a.lse[o] * kLog2e;
  }
}

// --------------------------------------------------------------------------
// 2. dK / dV
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void tree_attn_dkdv_kernel(BwdArgs a) {
  using C = DkdvCfg<T, D>;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int QB = C::QB, NSUB = C::NSUB, KC = C::KC, DB = C::DB;
  using QT = Tile<D, QB>;  // Q / dO tiles of a step
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);

  const I8 it = load_plan8(a.items, blockIdx.x);
  const int k0 = it.v[0], k1 = it.v[1], g = it.v[2], eb = it.v[3], ee = it.v[4];
  const int slot = it.v[5];
  if (eb >= ee) return;  // an empty item that pads the launch order
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
  const int wk0 = k0 + 32 * wave;        // first key of this wave

  auto q_tile = [&](int buf, int plane) {
    return lds + C::Q_OFF + (buf * C::NP + plane) * C::Q_PLANE;
  };
  auto do_tile = [&](int buf, int plane) {
    return lds + C::DO_OFF + (buf * C::NP + plane) * C::Q_PLANE;
  };
  auto ld_tile = [&](int buf) { return (LDS_PTR(float))(lds + C::LD_OFF + buf * C::LD_BYTES); };

  // Prefetch of the next step: Q / dO rows (buffer loads straight to LDS for
  // bf16, through registers for fp32) and one LSE or D value per thread.
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
      const float* src = tid < QB ? a.neg_lse2 : a.neg_d;
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
            __bf16 hs, ls;
            split_bits(f[s2], hs, ls);
            h[s2] = hs;
            l[s2] = ls;
          }
          LDS_PTR(char) hi = t ? do_tile(buf, 0) : q_tile(buf, 0);
          LDS_PTR(char) lo = t ? do_tile(buf, 1) : q_tile(buf, 1);
          *reinterpret_cast<LDS_PTR(bf16x4)>(hi + QT::elem_off(r, cc * 4)) = h;
          *reinterpret_cast<LDS_PTR(bf16x4)>(lo + QT::elem_off(r, cc * 4)) = l;
        }
      }
    }
    if (tid < 2 * QB) ld_tile(buf)[tid] = ld_reg;
  };

  // this wave's K / V operands (B operands of S = Q K^T and dP = dO V^T)
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
  const int qrow_a = swap23(l32);  // A-operand row of S / dP

  Blk cur;
  load_entry(cur, eb, ee, a.entries);
  issue(cur, 0);
  commit(0);
  int step = 0;
  while (true) {
    Blk nxt = cur;
    const bool has_next = advance<QB>(nxt, ee, a.entries);
    const int buf = step & 1;
    wait_vm();
    __syncthreads();  // this step's rows are in LDS; the other buffer is free
    if (has_next) issue(nxt, buf ^ 1);

    LDS_PTR(float) ldv = ld_tile(buf);
#pragma unroll 1
    for (int sb = 0; sb < NSUB; ++sb) {
      const int qs0 = cur.qb + 32 * sb;  // first row of the sub-block
      // wave-uniform: no row of the sub-block sees any key of this wave
      // (a key limit, causal = -(limit + 1), hides keys >= limit from all rows)
      const int klimit = cur.causal < 0 ? -cur.causal - 1 : k1;
      if (qs0 >= cur.qe || wk0 >= klimit || (cur.causal > 0 && wk0 > qs0 + 31)) continue;
      // -LSE * log2(e) and -D of the 16 rows this lane holds: rows
      // 32 sb + 8 half + (0..7) and 32 sb + 16 + 8 half + (0..7)
      f32x4 lse4[4], dv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 32 * sb + 16 * (i >> 1) + 8 * half + 4 * (i & 1);
        lse4[i] = *reinterpret_cast<const LDS_PTR(f32x4)>(ldv + r0);
        dv4[i] = *reinterpret_cast<const LDS_PTR(f32x4)>(ldv + QB + r0);
      }
      // S = Q K^T and dP = dO V^T for this wave's 32 keys and 32 query rows;
      // register v of this lane is query row 32 sb + 16 (v / 8) + 8 half + v % 8.
      // The row operands of the phase are all read before the fence so that
      // the LDS reads stream while the MFMAs run.
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[v] = 0.f;
        pacc[v] = 0.f;
      }
      {
        Frag<SPLIT> qa_f[KC], da_f[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          qa_f[kc].h = row_operand<QT>(q_tile(buf, 0), 32 * sb + qrow_a, 2 * kc + half);
          da_f[kc].h = row_operand<QT>(do_tile(buf, 0), 32 * sb + qrow_a, 2 * kc + half);
          if constexpr (SPLIT) {
            qa_f[kc].l = row_operand<QT>(q_tile(buf, 1), 32 * sb + qrow_a, 2 * kc + half);
            da_f[kc].l = row_operand<QT>(do_tile(buf, 1), 32 * sb + qrow_a, 2 * kc + half);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          mma<SPLIT>(sacc, qa_f[kc], kf[kc]);
          mma<SPLIT>(pacc, da_f[kc], vf[kc]);
        }
      }
      // P = 2^(c s - LSE log2 e) recomputed from the saved LSE; masked where
      // a row is past the range, a key past the tile, or (causal) key > row.
      const bool need_mask =
          qs0 + 32 > cur.qe || wk0 + 32 > klimit || (cur.causal > 0 && wk0 + 31 > qs0);
      float p[16], ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v)
        p[v] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(sacc[v], a.scale_log2, lse4[v >> 2][v & 3]));
      if (need_mask) {
        const int qlim = cur.qe - cur.qb;                       // local rows < qlim
        const int kq = cur.causal > 0 ? key - cur.qb : -(1 << 30);  // local rows >= kq
        const bool kok = key < klimit;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ql = 32 * sb + 16 * (v >> 3) + 8 * half + (v & 7);
          p[v] = (kok && ql < qlim && ql >= kq) ? p[v] : 0.f;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) ds[v] = p[v] * (pacc[v] + dv4[v >> 2][v & 3]);
      const Frag<SPLIT> pf0 = pack8<SPLIT>(p), pf1 = pack8<SPLIT>(p + 8);
      const Frag<SPLIT> sf0 = pack8<SPLIT>(ds), sf1 = pack8<SPLIT>(ds + 8);

      // dV += P^T dO, dK += dS^T Q (dO, Q read transposed from LDS); the
      // operands of all column blocks are read before the fence
      {
        Frag<SPLIT> bo[DB][2], bq[DB][2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int qc = 0; qc < 2; ++qc) {
            bo[db][qc].h = tr_operand<QT>(do_tile(buf, 0), 32 * sb + 16 * qc, 32 * db, lane);
            bq[db][qc].h = tr_operand<QT>(q_tile(buf, 0), 32 * sb + 16 * qc, 32 * db, lane);
            if constexpr (SPLIT) {
              bo[db][qc].l = tr_operand<QT>(do_tile(buf, 1), 32 * sb + 16 * qc, 32 * db, lane);
              bq[db][qc].l = tr_operand<QT>(q_tile(buf, 1), 32 * sb + 16 * qc, 32 * db, lane);
            }
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int qc = 0; qc < 2; ++qc) {
            mma<SPLIT>(dv_acc[db], qc ? pf1 : pf0, bo[db][qc]);
            mma<SPLIT>(dk_acc[db], qc ? sf1 : sf0, bq[db][qc]);
          }
      }
    }

    if (!has_next) break;
    commit(buf ^ 1);
    cur = nxt;
    ++step;
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
// 2b. dK / dV for bf16 inputs, software-pipelined over 32-row query steps.
//
// The work of step j splits into three independent parts: A(j), the products
// S = Q K^T and dP = dO V^T; B(j), the element-wise P = 2^(c S - LSE log2 e)
// and dS = P (dP - D); and C(j), the updates dV += P^T dO and dK += dS^T Q.
// Iteration j issues C(j-1) and A(j+1) on the matrix cores while the vector
// ALUs run B(j), so the element-wise work of a wave hides under its own
// MFMAs.  Q, dO and the row terms go from memory straight into a ring of
// six LDS buffers (inline-asm LDS DMA, which the compiler's wait analysis
// does not see; the kernel counts its own loads): iteration j waits for step
// j + 1, passes a barrier and issues the loads of step j + 3, so each step
// has two iterations to arrive.  Iteration j reads the buffers of steps
// j - 1 .. j + 1; the barrier makes sure no wave still reads the buffer of
// step j - 3 that the new loads overwrite.  The S and dP MFMAs are inline
// asm as well, to keep their results out of the accumulation registers.
//
// No branch masks anything inside the loop:
//  * rows past a query range read as zeros (each buffer resource ends at the
//    range), so Q = dO = 0 and -LSE log2 e = -D = 0 there; P = 1 but
//    dP - D = 0 and dO = 0, so neither dK nor dV changes;
//  * keys past the tile only reach rows of dK / dV that are never stored;
//  * under the causal mask S starts from -inf where key > row, so P = 0.
template <int D>
struct DkdvPipeCfg {
  static constexpr int KC = D / 16, DB = D / 32;
  static constexpr int ROWS = 32;                // query rows per step
  static constexpr int NB = 6;                   // LDS ring buffers
  static constexpr int TILE = ROWS * D * 2;      // one bf16 Q or dO tile
  static constexpr int Q_OFF = 0, DO_OFF = TILE;
  static constexpr int NL_OFF = 2 * TILE;        // -LSE log2 e (64 floats, 32 used)
  static constexpr int ND_OFF = 2 * TILE + 256;  // -D (64 floats, 32 used)
  static constexpr int BUF = 2 * TILE + 512;
  static constexpr int SPARE_OFF = NB * BUF;     // target of the extra row-term loads
  static constexpr int BYTES = NB * BUF + 256;
};

namespace {

// A 32-row query step of a backward item: rows [r0, min(r0 + 32, qe)) of
// query head h, taken from entry e.  e == entry_end marks "no step".
struct Step {
  int e, r0, qe, h, causal;
};

__device__ __forceinline__ void step_at(Step& s, int e, int ee, const I4* entries) {
  s.e = e;
  if (e < ee) {
    const I4 en = load_plan4(entries, e);
    s.h = en.x;
    s.r0 = en.y;
    s.qe = en.z;
    s.causal = en.w;
  } else {
    s.h = 0;
    s.r0 = 0;
    s.qe = 0;
    s.causal = 0;
  }
}

__device__ __forceinline__ void step_next(Step& s, int ee, const I4* entries) {
  s.r0 += 32;
  if (s.r0 >= s.qe) step_at(s, s.e < ee ? s.e + 1 : ee, ee, entries);
}

// The step whose rows are being loaded, with the byte addresses of its first
// Q / dO row and row term, so that moving on within an entry is a few scalar
// adds rather than a fresh row-times-stride product.
struct LoadStep {
  Step s;
  const char* q;   // &Q[r0, h, 0]
  const char* d;   // &dO[r0, h, 0]
  const char* t;   // &rterm[h, r0] (-LSE log2 e or -D)
};

__device__ __forceinline__ void load_at(LoadStep& l, int e, int ee, const I4* entries,
                                        const char* q, const char* d, const char* t,
                                        int64_t row_bytes, int64_t head_bytes, int64_t n_tokens) {
  step_at(l.s, e, ee, entries);
  const int64_t r0 = l.s.r0, h = l.s.h;
  l.q = q + r0 * row_bytes + h * head_bytes;
  l.d = d + r0 * row_bytes + h * head_bytes;
  l.t = t + 4 * (h * n_tokens + r0);
}

__device__ __forceinline__ void load_next(LoadStep& l, int ee, const I4* entries, const char* q,
                                          const char* d, const char* t, int64_t row_bytes,
                                          int64_t head_bytes, int64_t n_tokens) {
  l.s.r0 += 32;
  l.q += 32 * row_bytes;
  l.d += 32 * row_bytes;
  l.t += 4 * 32;
  if (l.s.r0 >= l.s.qe)
    load_at(l, l.s.e < ee ? l.s.e + 1 : ee, ee, entries, q, d, t, row_bytes, head_bytes,
            n_tokens);
}

// P and dS of one step packed as A operands of the dV / dK products: p[c] /
// s[c] hold this lane's key against rows 16 c + 8 (lane / 32) + (0..7).
struct PdsPack {
  bf16x8 p[2], s[2];
};

// S and dP MFMAs of the pipelined kernel, written as inline asm so that
// their results land in ordinary VGPRs.  At one wave per SIMD the compiler
// gives every MFMA result to the accumulation registers, and each element
// would then need a v_accvgpr_read -- one more instruction for a wave that
// can issue only one every four cycles.  The compiler does not see these
// statements as MFMAs and inserts no hazard wait states around them, so the
// kernel's order keeps them apart from every other access of their
// registers: the first read of S or dP comes two MFMA slots into the next
// iteration, well over the sixteen wait states an 8-pass XDL result needs
// before a VALU op may read or overwrite it (CDNA3 / CDNA4 ISA, dependency
// rules).  Within a chain the accumulator is read back as source C in the
// same registers, which needs none.  Their A operands come from LDS loads
// and their B operands from registers loaded before the loop, never from a
// VALU op just before; a CPU test checks the compiled code for all of these
// distances on every path.
__device__ __forceinline__ void mfma_v_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// The LDS-DMA loads of one query step of the pipelined kernel in one
// assembly block (see TileLoader for the lane layout): PER loads of the Q
// tile from M0 = mq on, in 1 KiB steps, the same for dO at DSTEP bytes past
// the last Q load, and one row-term dword per lane to M0 = mt.  One hazard
// pad (an SGPR written by a VALU op needs five wait states before a vector
// memory op reads it), one M0 save / restore, and the one wait state an
// LDS DMA needs after each M0 write.
template <int PER, int DSTEP>
__device__ __forceinline__ void step_loads(unsigned mq, unsigned mt, const int (&voff)[PER],
                                           int vt, rsrc_t rq, rsrc_t rd, rsrc_t rt) {
  static_assert(PER == 1 || PER == 2, "one or two loads per wave and tile");
  unsigned saved;
  if constexpr (PER == 2) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, %9\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %7, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %4, %7, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %5, %8, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(mq), "s"(mt), "v"(voff[0]), "v"(voff[1]), "v"(vt), "s"(rq), "s"(rd), "s"(rt),
          "i"(DSTEP)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, %8\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %4, %7, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(mq), "s"(mt), "v"(voff[0]), "v"(vt), "s"(rq), "s"(rd), "s"(rt), "i"(DSTEP)
        : "memory", "scc");
  }
}

// Waits until at most n LDS (and scalar memory) operations of this wave are
// outstanding.  n must fold to a constant once the caller is unrolled; the
// switch turns it into the immediate the instruction needs (gfx9 s_waitcnt:
// lgkmcnt in bits 11:8, vmcnt and expcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_lgkm_c() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}
__device__ __forceinline__ void wait_lgkm(int n) {
  switch (n) {
    case 0: wait_lgkm_c<0>(); break;
    case 1: wait_lgkm_c<1>(); break;
    case 2: wait_lgkm_c<2>(); break;
    case 3: wait_lgkm_c<3>(); break;
    case 4: wait_lgkm_c<4>(); break;
    case 5: wait_lgkm_c<5>(); break;
    case 6: wait_lgkm_c<6>(); break;
    case 7: wait_lgkm_c<7>(); break;
    case 8: wait_lgkm_c<8>(); break;
    case 9: wait_lgkm_c<9>(); break;
    case 10: wait_lgkm_c<10>(); break;
    case 11: wait_lgkm_c<11>(); break;
    case 12: wait_lgkm_c<12>(); break;
    case 13: wait_lgkm_c<13>(); break;
    case 14: wait_lgkm_c<14>(); break;
    default: wait_lgkm_c<15>(); break;
  }
}

// Empty asm use: the value must be computed before this point, which keeps
// the compiler from sinking element-wise work out of its MFMA slot.
__device__ __forceinline__ void keep(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(const bf16x8& x) { asm volatile("" ::"v"(x)); }

}  // namespace

// LIM: the plan has key-limit entries (key tiles that cross from a parent
// into the child stored after it); the variant without them keeps the
// per-step mask test to the causal case.
template <int D, bool LIM>
__global__ __launch_bounds__(256, 1) void tree_attn_dkdv_pipe_kernel(BwdArgs a) {
  using C = DkdvPipeCfg<D>;
  constexpr int KC = C::KC, DB = C::DB, NB = C::NB, BUF = C::BUF;
  using QT = Tile<D, 32>;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);

  const I8 it = load_plan8(a.items, blockIdx.x);
  const int k0 = it.v[0], k1 = it.v[1], g = it.v[2], eb = it.v[3], ee = it.v[4];
  const int slot = it.v[5];
  if (eb >= ee) return;  // an empty item that pads the launch order
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t last = a.n_tokens - 1;
  const int64_t qs = static_cast<int64_t>(a.hq) * D;
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  const __bf16* Qall = static_cast<const __bf16*>(a.q);
  const __bf16* dOall = static_cast<const __bf16*>(a.dout);
  const int wk0 = k0 + 32 * wave;  // first key of this wave
  const int key = wk0 + l32;       // this lane's key (column of S)

  // Per-lane LDS offsets; every other term of an operand address is a
  // compile-time immediate (see Tile): row operands of chunk pair kc / 2,
  // transposed operands of rows (16 qc ..) and columns (32 db ..).
  const int qrow_a = swap23(l32);
  int ro[2];
  ro[0] = QT::chunk_off(qrow_a, half);
  ro[1] = QT::chunk_off(qrow_a, 2 + half);
  int tro[2];
  {
    const int grp = lane >> 4, L = lane & 15;
    const int r = 8 * (grp >> 1) + (L >> 2);
    const int c = 16 * (grp & 1) + 4 * (L & 3);
    tro[0] = QT::elem_off(r, c);
    tro[1] = QT::elem_off(r + 4, c);
  }
  const int ldo = 32 * half;  // byte offset of row 8 * half in a row-term array

  // The first iteration's dK / dV products read the last ring buffer with
  // zero P / dS; clear it so that stale LDS bits cannot form NaNs.
  {
    const i32x4 z = {0, 0, 0, 0};
    for (int i = tid; i < BUF / 16; i += 256) lds_write16(lds + (NB - 1) * BUF, 16 * i, z);
  }

  // Loads of one step go straight from memory into a ring buffer (see
  // TileLoader): C::PER 16-byte chunks of Q and of dO per thread, and one
  // row term per lane -- -LSE log2 e for wave 0, -D for wave 1; waves 2 and 3
  // repeat wave 0's load into a spare slot, so that every wave issues the
  // same number of loads per step and can count them in its waits.
  // Resources end at the step's last row, so rows past a query range, and
  // steps past the end (empty resources), read as zeros.
  TileLoader<D, 32, 4> tl;
  const char* rterm =
      reinterpret_cast<const char*>(wave == 1 ? a.neg_d : a.neg_lse2);
  const int rterm_off = wave == 1 ? C::ND_OFF : C::NL_OFF;
  // A step covers at most 32 rows, so its byte counts fit 32 bits.
  const int64_t row_bytes = qs * 2, head_bytes = D * 2;
  const uint32_t row_bytes32 = static_cast<uint32_t>(row_bytes);
  tl.init(static_cast<int>(row_bytes32), wave, lane);
  const char* Qb = reinterpret_cast<const char*>(Qall);
  const char* dOb = reinterpret_cast<const char*>(dOall);
  constexpr int TPER = TileLoader<D, 32, 4>::PER;
  constexpr int LPS = 2 * TPER + 1;  // loads per wave and step
  auto lds_addr = [&](LDS_PTR(char) p) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<__SIZE_TYPE__>(p)));
  };
  auto issue = [&](const LoadStep& l, int boff) __attribute__((always_inline)) {
    // rows of the step, at most 32; a step past the item's last entry has
    // r0 = qe = 0 (step_at), and a cursor never stands at r0 > qe, so this
    // is never negative and needs no test of the entry index
    const uint32_t rows = static_cast<uint32_t>(min(l.s.qe - l.s.r0, 32));
    const uint32_t nq = rows * row_bytes32;
    step_loads<TPER, C::TILE - (TPER - 1) * 1024>(
        lds_addr(lds + boff + C::Q_OFF + tl.lds0),
        lds_addr(wave < 2 ? lds + boff + rterm_off : lds + C::SPARE_OFF), tl.voff, 4 * lane,
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(l.q), static_cast<short>(0),
                                          static_cast<int>(nq), kRsrcFlags),
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(l.d), static_cast<short>(0),
                                          static_cast<int>(nq), kRsrcFlags),
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(l.t), static_cast<short>(0),
                                          static_cast<int>(4 * rows), kRsrcFlags));
  };

  // this wave's K / V operands (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[KC], vf[KC];
  {
    const int64_t r = key < last ? key : last;
    const __bf16* kp = static_cast<const __bf16*>(a.k) + r * ks + static_cast<int64_t>(g) * D;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + r * ks + static_cast<int64_t>(g) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = *reinterpret_cast<const bf16x8*>(kp + 16 * kc + 8 * half);
      vf[kc] = *reinterpret_cast<const bf16x8*>(vp + 16 * kc + 8 * half);
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

  auto nexto = [&](int o) __attribute__((always_inline)) { return o + BUF == NB * BUF ? 0 : o + BUF; };

  // MFMA slots of one iteration: first the dV / dK updates of the previous
  // step (slot i < NC: column block i / 4, row chunk (i / 2) % 2, dV for even
  // i and dK for odd i), then S and dP of the next step (slot NC + 2 kc for S,
  // NC + 2 kc + 1 for dP).
  constexpr int NC = 4 * DB, NS = NC + 2 * KC;
  constexpr int LA = 4;  // operands are read this many slots ahead
  constexpr int NRT = 8;  // row-term reads of a step (-LSE log2 e and -D, 4 x 16 bytes each)
  // LDS reads of an iteration, in issue order: its first LA operands (read
  // during the previous iteration), the row terms of its step, then the
  // operand LA slots ahead in every slot; the last LA slots read the next
  // iteration's first operands instead.  A transposed (dK / dV) operand
  // takes two reads.
  auto slot_reads = [&](int t) constexpr {
    const int k = t + LA;  // operand read in slot t
    return k < NC || k >= NS ? 2 : 1;
  };
  // reads up to and including operand k
  auto through_op = [&](int k) constexpr {
    if (k < LA) return 2 * (k + 1);
    int n = 2 * LA + NRT;
    for (int t = 0; t + LA <= k; ++t) n += slot_reads(t);
    return n;
  };
  // reads issued after operand i + 1 once slot i has issued its own.  Even
  // slots wait for their operand and the next one together: one s_waitcnt
  // per two MFMAs, each an issue slot of the only wave on the SIMD.  (The
  // compiler adds a wait of its own before any use these do not cover.)
  auto younger = [&](int i) constexpr {
    int n = 2 * LA + NRT;
    for (int t = 0; t <= i; ++t) n += slot_reads(t);
    return n - through_op(i + 1);
  };
  auto fetch = [&](int i, LDS_PTR(char) bprev, LDS_PTR(char) bnext)
                   __attribute__((always_inline)) -> bf16x8 {
    if (i < NC) {
      const int imm = (i >> 2) * QT::SUB + ((i >> 1) & 1) * 1024;
      LDS_PTR(char) t = bprev + ((i & 1) ? C::Q_OFF : C::DO_OFF);
      const bf16x4 lo = lds_read_tr(t, tro[0] + imm);
      const bf16x4 hi = lds_read_tr(t, tro[1] + imm);
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[e + 4] = hi[e];
      }
      return r;
    }
    const int kc = (i - NC) >> 1;
    LDS_PTR(char) t = bnext + (((i - NC) & 1) ? C::DO_OFF : C::Q_OFF);
    return lds_read16(t, ro[kc & 1] + (kc >> 1) * QT::SUB);
  };
  // S and dP of the step whose element-wise part runs next; P / dS of the
  // step whose updates run next
  f32x16 sacc, pacc;
  PdsPack pk;
  auto mfma_slot = [&](int i, const bf16x8& op) __attribute__((always_inline)) {
    if (i < NC) {
      const int db = i >> 2, qc = (i >> 1) & 1;
      if (i & 1) dk_acc[db] = mfma32(pk.s[qc], op, dk_acc[db]);
      else dv_acc[db] = mfma32(pk.p[qc], op, dv_acc[db]);
    } else {
      const int kc = (i - NC) >> 1;
      f32x16& acc = ((i - NC) & 1) ? pacc : sacc;
      const bf16x8& b = ((i - NC) & 1) ? vf[kc] : kf[kc];
      if (kc == 0) mfma_v_first(acc, op, b);
      else mfma_v_acc(acc, op, b);
    }
  };

  // The first LA operands of an iteration, read during the previous one so
  // that its first MFMAs need not wait out an LDS round trip.
  bf16x8 carry[LA];

  // One pipelined iteration j: C(j-1) then A(j+1) on the matrix cores, B(j)
  // on the vector ALUs beside them.  During the C slots each element's S and
  // dP leave the accumulators (x = c s - LSE log2 e, y = dP - D), so the A
  // slots may overwrite them; during the A slots P = 2^x, dS = P y and the
  // bf16 packs are formed, after the last C slot has read the old packs.
  // The fences keep this order.  Under the causal mask (rare steps) x is set
  // to -inf where key > row between the halves.  work(i) is scalar work
  // (loads, step bookkeeping) placed in C slot i, where the matrix core is
  // busy with that slot's MFMA.
  auto iteration = [&](int bp, int bc, int bn, bool masked, int delta, int rmask,
                       auto&& work) __attribute__((always_inline)) {
    LDS_PTR(char) bprev = lds + bp;
    LDS_PTR(char) bcur = lds + bc;
    LDS_PTR(char) bnext = lds + bn;
    bf16x8 op[NS];
#pragma unroll
    for (int i = 0; i < LA; ++i) op[i] = carry[i];
    f32x4 nl[4], nd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = ldo + 64 * (i >> 1) + 16 * (i & 1);
      nl[i] = *reinterpret_cast<const LDS_PTR(f32x4)>(bcur + C::NL_OFF + off);
      nd[i] = *reinterpret_cast<const LDS_PTR(f32x4)>(bcur + C::ND_OFF + off);
    }
    float x[16], y[16];
    // C slots 0 and 1 leave S and dP alone (the MFMAs that wrote them may
    // still run, and the row terms are still on their way); slots 2 .. NC - 1
    // take the 16 elements between them
    auto c_first = [&](int i) constexpr { return i < 2 ? 0 : ((i - 2) * 16) / (NC - 2); };
    constexpr int EA = 16 / (NS - NC);  // elements per A slot
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      op[i + LA] = fetch(i + LA, bprev, bnext);
      if ((i & 1) == 0) wait_lgkm(younger(i));
      mfma_slot(i, op[i]);
#pragma unroll
      for (int e = c_first(i); e < c_first(i + 1); ++e) {
        x[e] = __builtin_fmaf(sacc[e], a.scale_log2, nl[e >> 2][e & 3]);
        y[e] = pacc[e] + nd[e >> 2][e & 3];
        keep(x[e]);
        keep(y[e]);
      }
      work(i);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 16 * (v >> 3) + 8 * half + (v & 7);
        x[v] = l32 - (r & rmask) > delta ? -__builtin_inff() : x[v];
      }
    }
#pragma unroll
    for (int i = NC; i < NS; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + LA < NS) {
        op[i + LA] = fetch(i + LA, bprev, bnext);
      } else {
        // the next iteration's first operands (its C slots read step j's tiles)
        carry[i + LA - NS] = fetch(i + LA - NS, bcur, bcur);
      }
      if (((i - NC) & 1) == 0) wait_lgkm(younger(i));
      mfma_slot(i, op[i]);
#pragma unroll
      for (int e = EA * (i - NC); e < EA * (i - NC + 1); ++e) {
        const float pe = __builtin_amdgcn_exp2f(x[e]);
        pk.p[e >> 3][e & 7] = to_bf16(pe);
        pk.s[e >> 3][e & 7] = to_bf16(pe * y[e]);
      }
      if ((EA * (i - NC + 1)) % 8 == 0) {
        const int c = (EA * (i - NC + 1)) / 8 - 1;
        keep(pk.p[c]);
        keep(pk.s[c]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  LoadStep ld;
  auto ld_next = [&]() __attribute__((always_inline)) {
    load_next(ld, ee, a.entries, Qb, dOb, rterm, row_bytes, head_bytes, a.n_tokens);
  };
  load_at(ld, eb, ee, a.entries, Qb, dOb, rterm, row_bytes, head_bytes, a.n_tokens);
  Step cur = ld.s;  // step j
  Step nx = cur;
  step_next(nx, ee, a.entries);  // step j + 1
  issue(ld, 0);  // steps 0, 1 and 2 (zeros where there is none)
  ld_next();
  issue(ld, BUF);
  ld_next();
  issue(ld, 2 * BUF);
  ld_next();
  wait_vmcnt<2 * LPS>();  // step 0 is in
  // ring buffers as byte offsets: previous, current and next step
  int bp = (NB - 1) * BUF, bc = 0, bn = BUF;
  __syncthreads();
  // A of step 0; the first C(-1) runs on zero packs and a cleared buffer
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pk.p[c][e] = to_bf16(0.f);
      pk.s[c][e] = to_bf16(0.f);
    }
  {
    LDS_PTR(char) b0 = lds + bc;
#pragma unroll
    for (int i = NC; i < NS; ++i) mfma_slot(i, fetch(i, b0, b0));
#pragma unroll
    for (int i = 0; i < LA; ++i) carry[i] = fetch(i, lds + bp, lds + bp);
  }

  int bw = 3 * BUF;  // buffer of step j + 3
  // Iteration j: step j + 1 (loaded during iteration j - 2) must be in for
  // every wave, and every wave past iteration j - 1; then step j + 3 goes to
  // the buffer of step j - 3, leaving the load of step j + 2 in flight.
  // Iteration j reads only the buffers of steps j - 1 .. j + 1.  This runs
  // in the first C slots of the iteration, beside their MFMAs, the same in
  // every iteration (no branch).  The barrier needs no memory fence: every
  // LDS read of iteration j - 1 was waited for before the MFMA that used it,
  // and the tiles arrive by LDS DMA, whose completion the vmcnt wait covers.
  while (true) {
    const bool more = nx.e < ee;
    // A causal entry (w = 1) masks key > row, i.e. l32 - r > r0 - wk0; a
    // key limit (w = -(limit + 1)) masks key >= limit on every row, i.e.
    // l32 > limit - 1 - wk0.
    int delta = cur.r0 - wk0, rmask = -1;
    bool masked = cur.causal && delta < 32;
    if constexpr (LIM) {
      const bool lim = cur.causal < 0;
      delta = lim ? -cur.causal - 2 - wk0 : delta;
      masked = lim ? delta < 31 : (cur.causal != 0 && delta < 32);
      rmask = lim ? 0 : -1;
    }
    iteration(bp, bc, bn, masked, delta, rmask, [&](int i) __attribute__((always_inline)) {
      if (i == 1) {
        wait_vmcnt<LPS>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else if (i == 2) {
        issue(ld, bw);
        bw = nexto(bw);
      } else if (i == 3) {
        ld_next();
      }
      if (i == 7) {
        cur = nx;
        step_next(nx, ee, a.entries);
      }
    });
    bp = bc;
    bc = bn;
    bn = nexto(bn);
    if (!more) break;
  }
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup has left
  // the last S / dP MFMAs may still be writing registers that the code
  // below reuses: sixteen wait states
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  // C of the last step (its buffer is bp now)
  {
    LDS_PTR(char) bl = lds + bp;
#pragma unroll
    for (int i = 0; i < NC; ++i) mfma_slot(i, fetch(i, bl, bl));
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
        __bf16* dk = static_cast<__bf16*>(a.dk) + static_cast<int64_t>(kr) * ks +
                     static_cast<int64_t>(g) * D;
        __bf16* dv = static_cast<__bf16*>(a.dv) + static_cast<int64_t>(kr) * ks +
                     static_cast<int64_t>(g) * D;
        dk[d] = to_bf16(dkv);
        dv[d] = to_bf16(dvv);
      } else {
        const int64_t so = (static_cast<int64_t>(slot) * kBwdKeys + kl) * D + d;
        a.dk_slots[so] = dkv;
        a.dv_slots[so] = dvv;
      }
    }
  }
}

// --------------------------------------------------------------------------
// 3. dQ: query-tile centric, like the forward pass
template <typename T, int D>
struct DqCfg {
  static constexpr bool SPLIT = IsSplit<T>::value;
  static constexpr int NP = SPLIT ? 2 : 1;
  static constexpr int NBUF = (SPLIT && D == 128) ? 1 : 2;
  static constexpr int PLANE = kFwdKeys * D * 2;
  static constexpr int BYTES = NBUF * 2 * NP * PLANE;
};

template <typename T, int D>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void tree_attn_dq_kernel(BwdArgs a) {
  using C = DqCfg<T, D>;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int NP = C::NP, NBUF = C::NBUF;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int PLANE = C::PLANE;
  using KT = Tile<D, kFwdKeys>;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  LDS_PTR(char) lds = (LDS_PTR(char))(smem_dyn);
  auto k_tile = [&](int buf, int plane) { return lds + ((buf * 2 + 0) * NP + plane) * PLANE; };
  auto v_tile = [&](int buf, int plane) { return lds + ((buf * 2 + 1) * NP + plane) * PLANE; };

  // workgroup -> (query tile, kv head, query head), as in the forward pass
  const int b = blockIdx.x;
  const int xcd = b % kXcds, wslot = b / kXcds;
  const int64_t gi = static_cast<int64_t>(wslot / a.gsize) * kXcds + xcd;
  if (gi >= a.n_groups) return;
  const int tile = static_cast<int>(gi / a.hkv);
  const int g = static_cast<int>(gi % a.hkv);
  const int h = g * a.gsize + wslot % a.gsize;
  const I4 t = load_plan4(a.tiles, tile);
  const int q0 = t.x, q1 = t.y;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t last = a.n_tokens - 1;
  const int64_t qs = static_cast<int64_t>(a.hq) * D;
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  const T* K = static_cast<const T*>(a.k) + static_cast<int64_t>(g) * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<int64_t>(g) * D;
  const int qrow = q0 + 32 * wave + l32;  // this lane's query row
  const int wave_q0 = q0 + 32 * wave;

  // Q and dO of this lane's row (B operands of S^T = K Q^T and dP^T = V dO^T)
  Frag<SPLIT> qf[KC], df[KC];
  float nl2, ndq;  // -LSE * log2(e) and -D of this lane's row
  {
    const int64_t r = qrow < last ? qrow : last;
    const T* qp = static_cast<const T*>(a.q) + r * qs + static_cast<int64_t>(h) * D + 8 * half;
    const T* dp = static_cast<const T*>(a.dout) + r * qs + static_cast<int64_t>(h) * D + 8 * half;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qf[kc] = load_frag8(qp + 16 * kc);
      df[kc] = load_frag8(dp + 16 * kc);
    }
    nl2 = a.neg_lse2[static_cast<int64_t>(h) * a.n_tokens + r];
    ndq = a.neg_d[static_cast<int64_t>(h) * a.n_tokens + r];
  }

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

  f32x16 qacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) qacc[db][v] = 0.f;

  int ri = t.z;
  I4 rg = load_plan4(a.ranges, ri);
  int kt = rg.x;
  issue(kt, 0);
  commit(0);
  int step = 0;
  while (true) {
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
    __syncthreads();
    if (NBUF == 2 && has_next) issue(nkt, buf ^ 1);

    const int k1 = rg.y;
    const bool causal = rg.z != 0;
    // skipped when every key lies past this wave's rows or the wave has no
    // rows (the last tile of a node)
    if (!(causal && kt > wave_q0 + 31) && wave_q0 < q1) {
      // S^T and dP^T for keys kt + 32 kb + (0..31); register v of this lane
      // is key 16 (v / 8) + 8 half + v % 8 of the block (A rows swap23).
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          sacc[kb][v] = 0.f;
          pacc[kb][v] = 0.f;
        }
        const int krow = 32 * kb + swap23(l32);
        // row operands (K, then V) in four batches of KC / 2 fragments: the
        // smallest batches that keep the kernel within 256 VGPRs without
        // spilling
        constexpr int HB = KC / 2;
#pragma unroll
        for (int part = 0; part < 4; ++part) {
          const int kv = part >> 1, kc0 = (part & 1) * HB;
          Frag<SPLIT> fr[HB];
#pragma unroll
          for (int kc = 0; kc < HB; ++kc) {
            fr[kc].h =
                row_operand<KT>(kv ? v_tile(buf, 0) : k_tile(buf, 0), krow, 2 * (kc0 + kc) + half);
            if constexpr (SPLIT)
              fr[kc].l = row_operand<KT>(kv ? v_tile(buf, 1) : k_tile(buf, 1), krow,
                                         2 * (kc0 + kc) + half);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kc = 0; kc < HB; ++kc) {
            if (kv) mma<SPLIT>(pacc[kb], fr[kc], df[kc0 + kc]);
            else mma<SPLIT>(sacc[kb], fr[kc], qf[kc0 + kc]);
          }
        }
      }
      // P = 2^(c s - LSE log2 e); dS = P (dP - D); masked entries give 0.
      // Only edge and diagonal steps mask (a wave-uniform branch; the empty
      // asm keeps the compiler from flattening it into selects on every
      // step).
      const bool need_mask = (kt + kFwdKeys > k1) || (causal && kt + kFwdKeys - 1 > wave_q0);
      if (need_mask) {
        asm volatile("");
        const int klim = (causal ? (k1 < qrow + 1 ? k1 : qrow + 1) : k1) - kt;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = 32 * kb + 16 * (v >> 3) + 8 * half + (v & 7);
            sacc[kb][v] = kl < klim ? sacc[kb][v] : -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], a.scale_log2, nl2));
          sacc[kb][v] = p * (pacc[kb][v] + ndq);
        }
      // dQ^T += K^T dS^T over four 16-key chunks (K read transposed)
      Frag<SPLIT> sf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) x[s] = sacc[c >> 1][8 * (c & 1) + s];
        sf[c] = pack8<SPLIT>(x);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Frag<SPLIT> kt_f[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          kt_f[db].h = tr_operand<KT>(k_tile(buf, 0), 16 * c, 32 * db, lane);
          if constexpr (SPLIT) kt_f[db].l = tr_operand<KT>(k_tile(buf, 1), 16 * c, 32 * db, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) mma<SPLIT>(qacc[db], kt_f[db], sf[c]);
      }
    }

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

  if (qrow < q1) {
    // a key part of a split tile writes its fp32 partial sum, which
    // tree_attn_dq_sum_kernel adds up; a whole tile writes dQ
    const int part = load_plan1(a.part, tile);
    const float sc = a.scale;
    if (part >= 0) {
      float* op = a.dq_part +
                  ((static_cast<int64_t>(part) * a.hq + h) * kFwdRows + (qrow - q0)) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4(op + 32 * db + 8 * j + 4 * half, sc * qacc[db][4 * j],
                 sc * qacc[db][4 * j + 1], sc * qacc[db][4 * j + 2], sc * qacc[db][4 * j + 3]);
    } else {
      T* op =
          static_cast<T*>(a.dq) + static_cast<int64_t>(qrow) * qs + static_cast<int64_t>(h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4(op + 32 * db + 8 * j + 4 * half, sc * qacc[db][4 * j],
                 sc * qacc[db][4 * j + 1], sc * qacc[db][4 * j + 2], sc * qacc[db][4 * j + 3]);
    }
  }
}

// dQ of a split query tile: the fixed-order sum of its key parts' partial
// sums (deterministic), rounded once.  One workgroup per (split tile, query
// head); D / 8 threads per row, 8 columns each.
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_dq_sum_kernel(BwdArgs a) {
  const I4 c = load_plan4(a.combine, blockIdx.x);
  const int q0 = c.x, q1 = c.y, s0 = c.z, ns = c.w;
  const int h = blockIdx.y;
  constexpr int TPR = D / 8, RPP = 256 / TPR;
  const int col = (threadIdx.x % TPR) * 8;
  for (int r = q0 + static_cast<int>(threadIdx.x) / TPR; r < q1; r += RPP) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const int64_t row = (static_cast<int64_t>(s0 + s) * a.hq + h) * kFwdRows + (r - q0);
      const f32x4* p = reinterpret_cast<const f32x4*>(a.dq_part + row * D + col);
      const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += x0[e];
        acc[e + 4] += x1[e];
      }
    }
    T* op = static_cast<T*>(a.dq) + static_cast<int64_t>(r) * a.hq * D +
            static_cast<int64_t>(h) * D + col;
    store4(op, acc[0], acc[1], acc[2], acc[3]);
    store4(op + 4, acc[4], acc[5], acc[6], acc[7]);
  }
}

// --------------------------------------------------------------------------
// 4. post: partial-slot reduction (fixed order: deterministic dK / dV)
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_bwd_reduce_kernel(BwdArgs a) {
  const I8 r = load_plan8(a.reduce, blockIdx.x);
  const int k0 = r.v[0], k1 = r.v[1], g = r.v[2], sb = r.v[3], ns = r.v[4];
  const int64_t ks = static_cast<int64_t>(a.hkv) * D;
  // this block's share of the tile's (k1 - k0) * D elements
  const int n = (k1 - k0) * D;
  const int per = (n + static_cast<int>(gridDim.y) - 1) / static_cast<int>(gridDim.y);
  const int i0 = static_cast<int>(blockIdx.y) * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  for (int i = i0 + static_cast<int>(threadIdx.x); i < i1; i += 256) {
    const int kl = i / D, d = i % D;
    float sk = 0.f, sv = 0.f;
    for (int s = 0; s < ns; ++s) {
      const int64_t so = (static_cast<int64_t>(sb + s) * kBwdKeys + kl) * D + d;
      sk += a.dk_slots[so];
      sv += a.dv_slots[so];
    }
    const int64_t o = static_cast<int64_t>(k0 + kl) * ks + static_cast<int64_t>(g) * D + d;
    if (a.acc_dk) {
      // each (key row, kv head) belongs to one reduction entry: no races
      a.acc_dk[o] += sk;
      a.acc_dv[o] += sv;
    } else {
      static_cast<T*>(a.dk)[o] = static_cast<T>(sk);
      static_cast<T*>(a.dv)[o] = static_cast<T>(sv);
    }
  }
}

// Conversion of fp32 accumulators to the tensors' dtype (after a sequence
// of accumulating backward calls): 4 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void tree_attn_cast_kernel(const float* src, T* dst,
                                                            int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 x = *reinterpret_cast<const float4*>(src + i);
    dst[i] = static_cast<T>(x.x);
    dst[i + 1] = static_cast<T>(x.y);
    dst[i + 2] = static_cast<T>(x.z);
    dst[i + 3] = static_cast<T>(x.w);
  } else {
    for (int64_t j = i; j < n; ++j) dst[j] = static_cast<T>(src[j]);
  }
}

// --------------------------------------------------------------------------
// launchers

template <typename T, int D>
static hipError_t pre_t(const BwdArgs& a, hipStream_t s) {
  const int64_t per = 256 / (D / 8);
  if (a.pre_tiles) {
    if (a.n_pre_tiles == 0) return hipSuccess;
    // a forward query tile holds at most kFwdRows tokens
    const int64_t blocks = (static_cast<int64_t>(kFwdRows) * a.hq + per - 1) / per;
    hipLaunchKernelGGL((tree_attn_bwd_pre_kernel<T, D>),
                       dim3(static_cast<unsigned>(a.n_pre_tiles), static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int64_t rows = a.n_tokens * a.hq;
  const int64_t blocks = (rows + per - 1) / per;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((tree_attn_bwd_pre_kernel<T, D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dkdv_t(const BwdArgs& a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  // bf16: the software-pipelined kernel; fp32: the kernel with fp32 MFMAs
  // (the only instantiation of tree_attn_dkdv_kernel)
  void (*kern)(BwdArgs);
  int bytes;
  if constexpr (IsSplit<T>::value) {
    kern = tree_attn_dkdv_kernel<T, D>;
    bytes = DkdvCfg<T, D>::BYTES;
  } else {
    kern = a.has_limit ? tree_attn_dkdv_pipe_kernel<D, true> : tree_attn_dkdv_pipe_kernel<D, false>;
    bytes = DkdvPipeCfg<D>::BYTES;
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_items)), dim3(256), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dq_t(const BwdArgs& a, hipStream_t s) {
  if (a.dq_blocks <= 0) return hipSuccess;
  constexpr int bytes = DqCfg<T, D>::BYTES;
  auto kern = tree_attn_dq_kernel<T, D>;
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.dq_blocks)), dim3(256), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dq_sum_t(const BwdArgs& a, hipStream_t s) {
  if (a.n_combine <= 0) return hipSuccess;
  hipLaunchKernelGGL((tree_attn_dq_sum_kernel<T, D>),
                     dim3(static_cast<unsigned>(a.n_combine), static_cast<unsigned>(a.hq)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t post_t(const BwdArgs& a, hipStream_t s) {
  if (a.n_reduce == 0) return hipSuccess;
  // 16 blocks per split key tile: enough parallel streams over the slots
  hipLaunchKernelGGL((tree_attn_bwd_reduce_kernel<T, D>),
                     dim3(static_cast<unsigned>(a.n_reduce), 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Every kernel variant is instantiated explicitly so that the host pass
// always emits its launch stub.
#define TREE_ATTN_INSTANTIATE(T, D)                                          \
  template __global__ void tree_attn_bwd_pre_kernel<T, D>(BwdArgs);         \
  template __global__ void tree_attn_dq_kernel<T, D>(BwdArgs);              \
  template __global__ void tree_attn_dq_sum_kernel<T, D>(BwdArgs);          \
  template __global__ void tree_attn_bwd_reduce_kernel<T, D>(BwdArgs);
template __global__ void tree_attn_dkdv_pipe_kernel<128, false>(BwdArgs);
template __global__ void tree_attn_dkdv_pipe_kernel<64, false>(BwdArgs);
template __global__ void tree_attn_dkdv_pipe_kernel<128, true>(BwdArgs);
template __global__ void tree_attn_dkdv_pipe_kernel<64, true>(BwdArgs);
template __global__ void tree_attn_dkdv_kernel<float, 128>(BwdArgs);
template __global__ void tree_attn_dkdv_kernel<float, 64>(BwdArgs);
TREE_ATTN_INSTANTIATE(__bf16, 128)
TREE_ATTN_INSTANTIATE(__bf16, 64)
TREE_ATTN_INSTANTIATE(float, 128)
TREE_ATTN_INSTANTIATE(float, 64)
#undef TREE_ATTN_INSTANTIATE

#define TREE_ATTN_DISPATCH(FN)                                     \
  if (dtype == 0 && head_dim == 128) return FN<__bf16, 128>(a, s); \
  if (dtype == 0 && head_dim == 64) return FN<__bf16, 64>(a, s);   \
  if (dtype == 1 && head_dim == 128) return FN<float, 128>(a, s);  \
  if (dtype == 1 && head_dim == 64) return FN<float, 64>(a, s);    \
  return hipErrorInvalidValue;

hipError_t launch_bwd_pre(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(pre_t)
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(dkdv_t)
}
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(dq_t)
}
hipError_t launch_bwd_post(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(post_t)
}
hipError_t launch_bwd_dq_sum(const BwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  TREE_ATTN_DISPATCH(dq_sum_t)
}

hipError_t launch_cast(const float* src, void* dst, int64_t n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 1023) / 1024;
  if (dtype == 0)
    hipLaunchKernelGGL(tree_attn_cast_kernel<__bf16>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, src, static_cast<__bf16*>(dst), n);
  else if (dtype == 1)
    hipLaunchKernelGGL(tree_attn_cast_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, src, static_cast<float*>(dst), n);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tree_attn
