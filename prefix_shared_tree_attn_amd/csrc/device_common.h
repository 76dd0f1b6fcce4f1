// Device helpers shared by the tree-attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, one 64-lane wave):
//   A operand (32 x 16): lane l holds A[l % 32][8 * (l / 32) + s], s = 0..7
//   B operand (16 x 32): lane l holds B[8 * (l / 32) + s][l % 32]
//   C (32 x 32, fp32):   lane l, register v holds C[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32]
// The reduction index k can be relabelled freely as long as A and B agree.
//
// ds_read_tr16_b64 (gfx950): in each group of 16 lanes, lane L supplies the
// address of 4 consecutive 16-bit elements; lane j of the group receives
// element j % 4 of the address given by lane 4 * i + j / 4 as its element i.
// Reading a row-major [row][col] tile with lane L pointing at
// (row0 + L / 4, col0 + 4 * (L % 4)) therefore returns, in lane j, the
// column col0 + j of rows row0 .. row0 + 3: a transposed operand straight
// from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "planner.h"

namespace tree_attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// fp32 values travel through the bf16 tile and fragment machinery as two
// 16-bit planes: hi holds the upper and lo the lower 16 bits of each fp32
// bit pattern (stored in bf16-typed slots; the split is exact, no rounding),
// so LDS tiles, transposed reads and operand layouts are those of bf16.
__device__ __forceinline__ void split_bits(float x, __bf16& hi, __bf16& lo) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  hi = __builtin_bit_cast(__bf16, static_cast<uint16_t>(u >> 16));
  lo = __builtin_bit_cast(__bf16, static_cast<uint16_t>(u & 0xFFFFu));
}
__device__ __forceinline__ float join_bits(__bf16 hi, __bf16 lo) {
  const uint32_t h = __builtin_bit_cast(uint16_t, hi), l = __builtin_bit_cast(uint16_t, lo);
  return __builtin_bit_cast(float, (h << 16) | l);
}

// An MFMA operand fragment: this lane's 8 values of a 32 x 16 (A) or
// 16 x 32 (B) operand.  bf16: one register quad, one 32x32x16 MFMA.  fp32
// (SPLIT): the two 16-bit planes (split_bits); mma rebuilds the fp32 values
// and issues eight v_mfma_f32_32x32x2_f32, the s-th taking this lane's
// value s, so that lane halves 0 and 1 contribute reduction indices s and
// 8 + s -- together the same 16 reduction indices as the bf16 MFMA, with
// fp32 products and fp32 accumulation.
template <bool SPLIT>
struct Frag;
template <>
struct Frag<false> {
  bf16x8 h;
};
template <>
struct Frag<true> {
  bf16x8 h, l;
};

template <bool SPLIT>
__device__ __forceinline__ void mma(f32x16& c, const Frag<SPLIT>& a, const Frag<SPLIT>& b) {
  if constexpr (SPLIT) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(join_bits(a.h[s], a.l[s]),
                                               join_bits(b.h[s], b.l[s]), c, 0, 0, 0);
  } else {
    c = mfma32(a.h, b.h, c);
  }
}

// Packs eight fp32 values into an operand fragment (bf16 rounding, or the
// exact 16-bit planes for fp32).
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> pack8(const float* x) {
  Frag<SPLIT> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if constexpr (SPLIT) {
      __bf16 hi, lo;
      split_bits(x[s], hi, lo);
      f.h[s] = hi;
      f.l[s] = lo;
    } else {
      f.h[s] = to_bf16(x[s]);
    }
  }
  return f;
}

// ---------------------------------------------------------------------------
// LDS tiles: ROWS rows x D bf16 columns, stored as D / 32 sub-tiles of 32
// columns, each with 64-byte rows.  The 16-byte chunk cc (0..3) of row r in a
// sub-tile sits at chunk cc ^ ((r >> 2) & 3).  Four consecutive rows share a
// 256-byte bank line, so
//  * 16 lanes reading the same chunk of 16 consecutive rows (row operands,
//    ds_read_b128) hit 16 distinct 16-byte slots, and
//  * a 16-lane transpose read of 4 consecutive rows x 32 bytes plus its
//    neighbour group's next 32 bytes (ds_read_tr16_b64) fill one bank line,
// both free of bank conflicts; and because the swizzle depends only on bits
// 2..3 of the row, the sub-tile and any row offset that is a multiple of 16
// stay compile-time immediates of the LDS instructions.
template <int D, int ROWS>
struct Tile {
  static constexpr int SUB = ROWS * 64;  // bytes of one 32-column sub-tile
  static constexpr int BYTES = (D / 32) * SUB;
  __device__ __forceinline__ static int swz(int r) { return (r >> 2) & 3; }
  // byte offset of the 16-byte chunk c (columns 8c .. 8c + 7) of row r
  __device__ __forceinline__ static int chunk_off(int r, int c) {
    return (c >> 2) * SUB + r * 64 + (((c & 3) ^ swz(r)) << 4);
  }
  // byte offset of element col of row r (col a multiple of 4 for 8-byte reads)
  __device__ __forceinline__ static int elem_off(int r, int col) {
    return (col >> 5) * SUB + r * 64 + ((((col >> 3) & 3) ^ swz(r)) << 4) + ((col & 7) << 1);
  }
};

__device__ __forceinline__ bf16x8 lds_read16(const LDS_PTR(char) base, int off) {
  return *reinterpret_cast<const LDS_PTR(bf16x8)>(base + off);
}
__device__ __forceinline__ void lds_write16(LDS_PTR(char) base, int off, const i32x4& v) {
  *reinterpret_cast<LDS_PTR(i32x4)>(base + off) = v;
}
__device__ __forceinline__ bf16x4 lds_read_tr(const LDS_PTR(char) base, int off) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LDS_PTR(s16x4)>(const_cast<LDS_PTR(char)>(base) + off));
  return __builtin_bit_cast(bf16x4, r);
}

// Transposed operand from an LDS tile: returns, for this lane, the 8 values
// tile[row0 + 8 * (lane / 32) + s][col0 + (lane % 32)], s = 0..7 -- an MFMA
// operand whose lane index runs along the tile's columns and whose reduction
// slots run along its rows.  `row0` must be a multiple of 16 and `col0` of 32.
template <class TL>
__device__ __forceinline__ bf16x8 tr_operand(const LDS_PTR(char) base, int row0, int col0,
                                             int lane) {
  const int grp = lane >> 4, L = lane & 15;
  // The lane's own row and column inside the 16 x 32 block, and the block's
  // place: row0 (a multiple of 16) adds whole 64-byte rows without touching
  // the swizzle, which depends on bits 2-3 of the row only, and col0 (a
  // multiple of 32) whole sub-tiles.  Kept apart, the block's part folds
  // into the reads' immediate offsets and the lane's part is computed once.
  const int r = 8 * (grp >> 1) + (L >> 2);
  const int c = 16 * (grp & 1) + 4 * (L & 3);
  const LDS_PTR(char) b = base + row0 * 64 + (col0 >> 5) * TL::SUB;
  const bf16x4 lo = lds_read_tr(b, TL::elem_off(r, c));
  const bf16x4 hi = lds_read_tr(b, TL::elem_off(r + 4, c));
  bf16x8 out;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    out[s] = lo[s];
    out[s + 4] = hi[s];
  }
  return out;
}

// Row operand from an LDS tile: the 8 values tile[row][c8 * 8 + s].
template <class TL>
__device__ __forceinline__ bf16x8 row_operand(const LDS_PTR(char) base, int row, int c8) {
  return lds_read16(base, TL::chunk_off(row, c8));
}

// Row index used for the A operand so that output register v of lane half h
// corresponds to row 16 * (v / 8) + 8 * h + v % 8: bits 2 and 3 of the MFMA
// row are swapped.  With it, the 16 fp32 outputs of a lane split into two
// halves of 8 consecutive reduction indices, which is exactly the B/A operand
// slot order of a following MFMA that reduces over that dimension.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Global memory helpers -----------------------------------------------------

// Plan arrays are read-only while a kernel runs.  Reading them through the
// constant address space gives uniform scalar loads; a vector load instead
// would make the compiler wait for every outstanding vector memory operation
// (s_waitcnt vmcnt(0)) before using the value -- including tile prefetches.
#define CONST_PTR(T) __attribute__((address_space(4))) const T*

__device__ __forceinline__ I4 load_plan4(const I4* p, int64_t i) {
  CONST_PTR(int) q = (CONST_PTR(int))(p) + 4 * i;
  return {q[0], q[1], q[2], q[3]};
}
__device__ __forceinline__ int load_plan1(const int32_t* p, int64_t i) {
  return *((CONST_PTR(int))(p) + i);
}
__device__ __forceinline__ I8 load_plan8(const I8* p, int64_t i) {
  CONST_PTR(int) q = (CONST_PTR(int))(p) + 8 * i;
  I8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r.v[j] = q[j];
  return r;
}
__device__ __forceinline__ i32x4 gload16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// 8 consecutive elements of a global row as an operand fragment.
__device__ __forceinline__ Frag<false> load_frag8(const __bf16* p) {
  Frag<false> f;
  f.h = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<true> load_frag8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return pack8<true>(x);
}

// Copies rows [row0, row0 + ROWS) of a global tensor (D elements per row
// starting at `base`, rows `row_stride` elements apart) into a bf16 LDS tile,
// or for fp32 inputs into the two 16-bit planes of one (split_bits).  Rows past
// `last_row` are clamped to it; callers mask their contributions.  All
// global loads are issued before the LDS writes.
template <typename T, int D, int ROWS, int NT>
__device__ __forceinline__ void load_tile(LDS_PTR(char) hi, LDS_PTR(char) lo, const T* base,
                                          int64_t row_stride, int64_t row0, int64_t last_row,
                                          int tid) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  constexpr int CPR = D / EPC;
  constexpr int TOTAL = ROWS * CPR;
  static_assert(TOTAL % NT == 0, "tile chunks must divide evenly among threads");
  constexpr int PER = TOTAL / NT;
  i32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    const int64_t row = row0 + r < last_row ? row0 + r : last_row;
    v[i] = gload16(base + row * row_stride + cc * EPC);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    if constexpr (sizeof(T) == 2) {
      lds_write16(hi, Tile<D, ROWS>::chunk_off(r, cc), v[i]);
    } else {
      const f32x4 f = __builtin_bit_cast(f32x4, v[i]);
      bf16x4 h, l;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        __bf16 hs, ls;
        split_bits(f[s], hs, ls);
        h[s] = hs;
        l[s] = ls;
      }
      *reinterpret_cast<LDS_PTR(bf16x4)>(hi + Tile<D, ROWS>::elem_off(r, cc * 4)) = h;
      *reinterpret_cast<LDS_PTR(bf16x4)>(lo + Tile<D, ROWS>::elem_off(r, cc * 4)) = l;
    }
  }
}

// Buffer resources (V#): a 64-bit base in scalar registers, no stride, and a
// byte range; loads past the range return zero and stores / atomics past it
// are dropped (the scalar offset counts toward the range).  Row tiles near
// the end of a tensor therefore need no clamping.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw 32-bit buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, const void* end) {
  const int64_t n = static_cast<const char*>(end) - static_cast<const char*>(base);
  const uint32_t r = n <= 0 ? 0u : (n >= 0xFFFFFFFFll ? 0xFFFFFFFFu : static_cast<uint32_t>(n));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(r), kRsrcFlags);
}

// Raw buffer resource over `rows` rows of `row_bytes` bytes from `base`: a
// tile of at most a few hundred rows, whose byte count fits 32 bits, so no
// 64-bit clamp is needed.  Lanes past the last row read zeros.
__device__ __forceinline__ rsrc_t tile_rsrc(const void* base, int rows, uint32_t row_bytes) {
  const uint32_t n = rows > 0 ? static_cast<uint32_t>(rows) * row_bytes : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(n), kRsrcFlags);
}

// Buffer loads straight to LDS (MUBUF with the lds bit): lane l writes its
// SIZE bytes to LDS address M0 + SIZE * l.  They are issued from inline
// assembly on purpose.  The compiler cannot relate a direct-to-LDS load to a
// later transposed LDS read (ds_read_b64_tr_b16 carries no alias
// information), so with the intrinsic it drains every outstanding load
// (vmcnt(0)) before each transposed read -- including the prefetch of the
// next tile, which then never overlaps the compute.  Issued this way the
// loads are invisible to that analysis: callers wait for them explicitly
// (s_waitcnt vmcnt) and synchronise before reading the destination.  The
// block saves and restores M0, and pads the hazards the assembler does not
// check inside inline assembly: an SGPR written by a vector instruction
// needs five wait states before a vector memory instruction reads it, and
// an M0 write one wait state before an LDS DMA uses it.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(LDS_PTR(char) dst, int voffset, rsrc_t rs) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4 transfers");
  const unsigned m0v =
      __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<__SIZE_TYPE__>(dst)));
  unsigned saved;
  if constexpr (SIZE == 16) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(voffset), "s"(rs)
        : "memory");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(voffset), "s"(rs)
        : "memory");
  }
}

// Loads a ROWS x D bf16 row tile into a swizzled LDS tile (Tile<D, ROWS>)
// with buffer loads straight to LDS (dma_to_lds): the wave's lanes fill
// consecutive 16-byte LDS slots, each lane fetching the logical chunk the
// swizzle puts at its slot.  Per-lane byte offsets are fixed for a given row
// stride, so a step only changes the buffer base.
template <int D, int ROWS, int NW>
struct TileLoader {
  static constexpr int PER = ROWS * (D / 8) / (64 * NW);
  static_assert(ROWS * (D / 8) % (64 * NW) == 0, "tile must split into whole wave loads");
  int voff[PER];
  int lds0;
  __device__ __forceinline__ void init(int row_stride_bytes, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int p = (wave * PER + j) * 64 + lane;
      const int sub = p / (ROWS * 4), rem = p % (ROWS * 4);
      const int r = rem >> 2;
      const int c = sub * 4 + ((rem & 3) ^ Tile<D, ROWS>::swz(r));
      voff[j] = r * row_stride_bytes + c * 16;
    }
    lds0 = wave * PER * 1024;
  }
  // The wave's PER loads go out in one assembly block: the hazard padding
  // and the M0 save / restore are paid once, and M0 steps 1 KiB (one wave's
  // 64 x 16 bytes) between loads, with the one wait state an M0 write needs
  // before an LDS DMA.
  __device__ __forceinline__ void issue(LDS_PTR(char) tile, rsrc_t rs) const {
    static_assert(PER == 1 || PER == 2 || PER == 4, "one, two or four loads per wave");
    const unsigned m0v = __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<__SIZE_TYPE__>(tile + lds0)));
    unsigned saved;
    if constexpr (PER == 1) {
      dma_to_lds<16>(tile + lds0, voff[0], rs);
    } else if constexpr (PER == 2) {
      asm volatile(
          "s_nop 4\n\t"
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %3, %4, 0 offen lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(m0v), "v"(voff[0]), "v"(voff[1]), "s"(rs)
          : "memory", "scc");
    } else {
      asm volatile(
          "s_nop 4\n\t"
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %4, %6, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %5, %6, 0 offen lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(m0v), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs)
          : "memory", "scc");
    }
  }
};

// Waits until this wave's vector memory operations (loads, direct-to-LDS
// loads, stores, atomics) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N vector memory loads of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Stores four consecutive fp32 values as output elements.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 x;
  x[0] = to_bf16(a);
  x[1] = to_bf16(b);
  x[2] = to_bf16(c);
  x[3] = to_bf16(d);
  *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 x;
  x[0] = a;
  x[1] = b;
  x[2] = c;
  x[3] = d;
  *reinterpret_cast<f32x4*>(p) = x;
}

template <typename T>
struct IsSplit {
  static constexpr bool value = false;
};
template <>
struct IsSplit<float> {
  static constexpr bool value = true;
};

}  // namespace tree_attn
