// Passes on either side of tree attention (gfx950): the inverse gather of
// unique-token rows to trajectory positions, its adjoint (a deterministic
// sum of trajectory rows onto unique tokens) and rotary embeddings at tree
// depth.
//
// After prefix compression every trajectory position refers to one unique
// token (AReaL-DTA, abstract: shared prefixes are one computation; HARTS,
// abstract: per-trajectory objectives keep their interface).  Per-token
// results such as log-probabilities are handed back to the trajectories by
// a gather; gradients coming from the trajectories are summed per unique
// token in a fixed order (no atomics, bitwise reproducible).  Rotary
// embeddings use the token's depth, which is its position on every path
// through it.  All three are bound by HBM bandwidth: rows are moved in
// 8- or 16-byte pieces when the row size and alignment allow it.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace tree_attn {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int v4i;

// One workgroup per output row at a time (grid-stride over rows); its
// threads copy the row's words, so no thread divides to find its row.
template <typename W>
__global__ __launch_bounds__(256) void gather_kernel(const W* __restrict__ src, W* __restrict__ dst,
                                                     const int32_t* __restrict__ index,
                                                     int64_t rows, int64_t row_words) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const W* s = src + static_cast<int64_t>(index[r]) * row_words;
    W* d = dst + r * row_words;
    // up to four loads in flight before their stores; the destination is
    // not read again here, so its stores bypass the caches (non-temporal)
    for (int64_t c = threadIdx.x; c < row_words; c += 4 * 256) {
      W v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k * 256 < row_words) v[k] = s[c + k * 256];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k * 256 < row_words) __builtin_nontemporal_store(v[k], d + c + k * 256);
    }
  }
}

// Rows of a few words: one thread per (row, word).
template <typename W>
__global__ __launch_bounds__(256) void gather_narrow_kernel(const W* __restrict__ src,
                                                            W* __restrict__ dst,
                                                            const int32_t* __restrict__ index,
                                                            int64_t rows, int row_words) {
  const int64_t total = rows * row_words;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = e / row_words;
    const int c = static_cast<int>(e - r * row_words);
    dst[e] = src[static_cast<int64_t>(index[r]) * row_words + c];
  }
}

__device__ __forceinline__ float load_f(const __bf16* p) { return static_cast<float>(*p); }
__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ void store_f(__bf16* p, float x) { *p = static_cast<__bf16>(x); }
__device__ __forceinline__ void store_f(float* p, float x) { *p = x; }

// dst[u, c] = sum over j in [offsets[u], offsets[u+1]) of src[positions[j], c],
// fp32 accumulation in the order of `positions`.  One thread per (row,
// group of VEC columns); consecutive threads take consecutive groups, so a
// wave reads whole rows with 16-byte accesses when VEC * sizeof(T) = 16.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void scatter_sum_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ positions,
                                                          int64_t rows, int64_t row_elems) {
  typedef __attribute__((__vector_size__(VEC * sizeof(T)))) T vec_t;
  const int64_t groups = row_elems / VEC;
  // wide rows: one workgroup per output row at a time; narrow rows: one
  // thread per (row, group)
  const bool wide = groups >= 64;
  const int64_t total = wide ? rows * 256 : rows * groups;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t u = wide ? e >> 8 : e / groups;
    const int64_t g0 = wide ? (e & 255) : e - u * groups;
    for (int64_t g = g0; g < (wide ? groups : g0 + 1); g += 256) {
    const int64_t c = g * VEC;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int32_t j = offsets[u]; j < offsets[u + 1]; ++j) {
      const vec_t v = *reinterpret_cast<const vec_t*>(src + static_cast<int64_t>(positions[j]) * row_elems + c);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += static_cast<float>(v[i]);
    }
    vec_t out;
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = static_cast<T>(acc[i]);
    *reinterpret_cast<vec_t*>(dst + u * row_elems + c) = out;
    }
  }
}

// Rotary embedding, rotate-half pairing: for each (token, head) and
// i < D/2 the pair (x_i, x_{i+D/2}) is rotated by angle
// pos[t] * theta^(-2i/D) (by minus that angle when inverse, which is the
// transpose, i.e. the backward of the forward rotation).  One thread per
// (token, i): the angle is reduced modulo 2 pi in double precision, its sine
// and cosine are taken once in single precision and applied to every head.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ x, const int32_t* __restrict__ pos,
                                                   int64_t n_tokens, int heads, int head_dim,
                                                   double log2_theta, int inverse) {
  typedef __attribute__((__vector_size__(VEC * sizeof(T)))) T vec_t;
  const int half = head_dim / 2;
  const int groups = half / VEC;
  const int64_t total = n_tokens * groups;
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e < 0x7FFFFFFF ? static_cast<int64_t>(static_cast<uint32_t>(e) /
                                                          static_cast<uint32_t>(groups))
                                     : e / groups;
    const int i0 = static_cast<int>(e - t * groups) * VEC;
    float sn[VEC], cs[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const double inv_freq = exp2(-(2.0 * (i0 + v) / head_dim) * log2_theta);
      const double ang = static_cast<double>(pos[t]) * inv_freq;
      const float r = static_cast<float>(ang - two_pi * rint(ang / two_pi));
      sincosf(r, &sn[v], &cs[v]);
      if (inverse) sn[v] = -sn[v];
    }
    T* row = x + t * static_cast<int64_t>(heads) * head_dim;
    for (int h = 0; h < heads; ++h) {
      T* p = row + static_cast<int64_t>(h) * head_dim + i0;
      const vec_t a = *reinterpret_cast<const vec_t*>(p);
      const vec_t b = *reinterpret_cast<const vec_t*>(p + half);
      vec_t ra, rb;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float av = static_cast<float>(a[v]), bv = static_cast<float>(b[v]);
        ra[v] = static_cast<T>(av * cs[v] - bv * sn[v]);
        rb[v] = static_cast<T>(av * sn[v] + bv * cs[v]);
      }
      *reinterpret_cast<vec_t*>(p) = ra;
      *reinterpret_cast<vec_t*>(p + half) = rb;
    }
  }
}

int64_t grid_for(int64_t work) {
  const int64_t blocks = (work + 255) / 256;
  return blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536;
}

// matches the thread mapping of scatter_sum_kernel
int64_t scatter_grid(int64_t rows, int64_t groups) {
  return grid_for(groups >= 64 ? rows * 256 : rows * groups);
}

}  // namespace

hipError_t launch_gather(const void* src, void* dst, const int32_t* index, int64_t rows,
                         int64_t row_bytes, hipStream_t s) {
  if (rows <= 0 || row_bytes <= 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  if (row_bytes % 16 == 0 && al % 16 == 0) {
    const int64_t w = row_bytes / 16;
    if (w >= 64)
      hipLaunchKernelGGL(gather_kernel<v4i>, dim3(rows < 65536 ? rows : 65536), dim3(256), 0, s,
                         static_cast<const v4i*>(src), static_cast<v4i*>(dst), index, rows, w);
    else
      hipLaunchKernelGGL(gather_narrow_kernel<v4i>, dim3(grid_for(rows * w)), dim3(256), 0, s,
                         static_cast<const v4i*>(src), static_cast<v4i*>(dst), index, rows,
                         static_cast<int>(w));
  } else if (row_bytes % 4 == 0 && al % 4 == 0 && row_bytes / 4 < (1 << 30)) {
    hipLaunchKernelGGL(gather_narrow_kernel<int32_t>, dim3(grid_for(rows * (row_bytes / 4))),
                       dim3(256), 0, s, static_cast<const int32_t*>(src),
                       static_cast<int32_t*>(dst), index, rows, static_cast<int>(row_bytes / 4));
  } else if (row_bytes % 2 == 0 && al % 2 == 0 && row_bytes / 2 < (1 << 30)) {
    hipLaunchKernelGGL(gather_narrow_kernel<int16_t>, dim3(grid_for(rows * (row_bytes / 2))),
                       dim3(256), 0, s, static_cast<const int16_t*>(src),
                       static_cast<int16_t*>(dst), index, rows, static_cast<int>(row_bytes / 2));
  } else {
    hipLaunchKernelGGL(gather_kernel<int8_t>, dim3(rows < 65536 ? rows : 65536), dim3(256), 0, s,
                       static_cast<const int8_t*>(src), static_cast<int8_t*>(dst), index, rows,
                       row_bytes);
  }
  return hipGetLastError();
}

hipError_t launch_scatter_sum(const void* src, void* dst, const int32_t* offsets,
                              const int32_t* positions, int64_t rows, int64_t row_elems, int dtype,
                              hipStream_t s) {
  if (rows <= 0 || row_elems <= 0) return hipSuccess;
  const bool al = (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0;
  if (dtype == 0) {
    const __bf16* sp = static_cast<const __bf16*>(src);
    __bf16* dp = static_cast<__bf16*>(dst);
    if (al && row_elems % 8 == 0)
      hipLaunchKernelGGL((scatter_sum_kernel<__bf16, 8>), dim3(scatter_grid(rows, row_elems / 8)),
                         dim3(256), 0, s, sp, dp, offsets, positions, rows, row_elems);
    else
      hipLaunchKernelGGL((scatter_sum_kernel<__bf16, 1>), dim3(scatter_grid(rows, row_elems)),
                         dim3(256), 0, s, sp, dp, offsets, positions, rows, row_elems);
  } else {
    const float* sp = static_cast<const float*>(src);
    float* dp = static_cast<float*>(dst);
    if (al && row_elems % 4 == 0)
      hipLaunchKernelGGL((scatter_sum_kernel<float, 4>), dim3(scatter_grid(rows, row_elems / 4)),
                         dim3(256), 0, s, sp, dp, offsets, positions, rows, row_elems);
    else
      hipLaunchKernelGGL((scatter_sum_kernel<float, 1>), dim3(scatter_grid(rows, row_elems)),
                         dim3(256), 0, s, sp, dp, offsets, positions, rows, row_elems);
  }
  return hipGetLastError();
}

hipError_t launch_rope(void* x, const int32_t* pos, int64_t n_tokens, int heads, int head_dim,
                       double log2_theta, int inverse, int dtype, hipStream_t s) {
  if (n_tokens <= 0 || heads <= 0) return hipSuccess;
  const int half = head_dim / 2;
  const bool vec = half % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
  const dim3 g(grid_for(n_tokens * (vec ? half / 4 : half)));
  if (dtype == 0) {
    __bf16* xp = static_cast<__bf16*>(x);
    if (vec)
      hipLaunchKernelGGL((rope_kernel<__bf16, 4>), g, dim3(256), 0, s, xp, pos, n_tokens, heads,
                         head_dim, log2_theta, inverse);
    else
      hipLaunchKernelGGL((rope_kernel<__bf16, 1>), g, dim3(256), 0, s, xp, pos, n_tokens, heads,
                         head_dim, log2_theta, inverse);
  } else {
    float* xp = static_cast<float*>(x);
    if (vec)
      hipLaunchKernelGGL((rope_kernel<float, 4>), g, dim3(256), 0, s, xp, pos, n_tokens, heads,
                         head_dim, log2_theta, inverse);
    else
      hipLaunchKernelGGL((rope_kernel<float, 1>), g, dim3(256), 0, s, xp, pos, n_tokens, heads,
                         head_dim, log2_theta, inverse);
  }
  return hipGetLastError();
}

}  // namespace tree_attn
