// Row copies of the permutation and of the all-to-all dispatch: a token's
// hidden row, loaded once, stored to every row it occupies in a permuted
// buffer. Internal to the HIP sources.
#pragma once

#include "common.h"

namespace moe {
namespace {

typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): an offset at or past the end
// reads zeros and drops stores, so vector tails need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The permuted rows are written once and read by a later kernel, long after
// they would have left the caches, so their stores carry the non-temporal
// policy (bit 1 of the cache-policy operand, NT on gfx950). Measured on
// 16384 tokens x 8 rows of 8 KB scattered in random order: 235 us with the
// default policy, 209 us non-temporal (non-temporal loads of x as well: 252).
constexpr int kNonTemporal = 2;
constexpr int kGatherVec = 2;  // 16-byte vectors per thread loaded before the stores

// Input-side routing: the row of pair (t, k) is x[t] scaled by the pair's
// weight, w * x evaluated in f32 and rounded once to the element type.
__device__ __forceinline__ int32x4_t scale_row(int32x4_t v, float s, const uint16_t*) {
  int32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t q = (uint32_t)v[i];
    o[i] = (int)pack_bf16x2(bf16_to_f32(q & 0xffffu) * s, bf16_to_f32(q >> 16) * s);
  }
  return o;
}

__device__ __forceinline__ int32x4_t scale_row(int32x4_t v, float s, const float*) {
  int32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_int(__int_as_float(v[i]) * s);
  return o;
}

// One block per token: the token's row is loaded once (kGatherVec vectors
// per thread, all in flight), then stored to each included pair's row.
// scale_row (above) gives input-side routing its weighted rows.
template <bool SCALED, typename ET>
__device__ __forceinline__ void gather_rows(const uint4* __restrict__ src, int nvec, int K,
                                            const int32_t* rows, const float* ws,
                                            uint4* __restrict__ x_perm) {
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  const __amdgpu_buffer_rsrc_t sr = row_rsrc(src, row_bytes);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kGatherVec * blockDim.x) {
    int32x4_t val[kGatherVec];
#pragma unroll
    for (int u = 0; u < kGatherVec; ++u) {
      const int v = v0 + u * blockDim.x;
      val[u] = __builtin_amdgcn_raw_buffer_load_b128(sr, v < nvec ? (uint32_t)v * 16u : row_bytes,
                                                     0, 0);
    }
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r < 0) continue;  // block-uniform
      const __amdgpu_buffer_rsrc_t dr = row_rsrc(x_perm + (size_t)r * nvec, row_bytes);
#pragma unroll
      for (int u = 0; u < kGatherVec; ++u) {
        const int v = v0 + u * blockDim.x;
        int32x4_t o = val[u];
        if constexpr (SCALED) o = scale_row(o, ws[k], (const ET*)nullptr);
        __builtin_amdgcn_raw_buffer_store_b128(
            o, dr, v < nvec ? (uint32_t)v * 16u : row_bytes, 0, kNonTemporal);
      }
    }
  }
}

}  // namespace
}  // namespace moe
