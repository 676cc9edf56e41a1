// Weighted combine of the expert outputs back into token order.
//
// Source: DeepSpeed PR #6964 "AutoTP for MoE models" (the routed output is
// the weighted sum of the selected experts' outputs, formed before the one
// reduction of the layer) and TensorRT-LLM PR #10985 review of torch_moe.py
// (_template_moe applies the routing weights on the output side).
//
// Token-major: one block per token reads the token's K (row, weight) pairs
// (weight 1 for every pair when no weights are given; with a shared-expert
// output, [EPMASK] ep_reduce_output's out = routed_out + shared_out, its row
// is added to the sum before the single rounding),
// gathers the included expert-output rows with 16-byte loads, accumulates in
// f32 in ascending k with fused multiply-adds and writes the token's output
// row once. Every output element is written by exactly one thread, so the
// result does not depend on scheduling.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

typedef int int32x4_t __attribute__((ext_vector_type(4)));
constexpr int kNonTemporal = 2;

// Buffer resource over one row of Y: [row, row + bytes). A resource of 0
// bytes (an excluded pair) makes every load return zeros without a memory
// access, so the loads need no branch.
//
// Y is read exactly once, so its loads carry the non-temporal cache policy
// (bit 1 of the buffer instruction's cache-policy operand, NT on gfx950):
// streamed rows do not displace other lines from L2. Measured on 1.07 GB of
// rows gathered in random order: 5.0 TB/s with the default policy, 5.8 TB/s
// non-temporal, against 6.4 TB/s for a plain sequential read of the same
// bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint16_t*,
                                      float* v) {
  const int32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32((uint32_t)q[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32((uint32_t)q[i] >> 16);
  }
}

__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, uint32_t off, const float*,
                                      float* v) {
  const int32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
  const int32x4_t b =
      __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16u), 0, kNonTemporal);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __int_as_float(a[i]);
    v[4 + i] = __int_as_float(b[i]);
  }
}

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 q;
  q.x = pack_bf16x2(v[0], v[1]);
  q.y = pack_bf16x2(v[2], v[3]);
  q.z = pack_bf16x2(v[4], v[5]);
  q.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = q;
}

__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One block per token. Each thread owns kVec vectors of 8 elements. The K
// row loads of both vectors are issued before any arithmetic (each through
// a resource over its own row, empty for an excluded pair), which keeps
// KMAX * kVec loads in flight per thread; the included pairs are then added in
// ascending k.
template <typename YT, typename OT, int KMAX, int kVec>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ w_masked, int K,
                                                      int H, OT* __restrict__ out,
                                                      int accumulate,
                                                      const void* __restrict__ shared,
                                                      int shared_bf16) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  __shared__ float wts[MOE_MAX_TOPK];
  if (threadIdx.x < K) {
    rows[threadIdx.x] = pair_row[(size_t)t * K + threadIdx.x];
    wts[threadIdx.x] = w_masked != nullptr ? w_masked[(size_t)t * K + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  const int nvec = H / 8;
  const uint32_t row_bytes = (uint32_t)H * (uint32_t)sizeof(YT);
  OT* o = out + (size_t)t * H;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kVec * blockDim.x) {
    float acc[kVec][8];
#pragma unroll
    for (int u = 0; u < kVec; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KMAX) {
      float yv[KMAX][kVec][8];
#pragma unroll
      for (int kk = 0; kk < KMAX; ++kk) {
        const int r = k0 + kk < K ? rows[k0 + kk] : -1;
        const __amdgpu_buffer_rsrc_t rr =
            row_rsrc(y + (size_t)(r >= 0 ? r : 0) * H, r >= 0 ? row_bytes : 0u);
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
          const int v = v0 + u * blockDim.x;
          load8(rr, v < nvec ? (uint32_t)v * 8u * (uint32_t)sizeof(YT) : row_bytes, y,
                yv[kk][u]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < KMAX; ++kk) {
        const int k = k0 + kk;
        if (k < K && rows[k] >= 0) {
          const float wk = wts[k];
#pragma unroll
          for (int u = 0; u < kVec; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(wk, yv[kk][u][i], acc[u][i]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int v = v0 + u * blockDim.x;
      if (v >= nvec) continue;
      if (shared != nullptr) {
        float sv[8];
        if (shared_bf16)
          load8(static_cast<const uint16_t*>(shared) + (size_t)t * H + v * 8, sv);
        else
          load8(static_cast<const float*>(shared) + (size_t)t * H + v * 8, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = acc[u][i] + sv[i];
      }
      if (accumulate) {
        float prev[8];
        load8(o + v * 8, prev);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = prev[i] + acc[u][i];
      }
      store8(o + v * 8, acc[u]);
    }
  }
}

template <typename YT, typename OT, int KMAX, int VEC>
void launch_kv(const void* y, const int32_t* pair_row, const float* w_masked, int T, int K,
               int H, void* out, int accumulate, const void* shared, int shared_bf16,
               hipStream_t stream) {
  // VEC vectors of 8 elements per thread: H / (8 VEC) threads, whole waves,
  // at most 256 (wider rows loop), so narrow rows leave no thread idle and
  // more tokens fit on a CU.
  const int threads = std::min(256, std::max(kWave, ceil_div(H / 8, VEC * kWave) * kWave));
  combine_kernel<YT, OT, KMAX, VEC><<<T, threads, 0, stream>>>(
      static_cast<const YT*>(y), pair_row, w_masked, K, H, static_cast<OT*>(out), accumulate,
      shared, shared_bf16);
}

template <typename YT, typename OT>
void launch_typed(const void* y, const int32_t* pair_row, const float* w_masked, int T, int K,
                  int H, void* out, int accumulate, const void* shared, int shared_bf16,
                  hipStream_t stream) {
  // 32 bytes of each row per thread (two bf16 vectors, one f32 vector);
  // K <= 4 keeps half the rows in flight, in half the registers, so more
  // blocks fit on a compute unit (K = 4 measured 3-6% faster that way)
  const bool k4 = K <= 4;
  const bool v1 = sizeof(YT) == 4;
  if (k4 && v1)
    launch_kv<YT, OT, 4, 1>(y, pair_row, w_masked, T, K, H, out, accumulate, shared,
                            shared_bf16, stream);
  else if (k4)
    launch_kv<YT, OT, 4, 2>(y, pair_row, w_masked, T, K, H, out, accumulate, shared,
                            shared_bf16, stream);
  else if (v1)
    launch_kv<YT, OT, 8, 1>(y, pair_row, w_masked, T, K, H, out, accumulate, shared,
                            shared_bf16, stream);
  else
    launch_kv<YT, OT, 8, 2>(y, pair_row, w_masked, T, K, H, out, accumulate, shared,
                            shared_bf16, stream);
}

}  // namespace

moe_status_t launch_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                            const float* w_masked, int T, int K, int H, void* out,
                            moe_dtype_t out_dt, int accumulate, hipStream_t stream,
                            const void* shared, moe_dtype_t shared_dt) {
  if (T == 0) return MOE_OK;
  const bool yb = y_dt == MOE_DTYPE_BF16;
  const bool ob = out_dt == MOE_DTYPE_BF16;
  const int sb = shared_dt == MOE_DTYPE_BF16 ? 1 : 0;
  if (yb && ob)
    launch_typed<uint16_t, uint16_t>(y, pair_row, w_masked, T, K, H, out, accumulate, shared, sb,
                                     stream);
  else if (yb)
    launch_typed<uint16_t, float>(y, pair_row, w_masked, T, K, H, out, accumulate, shared, sb,
                                  stream);
  else if (ob)
    launch_typed<float, uint16_t>(y, pair_row, w_masked, T, K, H, out, accumulate, shared, sb,
                                  stream);
  else
    launch_typed<float, float>(y, pair_row, w_masked, T, K, H, out, accumulate, shared, sb,
                               stream);
  return launch_status();
}

}  // namespace moe
