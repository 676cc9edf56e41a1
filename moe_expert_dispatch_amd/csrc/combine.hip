// Weighted combine of the expert outputs back into token order.
//
// Source: DeepSpeed PR #6964 "AutoTP for MoE models" (the routed output is
// the weighted sum of the selected experts' outputs, formed before the one
// reduction of the layer) and TensorRT-LLM PR #10985 review of torch_moe.py
// (_template_moe applies the routing weights on the output side).
//
// Token-major: one block per token reads the token's K (row, weight) pairs,
// gathers the included expert-output rows with 16-byte loads, accumulates in
// f32 in ascending k with fused multiply-adds and writes the token's output
// row once. Every output element is written by exactly one thread, so the
// result does not depend on scheduling.
#include "common.h"

namespace moe {
namespace {

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

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ w_masked, int K,
                                                      int H, OT* __restrict__ out,
                                                      int accumulate) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  __shared__ float wts[MOE_MAX_TOPK];
  if (threadIdx.x < K) {
    rows[threadIdx.x] = pair_row[(size_t)t * K + threadIdx.x];
    wts[threadIdx.x] = w_masked[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  const int nvec = H / 8;
  OT* o = out + (size_t)t * H;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r < 0) continue;
      const float wk = wts[k];
      float yv[8];
      load8(y + (size_t)r * H + v * 8, yv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wk, yv[i], acc[i]);
    }
    if (accumulate) {
      float prev[8];
      load8(o + v * 8, prev);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = prev[i] + acc[i];
    }
    store8(o + v * 8, acc);
  }
}

template <typename YT, typename OT>
void launch_typed(const void* y, const int32_t* pair_row, const float* w_masked, int T, int K,
                  int H, void* out, int accumulate, hipStream_t stream) {
  combine_kernel<YT, OT><<<T, 256, 0, stream>>>(static_cast<const YT*>(y), pair_row, w_masked,
                                                K, H, static_cast<OT*>(out), accumulate);
}

}  // namespace

moe_status_t launch_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                            const float* w_masked, int T, int K, int H, void* out,
                            moe_dtype_t out_dt, int accumulate, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const bool yb = y_dt == MOE_DTYPE_BF16;
  const bool ob = out_dt == MOE_DTYPE_BF16;
  if (yb && ob)
    launch_typed<uint16_t, uint16_t>(y, pair_row, w_masked, T, K, H, out, accumulate, stream);
  else if (yb)
    launch_typed<uint16_t, float>(y, pair_row, w_masked, T, K, H, out, accumulate, stream);
  else if (ob)
    launch_typed<float, uint16_t>(y, pair_row, w_masked, T, K, H, out, accumulate, stream);
  else
    launch_typed<float, float>(y, pair_row, w_masked, T, K, H, out, accumulate, stream);
  return launch_status();
}

}  // namespace moe
