// Quantization to FP8 (E4M3) with one scale per tensor.
//
// Source: TensorRT-LLM PR #10985 "MoE all-to-all paradigm", review of
// torch_moe.py: the FP8 MoE op runs the routed template with quantized
// expert operands. The pages give no scheme; the one implemented (stated
// with moe_quantize_fp8 in moe.h): code = E4M3 value nearest to
// clamp(x * (1 / scale), -448, 448), ties to the even code.
//
// v_cvt_pk_fp8_f32 rounds to nearest even but turns magnitudes past the
// 448 / 480 midpoint into NaN, so every value is clamped first.
#include "common.h"

namespace moe {
namespace {

typedef int int32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// four values -> four codes, first value in the lowest byte
__device__ __forceinline__ uint32_t q4(float a, float b, float c, float d, float inv) {
  const int lo =
      __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a * inv), clamp448(b * inv), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c * inv), clamp448(d * inv), lo,
                                                   true);
}

__device__ __forceinline__ float ld(const uint16_t* x, int64_t i) { return bf16_to_f32(x[i]); }
__device__ __forceinline__ float ld(const float* x, int64_t i) { return x[i]; }

// 16 values per thread: 16-byte loads and one 16-byte store; the last
// partial group (n % 16) element by element.
__device__ __forceinline__ void load16(const uint16_t* x, int64_t i0, float* v) {
  const int32x4_t* p = reinterpret_cast<const int32x4_t*>(x + i0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int32x4_t w = p[h];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * h + 2 * k] = bf16_to_f32((uint32_t)w[k] & 0xffffu);
      v[8 * h + 2 * k + 1] = bf16_to_f32((uint32_t)w[k] >> 16);
    }
  }
}
__device__ __forceinline__ void load16(const float* x, int64_t i0, float* v) {
  const float4* p = reinterpret_cast<const float4*>(x + i0);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 w = p[h];
    v[4 * h] = w.x;
    v[4 * h + 1] = w.y;
    v[4 * h + 2] = w.z;
    v[4 * h + 3] = w.w;
  }
}

template <typename XT>
__global__ __launch_bounds__(256) void quantize_kernel(const XT* __restrict__ x, int64_t n,
                                                       float inv, uint8_t* __restrict__ q) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16;
  if (i0 >= n) return;
  if (i0 + 16 <= n) {
    float v[16];
    load16(x, i0, v);
    int32x4_t out;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = (int)q4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3], inv);
    *reinterpret_cast<int32x4_t*>(q + i0) = out;
  } else {
    for (int64_t i = i0; i < n; ++i)
      q[i] = (uint8_t)(q4(ld(x, i), 0.0f, 0.0f, 0.0f, inv) & 0xffu);
  }
}

}  // namespace

moe_status_t launch_quantize_fp8(const void* x, bool x_bf16, int64_t n, float scale, uint8_t* q,
                                 hipStream_t stream) {
  if (n == 0) return MOE_OK;
  const float inv = 1.0f / scale;
  const int64_t threads = (n + 15) / 16;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (x_bf16)
    quantize_kernel<uint16_t>
        <<<blocks, 256, 0, stream>>>(static_cast<const uint16_t*>(x), n, inv, q);
  else
    quantize_kernel<float><<<blocks, 256, 0, stream>>>(static_cast<const float*>(x), n, inv, q);
  return launch_status();
}

}  // namespace moe
