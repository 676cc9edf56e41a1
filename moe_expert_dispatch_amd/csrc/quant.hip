// Quantization to FP8 (E4M3) with one scale per tensor.
//
// Source: TensorRT-LLM PR #10985 "MoE all-to-all paradigm", review of
// torch_moe.py: the FP8 MoE op runs the routed template with quantized
// expert operands. The pages give no scheme; the one implemented (stated
// with moe_quantize_fp8 in moe.h): code = E4M3 value nearest to
// clamp(x * (1 / scale), -448, 448), ties to the even code.
//
// The per-thread rule (quantize16, with the clamp before gfx950's converter)
// is in common.h: the fused forward also runs it as extra blocks of the
// permutation's scatter launch.
#include "common.h"

namespace moe {
namespace {

template <typename XT>
__global__ __launch_bounds__(256) void quantize_kernel(const XT* __restrict__ x, int64_t n,
                                                       float inv, uint8_t* __restrict__ q) {
  quantize16(x, n, inv, q, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
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
