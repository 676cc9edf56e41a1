// Grouped f32 GEMMs of the expert MLP (vector FMA, one output per thread).
//
// Same contract as the bf16 MFMA path (TensorRT-LLM PR #10985 review of
// torch_moe.py: gated MLP; SwiGLU gate). gfx950 has no fp32-input MFMA that
// matches f32 accuracy in one pass, and the f32 workload of this layer is
// tiny (a few hundred rows), so a direct dot-product kernel is used: each
// output finds its slot by binary search over `offsets` and reduces along K
// in order with f32 fused multiply-adds.
#include "common.h"

namespace moe {
namespace {

template <int OP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, int S,
    const float* __restrict__ W, int N, int Kd, int max_rows, float* __restrict__ C) {
  const int P_in = min(offsets[S], max_rows);
  const long long total = (long long)P_in * N;
  const size_t w_rows = (OP == 0) ? 2 * (size_t)N : (size_t)N;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int r = (int)(idx / N);
    const int j = (int)(idx - (long long)r * N);
    int lo = 0, hi = S;  // largest s with offsets[s] <= r: a non-empty slot
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= r) lo = mid; else hi = mid;
    }
    const float* a = A + (size_t)r * Kd;
    const float* w0 = W + ((size_t)lo * w_rows + j) * Kd;
    float d0 = 0.f;
    for (int k = 0; k < Kd; ++k) d0 = fmaf(a[k], w0[k], d0);
    float val = d0;
    if (OP == 0) {
      const float* w1 = w0 + (size_t)N * Kd;
      float d1 = 0.f;
      for (int k = 0; k < Kd; ++k) d1 = fmaf(a[k], w1[k], d1);
      val = d0 / (1.0f + expf(-d0)) * d1;
    }
    C[(size_t)r * N + j] = val;
  }
}

}  // namespace

moe_status_t launch_gemm_f32(moe_gemm_op_t op, const void* a, const int32_t* offsets, int S,
                             int max_rows, const void* w, int H, int I, void* c,
                             hipStream_t stream) {
  if (max_rows == 0) return MOE_OK;
  const int N = (op == MOE_GEMM_GATE_UP_SWIGLU) ? I : H;
  const int Kd = (op == MOE_GEMM_GATE_UP_SWIGLU) ? H : I;
  const long long outs = (long long)max_rows * N;
  long long blocks = (outs + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (op == MOE_GEMM_GATE_UP_SWIGLU)
    grouped_gemm_f32_kernel<0><<<(int)blocks, 256, 0, stream>>>(
        static_cast<const float*>(a), offsets, S, static_cast<const float*>(w), N, Kd, max_rows,
        static_cast<float*>(c));
  else
    grouped_gemm_f32_kernel<1><<<(int)blocks, 256, 0, stream>>>(
        static_cast<const float*>(a), offsets, S, static_cast<const float*>(w), N, Kd, max_rows,
        static_cast<float*>(c));
  return launch_status();
}

}  // namespace moe
