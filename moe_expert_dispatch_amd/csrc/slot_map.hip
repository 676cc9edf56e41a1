// Expert-parallel mask / remap and expert -> slot lookup, one thread per
// (token, k) pair (the per-pair rule is map_pair in common.h, which the fused
// router of moe_forward applies too).
//
// Source: vLLM ep_fused_moe_patch.py, ep_mask_and_remap (local mask for the
// rank's expert range, weights multiplied by the mask, local id = id - start,
// non-local ids spread by id mod E_local) and _ep_init (start = rank * E_local);
// TensorRT-LLM PR #4495, Description (expert id -> engine-side expert slot).
// The replica of a local expert is chosen by token index: t mod r.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void slot_map_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int P, int K, int start,
    int E_local, const int32_t* __restrict__ rep_off, const int32_t* __restrict__ rep_slots,
    int S, int32_t* __restrict__ slot, float* __restrict__ w_masked,
    uint8_t* __restrict__ mask) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  map_pair(p, p / K, ids[p], w[p], start, E_local, rep_off, rep_slots, S, slot, w_masked, mask);
}

}  // namespace

moe_status_t launch_slot_map(const int32_t* ids, const float* w, int T, int K, int start,
                             int E_local, const int32_t* rep_off, const int32_t* rep_slots,
                             int S, int32_t* slot, float* w_masked, uint8_t* mask,
                             hipStream_t stream) {
  const int P = T * K;
  if (P == 0) return MOE_OK;
  slot_map_kernel<<<ceil_div(P, 256), 256, 0, stream>>>(ids, w, P, K, start, E_local, rep_off,
                                                       rep_slots, S, slot, w_masked, mask);
  return launch_status();
}

}  // namespace moe
