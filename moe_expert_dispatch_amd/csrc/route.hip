// Router: softmax over the expert logits and top-K selection, one wave per
// token.
//
// Source: vLLM ep_fused_moe_patch.py, module docstring "EP expert dispatch"
// (top-k routing yields the same global expert ids on every rank) and the
// FusedMoE constructor (top_k, renormalize). Selection compares the f32
// logits exactly; ties go to the lower expert id; -0.0 equals +0.0.
//
// Each lane holds E/64 (rounded up) logits in registers. Candidates carry a
// 64-bit key: the logit mapped to an order-preserving unsigned integer in the
// high word and (0xffffffff - id) in the low word, so one unsigned max picks
// the largest logit and, among equal logits, the lowest id. K rounds of a
// wave-wide max select the experts; the winner's owner lane clears its key.
//
// Group-limited routing (the constructor's use_grouped_topk,
// num_expert_group and topk_group, which the pages only name; reading: the
// E experts form G consecutive groups scored by their largest logit): lane g
// gets group g's key (best ordered logit, 0xffffffff - g), topk_group rounds
// of a wave max pick the groups, and the keys of experts outside them are
// cleared before the K rounds. The softmax still runs over all E experts.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks below everything
  if ((u & 0x7fffffffu) == 0u) u = 0u;              // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


// G == 0: plain top-K over all experts; otherwise 1 <= TG <= G <= 64, E % G == 0.
template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int K, int renorm, int G, int TG,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // wave-uniform
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;

  float v[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + kWave * j;
    if (e < E) {
      v[j] = row[e];
      key[j] = ((uint64_t)ordered_bits(v[j]) << 32) | (0xffffffffu - (uint32_t)e);
    } else {
      v[j] = -INFINITY;
      key[j] = 0;  // never selected: every real candidate has a non-zero key
    }
  }

  if (G > 0) {
    const int Eg = E / G;
    uint64_t gkey = 0;
    for (int g = 0; g < G; ++g) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        if (e < E && e / Eg == g) {
          const uint32_t o = (uint32_t)(key[j] >> 32);
          m = o > m ? o : m;
        }
      }
      m = wave_max_u32(m);
      if (lane == g) gkey = ((uint64_t)m << 32) | (0xffffffffu - (uint32_t)g);
    }
    uint64_t keep = 0;  // selected groups, the same in every lane
    for (int r = 0; r < TG; ++r) {
      const uint64_t best = wave_max_u64(gkey);
      const int g = (int)(0xffffffffu - (uint32_t)best);
      keep |= 1ull << g;
      if (lane == g) gkey = 0;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((keep >> (e / Eg)) & 1ull)) key[j] = 0;
    }
  }

  // K rounds of wave max; lane k keeps the k-th selection.
  int my_id = 0;
  float my_logit = 0.f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + kWave * j == e) key[j] = 0;
    if (lane == k) {
      my_id = e;
      my_logit = row[e];
    }
  }

  // Softmax with the top logit as the shift: m = max_e l_e.
  const float m = __shfl(my_logit, 0, kWave);
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + kWave * j < E) part += expf(v[j] - m);
  const float denom = wave_sum(part);
  float p = (lane < K) ? expf(my_logit - m) / denom : 0.f;
  if (renorm) {
    const float s = wave_sum(p);
    p = p / s;
  }
  if (lane < K) {
    ids[(size_t)t * K + lane] = my_id;
    w[(size_t)t * K + lane] = p;
  }
}

}  // namespace

moe_status_t launch_route(const float* logits, int T, int E, int K, int renorm, int G, int TG,
                          int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const dim3 block(256);
  const dim3 grid(ceil_div(T, 256 / kWave));
  const int epl = ceil_div(E, kWave);
  if (epl <= 1)
    route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w);
  else if (epl <= 2)
    route_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w);
  else if (epl <= 4)
    route_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w);
  else if (epl <= 8)
    route_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w);
  else
    route_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w);
  return launch_status();
}

}  // namespace moe
