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
// Up to 256 experts (K <= 8 or the lane count, no groups) a token gets
// L = 8, 16 or 32 lanes of a wave (at most 8 logits per lane) instead of a
// whole wave: lane q holds experts q, q + L, ..., sorted once in the lane,
// and each round's maximum is the DPP maximum of the lanes' first keys inside
// the group; the lane that held it moves its list up (route_lanes_kernel). Both forms give the same ids; the weights are
// the same softmax with the sums taken in a different order, and moe_route,
// moe_forward and the fused route + slot map of moe_forward all take the
// same form for a given shape, so their bits agree.
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


// Inverse of ordered_bits for non-NaN keys (-0.0 comes back as +0.0, which
// gives the same exponentials).
__device__ __forceinline__ float from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Where the fused router writes the slot map (null slot: route only).
struct MapOut {
  int start, E_local, S;
  const int32_t* rep_off;
  const int32_t* rep_slots;
  int32_t* slot;
  float* w_masked;
  uint8_t* mask;
};

// Sorts n <= 8 keys into descending order with a comparator network
// (Batcher's odd-even merge sort: 1, 5 or 19 compare-exchanges).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[N]) {
  auto cx = [&](int a, int b) {
    const uint64_t hi = k[a] > k[b] ? k[a] : k[b];
    const uint64_t lo = k[a] > k[b] ? k[b] : k[a];
    k[a] = hi;
    k[b] = lo;
  };
  if constexpr (N == 2) {
    cx(0, 1);
  } else if constexpr (N == 4) {
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
  } else if constexpr (N == 8) {
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(1, 2); cx(5, 6);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 2); cx(3, 4); cx(5, 6);
  } else {
    static_assert(N == 1, "1, 2, 4 or 8 keys per lane");
  }
}

// L lanes per token, EPL logits per lane (a power of two); K <= L,
// E <= L * EPL. Lanes of
// tokens past T carry empty keys and store nothing, but stay active, so every
// DPP step reads live lanes.
template <int L, int EPL, bool MAP>
__global__ __launch_bounds__(256) void route_lanes_kernel(const float* __restrict__ logits,
                                                          int T, int E, int K, int renorm,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ w, MapOut mo) {
  const int q = threadIdx.x & (L - 1);
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / L);
  const bool live = t < T;
  const float* row = logits + (size_t)(live ? t : 0) * E;

  float v[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = q + L * j;
    if (live && e < E) {
      v[j] = row[e];
      key[j] = ((uint64_t)ordered_bits(v[j]) << 32) | (0xffffffffu - (uint32_t)e);
    } else {
      v[j] = -INFINITY;
      key[j] = 0;
    }
  }

  // K rounds; lane k of the group keeps the k-th selection's key. The
  // lane's keys are sorted once, so a round's candidate is key[0] and only
  // the lane holding the group's maximum (keys are unique) moves its list up.
  sort_desc<EPL>(key);
  uint64_t my_key = 0;
  uint64_t top = 0;
  for (int k = 0; k < K; ++k) {
    const uint64_t best = group_max_u64<L>(key[0]);
    // all ones in the lane that held it (as a bit mask: one select per word)
    const uint64_t mv = 0ull - (uint64_t)(key[0] == best);
#pragma unroll
    for (int j = 0; j + 1 < EPL; ++j) key[j] = (key[j + 1] & mv) | (key[j] & ~mv);
    key[EPL - 1] &= ~mv;
    if (q == k) my_key = best;
    if (k == 0) top = best;
  }

  // Softmax with the top logit as the shift.
  const float m = from_ordered((uint32_t)(top >> 32));
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (q + L * j < E) part += expf(v[j] - m);
  const float denom = group_sum<L>(part);
  float p = (q < K) ? expf(from_ordered((uint32_t)(my_key >> 32)) - m) / denom : 0.f;
  if (renorm) {
    const float s = group_sum<L>(p);
    p = p / s;
  }
  if (live && q < K) {
    const int id = (int)(0xffffffffu - (uint32_t)my_key);
    const int pi = t * K + q;
    ids[pi] = id;
    w[pi] = p;
    if constexpr (MAP)
      map_pair(pi, t, id, p, mo.start, mo.E_local, mo.rep_off, mo.rep_slots, mo.S, mo.slot,
               mo.w_masked, mo.mask);
  }
}

// G == 0: plain top-K over all experts; otherwise 1 <= TG <= G <= 64, E % G == 0.
// MAP: the slot map of each selected pair as well (as in the lane-group form).
template <int EPL, bool MAP>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int K, int renorm, int G, int TG,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w, MapOut mo) {
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
    int grp[EPL];  // group of each of the lane's experts (-1: none)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      grp[j] = e < E ? e / Eg : -1;
    }
    uint64_t gkey = 0;
    for (int g = 0; g < G; ++g) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if (grp[j] == g) {
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
    for (int j = 0; j < EPL; ++j)
      if (grp[j] >= 0 && !((keep >> grp[j]) & 1ull)) key[j] = 0;
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
      my_logit = from_ordered((uint32_t)(best >> 32));
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
    const int pi = t * K + lane;
    ids[pi] = my_id;
    w[pi] = p;
    if constexpr (MAP)
      map_pair(pi, t, my_id, p, mo.start, mo.E_local, mo.rep_off, mo.rep_slots, mo.S, mo.slot,
               mo.w_masked, mo.mask);
  }
}

// Lanes per token for the grouped-lane router (at most 8 logits per lane and
// K <= L), or 0 where the wave-per-token kernel runs (group-limited routing,
// more than 256 experts, K > 32).
int lanes_for(int E, int K, int G) {
  if (G != 0 || E > 256 || K > 32) return 0;
  if (E <= 64 && K <= 8) return 8;
  if (E <= 128 && K <= 16) return 16;
  return 32;
}

template <int L, bool MAP>
void launch_lanes(const float* logits, int T, int E, int K, int renorm, int32_t* ids, float* w,
                  const MapOut& mo, hipStream_t stream) {
  const int epl = ceil_div(E, L);
  const dim3 grid((unsigned)ceil_div(T, 256 / L));
  if (epl <= 1)
    route_lanes_kernel<L, 1, MAP><<<grid, 256, 0, stream>>>(logits, T, E, K, renorm, ids, w, mo);
  else if (epl <= 2)
    route_lanes_kernel<L, 2, MAP><<<grid, 256, 0, stream>>>(logits, T, E, K, renorm, ids, w, mo);
  else if (epl <= 4)
    route_lanes_kernel<L, 4, MAP><<<grid, 256, 0, stream>>>(logits, T, E, K, renorm, ids, w, mo);
  else
    route_lanes_kernel<L, 8, MAP><<<grid, 256, 0, stream>>>(logits, T, E, K, renorm, ids, w, mo);
}

// One wave per token (group-limited routing, more than 256 experts, K > 32).
template <bool MAP>
void launch_waves(const float* logits, int T, int E, int K, int renorm, int G, int TG,
                  int32_t* ids, float* w, const MapOut& mo, hipStream_t stream) {
  const dim3 block(256);
  const dim3 grid(ceil_div(T, 256 / kWave));
  const int epl = ceil_div(E, kWave);
  if (epl <= 1)
    route_kernel<1, MAP><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w, mo);
  else if (epl <= 2)
    route_kernel<2, MAP><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w, mo);
  else if (epl <= 4)
    route_kernel<4, MAP><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w, mo);
  else if (epl <= 8)
    route_kernel<8, MAP><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w, mo);
  else
    route_kernel<16, MAP><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, G, TG, ids, w,
                                                      mo);
}

template <bool MAP>
void launch_lanes_any(int L, const float* logits, int T, int E, int K, int renorm, int32_t* ids,
                      float* w, const MapOut& mo, hipStream_t stream) {
  if (L == 8)
    launch_lanes<8, MAP>(logits, T, E, K, renorm, ids, w, mo, stream);
  else if (L == 16)
    launch_lanes<16, MAP>(logits, T, E, K, renorm, ids, w, mo, stream);
  else
    launch_lanes<32, MAP>(logits, T, E, K, renorm, ids, w, mo, stream);
}

}  // namespace

moe_status_t launch_route_map(const float* logits, int T, int E, int K, int renorm, int G,
                              int TG, int32_t* ids, float* w, int start, int E_local,
                              const int32_t* rep_off, const int32_t* rep_slots, int S,
                              int32_t* slot, float* w_masked, uint8_t* mask,
                              hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const int L = lanes_for(E, K, G);
  const MapOut mo{start, E_local, S, rep_off, rep_slots, slot, w_masked, mask};
  if (L == 0)
    launch_waves<true>(logits, T, E, K, renorm, G, TG, ids, w, mo, stream);
  else
    launch_lanes_any<true>(L, logits, T, E, K, renorm, ids, w, mo, stream);
  return launch_status();
}

moe_status_t launch_route(const float* logits, int T, int E, int K, int renorm, int G, int TG,
                          int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  if (const int L = lanes_for(E, K, G)) {
    launch_lanes_any<false>(L, logits, T, E, K, renorm, ids, w, MapOut{}, stream);
    return launch_status();
  }
  launch_waves<false>(logits, T, E, K, renorm, G, TG, ids, w, MapOut{}, stream);
  return launch_status();
}

}  // namespace moe
