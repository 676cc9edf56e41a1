// All-to-all token dispatch of expert parallelism, on one device: the send
// side's packing and the return side's gather-sum.
//
// Source: TensorRT-LLM PR #10985 "MoE all-to-all paradigm", walkthrough
// sequence diagram (tokens are dispatched to the ranks responsible for their
// experts, each rank computes the MoE on its local experts, the results are
// gathered back) and the mapping configuration's max-num-tokens field, which
// sizes the exchange workspace. The expert partition follows vLLM
// ep_fused_moe_patch.py _ep_init (rank r owns [r * E_local, (r+1) * E_local)).
//
// A token goes once to every rank that owns at least one of its experts.
// Rank r's block is rows [r * cap, (r+1) * cap) of the send buffer (cap is
// the max token count, so a block never overflows); inside a block tokens
// keep ascending index. The packing is the counting-sort permutation over
// T x ep_size (token, rank) pseudo-pairs, keyed by rank and laid out in
// fixed-capacity blocks; each sent row also carries the token's routing so
// the receiving rank can run its own expert-parallel forward on the block.
#include "common.h"

namespace moe {
namespace {

// One thread per token: the (token, rank) pseudo-pair t * R + r is included
// iff rank r owns one of the token's valid experts.
__global__ __launch_bounds__(256) void a2a_route_kernel(const int32_t* __restrict__ ids, int T,
                                                        int K, int E_global, int E_local, int R,
                                                        int32_t* __restrict__ pslot,
                                                        uint8_t* __restrict__ pmask) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  uint32_t bits = 0;
  for (int k = 0; k < K; ++k) {
    const int e = ids[(size_t)t * K + k];
    if (e >= 0 && e < E_global) bits |= 1u << (e / E_local);
  }
  for (int r = 0; r < R; ++r) {
    pslot[(size_t)t * R + r] = r;
    pmask[(size_t)t * R + r] = (bits >> r) & 1u;
  }
}

// One thread per (send row, k): the routing of the token in that row, or an
// invalid expert id (-1) and weight 0 for an unused row, so a receiving
// forward over the whole block excludes it. Also writes send_token.
__global__ __launch_bounds__(256) void a2a_routing_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int K, int R, int cap,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ psorted,
    int32_t* __restrict__ send_token, int32_t* __restrict__ send_ids,
    float* __restrict__ send_w) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n = (long long)R * cap * K;
  if (i >= n) return;
  const int row = (int)(i / K);
  const int k = (int)(i - (long long)row * K);
  const int r = row / cap;
  const int used = offsets[r + 1] - offsets[r];
  int t = -1;
  if (row - r * cap < used) t = psorted[row] / R;
  if (k == 0) send_token[row] = t;
  send_ids[i] = t >= 0 ? ids[(size_t)t * K + k] : -1;
  send_w[i] = t >= 0 ? w[(size_t)t * K + k] : 0.0f;
}

}  // namespace

A2aLayout a2a_layout(int T, int R, int cap) {
  A2aLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return o;
  };
  L.pslot = take((size_t)T * R * 4);
  L.pmask = take((size_t)T * R);
  L.psorted = take((size_t)R * cap * 4);
  L.perm_ws = take(permute_plan(T, R, R).ws_bytes);
  L.total = off;
  return L;
}

moe_status_t launch_a2a_dispatch(const void* x, int elem_bytes, int T, int H, int K,
                                 const int32_t* ids, const float* w, int E_global, int R, int cap,
                                 int32_t* offsets, int32_t* token_pos, int32_t* send_token,
                                 void* send_x, int32_t* send_ids, float* send_w, void* ws,
                                 hipStream_t stream) {
  const A2aLayout L = a2a_layout(T, R, cap);
  char* base = static_cast<char*>(ws);
  int32_t* pslot = reinterpret_cast<int32_t*>(base + L.pslot);
  uint8_t* pmask = reinterpret_cast<uint8_t*>(base + L.pmask);
  int32_t* psorted = reinterpret_cast<int32_t*>(base + L.psorted);
  if (T > 0)
    a2a_route_kernel<<<ceil_div(T, 256), 256, 0, stream>>>(ids, T, K, E_global, E_global / R, R,
                                                           pslot, pmask);
  const moe_status_t st =
      launch_permute(x, elem_bytes, T, H, R, pslot, pmask, R, offsets, psorted, token_pos,
                     send_x, base + L.perm_ws, stream, cap);
  if (st != MOE_OK) return st;
  const long long n = (long long)R * cap * K;
  if (n > 0)
    a2a_routing_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
        ids, w, K, R, cap, offsets, psorted, send_token, send_ids, send_w);
  return launch_status();
}

}  // namespace moe
