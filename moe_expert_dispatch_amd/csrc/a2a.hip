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
// keep ascending index, so token t's row in rank r's block is r * cap plus
// the number of earlier tokens sent to r. Two launches:
//   1. count  one thread per token, one block per chunk of 256 tokens: the
//             token's mask of destination ranks, and the chunk's count per
//             rank (hist[r * nchunks + c]).
//   2. pack   one block per token: its rows from the counts of the earlier
//             chunks plus the masks of the chunk's earlier tokens (each block
//             derives its own, so no scan launch sits between the two), then
//             the token's routing and hidden row are written to each of its
//             rows. Extra blocks write the rank offsets and mark the unused
//             rows of every block. Each sent row also carries the token's
//             routing so the receiving rank can run its own expert-parallel
//             forward on the block.
#include "common.h"
#include "row_gather.h"

namespace moe {
namespace {

constexpr int kA2aChunk = 256;  // tokens per counting block, one thread each
constexpr int kFillRows = 256;  // send rows per fill-block step

// Ranks owning at least one of token t's valid experts, as a bit mask.
__device__ __forceinline__ uint32_t dest_ranks(const int32_t* __restrict__ ids, int t, int K,
                                               int E_global, int E_local) {
  uint32_t bits = 0;
  for (int k = 0; k < K; ++k) {
    const int e = ids[(size_t)t * K + k];
    if (e >= 0 && e < E_global) bits |= 1u << (e / E_local);
  }
  return bits;
}

__global__ __launch_bounds__(kA2aChunk) void a2a_count_kernel(
    const int32_t* __restrict__ ids, int T, int K, int E_global, int E_local, int R, int nchunks,
    uint32_t* __restrict__ bits, int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[MOE_MAX_A2A_RANKS];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  if (tid < R) cnt[tid] = 0;
  __syncthreads();
  const int t = c * kA2aChunk + tid;
  const uint32_t b = t < T ? dest_ranks(ids, t, K, E_global, E_local) : 0u;
  if (t < T) bits[t] = b;
  for (int r = 0; r < R; ++r) {
    const uint64_t m = __ballot((b >> r) & 1u);
    if (lane_id() == 0 && m != 0) atomicAdd(&cnt[r], __popcll(m));
  }
  __syncthreads();
  if (tid < R) hist[(size_t)tid * nchunks + c] = cnt[tid];
}

// Blocks [0, T): token blockIdx.x. Blocks [T, gridDim.x): rank totals, the
// offsets (first of them) and the unused rows' routing (-1 / 0).
__global__ __launch_bounds__(kA2aChunk) void a2a_pack_kernel(
    const uint4* __restrict__ x, int T, int nvec, const int32_t* __restrict__ ids,
    const float* __restrict__ w, int K, int R, int cap, int nchunks,
    const uint32_t* __restrict__ bits, const int32_t* __restrict__ hist,
    int32_t* __restrict__ offsets, int32_t* __restrict__ token_pos,
    int32_t* __restrict__ send_token, uint4* __restrict__ send_x,
    int32_t* __restrict__ send_ids, float* __restrict__ send_w) {
  __shared__ int32_t cnt[MOE_MAX_A2A_RANKS];
  __shared__ int32_t rows[MOE_MAX_A2A_RANKS];
  const int tid = threadIdx.x;
  if (tid < R) cnt[tid] = 0;
  if ((int)blockIdx.x < T) {
    const int t = blockIdx.x;
    const int c = t / kA2aChunk;
    const int i = t - c * kA2aChunk;
    // the row's first vectors are requested before its destinations are known
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const __amdgpu_buffer_rsrc_t sr = row_rsrc(x + (size_t)t * nvec, row_bytes);
    int32x4_t val[kGatherVec];
    auto load = [&](int v0) {
#pragma unroll
      for (int u = 0; u < kGatherVec; ++u) {
        const int v = v0 + u * kA2aChunk;
        val[u] = __builtin_amdgcn_raw_buffer_load_b128(
            sr, v < nvec ? (uint32_t)v * 16u : row_bytes, 0, 0);
      }
    };
    load(tid);
    // tokens before t sent to each rank: the earlier chunks' counts, then
    // the earlier tokens of this chunk (one per thread)
    const uint32_t bj = tid < i ? bits[(size_t)c * kA2aChunk + tid] : 0u;
    const uint32_t bt = bits[t];
    __syncthreads();
    for (int idx = tid; idx < R * c; idx += kA2aChunk) {
      const int r = idx / c;
      const int v = hist[(size_t)r * nchunks + (idx - r * c)];
      if (v != 0) atomicAdd(&cnt[r], v);
    }
    for (int r = 0; r < R; ++r) {
      const uint64_t m = __ballot((bj >> r) & 1u);
      if (lane_id() == 0 && m != 0) atomicAdd(&cnt[r], __popcll(m));
    }
    __syncthreads();
    if (tid < R) {
      const int row = ((bt >> tid) & 1u) ? tid * cap + cnt[tid] : -1;
      rows[tid] = row;
      token_pos[(size_t)t * R + tid] = row;
      if (row >= 0) send_token[row] = t;
    }
    __syncthreads();
    for (int idx = tid; idx < R * K; idx += kA2aChunk) {
      const int r = idx / K;
      const int k = idx - r * K;
      const int row = rows[r];
      if (row >= 0) {
        send_ids[(size_t)row * K + k] = ids[(size_t)t * K + k];
        send_w[(size_t)row * K + k] = w[(size_t)t * K + k];
      }
    }
    for (int v0 = tid; v0 < nvec; v0 += kGatherVec * kA2aChunk) {
      if (v0 != tid) load(v0);
      for (int r = 0; r < R; ++r) {
        const int row = rows[r];
        if (row < 0) continue;  // block-uniform
        const __amdgpu_buffer_rsrc_t dr = row_rsrc(send_x + (size_t)row * nvec, row_bytes);
#pragma unroll
        for (int u = 0; u < kGatherVec; ++u) {
          const int v = v0 + u * kA2aChunk;
          __builtin_amdgcn_raw_buffer_store_b128(
              val[u], dr, v < nvec ? (uint32_t)v * 16u : row_bytes, 0, kNonTemporal);
        }
      }
    }
  } else {
    __syncthreads();
    for (int idx = tid; idx < R * nchunks; idx += kA2aChunk) {
      const int v = hist[idx];
      if (v != 0) atomicAdd(&cnt[idx / nchunks], v);
    }
    __syncthreads();
    const int f = (int)blockIdx.x - T;
    const int F = (int)gridDim.x - T;
    if (f == 0 && tid == 0) {
      int run = 0;
      offsets[0] = 0;
      for (int r = 0; r < R; ++r) {
        run += cnt[r];
        offsets[r + 1] = run;
      }
    }
    const int64_t nrows = (int64_t)R * cap;
    for (int64_t row = (int64_t)f * kFillRows + tid; row < nrows; row += (int64_t)F * kFillRows) {
      const int r = (int)(row / cap);
      if (row - (int64_t)r * cap < cnt[r]) continue;  // a sent token's row
      send_token[row] = -1;
      for (int k = 0; k < K; ++k) {
        send_ids[row * K + k] = -1;
        send_w[row * K + k] = 0.0f;
      }
    }
  }
}

}  // namespace

A2aLayout a2a_layout(int T, int R, int cap) {
  (void)cap;
  A2aLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t nchunks = (size_t)ceil_div(T, kA2aChunk);
  L.bits = take((size_t)T * 4);
  L.hist = take((size_t)R * nchunks * 4);
  L.total = off > 0 ? off : 256;  // nonzero: a size of 0 reports invalid arguments
  return L;
}

moe_status_t launch_a2a_dispatch(const void* x, int elem_bytes, int T, int H, int K,
                                 const int32_t* ids, const float* w, int E_global, int R, int cap,
                                 int32_t* offsets, int32_t* token_pos, int32_t* send_token,
                                 void* send_x, int32_t* send_ids, float* send_w, void* ws,
                                 hipStream_t stream) {
  const A2aLayout L = a2a_layout(T, R, cap);
  char* base = static_cast<char*>(ws);
  uint32_t* bits = reinterpret_cast<uint32_t*>(base + L.bits);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  const int nchunks = ceil_div(T, kA2aChunk);
  if (nchunks > 0)
    a2a_count_kernel<<<nchunks, kA2aChunk, 0, stream>>>(ids, T, K, E_global, E_global / R, R,
                                                        nchunks, bits, hist);
  const int64_t nrows = (int64_t)R * cap;
  const int64_t fsteps = (nrows + kFillRows - 1) / kFillRows;
  const int fill = (int)(fsteps < 1 ? 1 : (fsteps > 256 ? 256 : fsteps));
  a2a_pack_kernel<<<(unsigned)(T + fill), kA2aChunk, 0, stream>>>(
      static_cast<const uint4*>(x), T, H * elem_bytes / 16, ids, w, K, R, cap, nchunks, bits,
      hist, offsets, token_pos, send_token, static_cast<uint4*>(send_x), send_ids, send_w);
  return launch_status();
}

}  // namespace moe
