// Counting-sort permutation of the included (token, slot) pairs by slot, and
// the gather of hidden rows into that order.
//
// Source: vLLM ep_fused_moe_patch.py, module docstring "EP expert dispatch":
// per-expert compute over the tokens routed to each expert, skipping empty
// experts, and the ragged gather that drops non-local pairs before compute.
//
// The result is a pure function of (slot, mask): within a slot, pairs keep
// ascending pair index. Four kernels, all deterministic:
//   1. count   one block per chunk of pairs: LDS histogram over slots,
//              written slot-major: hist[s * nchunks + c].
//   2. scan    one block: exclusive scan of hist in slot-major order, which
//              yields each (slot, chunk) base row; offsets[s] = base of
//              (s, chunk 0) and offsets[S] = P_in.
//   3. scatter one wave per chunk walks its pairs in order, 64 at a time;
//              lanes holding the same slot are ranked with a ballot, so the
//              order inside a chunk is the pair order.
//   4. gather  token-major: each token's row is read once and written to
//              the K rows its included pairs occupy (16-byte vectors).
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ bool included(const int32_t* slot, const uint8_t* mask, int p,
                                         int P, int S, int* s_out) {
  if (p >= P) return false;
  const int s = slot[p];
  *s_out = s;
  return mask[p] != 0 && s >= 0 && s < S;
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ slot,
                                                    const uint8_t* __restrict__ mask, int P,
                                                    int S, int chunk, int nchunks,
                                                    int32_t* __restrict__ hist) {
  extern __shared__ int32_t lds_hist[];
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < S; i += blockDim.x) lds_hist[i] = 0;
  __syncthreads();
  const int p0 = c * chunk;
  const int p1 = min(p0 + chunk, P);
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    int s;
    if (included(slot, mask, p, P, S, &s)) atomicAdd(&lds_hist[s], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += blockDim.x) hist[(size_t)i * nchunks + c] = lds_hist[i];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ hist, int S,
                                                            int nchunks,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int32_t partial[kScanThreads];
  const int N = S * nchunks;
  const int tid = threadIdx.x;
  const int seg = ceil_div(N, kScanThreads);
  const int lo = min(tid * seg, N);
  const int hi = min(lo + seg, N);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += hist[i];
  partial[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums.
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = tid >= off ? partial[tid - off] : 0;
    __syncthreads();
    partial[tid] += v;
    __syncthreads();
  }
  int run = partial[tid] - sum;  // exclusive prefix of this segment
  for (int i = lo; i < hi; ++i) {
    const int v = hist[i];
    hist[i] = run;
    run += v;
  }
  __syncthreads();
  const int total = partial[kScanThreads - 1];
  for (int s = tid; s < S; s += kScanThreads)
    offsets[s] = nchunks > 0 ? hist[(size_t)s * nchunks] : 0;
  if (tid == 0) offsets[S] = total;
}

__global__ __launch_bounds__(kWave) void scatter_kernel(const int32_t* __restrict__ slot,
                                                        const uint8_t* __restrict__ mask, int P,
                                                        int S, int chunk, int nchunks,
                                                        const int32_t* __restrict__ base,
                                                        int32_t* __restrict__ sorted_pairs,
                                                        int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t counter[];
  const int c = blockIdx.x;
  const int lane = lane_id();
  for (int i = lane; i < S; i += kWave) counter[i] = base[(size_t)i * nchunks + c];
  __syncthreads();
  const int p0 = c * chunk;
  const int p1 = min(p0 + chunk, P);
  for (int pb = p0; pb < p1; pb += kWave) {
    const int p = pb + lane;
    int s = -1;
    const bool inc = (p < p1) && included(slot, mask, p, P, S, &s);
    int row = -1;
    uint64_t active = __ballot(inc);
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int ls = __shfl(s, leader, kWave);
      const uint64_t same = __ballot(inc && s == ls);
      const int b = counter[ls];
      if (inc && s == ls) row = b + __popcll(same & lanemask_lt());
      if (lane == leader) counter[ls] = b + __popcll(same);
      active &= ~same;
    }
    if (p < p1) {
      pair_row[p] = row;
      if (row >= 0) sorted_pairs[row] = p;
    }
  }
}

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x, int T,
                                                     int nvec, int K,
                                                     const int32_t* __restrict__ pair_row,
                                                     uint4* __restrict__ x_perm) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  if (threadIdx.x < K) rows[threadIdx.x] = pair_row[(size_t)t * K + threadIdx.x];
  __syncthreads();
  const uint4* src = x + (size_t)t * nvec;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    const uint4 val = src[v];
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r >= 0) x_perm[(size_t)r * nvec + v] = val;
    }
  }
}

}  // namespace

PermutePlan permute_plan(int T, int K, int S) {
  PermutePlan pl;
  pl.P = T * K;
  const int cap = S > 0 ? (65536 / S > 0 ? 65536 / S : 1) : 1;
  const int units = ceil_div(pl.P, 256);
  const int n = units < cap ? units : cap;
  pl.chunk = 256 * (n > 0 ? ceil_div(units, n) : 1);
  pl.nchunks = pl.P > 0 ? ceil_div(pl.P, pl.chunk) : 0;
  const int bound = n > 0 ? n : 1;  // min(units, cap), monotone in P
  pl.ws_bytes = (size_t)S * (size_t)bound * sizeof(int32_t);
  return pl;
}

moe_status_t launch_permute(const void* x, int elem_bytes, int T, int H, int K,
                            const int32_t* slot, const uint8_t* mask, int S, int32_t* offsets,
                            int32_t* sorted_pairs, int32_t* pair_row, void* x_perm, void* ws,
                            hipStream_t stream) {
  const PermutePlan pl = permute_plan(T, K, S);
  int32_t* hist = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)S * sizeof(int32_t);
  if (pl.nchunks > 0) {
    count_kernel<<<pl.nchunks, 256, lds, stream>>>(slot, mask, pl.P, S, pl.chunk, pl.nchunks,
                                                  hist);
  }
  scan_kernel<<<1, kScanThreads, 0, stream>>>(hist, S, pl.nchunks, offsets);
  if (pl.nchunks > 0) {
    scatter_kernel<<<pl.nchunks, kWave, lds, stream>>>(slot, mask, pl.P, S, pl.chunk,
                                                      pl.nchunks, hist, sorted_pairs, pair_row);
  }
  if (x_perm != nullptr && T > 0) {
    const int nvec = H * elem_bytes / 16;
    gather_kernel<<<T, 256, 0, stream>>>(static_cast<const uint4*>(x), T, nvec, K, pair_row,
                                         static_cast<uint4*>(x_perm));
  }
  return launch_status();
}

}  // namespace moe
