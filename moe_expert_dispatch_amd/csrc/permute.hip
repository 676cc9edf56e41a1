// Counting-sort permutation of the included (token, slot) pairs by slot, and
// the gather of hidden rows into that order.
//
// Source: vLLM ep_fused_moe_patch.py, module docstring "EP expert dispatch":
// per-expert compute over the tokens routed to each expert, skipping empty
// experts, and the ragged gather that drops non-local pairs before compute.
//
// The result is a pure function of (slot, mask): within a slot, pairs keep
// ascending pair index. Chunks are runs of whole tokens. Two index launches
// and the row gather, all deterministic:
//   1. count   one block per chunk: LDS histogram over slots, written
//              slot-major: hist[s * nchunks + c].
//   2. rank    one block per chunk. The block derives its own base rows from
//              all histograms (slot totals, their exclusive scan over slots,
//              plus the counts of the earlier chunks of each slot; chunk 0
//              also writes offsets), so no separate scan launch sits between
//              the two. Batches of 64 pairs are then ranked with one ballot
//              per bit of the slot id and per-batch counts scanned in LDS,
//              so the order inside a chunk is the pair order.
//   3. gather  token-major, one block per token: the token's row is read
//              once and written to the K rows its included pairs occupy
//              (16-byte vectors). (Folded into the ranking launch, with one
//              block per chunk, it had too few blocks on small layers and
//              was no faster on the largest.)
#include <mutex>

#include "common.h"
#include "row_gather.h"

// Histogram memory of moe_permute_noalloc: one static array per device
// (each GPU the library runs on holds its own copy until the process ends).
// 65536 entries cover every permutation the plan below admits (at most
// 65536 / S chunks of S slots). In host code this name only stands for the
// array: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) int32_t scratch[moe::kPermuteScratchInts];

namespace moe {
namespace {

__device__ __forceinline__ bool included(const int32_t* slot, const uint8_t* mask, int p,
                                         int P, int S, int* s_out) {
  if (p >= P) return false;
  const int s = slot[p];
  *s_out = s;
  return mask[p] != 0 && s >= 0 && s < S;
}

constexpr int kSub = 512;      // pairs per sub-chunk (8 batches of 64, 2 per wave)
constexpr int kBatches = kSub / kWave;

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

constexpr int kRankThreads = 512;  // 8 waves: one batch of 64 pairs each per sub-chunk
constexpr int kRankWaves = kRankThreads / kWave;
static_assert(kBatches == kRankWaves, "one batch per wave");
// Histogram rows a wave sums at a time, and 64-entry column blocks of each:
// all kBaseRows * kBaseCols loads in flight. Four rows keep the ranking at 49
// registers, so it leaves room for the quantization blocks that share its
// launch (sixteen rows: 157 registers, three waves per SIMD, and the FP8
// permute stage 25-30% slower); the ranking alone is no slower for it.
constexpr int kBaseRows = 4;
constexpr int kBaseCols = 4;

// Base rows of chunk c, from the per-chunk histograms hist[s * nchunks + j]
// (counts): tot[s] = sum over j of hist[s][j], pre[s] = sum over j < c;
// the slot's first row is the exclusive scan of tot over slots.
// running[s] = first row + pre[s].
// Chunk 0 writes offsets[s] (the scan) and offsets[S] (all included pairs).
// tot and wsum are LDS scratch ([S], [kRankWaves]).
__device__ __forceinline__ void chunk_bases(const int32_t* __restrict__ hist, int S, int nchunks,
                                            int c, int32_t* running, int32_t* tot,
                                            int32_t* wsum, int32_t* __restrict__ offsets) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  // wave w sums rows s = w, w + 8, ... (kBaseRows rows at a time); lane l
  // reads entries j = l, l + 64, ... of each (kBaseCols per row at a time),
  // so each step has kBaseRows * kBaseCols loads in flight
  const int rows_w = wave < S ? ceil_div(S - wave, kRankWaves) : 0;
  for (int r0 = 0; r0 < rows_w; r0 += kBaseRows) {
    int tsum[kBaseRows], psum[kBaseRows];
#pragma unroll
    for (int i = 0; i < kBaseRows; ++i) tsum[i] = psum[i] = 0;
    for (int j0 = 0; j0 < nchunks; j0 += kBaseCols * kWave) {
      int v[kBaseRows][kBaseCols];
#pragma unroll
      for (int i = 0; i < kBaseRows; ++i) {
        const int srow = wave + kRankWaves * (r0 + i);
#pragma unroll
        for (int m = 0; m < kBaseCols; ++m) {
          const int j = j0 + m * kWave + lane;
          v[i][m] = (r0 + i < rows_w && j < nchunks) ? hist[(size_t)srow * nchunks + j] : 0;
        }
      }
#pragma unroll
      for (int i = 0; i < kBaseRows; ++i) {
#pragma unroll
        for (int m = 0; m < kBaseCols; ++m) {
          tsum[i] += v[i][m];
          psum[i] += j0 + m * kWave + lane < c ? v[i][m] : 0;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBaseRows; ++i) {
      const int t = wave_sum_i32(tsum[i]);
      const int q = wave_sum_i32(psum[i]);
      if (lane == 0 && r0 + i < rows_w) {
        const int srow = wave + kRankWaves * (r0 + i);
        tot[srow] = t;
        running[srow] = q;
      }
    }
  }
  __syncthreads();
  // exclusive scan of tot over the slots: thread t owns slots 2t, 2t + 1
  // (S <= 1024 = 2 * kRankThreads)
  const int a = 2 * tid < S ? tot[2 * tid] : 0;
  const int b = 2 * tid + 1 < S ? tot[2 * tid + 1] : 0;
  int incl = a + b;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kRankWaves; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  const int first = before + incl - (a + b);  // first row of slot 2t
  if (2 * tid < S) {
    running[2 * tid] += first;
    if (c == 0) offsets[2 * tid] = first;
  }
  if (2 * tid + 1 < S) {
    running[2 * tid + 1] += first + a;
    if (c == 0) offsets[2 * tid + 1] = first + a;
  }
  if (c == 0 && tid == 0) offsets[S] = total;
  __syncthreads();
}

// Ranking and scatter of chunk c (one block of kRankThreads). The chunk is
// walked in sub-chunks of 512 pairs = 8 batches of 64, one per wave. Inside a
// batch a lane's rank is the number of lower lanes holding the same slot
// (lane order = pair order), found from one ballot per bit of the slot id;
// per-batch slot counts, scanned over the batches, give each batch's base
// row, so the order inside a slot is the pair order.
__device__ __forceinline__ void rank_chunk(int c, const int32_t* __restrict__ slot,
                                           const uint8_t* __restrict__ mask, int P, int S,
                                           int chunk, int nchunks,
                                           const int32_t* __restrict__ hist,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ sorted_pairs,
                                           int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t lds[];
  int32_t* running = lds;            // [S] next free row per slot
  int32_t* tot = lds + S;            // [S] slot totals (base computation)
  int32_t* bcount = lds + 2 * S;     // [kBatches][S] counts, then base rows
  int32_t* wsum = lds + (2 + kBatches) * S;  // [kRankWaves]
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int p0 = c * chunk;
  const int p1 = min(p0 + chunk, P);
  const int sbits = S > 1 ? 32 - __clz(S - 1) : 0;  // bits of the largest slot id
  // the first sub-chunk's pairs are loaded before the bases are summed, so
  // the two memory round trips overlap
  int s_first = -1;
  const bool inc_first =
      p0 + wave * kWave + lane < p1 && included(slot, mask, p0 + wave * kWave + lane, P, S, &s_first);
  chunk_bases(hist, S, nchunks, c, running, tot, wsum, offsets);
  for (int q0 = p0; q0 < p1; q0 += kSub) {
    for (int i = tid; i < kBatches * S; i += kRankThreads) bcount[i] = 0;
    __syncthreads();
    const int b = wave;  // this wave's batch
    const int p = q0 + b * kWave + lane;
    int s = s_first;
    const bool inc = q0 == p0 ? inc_first : p < p1 && included(slot, mask, p, P, S, &s);
    // Lanes holding the same slot: the included lanes whose slot id agrees
    // with this lane's in every bit, one ballot per bit of S - 1 (no loop
    // over the batch's distinct slots, no cross-lane reads).
    uint64_t same = __ballot(inc);
    for (int bit = 0; bit < sbits; ++bit) {
      const bool on = (s >> bit) & 1;
      const uint64_t ones = __ballot(inc && on);
      same &= on ? ones : ~ones;
    }
    const uint64_t below = same & lanemask_lt();
    const int rank = __popcll(below);
    if (inc && below == 0) bcount[b * S + s] = __popcll(same);  // first lane of its slot
    __syncthreads();
    for (int i = tid; i < S; i += kRankThreads) {
      int run = running[i];
      for (int bb = 0; bb < kBatches; ++bb) {
        const int t = bcount[bb * S + i];
        bcount[bb * S + i] = run;
        run += t;
      }
      running[i] = run;
    }
    __syncthreads();
    if (p < p1) {
      const int row = inc ? bcount[b * S + s] + rank : -1;
      pair_row[p] = row;
      if (row >= 0) sorted_pairs[row] = p;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kRankThreads) void rank_kernel(
    const int32_t* __restrict__ slot, const uint8_t* __restrict__ mask, int P, int S, int chunk,
    int nchunks, const int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_row) {
  rank_chunk(blockIdx.x, slot, mask, P, S, chunk, nchunks, hist, offsets, sorted_pairs,
             pair_row);
}

// The ranking with a quantization riding along: blocks [0, rblocks) rank
// their chunk, the remaining blocks quantize 16 values per thread. The two
// are independent, so the quantization's HBM traffic overlaps the
// latency-bound ranking instead of following it. The branch is uniform per
// block, so the ranking's barriers are reached by whole blocks.
__global__ __launch_bounds__(kRankThreads) void rank_quant_kernel(
    const int32_t* __restrict__ slot, const uint8_t* __restrict__ mask, int P, int S, int chunk,
    int nchunks, int rblocks, const int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_row,
    FusedQuant fq) {
  if ((int)blockIdx.x < rblocks)
    rank_chunk(blockIdx.x, slot, mask, P, S, chunk, nchunks, hist, offsets,
               sorted_pairs, pair_row);
  else
    quantize16(fq.x, fq.n, fq.inv, fq.q,
               (int64_t)(blockIdx.x - (unsigned)rblocks) * blockDim.x + threadIdx.x);
}

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x, int T,
                                                     int nvec, int K,
                                                     const int32_t* __restrict__ pair_row,
                                                     uint4* __restrict__ x_perm) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  if (threadIdx.x < K) rows[threadIdx.x] = pair_row[(size_t)t * K + threadIdx.x];
  __syncthreads();
  gather_rows<false, uint16_t>(x + (size_t)t * nvec, nvec, K, rows, nullptr, x_perm);
}

template <typename ET>
__global__ __launch_bounds__(256) void gather_scaled_kernel(const uint4* __restrict__ x, int T,
                                                            int nvec, int K,
                                                            const int32_t* __restrict__ pair_row,
                                                            const float* __restrict__ pair_w,
                                                            uint4* __restrict__ x_perm) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  __shared__ float ws[MOE_MAX_TOPK];
  if (threadIdx.x < K) {
    rows[threadIdx.x] = pair_row[(size_t)t * K + threadIdx.x];
    ws[threadIdx.x] = pair_w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  gather_rows<true, ET>(x + (size_t)t * nvec, nvec, K, rows, ws, x_perm);
}

}  // namespace

PermutePlan permute_plan(int T, int K, int S) {
  PermutePlan pl;
  pl.P = T * K;
  // About one chunk per 512 pairs, at most max(1, 65536 / S) chunks (so the
  // histograms stay small: each ranking block reads all of them); a chunk is
  // a run of whole tokens, so the block that ranks it can also gather them.
  const int cap = S > 0 ? (65536 / S > 0 ? 65536 / S : 1) : 1;
  const int units = ceil_div(pl.P, kSub);
  const int n = units < cap ? units : cap;
  const int tokens = n > 0 ? ceil_div(T, n) : 1;  // tokens per chunk
  pl.chunk = tokens * K;
  pl.nchunks = pl.P > 0 ? ceil_div(T, tokens) : 0;  // <= n
  const int bound = n > 0 ? n : 1;  // min(units, cap), monotone in P
  // histograms, padded to whole 16-byte vectors
  pl.ws_bytes = ((size_t)S * (size_t)bound * sizeof(int32_t) + 15) / 16 * 16;
  return pl;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

moe_status_t permute_scratch(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {  // first call on this device: it is current
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe_status_t launch_permute(const void* x, int elem_bytes, int T, int H, int K,
                            const int32_t* slot, const uint8_t* mask, int S, int32_t* offsets,
                            int32_t* sorted_pairs, int32_t* pair_row, void* x_perm, void* ws,
                            hipStream_t stream, const float* pair_w,
                            const FusedQuant* quant) {
  const PermutePlan pl = permute_plan(T, K, S);
  int32_t* hist = static_cast<int32_t*>(ws);
  if (pl.nchunks > 0) {
    count_kernel<<<pl.nchunks, 256, (size_t)S * sizeof(int32_t), stream>>>(
        slot, mask, pl.P, S, pl.chunk, pl.nchunks, hist);
  }
  // at least one ranking block: chunk 0 writes offsets (all zero when empty)
  const int rblocks = pl.nchunks > 0 ? pl.nchunks : 1;
  const size_t lds_rank = ((size_t)(2 + kBatches) * S + kRankWaves) * sizeof(int32_t);
  const int64_t qblocks = (quant != nullptr && quant->n > 0)
                              ? ((quant->n + 15) / 16 + kRankThreads - 1) / kRankThreads
                              : 0;
  if (qblocks > 0)
    rank_quant_kernel<<<(unsigned)(rblocks + qblocks), kRankThreads, lds_rank, stream>>>(
        slot, mask, pl.P, S, pl.chunk, pl.nchunks, rblocks, hist, offsets,
        sorted_pairs, pair_row, *quant);
  else
    rank_kernel<<<rblocks, kRankThreads, lds_rank, stream>>>(slot, mask, pl.P, S, pl.chunk,
                                                             pl.nchunks, hist, offsets,
                                                             sorted_pairs, pair_row);
  if (x_perm != nullptr && T > 0) {
    const int nvec = H * elem_bytes / 16;
    const uint4* x4 = static_cast<const uint4*>(x);
    uint4* xp4 = static_cast<uint4*>(x_perm);
    if (pair_w == nullptr)
      gather_kernel<<<T, 256, 0, stream>>>(x4, T, nvec, K, pair_row, xp4);
    else if (elem_bytes == 2)
      gather_scaled_kernel<uint16_t><<<T, 256, 0, stream>>>(x4, T, nvec, K, pair_row, pair_w,
                                                            xp4);
    else
      gather_scaled_kernel<float><<<T, 256, 0, stream>>>(x4, T, nvec, K, pair_row, pair_w, xp4);
  }
  return launch_status();
}

}  // namespace moe
