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
//   2. scan    one block, one pass: exclusive scan of hist in slot-major
//              order, which yields each (slot, chunk) base row;
//              offsets[s] = base of (s, chunk 0) and offsets[S] = P_in.
//   3. scatter one block per chunk: batches of 64 pairs are ranked with a
//              ballot per slot and per-batch counts are scanned in LDS, so
//              the order inside a chunk is the pair order.
//   4. gather  token-major: each token's row is read once and written to
//              the K rows its included pairs occupy (16-byte vectors).
#include <mutex>

#include "common.h"

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

constexpr int kScanThreads = 1024;
constexpr int kScanVec = 16;  // 16-byte vectors per thread: 64 entries, and
                              // S * nchunks <= 65536 (permute_plan)

// Exclusive scan of hist[0..N) in place, N = S * nchunks, in one pass: thread
// t owns the contiguous entries [t * per, (t + 1) * per) (per a multiple of 4,
// at most 64), loads them with up to 16 vector loads all in flight, and one
// block scan of the per-thread sums gives every thread its base. The
// workspace is padded to whole vectors; entries at or past N count as 0 and
// are not written.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ hist, int S,
                                                            int nchunks,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int32_t wsum[kScanThreads / kWave];
  const int N = S * nchunks;
  const int per = 4 * ceil_div(N, 4 * kScanThreads);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int lo = tid * per;
  int4 q[kScanVec];
#pragma unroll
  for (int k = 0; k < kScanVec; ++k) {
    const int i = lo + 4 * k;
    q[k] = (4 * k < per && i < N) ? *reinterpret_cast<const int4*>(hist + i)
                                   : make_int4(0, 0, 0, 0);
  }
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kScanVec; ++k) {
    const int i = lo + 4 * k;
    const bool in = 4 * k < per;
    q[k].x = in && i < N ? q[k].x : 0;
    q[k].y = in && i + 1 < N ? q[k].y : 0;
    q[k].z = in && i + 2 < N ? q[k].z : 0;
    q[k].w = in && i + 3 < N ? q[k].w : 0;
    sum += q[k].x + q[k].y + q[k].z + q[k].w;
  }
  // inclusive scan of the per-thread sums: within the wave, then across waves
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kScanThreads / kWave ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kScanThreads / kWave; off <<= 1) {
      const int o = __shfl_up(w, off, kWave);
      if (lane >= off) w += o;
    }
    if (lane < kScanThreads / kWave) wsum[lane] = w;
  }
  __syncthreads();
  int run = incl - sum + (wave > 0 ? wsum[wave - 1] : 0);
#pragma unroll
  for (int k = 0; k < kScanVec; ++k) {
    const int i = lo + 4 * k;
    if (4 * k < per && i < N) {
      int4 e;
      e.x = run;
      e.y = e.x + q[k].x;
      e.z = e.y + q[k].y;
      e.w = e.z + q[k].z;
      run = e.w + q[k].w;
      if (i + 3 < N) {
        *reinterpret_cast<int4*>(hist + i) = e;
      } else {
        hist[i] = e.x;
        if (i + 1 < N) hist[i + 1] = e.y;
        if (i + 2 < N) hist[i + 2] = e.z;
      }
    }
  }
  __syncthreads();  // the scanned entries are visible to the whole block
  for (int s = tid; s < S; s += kScanThreads)
    offsets[s] = nchunks > 0 ? hist[(size_t)s * nchunks] : 0;
  if (tid == 0) offsets[S] = wsum[kScanThreads / kWave - 1];
}

// One block (4 waves) per chunk. The chunk is walked in sub-chunks of 512
// pairs = 8 batches of 64; wave w ranks batches 2w and 2w+1. Inside a batch the
// lanes holding the same slot are ranked with a ballot (lane order = pair
// order); per-batch slot counts, scanned over the batches, give each batch's
// base row, so the order inside a slot is the pair order.
// seg_cap > 0: slot s's rows start at s * seg_cap instead of offsets[s]
// (fixed-capacity blocks, one per slot).
__device__ __forceinline__ void scatter_chunk(int c, const int32_t* __restrict__ slot,
                                              const uint8_t* __restrict__ mask, int P, int S,
                                              int chunk, int nchunks,
                                              const int32_t* __restrict__ base,
                                              const int32_t* __restrict__ offsets, int seg_cap,
                                              int32_t* __restrict__ sorted_pairs,
                                              int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t lds[];
  int32_t* running = lds;       // [S] next free row per slot
  int32_t* bcount = lds + S;    // [kBatches][S] counts, then base rows
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  for (int i = tid; i < S; i += blockDim.x) running[i] = base[(size_t)i * nchunks + c];
  const int p0 = c * chunk;
  const int p1 = min(p0 + chunk, P);
  for (int q0 = p0; q0 < p1; q0 += kSub) {
    for (int i = tid; i < kBatches * S; i += blockDim.x) bcount[i] = 0;
    __syncthreads();
    constexpr int kPer = kBatches / 4;  // batches per wave
    int s[kPer], rank[kPer];
    bool inc[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int p = q0 + (wave * kPer + m) * kWave + lane;
      s[m] = -1;
      inc[m] = p < p1 && included(slot, mask, p, P, S, &s[m]);
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int b = wave * kPer + m;
      rank[m] = 0;
      uint64_t active = __ballot(inc[m]);
      while (active) {
        const int leader = __ffsll((unsigned long long)active) - 1;
        const int ls = __shfl(s[m], leader, kWave);
        const uint64_t same = __ballot(inc[m] && s[m] == ls);
        if (inc[m] && s[m] == ls) rank[m] = __popcll(same & lanemask_lt());
        if (lane == leader) bcount[b * S + ls] = __popcll(same);
        active &= ~same;
      }
    }
    __syncthreads();
    for (int i = tid; i < S; i += blockDim.x) {
      int run = running[i];
      for (int b = 0; b < kBatches; ++b) {
        const int t = bcount[b * S + i];
        bcount[b * S + i] = run;
        run += t;
      }
      running[i] = run;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int b = wave * kPer + m;
      const int p = q0 + b * kWave + lane;
      if (p < p1) {
        int row = inc[m] ? bcount[b * S + s[m]] + rank[m] : -1;
        if (seg_cap > 0 && row >= 0) row += s[m] * seg_cap - offsets[s[m]];
        pair_row[p] = row;
        if (row >= 0) sorted_pairs[row] = p;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ slot,
                                                      const uint8_t* __restrict__ mask, int P,
                                                      int S, int chunk, int nchunks,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets,
                                                      int seg_cap,
                                                      int32_t* __restrict__ sorted_pairs,
                                                      int32_t* __restrict__ pair_row) {
  scatter_chunk(blockIdx.x, slot, mask, P, S, chunk, nchunks, base, offsets, seg_cap,
                sorted_pairs, pair_row);
}

// The scatter with a quantization riding along: blocks [0, nchunks) scatter
// their chunk, the remaining blocks quantize 16 values per thread. The two
// are independent, so the quantization's HBM traffic overlaps the
// latency-bound scatter instead of following it. The branch is uniform per
// block, so the scatter's barriers are reached by whole blocks.
__global__ __launch_bounds__(256) void scatter_quant_kernel(
    const int32_t* __restrict__ slot, const uint8_t* __restrict__ mask, int P, int S, int chunk,
    int nchunks, const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
    int seg_cap, int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_row,
    FusedQuant fq) {
  if ((int)blockIdx.x < nchunks)
    scatter_chunk(blockIdx.x, slot, mask, P, S, chunk, nchunks, base, offsets, seg_cap,
                  sorted_pairs, pair_row);
  else
    quantize16(fq.x, fq.n, fq.inv, fq.q,
               (int64_t)(blockIdx.x - (unsigned)nchunks) * blockDim.x + threadIdx.x);
}

typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): an offset at or past the end
// reads zeros and drops stores, so vector tails need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The permuted rows are written once and read by a later kernel, long after
// they would have left the caches, so their stores carry the non-temporal
// policy (bit 1 of the cache-policy operand, NT on gfx950). Measured on
// 16384 tokens x 8 rows of 8 KB scattered in random order: 235 us with the
// default policy, 209 us non-temporal (non-temporal loads of x as well: 252).
constexpr int kNonTemporal = 2;
constexpr int kGatherVec = 2;  // 16-byte vectors per thread loaded before the stores

// One block per token: the token's row is loaded once (kGatherVec vectors
// per thread, all in flight), then stored to each included pair's row.
// scale_row (below) gives input-side routing its weighted rows.
template <bool SCALED, typename ET>
__device__ __forceinline__ void gather_rows(const uint4* __restrict__ x, int nvec, int K,
                                            const int32_t* rows, const float* ws,
                                            uint4* __restrict__ x_perm);

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

// Input-side routing: the row of pair (t, k) is x[t] scaled by the pair's
// weight, w * x evaluated in f32 and rounded once to the element type.
__device__ __forceinline__ int32x4_t scale_row(int32x4_t v, float s, const uint16_t*) {
  int32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t q = (uint32_t)v[i];
    o[i] = (int)pack_bf16x2(bf16_to_f32(q & 0xffffu) * s, bf16_to_f32(q >> 16) * s);
  }
  return o;
}

__device__ __forceinline__ int32x4_t scale_row(int32x4_t v, float s, const float*) {
  int32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_int(__int_as_float(v[i]) * s);
  return o;
}

template <bool SCALED, typename ET>
__device__ __forceinline__ void gather_rows(const uint4* __restrict__ src, int nvec, int K,
                                            const int32_t* rows, const float* ws,
                                            uint4* __restrict__ x_perm) {
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  const __amdgpu_buffer_rsrc_t sr = row_rsrc(src, row_bytes);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kGatherVec * blockDim.x) {
    int32x4_t val[kGatherVec];
#pragma unroll
    for (int u = 0; u < kGatherVec; ++u) {
      const int v = v0 + u * blockDim.x;
      val[u] = __builtin_amdgcn_raw_buffer_load_b128(sr, v < nvec ? (uint32_t)v * 16u : row_bytes,
                                                     0, 0);
    }
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r < 0) continue;  // block-uniform
      const __amdgpu_buffer_rsrc_t dr = row_rsrc(x_perm + (size_t)r * nvec, row_bytes);
#pragma unroll
      for (int u = 0; u < kGatherVec; ++u) {
        const int v = v0 + u * blockDim.x;
        int32x4_t o = val[u];
        if constexpr (SCALED) o = scale_row(o, ws[k], (const ET*)nullptr);
        __builtin_amdgcn_raw_buffer_store_b128(
            o, dr, v < nvec ? (uint32_t)v * 16u : row_bytes, 0, kNonTemporal);
      }
    }
  }
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
  // At most max(1, 65536 / S) chunks, so the scan stays small; chunks are
  // whole sub-chunks of 512 pairs.
  const int cap = S > 0 ? (65536 / S > 0 ? 65536 / S : 1) : 1;
  const int units = ceil_div(pl.P, kSub);
  const int n = units < cap ? units : cap;
  pl.chunk = kSub * (n > 0 ? ceil_div(units, n) : 1);
  pl.nchunks = pl.P > 0 ? ceil_div(pl.P, pl.chunk) : 0;
  const int bound = n > 0 ? n : 1;  // min(units, cap), monotone in P
  // histograms, padded to whole 16-byte vectors for the scan
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
                            hipStream_t stream, int seg_cap, const float* pair_w,
                            const FusedQuant* quant) {
  const PermutePlan pl = permute_plan(T, K, S);
  // the one-pass scan covers up to 64 entries per thread
  if ((long long)S * pl.nchunks > (long long)kScanThreads * 4 * kScanVec)
    return MOE_ERR_UNSUPPORTED;
  int32_t* hist = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)S * sizeof(int32_t);
  if (pl.nchunks > 0) {
    count_kernel<<<pl.nchunks, 256, lds, stream>>>(slot, mask, pl.P, S, pl.chunk, pl.nchunks,
                                                  hist);
  }
  scan_kernel<<<1, kScanThreads, 0, stream>>>(hist, S, pl.nchunks, offsets);
  const int64_t qblocks =
      (quant != nullptr && quant->n > 0) ? ((quant->n + 15) / 16 + 255) / 256 : 0;
  if (pl.nchunks > 0 || qblocks > 0) {
    const size_t lds_scatter = (size_t)(1 + kBatches) * S * sizeof(int32_t);
    if (qblocks > 0)
      scatter_quant_kernel<<<(unsigned)(pl.nchunks + qblocks), 256, lds_scatter, stream>>>(
          slot, mask, pl.P, S, pl.chunk, pl.nchunks, hist, offsets, seg_cap, sorted_pairs,
          pair_row, *quant);
    else
      scatter_kernel<<<pl.nchunks, 256, lds_scatter, stream>>>(slot, mask, pl.P, S, pl.chunk,
                                                              pl.nchunks, hist, offsets,
                                                              seg_cap, sorted_pairs, pair_row);
  }
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
