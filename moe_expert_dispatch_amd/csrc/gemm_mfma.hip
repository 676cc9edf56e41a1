// Grouped GEMMs of the expert MLP on gfx950 matrix cores (MFMA): bf16, and
// FP8 (E4M3) with per-slot scales.
//
// Source: TensorRT-LLM PR #10985 review of torch_moe.py (gated MLP with an
// activation function over stacked per-expert parameters; FP8 variants of the
// quantized MoE ops) and vLLM ep_fused_moe_patch.py docstring (per-expert
// compute that skips experts with no tokens). The gate is SwiGLU,
// silu(z) = z / (1 + exp(-z)).
//
// One persistent launch covers every slot. Rows of slot s are the contiguous
// block a[offsets[s] .. offsets[s+1]) produced by the permutation, so each
// slot is a dense [n_s, Kd] x [Kd, N] product. Work items are
// (row tile, column tile) pairs; the row tiles of all slots are numbered
// through a prefix over ceil(n_s / BM) that every block rebuilds in LDS from
// `offsets`, so slots with no rows produce no items and no host readback of
// the row counts is needed.
//
// Two kernels share the tiling, item order and epilogue math: a
// direct-to-LDS kernel (further below) for K a multiple of 64 (K >= 128),
// and a register-staged kernel for every other K (a multiple of 8).
//
// Tiles: BM = 256 rows x 256 weight rows. Register-staged kernel: BK = 64,
// 256 threads (4 waves in a 2 x 2 layout, 128 x 128 per wave). For the
// gate/up product the 256 weight rows are 128 gate rows and the matching 128
// up rows, so each block produces a 256 x 128 tile of silu(G) * U without
// ever storing G or U. For the down product they are 256 output columns.
// Both operands are
// K-contiguous in HBM and in LDS; LDS rows are 128 bytes with the 16-byte
// chunks XOR-swizzled by (row mod 8), which keeps the MFMA fragment reads
// free of bank conflicts. Two LDS stages: the next K-slice is fetched into
// registers while the current one feeds the MFMAs.
//
// MFMA: v_mfma_f32_32x32x16_bf16 with the weight fragment as the first
// operand and the activation fragment as the second. Lane l supplies 8
// consecutive K values (block l/32 of the 16) of weight row (l mod 32) and of
// token row (l mod 32); the same K block for both operands, so the pairing
// of K values is consistent. Accumulator register v of lane l then holds
// output column 8*(v/4) + 4*(l/32) + (v mod 4) of token row (l mod 32): four
// runs of 4 consecutive columns, stored as 8-byte words. Fragments are
// double-buffered in registers so the LDS reads of the next K-16 step overlap
// the MFMAs of the current one.
//
// Item order: with G blocks (one per CU), round r gives block b the item
// r*G + (b mod 8)*(G/8) + b/8. Blocks b, b+8, ... run on the same XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin), so each XCD works
// on a contiguous run of 32 items per round. Items are numbered in groups of
// GM row tiles x GN column tiles (GN = min(column tiles, 4), GM = 32 / GN),
// so one XCD's 32 concurrent items share GM activation tiles and GN weight
// panels in its L2; partial groups at the row and column ends are numbered
// without holes (item_tile).
#include <type_traits>

#include "common.h"
#include "item_order.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;
constexpr int BK = 64;
constexpr int BROWS = 256;  // weight rows per stage
constexpr int NTHR = 256;
constexpr int XCD_ITEMS = 32;  // concurrent items per XCD per round
constexpr int kGroupCols = 4;  // column tiles per item group (8 row tiles x 4)
constexpr int A_VEC = BM * BK / 8;     // 16-byte vectors per A stage (1024)
constexpr int B_VEC = BROWS * BK / 8;  // 2048
constexpr int STAGE_VEC = A_VEC + B_VEC;

__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

typedef int int32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr uint32_t kOOB = 0x80000000u;  // beyond every resource size used here

// Raw buffer resource over [base, base + bytes): stride 0, gfx9 data format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const int32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// Builds tp[0..S] = prefix over slots of ceil(n_s / BM) in LDS. All NT threads
// of the block must call it (it contains barriers); scratch holds NT ints.
template <int NT>
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int S, int32_t* tp,
                                  int32_t* scratch) {
  const int tid = threadIdx.x;
  const int per = ceil_div(S, NT);
  const int lo = min(tid * per, S);
  const int hi = min(lo + per, S);
  int sum = 0;
  for (int s = lo; s < hi; ++s) sum += ceil_div(offsets[s + 1] - offsets[s], BM);
  scratch[tid] = sum;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += v;
    __syncthreads();
  }
  int run = scratch[tid] - sum;
  for (int s = lo; s < hi; ++s) {
    tp[s] = run;
    run += ceil_div(offsets[s + 1] - offsets[s], BM);
  }
  if (tid == NT - 1) tp[S] = scratch[NT - 1];
  __syncthreads();
}

// Block-uniform values read from LDS or memory are moved to scalar registers,
// so buffer descriptors built from them are known to be uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Largest s in [0, S) with tp[s] <= rt (always a non-empty slot).
__device__ __forceinline__ int find_slot(const int32_t* tp, int S, int rt) {
  int lo = 0, hi = S;  // invariant: tp[lo] <= rt < tp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tp[mid] <= rt) lo = mid; else hi = mid;
  }
  return lo;
}

// OP 0: gate/up + SwiGLU (Kd = H, N = I, weight rows per slot 2I).
// OP 1: down (Kd = I, N = H, weight rows per slot H).
template <int OP>
__global__ __launch_bounds__(NTHR, 1) void grouped_gemm_bf16_kernel(
    const uint4* __restrict__ A, const int32_t* __restrict__ offsets, int S,
    const uint4* __restrict__ W, int N, int Kd, uint16_t* __restrict__ C) {
  __shared__ uint4 smem[2 * STAGE_VEC];
  __shared__ int32_t tp[MOE_MAX_SLOTS + 1];
  __shared__ int32_t scan_scratch[NTHR];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave >> 1;  // 128-row half of the tile
  const int wn = wave & 1;   // 128-weight-row half of the tile
  const int kvec = Kd / 8;   // 16-byte vectors per row
  const size_t w_rows = (OP == 0) ? 2 * (size_t)N : (size_t)N;
  const int BN = (OP == 0) ? BROWS / 2 : BROWS;  // output columns per tile
  const int CT = ceil_div(N, BN);
  const int GN = CT < kGroupCols ? CT : kGroupCols;
  const int GM = XCD_ITEMS / GN;
  const int nk = ceil_div(Kd, BK);

  build_tile_prefix<NTHR>(offsets, S, tp, scan_scratch);
  const int RT = uniform(tp[S]);
  const int total = RT * CT;

  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int first = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  for (int item = first; item < total; item += G) {
    int rt, ct;
    item_tile(item, RT, CT, GM, GN, &rt, &ct);
    const int s = uniform(find_slot(tp, S, rt));
    const int row0 = uniform(offsets[s] + (rt - tp[s]) * BM);
    const int rows = uniform(min(BM, offsets[s + 1] - row0));
    const int col0 = ct * BN;
    const uint4* Ab = A + (size_t)row0 * kvec;
    const uint4* Wb = W + (size_t)s * w_rows * kvec;

    // Global loads are raw buffer loads: every byte offset sits in the 32-bit
    // per-lane offset, so the hardware range check (offset >= the resource's
    // size reads as 0) zero-fills rows past the slot's end; K and column tails
    // use an offset that is always out of range.
    const __amdgpu_buffer_rsrc_t ra_rsrc =
        make_rsrc(Ab, (uint32_t)rows * (uint32_t)Kd * 2u);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        make_rsrc(Wb, (uint32_t)w_rows * (uint32_t)Kd * 2u);
    const uint32_t row_bytes = (uint32_t)Kd * 2u;
    const uint32_t a_vo = (uint32_t)(tid >> 3) * row_bytes + (uint32_t)(tid & 7) * 16u;
    uint32_t b_vo[B_VEC / NTHR];
#pragma unroll
    for (int i = 0; i < B_VEC / NTHR; ++i) {
      const int r = i * (NTHR / 8) + (tid >> 3);
      int j, wrow;
      if (OP == 0) {
        j = col0 + (r & (BROWS / 2 - 1));
        wrow = (r >= BROWS / 2) ? N + j : j;
      } else {
        j = col0 + r;
        wrow = j;
      }
      b_vo[i] = j < N ? (uint32_t)wrow * row_bytes + (uint32_t)(tid & 7) * 16u : kOOB;
    }

    uint4 ra[A_VEC / NTHR], rb[B_VEC / NTHR];
    auto load_stage = [&](int kt) {
      const uint32_t kb = (uint32_t)kt * (BK * 2);
      const bool k_ok = kt * (BK / 8) + (tid & 7) < kvec;
#pragma unroll
      for (int i = 0; i < A_VEC / NTHR; ++i)
        ra[i] = buf_load16(ra_rsrc, k_ok ? a_vo + (uint32_t)i * (NTHR / 8) * row_bytes + kb : kOOB);
#pragma unroll
      for (int i = 0; i < B_VEC / NTHR; ++i)
        rb[i] = buf_load16(rb_rsrc, (k_ok && b_vo[i] != kOOB) ? b_vo[i] + kb : kOOB);
    };
    auto store_stage = [&](int buf) {
      uint4* sa = smem + buf * STAGE_VEC;
      uint4* sb = sa + A_VEC;
#pragma unroll
      for (int i = 0; i < A_VEC / NTHR; ++i) {
        const int idx = i * NTHR + tid;
        sa[swz(idx >> 3, idx & 7)] = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_VEC / NTHR; ++i) {
        const int idx = i * NTHR + tid;
        sb[swz(idx >> 3, idx & 7)] = rb[i];
      }
    };

    // acc[j][i]: weight-row subtile j (32 rows) x activation-row subtile i (32 rows).
    floatx16 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

    // LDS rows read by this lane: activation subtile i and weight subtile j.
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (OP == 0)  // j < 2: gate rows, j >= 2: the matching up rows
        b_row[j] = (j < 2 ? 0 : BROWS / 2) + wn * 64 + (j & 1) * 32 + (lane & 31);
      else
        b_row[j] = wn * 128 + j * 32 + (lane & 31);
    }

    __syncthreads();  // the previous item's readers are done with both buffers
    load_stage(0);
    store_stage(0);
    __syncthreads();

    // One K-step over LDS buffer `cur`; with HAS_NEXT it also fetches K-slice
    // kt+1 from global memory and stores it into the other buffer. The
    // scheduling groups at the end interleave, per K-16 sub-step, the 16 MFMAs
    // with the LDS reads of the next sub-step's fragments, the global loads of
    // the next stage (first sub-step) and its LDS stores (last sub-step).
    auto kstep = [&](int kt, auto has_next) {
      constexpr bool HAS_NEXT = decltype(has_next)::value;
      const int cur = kt & 1;
      const uint4* sa = smem + cur * STAGE_VEC;
      const uint4* sb = sa + A_VEC;
      bf16x8_t fa[2][4], fb[2][4];
      auto load_frags = [&](int kk, int buf) {
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = sa[swz(a_row[i], ch)];
          fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(&v);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = sb[swz(b_row[j], ch)];
          fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(&v);
        }
      };
      load_frags(0, 0);
      if (HAS_NEXT) load_stage(kt + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) load_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i],
                                                                acc[j][i], 0, 0, 0);
      }
      if (HAS_NEXT) store_stage(cur ^ 1);
      // Instruction groups: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read, 0x200 DS write.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // fragments of sub-step 0
#pragma unroll
      for (int x = 0; x < 8; ++x) {                         // sub-step 0
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (HAS_NEXT) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {                        // sub-steps 1 and 2
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {                        // sub-step 3
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (HAS_NEXT) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __syncthreads();
    };
    for (int kt = 0; kt + 1 < nk; ++kt) kstep(kt, std::true_type{});
    kstep(nk - 1, std::false_type{});

    // Epilogue: f32 accumulators -> (SwiGLU) -> bf16, rounded once; each lane
    // stores runs of 4 consecutive columns of one row as 8-byte words.
    uint16_t* Cb = C + (size_t)row0 * N;
    const int cq = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = a_row[i];
      if (r >= rows) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // run of 4 columns: accumulator registers 4g..4g+3
        if (OP == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = col0 + wn * 64 + j * 32 + 8 * g + cq;
            if (col < N) {
              float o[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float gt = acc[j][i][4 * g + v];
                const float up = acc[j + 2][i][4 * g + v];
                o[v] = gt / (1.0f + expf(-gt)) * up;
              }
              *reinterpret_cast<uint2*>(Cb + (size_t)r * N + col) =
                  make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = col0 + wn * 128 + j * 32 + 8 * g + cq;
            if (col < N)
              *reinterpret_cast<uint2*>(Cb + (size_t)r * N + col) =
                  make_uint2(pack_bf16x2(acc[j][i][4 * g], acc[j][i][4 * g + 1]),
                             pack_bf16x2(acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel, used for bf16 when K % 64 == 0 and K >= 128, and for
// every FP8 product (K % 128 == 0, K >= 256). Same tiles, item order and
// SwiGLU as above, with 8 waves (two per SIMD, so each SIMD has two
// instruction streams) in a 2 x 4 layout of 128 x 64 wave tiles, and the
// operands moved by buffer_load_dwordx4 ... lds: no registers hold
// prefetched data. The schedule below is the bf16 one; the FP8 slice
// schedule is described with its fragments further down.
//
// LDS holds two buffers of one 64-wide K-slice each (64 KB: 256 activation
// rows and 256 weight rows of 128 bytes). Chunk c of row r sits at
// c ^ ((r >> 1) & 7), which keeps the 32-row fragment reads free of bank
// conflicts. One DMA instruction fills 1 KB of LDS linearly (lane L writes
// bytes 16L..16L+15), i.e. 8 whole rows, so lane L fetches the global chunk
// that belongs at that position and every request is a full 128-byte line.
//
// The fragment reads are inline ds_read_b128 with explicit lgkmcnt waits, and
// DMA completion uses explicit vmcnt waits: the compiler's own tracking of
// LDS DMA would otherwise drain every pending load before each LDS read. Per
// slice d (buffer d & 1), in four K-16 blocks:
//   blocks 0-2: MFMAs on block kb (fragments in registers), each followed by
//               one LDS read of block kb+1;
//   wait:       block-3 reads complete; this wave's DMA of slice d+1
//               complete (vmcnt 0); workgroup barrier, after which slice d+1
//               is complete for every wave and buffer d & 1 is not read by
//               anyone;
//   block 3:    MFMAs, each with one DMA instruction of slice d+2 (into
//               buffer d & 1) and one LDS read of block 0 of slice d+1.
// Every slice issues the same 8 DMA instructions per wave (slices past the
// end use an out-of-range offset and move nothing), so the vmcnt accounting
// is constant. A bf16 wave with at most 64 real rows runs the same schedule
// with only its first two 32-row fragments (half the MFMAs and reads); a
// wave with none (the lower half of an item of at most 128 rows) only
// issues its DMAs and takes the barriers. The next item's first two slices (only slice 0 for the staged
// bf16 down epilogue, which occupies stage 1) are requested before an item's
// epilogue stores, so their fetch overlaps the epilogue. The wait for slice 0
// is then vmcnt(8): the 8 DMAs of slice 1 are younger, and loads complete in
// order, so whatever the stores do, no DMA of slice 0 can be outstanding.
constexpr int NTHR8 = 512;  // 8 waves: 2 per SIMD
constexpr int WBK = 64;
constexpr int WA_VEC = BM * WBK / 8;                // 2048 vectors: A part of a stage
constexpr int WSTAGE_VEC = (BM + BROWS) * WBK / 8;  // 4096 vectors = 64 KB
constexpr int WSTAGE_BYTES = WSTAGE_VEC * 16;
constexpr int WDMA = 8;  // DMA instructions per wave per slice

__device__ __forceinline__ int wswz(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int OFF>
__device__ __forceinline__ void lds_read16(bf16x8_t& d, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}

template <int OFF>
__device__ __forceinline__ void lds_read16(int32x4_t& d, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}

template <int OFF>
__device__ __forceinline__ void lds_write16(uint32_t addr, int32x4_t v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(OFF));
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}

template <int OP>
constexpr int bfragw_off(int j) {  // byte offset of weight fragment j (0..1) of a wave
  return (OP == 0 ? j * (BROWS / 2) : j * 32) * 128;
}

// bf16 K-loop fragment reads per K-16 block: four row fragments and two
// weight fragments (two and two when the wave computes only its first two
// row fragments). Read order: the first weight fragment, the row fragments,
// the second weight fragment -- the order in which the MFMAs (weight
// fragment j over row fragments i) first need them.
template <int NI>
constexpr int frag_reads() { return NI == 4 ? 6 : 4; }
template <int NI>  // read8 index (0..3 row fragments, 4, 5 weight fragments) of read y
constexpr int frag_read_order(int y) { return y == 0 ? 4 : (y == frag_reads<NI>() - 1 ? 5 : y - 1); }

struct WItem {
  int rows, row0, col0;
  __amdgpu_buffer_rsrc_t ra, rb, rc;
  uint32_t a_off[4], b_off[4];
  float sc;  // FP8: input scale times the slot's weight scale
};

typedef int int32x8_t __attribute__((ext_vector_type(8)));
typedef int int32x2_t __attribute__((ext_vector_type(2)));

// FP8 (E4M3) operands: a 128-wide K-slice is the same 128 bytes per row as a
// 64-wide bf16 slice, so stages, DMA and swizzle are shared; a slice is two
// k-blocks of v_mfma_f32_32x32x64_f8f6f4, each lane holding 32 bytes (two
// 16-byte chunks) of a row.
// XP: the cross-item prefetch (bf16 only; the launcher selects it when the
// number of 64-wide K-slices is even and at least 4). Kept a template
// parameter: one kernel holding both item schedules spills.
template <int OP, bool GATHER, bool FP8, bool XP = false>
__global__ __launch_bounds__(NTHR8, 1) void grouped_gemm_dma_kernel(
    const uint4* __restrict__ A, const int32_t* __restrict__ offsets, int S,
    const uint4* __restrict__ W, int N, int Kd, void* __restrict__ C,
    const int32_t* __restrict__ gather, int topk, int a_rows, float a_scale,
    const float* __restrict__ w_scale, float out_inv) {
  __shared__ uint4 smem[2 * WSTAGE_VEC];
  __shared__ int32_t tp[MOE_MAX_SLOTS + 1];
  __shared__ int32_t scan_scratch[NTHR8];


  const int tid = threadIdx.x;
  const int lane = lane_id();
  // 0..7. bf16 gate/up: in a scalar register, so the DMAs' LDS destinations
  // (M0) are scalar arithmetic (0.7% faster on the redundant-slot layer). The
  // down kernel measured 0.6% slower that way, and the FP8 kernels have no
  // scalar registers to spare (they spill).
  const int wave = (FP8 || OP == 1) ? tid / kWave : uniform(tid / kWave);
  const int wm = uniform(wave >> 2);  // 128-row half of the tile
  const int wn = wave & 3;       // quarter of the weight rows
  const size_t w_rows = (OP == 0) ? 2 * (size_t)N : (size_t)N;
  const int BN = (OP == 0) ? BROWS / 2 : BROWS;
  const int CT = ceil_div(N, BN);
  const int GN = CT < kGroupCols ? CT : kGroupCols;
  const int GM = XCD_ITEMS / GN;
  constexpr int EB = FP8 ? 1 : 2;                       // operand bytes (A and W are uint4*)
  constexpr uint32_t OB = (FP8 && OP == 0) ? 1u : 2u;   // output bytes
  const uint32_t row_bytes = (uint32_t)Kd * EB;
  const int nd = (int)(row_bytes / (WBK * 2));  // K-slices of 128 bytes per row

  build_tile_prefix<NTHR8>(offsets, S, tp, scan_scratch);
  const int RT = uniform(tp[S]);
  const int total = RT * CT;
  const int G = gridDim.x;
  const int b = blockIdx.x;

  const int a_row0 = wm * 128 + (lane & 31);
  const int b_row0 = (OP == 0 ? wn * 32 : wn * 64) + (lane & 31);
  // Lane offsets of K-16 block kb of the lane's first A and B fragment rows.
  uint32_t a_lane[4], b_lane[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    // bf16: the chunk of K-16 block kb. FP8 (kb < 2): the first of the two
    // chunks of K-64 block kb; the second is chunk ^ 1, i.e. offset ^ 16.
    const int ch = FP8 ? 4 * kb + 2 * (lane >> 5) : 2 * kb + (lane >> 5);
    a_lane[kb] = (uint32_t)wswz(a_row0, ch) * 16u;
    b_lane[kb] = WA_VEC * 16u + (uint32_t)wswz(b_row0, ch) * 16u;
  }
  const uint32_t smem_base = lds_addr(smem);

  // gather: the pair indices through a buffer resource (sorted rows only)
  const __amdgpu_buffer_rsrc_t g_rsrc =
      make_rsrc(gather, GATHER ? (uint32_t)a_rows * (uint32_t)topk * 4u : 0u);
  auto next_item = [&](int w, int* rt, int* ct) {
    if (w < total) item_tile(w, RT, CT, GM, GN, rt, ct);
    return w;
  };
  auto setup = [&](int rt, int ct, WItem& x) {
    const int s = uniform(find_slot(tp, S, rt));
    x.row0 = uniform(offsets[s] + (rt - tp[s]) * BM);
    x.rows = uniform(min(BM, offsets[s + 1] - x.row0));
    x.col0 = ct * BN;
    if constexpr (GATHER)
      x.ra = make_rsrc(A, (uint32_t)a_rows * row_bytes);
    else
      x.ra = make_rsrc(A + (size_t)x.row0 * (Kd / (16 / EB)), (uint32_t)x.rows * row_bytes);
    x.rb = make_rsrc(W + (size_t)s * w_rows * (Kd / (16 / EB)), (uint32_t)w_rows * row_bytes);
    x.rc = make_rsrc(static_cast<char*>(C) + (size_t)x.row0 * N * OB,
                     (uint32_t)x.rows * (uint32_t)N * OB);
    if constexpr (FP8) x.sc = a_scale * w_scale[s];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i;  // 8-row block of the stage
      const int r = q * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ ((r >> 1) & 7);
      if constexpr (GATHER)  // pair index via a 32-bit offset (no 64-bit lane addresses);
                             // gather_offsets() turns it into the token row's offset
        x.a_off[i] = r < x.rows ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                      g_rsrc, (uint32_t)(x.row0 + r) * 4u, 0, 0)
                                : kOOB;
      else
        x.a_off[i] = (uint32_t)r * row_bytes + (uint32_t)ch * 16u;
      int j, wrow;
      if (OP == 0) {
        j = x.col0 + (r & (BROWS / 2 - 1));
        wrow = (r >= BROWS / 2) ? N + j : j;
      } else {
        j = x.col0 + r;
        wrow = j;
      }
      uint32_t cb = (uint32_t)ch * 16u;
      // FP8: recomputed per item rather than held in registers across the loop
      if constexpr (FP8) asm volatile("" : "+v"(cb));
      x.b_off[i] = j < N ? (uint32_t)wrow * row_bytes + cb : kOOB;
    }
  };
  // Pair index -> byte offset of its token's row (the index loads were issued
  // by setup, so their latency overlaps whatever ran in between).
  auto gather_offsets = [&](WItem& x) {
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 8 + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        x.a_off[i] = x.a_off[i] != kOOB
                         ? (x.a_off[i] / (uint32_t)topk) * row_bytes + (uint32_t)ch * 16u
                         : kOOB;
      }
    }
  };
  // DMA instruction q (0..7) of slice d into buffer d & 1: 8 rows x 128
  // bytes, i.e. whole cache lines.
  // `chk` false: the caller knows d < nd. An out-of-range row or column
  // offset (kOOB) stays out of range with the slice offset added (every
  // resource is under 2 GiB), so it needs no test of its own.
  auto dma = [&](const WItem& x, int q, int d, bool chk = true) {
    const bool live = !chk || d < nd;
    const uint32_t kb = (uint32_t)d * (WBK * 2);
    uint4* stage = smem + (d & 1) * WSTAGE_VEC;
    if (q < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x.ra, (lds_ptr_t)(stage + (wave * 4 + q) * 64), 16, live ? x.a_off[q] + kb : kOOB, 0,
          0, 0);
    } else {
      const int i = q - 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x.rb, (lds_ptr_t)(stage + WA_VEC + (wave * 4 + i) * 64), 16,
          live ? x.b_off[i] + kb : kOOB, 0, 0, 0);
    }
  };
  auto issue_slice = [&](const WItem& x, int d) {
#pragma unroll
    for (int q = 0; q < WDMA; ++q) dma(x, q, d);
  };
  auto issue_prologue = [&](const WItem& x) {
    issue_slice(x, 0);
    issue_slice(x, 1);
  };

  floatx16 acc[2][4];
  bf16x8_t f0a[4], f0b[2], f1a[4], f1b[2];
  WItem cur;
  auto read8 = [&](int x, bf16x8_t* fa, bf16x8_t* fb, uint32_t aa, uint32_t ba) {
    switch (x) {
      case 0: lds_read16<0 * 4096>(fa[0], aa); break;
      case 1: lds_read16<1 * 4096>(fa[1], aa); break;
      case 2: lds_read16<2 * 4096>(fa[2], aa); break;
      case 3: lds_read16<3 * 4096>(fa[3], aa); break;
      case 4: lds_read16<bfragw_off<OP>(0)>(fb[0], ba); break;
      default: lds_read16<bfragw_off<OP>(1)>(fb[1], ba); break;
    }
  };
  auto wait_frags = [&](bf16x8_t* fa, bf16x8_t* fb) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1]));
  };
  auto mfma1 = [&](int x, const bf16x8_t* fa, const bf16x8_t* fb) {
    const int j = x >> 2, i = x & 3;
    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
  };
  auto mfma1_first = [&](int x, const bf16x8_t* fa, const bf16x8_t* fb) {
    const int j = x >> 2, i = x & 3;
    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], floatx16{}, 0, 0, 0);
  };

  // Epilogue: accumulator groups g and g+1 (4 columns each per lane half) are
  // exchanged between the lane halves, after which lane l holds 8
  // consecutive columns of row l mod 32 (group g for l < 32, g+1 above) and
  // writes them as one 16-byte store.
  auto pack8 = [&](const float* lo, const float* hi) {
    uint32_t x0 = pack_bf16x2(lo[0], lo[1]), x1 = pack_bf16x2(lo[2], lo[3]);
    uint32_t y0 = pack_bf16x2(hi[0], hi[1]), y1 = pack_bf16x2(hi[2], hi[3]);
    const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    return int32x4_t{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
  };
  auto store8 = [&](const WItem& x, uint32_t r, int col, const float* lo, const float* hi) {
    __builtin_amdgcn_raw_buffer_store_b128(
        pack8(lo, hi), x.rc, col < N ? (r * (uint32_t)N + (uint32_t)col) * 2u : kOOB, 0, 0);
  };
  // FP8 output: 4 + 4 codes per lane exchanged like store8, one 8-byte store.
  auto store8q = [&](const WItem& x, uint32_t r, int col, const float* lo, const float* hi) {
    const uint32_t xq = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        lo[2], lo[3], __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false), true);
    const uint32_t yq = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        hi[2], hi[3], __builtin_amdgcn_cvt_pk_fp8_f32(hi[0], hi[1], 0, false), true);
    const auto q = __builtin_amdgcn_permlane32_swap(xq, yq, false, false);
    __builtin_amdgcn_raw_buffer_store_b64(
        int32x2_t{(int)q[0], (int)q[1]}, x.rc,
        col < N ? r * (uint32_t)N + (uint32_t)col : kOOB, 0, 0);
  };
  // bf16 down product: a lane's 16-byte pieces cover 32 bytes of a row per
  // store, so each wave writes its 128 x 64 tile, 64 rows at a time (bf16,
  // rows of 128 bytes, chunk c of row r at c ^ ((r >> 1) & 7)), into its own
  // 8 KB of stage 1, reads it back as 8 rows x 8 chunks per instruction and
  // stores whole 128-byte lines. Reads and writes are conflict-free (each
  // half-wave touches every 16-byte bank group twice). Stage 0 is left to
  // the next item's first K-slice, whose DMA is issued before this epilogue;
  // the caller keeps the DMA of the second slice (into stage 1) behind a
  // barrier until every wave has read its tile.
  // (The FP8 down kernel stores directly: the staging addresses do not fit
  // beside its K-loop's registers without spilling.)
  constexpr bool STAGED = OP == 1 && !FP8;
  // The next item's slice 0 is requested before this item's epilogue stores,
  // except in the gathered bf16 gate/up kernel, whose SwiGLU epilogue has no
  // registers left for it.
  constexpr bool EARLY = !(GATHER && !FP8);
  // xp: the next item's slice 0 (and, except with the staged epilogue,
  // slice 1) was already requested by the last K-slices of this item.
  auto issue_next = [&](const WItem& x, auto before_epilogue, bool xp) {
    if constexpr (decltype(before_epilogue)::value) {
      if constexpr (EARLY) {
        if (!xp) {
          gather_offsets(cur);
          issue_slice(x, 0);
        }
      }
    } else {
      if constexpr (!EARLY) {
        if (!xp) {
          gather_offsets(cur);
          issue_slice(x, 0);
        }
      }
      if (!xp || STAGED) issue_slice(x, 1);
    }
  };
  auto epilogue_down = [&](const WItem& x) {
    // addresses derived per item from the lane index recomputed here (opaque
    // to the compiler), so that neither it nor anything derived from it is
    // held in a register across the K-loop
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const uint32_t eb = smem_base + (uint32_t)WSTAGE_BYTES + (uint32_t)wave * 8192u;
    const uint32_t p = (uint32_t)((ln >> 5) ^ ((ln >> 1) & 7));
    const uint32_t wrow = eb + (uint32_t)(ln & 31) * 128u;
    // instruction t of a half reads its rows 8t .. 8t+7: row 8t + lane/8,
    // chunk lane % 8
    const uint32_t c = (uint32_t)(ln & 7);
    const uint32_t rbase = eb + (uint32_t)(ln >> 3) * 128u;
    const uint32_t ra0 = rbase + ((c ^ (uint32_t)(ln >> 4)) * 16u);
    const uint32_t ra1 = rbase + ((c ^ (uint32_t)(4 | (ln >> 4))) * 16u);
    const int col = x.col0 + wn * 64 + 8 * (int)c;
    const bool col_ok = col < N;
    uint32_t nb = (uint32_t)N * 2u;  // row pitch in bytes, opaque like ln
    asm volatile("" : "+s"(nb));
    // byte offset of row wm*128 + lane/8, column col; +8 rows per instruction
    const uint32_t obase = (uint32_t)(wm * 128 + (ln >> 3)) * nb + (uint32_t)col * 2u;
    auto half = [&](auto hc) {  // accumulator rows 64h .. 64h + 63
      constexpr int h = decltype(hc)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // (g, j) = (0, 0), (2, 0), (0, 1), (2, 1)
        const int g = 2 * (q & 1), j = q >> 1;
        const uint32_t wa = wrow + (((uint32_t)(g + 4 * j) ^ p) * 16u);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * h + ii;
          float o[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) o[v] = acc[j][i][4 * g + v];
          const int32x4_t val = pack8(o, o + 4);
          if (ii == 0)
            lds_write16<0>(wa, val);
          else
            lds_write16<4096>(wa, val);
        }
      }
      // the previous half's reads completed before its stores (wait below),
      // and LDS operations of one wave run in order
      int32x4_t v[8];
      lds_read16<0 * 1024>(v[0], ra0);
      lds_read16<1 * 1024>(v[1], ra1);
      lds_read16<2 * 1024>(v[2], ra0);
      lds_read16<3 * 1024>(v[3], ra1);
      lds_read16<4 * 1024>(v[4], ra0);
      lds_read16<5 * 1024>(v[5], ra1);
      lds_read16<6 * 1024>(v[6], ra0);
      lds_read16<7 * 1024>(v[7], ra1);
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                     "+v"(v[6]), "+v"(v[7]));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(
            v[u], x.rc, col_ok ? obase + (uint32_t)(8 * (8 * h + u)) * nb : kOOB, 0, 0);
    };
    half(std::integral_constant<int, 0>{});
    half(std::integral_constant<int, 1>{});
  };
  auto epilogue = [&](const WItem& x) {
    if constexpr (STAGED) {
      epilogue_down(x);
      return;
    }
    const int ch = 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = (uint32_t)(wm * 128 + i * 32 + (lane & 31));
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        if (OP == 0) {
          float o[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            float gt = acc[0][i][4 * g + v];
            float up = acc[1][i][4 * g + v];
            if constexpr (FP8) {
              gt *= x.sc;
              up *= x.sc;
            }
            o[v] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;  // silu(g) * u
            if constexpr (FP8)  // quantized with the output scale, clamped to +-448
              o[v] = fminf(fmaxf(o[v] * out_inv, -448.0f), 448.0f);
          }
          if constexpr (FP8)
            store8q(x, r, x.col0 + wn * 32 + 8 * g + ch, o, o + 4);
          else
            store8(x, r, x.col0 + wn * 32 + 8 * g + ch, o, o + 4);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float o[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              o[v] = acc[j][i][4 * g + v];
              if constexpr (FP8) o[v] *= x.sc;
            }
            store8(x, r, x.col0 + wn * 64 + j * 32 + 8 * g + ch, o, o + 4);
          }
        }
      }
    }
  };

  // One K-slice d = four K-16 blocks. Block kb+1 is read while block kb
  // is computed; before the last block, this wave's DMA of slice d+1 is
  // waited for and the workgroup synchronises, after which slice d+1 is
  // visible everywhere and buffer d & 1 is no longer read, so the DMA of
  // slice d+2 goes there while block 0 of slice d+1 is read.
  // NI (4 or 2) is the number of the wave's 32-row fragments computed: with
  // at most 64 real rows in the wave's 128, fragments 2 and 3 are padding,
  // so only MFMAs (j, i < 2) run and only their fragments are read; the DMAs
  // and the barrier are the same (two DMAs per MFMA in the last block).
  // Waits until at most N LDS operations are outstanding; the two fragments
  // the next MFMA reads are its operands, so the MFMA cannot move above it.
  auto lgkm_wait = [&](auto nc, bf16x8_t& wb, bf16x8_t& wa) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(wb), "+v"(wa) : "n"(decltype(nc)::value));
  };
  // Block 3 of slice d requests slice fd (d + 2 inside an item; with the
  // cross-item prefetch the next item's slice 0 or 1) into stage fd & 1;
  // `go` converts the next item's gathered row indices first (their loads
  // were drained by this slice's full wait).
  auto dstep = [&](int d, auto first, auto chk, auto nic, int fd, bool go) {
    constexpr int NI = decltype(nic)::value;
    constexpr int NX = NI == 4 ? 8 : 4;  // MFMAs per K-16 block
    constexpr int NR = frag_reads<NI>();  // fragment reads per K-16 block
    // MFMA / fragment index of step y: (j, i) = (x >> 2, x & 3)
    auto xm = [](int y) { return NI == 4 ? y : ((y & 1) | ((y >> 1) << 2)); };
    const uint32_t base = smem_base + (uint32_t)(d & 1) * WSTAGE_BYTES;
    const uint32_t nbase = smem_base + (uint32_t)((d + 1) & 1) * WSTAGE_BYTES;
    // Gate/up, K-16 blocks 0-2: MFMA y on the current fragments, then read y
    // of the next block's fragments. LDS reads complete in order, so before MFMA
    // y < NR - 1 the reads it needs are done once at most NR - 2 are
    // outstanding: this block's y reads plus the previous block's reads that
    // come after the ones MFMA y uses (frag_read_order puts those first).
    auto kblk = [&](bf16x8_t* ca, bf16x8_t* cb, bf16x8_t* na, bf16x8_t* nb, uint32_t ra,
                    uint32_t rb, auto firstc) {
#pragma unroll
      for (int y = 0; y < NX; ++y) {
        const int x = xm(y);
        if (y < NR - 1) lgkm_wait(std::integral_constant<int, NR - 2>{}, cb[x >> 2], ca[x & 3]);
        if constexpr (decltype(firstc)::value)
          mfma1_first(x, ca, cb);
        else
          mfma1(x, ca, cb);
        if (y < NR) read8(frag_read_order<NI>(y), na, nb, ra, rb);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (OP == 0) {
      kblk(f0a, f0b, f1a, f1b, base + a_lane[1], base + b_lane[1], first);
      kblk(f1a, f1b, f0a, f0b, base + a_lane[2], base + b_lane[2], std::false_type{});
      kblk(f0a, f0b, f1a, f1b, base + a_lane[3], base + b_lane[3], std::false_type{});
    } else {
      // down product: reads in MFMA order ahead of each MFMA and one full wait
      // per block (measured 0.7% faster here than the per-MFMA waits)
      auto rd = [](int y) { return NI == 4 ? y < 6 : true; };
      auto oblk = [&](bf16x8_t* ca, bf16x8_t* cb, bf16x8_t* na, bf16x8_t* nb, uint32_t ra,
                      uint32_t rb, auto firstc) {
        wait_frags(ca, cb);
#pragma unroll
        for (int y = 0; y < NX; ++y) {
          if (rd(y)) read8(xm(y), na, nb, ra, rb);
          if constexpr (decltype(firstc)::value)
            mfma1_first(xm(y), ca, cb);
          else
            mfma1(xm(y), ca, cb);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      oblk(f0a, f0b, f1a, f1b, base + a_lane[1], base + b_lane[1], first);
      oblk(f1a, f1b, f0a, f0b, base + a_lane[2], base + b_lane[2], std::false_type{});
      oblk(f0a, f0b, f1a, f1b, base + a_lane[3], base + b_lane[3], std::false_type{});
    }
    // block 3: after this wave's DMA of slice d+1 and the workgroup barrier,
    // slice d+1 is complete and stage d & 1 is read by no one
    wait_frags(f1a, f1b);
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (GATHER) {
      if (go) {
        __builtin_amdgcn_sched_barrier(0);
        gather_offsets(cur);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int y = 0; y < NX; ++y) {
      if constexpr (OP == 0) {
        mfma1(xm(y), f1a, f1b);
        dma(cur, (8 / NX) * y, fd, decltype(chk)::value);
        if constexpr (NX == 4) dma(cur, 2 * y + 1, fd, decltype(chk)::value);
        if (y < NR) read8(frag_read_order<NI>(y), f0a, f0b, nbase + a_lane[0], nbase + b_lane[0]);
      } else {
        dma(cur, (8 / NX) * y, fd, decltype(chk)::value);
        if constexpr (NX == 4) dma(cur, 2 * y + 1, fd, decltype(chk)::value);
        if (NI == 4 ? y < 6 : true) read8(xm(y), f0a, f0b, nbase + a_lane[0], nbase + b_lane[0]);
        mfma1(xm(y), f1a, f1b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // FP8 fragments of one K-64 block, each reloaded right after its last use
  // (double buffering them would not fit the registers). MFMA x (0..7) of a
  // block uses weight fragment j = x >> 2 and row fragment i = x & 3. The
  // next block's fragments are read in the order B0 (after MFMA 3), A0 (after
  // 4), A1 (5), A2 (6), A3 and B1 (7), two 16-byte reads each, so before MFMA
  // x the reads allowed outstanding are 8, 6, 4, 2 for x = 0..3 and 2 (the
  // next block's B0) for x = 4.
  int32x8_t ga[4], gb[2];
  // the two 16-byte halves of a fragment, read into one 8-register tuple
  auto rd32 = [&](int32x8_t& f, uint32_t a0, uint32_t a1, auto offc) {
    constexpr int off = decltype(offc)::value;
    int32x4_t lo, hi;
    lds_read16<off>(lo, a0);
    lds_read16<off>(hi, a1);
    f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto rdf = [&](int f, auto kbc, uint32_t base) {
    constexpr int kb = decltype(kbc)::value;
    const uint32_t a0 = base + a_lane[kb], a1 = base + (a_lane[kb] ^ 16u);
    const uint32_t b0 = base + b_lane[kb], b1 = base + (b_lane[kb] ^ 16u);
    switch (f) {
      case 0: rd32(ga[0], a0, a1, std::integral_constant<int, 0 * 4096>{}); break;
      case 1: rd32(ga[1], a0, a1, std::integral_constant<int, 1 * 4096>{}); break;
      case 2: rd32(ga[2], a0, a1, std::integral_constant<int, 2 * 4096>{}); break;
      case 3: rd32(ga[3], a0, a1, std::integral_constant<int, 3 * 4096>{}); break;
      case 4: rd32(gb[0], b0, b1, std::integral_constant<int, bfragw_off<OP>(0)>{}); break;
      default: rd32(gb[1], b0, b1, std::integral_constant<int, bfragw_off<OP>(1)>{}); break;
    }
  };
  auto wfr = [&](int x, bool last) {  // wait for the fragments MFMA x needs first
    switch (x) {
      case 0: asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(gb[0]), "+v"(ga[0])); break;
      case 1: asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(ga[1])); break;
      case 2: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(ga[2])); break;
      case 3: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(ga[3])); break;
      default:
        if (last)
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(gb[1]));
        else
          asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(gb[1]));
        break;
    }
  };
  auto wait_all8 = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(ga[0]), "+v"(ga[1]), "+v"(ga[2]), "+v"(ga[3]), "+v"(gb[0]), "+v"(gb[1]));
  };
  auto mf8 = [&](int x, auto first) {
    const int j = x >> 2, i = x & 3;
    if constexpr (decltype(first)::value)
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[j], ga[i], floatx16{}, 0, 0, 0,
                                                                  0, 0, 0);
    else
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[j], ga[i], acc[j][i], 0, 0, 0,
                                                                  0, 0, 0);
  };
  // K-64 block kb of slice d. Block 0 reloads block 1 from the same stage.
  // Block 1 first waits for its last fragments, for this wave's DMA of slice
  // d+1 and at the workgroup barrier (after which slice d+1 is complete and
  // stage d & 1 is read by no one); then it reloads block 0 of slice d+1
  // from the other stage and issues the DMA of slice d+2 into stage d & 1,
  // two instructions after each of its last four MFMAs. In the item's last
  // slice (`last`), block 1 reloads and moves nothing.
  auto kblock = [&](int d, auto kbc, auto first, auto lastc) {
    constexpr int kb = decltype(kbc)::value;
    constexpr bool tail = kb == 1 && decltype(lastc)::value;
    const uint32_t base = smem_base + (uint32_t)(d & 1) * WSTAGE_BYTES;
    const uint32_t rb = kb == 0 ? base : smem_base + (uint32_t)((d + 1) & 1) * WSTAGE_BYTES;
    const std::integral_constant<int, kb == 0 ? 1 : 0> rk;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      if (x < 4) wfr(x, false);
      if (x == 4) {
        if constexpr (kb == 1) {
          wfr(4, true);
          vm_wait<0>();
          __builtin_amdgcn_s_barrier();
          if constexpr (!tail) rdf(4, rk, rb);
        } else {
          wfr(4, false);
        }
      }
      mf8(x, first);  // each accumulator is written by one MFMA per block
      if (kb == 0 && x == 3) rdf(4, rk, rb);
      if (!tail && x >= 4) rdf(x - 4, rk, rb);
      if (!tail && x == 7) rdf(5, rk, rb);
      if constexpr (kb == 1 && !tail) {
        if (x >= 4) {
          dma(cur, 2 * (x - 4), d + 2);
          dma(cur, 2 * (x - 4) + 1, d + 2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A slice for waves whose rows are all padding (the lower 128 rows of an
  // item with at most 128 rows): only their share of the operand DMAs and
  // the barrier, no fragment reads or MFMAs.
  auto pass_step = [&](int fd, bool go) {
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (GATHER) {
      if (go) gather_offsets(cur);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) dma(cur, x, fd);
  };

  int rt, ct;
  int item = next_item((G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b, &rt, &ct);
  if (item < total) {
    setup(rt, ct, cur);
    gather_offsets(cur);
    issue_prologue(cur);
  }
  while (item < total) {
    const bool skip = wm == 1 && cur.rows <= BM / 2;
    vm_wait<WDMA>();
    __builtin_amdgcn_s_barrier();
    int nxt = 0;
    WItem done;
    bool has_next = false;
    auto next_setup = [&]() {
      nxt = next_item(item + G, &rt, &ct);
      done = cur;
      has_next = nxt < total;
      if (has_next) setup(rt, ct, cur);
    };
    // Cross-item prefetch (bf16, an even number of K-slices, at least 4):
    // the next item is set up before the second-to-last slice, whose block 3
    // requests the next item's slice 0 into stage 0 instead of an
    // out-of-range slice; the last slice requests its slice 1 into stage 1,
    // except with the staged down epilogue, which needs stage 1 (it is then
    // requested after the epilogue as before). The next item's gathered row
    // indices are converted after the second-to-last slice's full wait.
    constexpr bool xp = XP && !FP8;
    // Without it: with the gather, the next item is set up before the last
    // slice, whose full wait then covers setup's index loads: they have
    // completed before any epilogue store is issued. (A store can complete
    // before an older load, so no wait may count across the stores.) The
    // last slice's DMAs are out of range whatever item they name.
    const int dlast = GATHER ? nd - 1 : nd;
    // The epilogue sits inside the computing branch, so the accumulators are
    // not live across the pass-only slices.
    if (!skip) {
      if constexpr (FP8) {
        const std::integral_constant<int, 0> k0;
        const std::integral_constant<int, 1> k1;
        // block 0 of slice 0, in the order the waits assume
        rdf(4, k0, smem_base);
#pragma unroll
        for (int f = 0; f < 4; ++f) rdf(f, k0, smem_base);
        rdf(5, k0, smem_base);
        const std::false_type no;
        kblock(0, k0, std::true_type{}, no);
        kblock(0, k1, no, no);
        for (int d = 1; d < nd - 1; ++d) {
          kblock(d, k0, no, no);
          kblock(d, k1, no, no);
        }
        kblock(nd - 1, k0, no, no);
        kblock(nd - 1, k1, no, std::true_type{});
        vm_wait<0>();
        wait_all8();
      } else {
        const std::true_type checked;
        const std::false_type unchecked;
        const std::false_type later;
        auto kloop = [&](auto nic) {
          constexpr int NI = decltype(nic)::value;
          if constexpr (NI == 2) {  // padding rows: defined, never stored
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[j][2] = acc[j][3] = floatx16{};
            f0a[2] = f0a[3] = f1a[2] = f1a[3] = bf16x8_t{};
          }
#pragma unroll
          for (int y = 0; y < frag_reads<NI>(); ++y) {
            // gate/up: the order its per-MFMA waits assume; down: MFMA order
            const int x = OP == 0 ? frag_read_order<NI>(y)
                                  : (NI == 4 ? y : ((y & 1) | ((y >> 1) << 2)));
            read8(x, f0a, f0b, smem_base + a_lane[0], smem_base + b_lane[0]);
          }
          dstep(0, std::true_type{}, checked, nic, 2, false);
          // the DMA of slice d + 2 is in range for d < nd - 2
          int d = 1;
          if constexpr (xp) {
            for (; d < nd - 2; ++d) dstep(d, later, unchecked, nic, d + 2, false);
            next_setup();
            dstep(nd - 2, later, checked, nic, has_next ? 0 : nd, has_next);
            dstep(nd - 1, later, checked, nic, has_next && !STAGED ? 1 : nd + 1, false);
          } else {
            for (; d < dlast && d < nd - 2; ++d) dstep(d, later, unchecked, nic, d + 2, false);
            for (; d < dlast; ++d) dstep(d, later, checked, nic, d + 2, false);
            if constexpr (GATHER) {
              next_setup();
              dstep(nd - 1, later, checked, nic, nd + 1, false);
            }
          }
        };
        // at most 64 real rows in this wave's 128: fragments 2 and 3 are padding
        if (cur.rows - wm * 128 <= 64)
          kloop(std::integral_constant<int, 2>{});
        else
          kloop(std::integral_constant<int, 4>{});
        // with the prefetch (no staged epilogue) the next item's slice 1
        // stays in flight through the epilogue
        if (!xp || STAGED) vm_wait<0>();
        wait_frags(f0a, f0b);
      }
      __builtin_amdgcn_s_barrier();
      if constexpr (!GATHER) {
        if (!xp) next_setup();
      } else if constexpr (FP8) {
        // FP8 fragments leave no registers for setup inside the K-loop: the
        // next item is set up here and its index loads drained before any
        // epilogue store.
        next_setup();
        vm_wait<0>();
      }
      if (has_next) issue_next(cur, std::true_type{}, xp);
      epilogue(done);
      // staged down: every wave has read its tile before slice 1 enters stage 1
      if constexpr (STAGED) __builtin_amdgcn_s_barrier();
    } else {
      if constexpr (xp) {
        for (int d = 0; d < nd - 2; ++d) pass_step(d + 2, false);
        next_setup();
        pass_step(has_next ? 0 : nd, has_next);
        pass_step(has_next && !STAGED ? 1 : nd + 1, false);
        if (STAGED) vm_wait<0>();
      } else {
        for (int d = 0; d < dlast; ++d) pass_step(d + 2, false);
        if constexpr (GATHER) {
          next_setup();
          pass_step(nd + 1, false);
        }
        vm_wait<0>();
      }
      __builtin_amdgcn_s_barrier();
      if constexpr (!GATHER) {
        if (!xp) next_setup();
      }
      if (has_next) issue_next(cur, std::true_type{}, xp);
      if constexpr (STAGED) __builtin_amdgcn_s_barrier();  // the computing waves' second one
    }
    if (has_next) issue_next(cur, std::false_type{}, xp);
    item = nxt;
  }
  vm_wait<0>();
}

}  // namespace

namespace {

int gemm_grid(int max_rows, int S, int N, int BN, int max_blocks) {
  // Upper bound on items: sum_s ceil(n_s/BM) <= ceil(max_rows/BM) + min(S, max_rows),
  // plus the holes of partial item groups.
  const long long max_items =
      (long long)(ceil_div(max_rows, BM) + (S < max_rows ? S : max_rows) + XCD_ITEMS) *
      (ceil_div(N, BN) + 8);
  int G = device_cu_count();
  if (max_blocks > 0 && max_blocks < G) G = max_blocks;
  return max_items < G ? (int)max_items : G;
}

// The direct-to-LDS kernel needs whole 64-wide K-slices, at least two.
bool dma_ok(int Kd) { return Kd % WBK == 0 && Kd >= 2 * WBK; }
// The cross-item prefetch: an even number of K-slices (the next item's first
// two slices land in the stages the current item's last two would use), at
// least four.
bool xp_ok(int Kd) { return (Kd / WBK) % 2 == 0 && Kd / WBK >= 4; }

}  // namespace

moe_status_t launch_gemm_bf16(moe_gemm_op_t op, const void* a, const int32_t* offsets, int S,
                              int max_rows, const void* w, int H, int I, void* c,
                              hipStream_t stream, int max_blocks) {
  if (max_rows == 0) return MOE_OK;
  const int N = (op == MOE_GEMM_GATE_UP_SWIGLU) ? I : H;
  const int Kd = (op == MOE_GEMM_GATE_UP_SWIGLU) ? H : I;
  const int BN = (op == MOE_GEMM_GATE_UP_SWIGLU) ? BROWS / 2 : BROWS;
  const int G = gemm_grid(max_rows, S, N, BN, max_blocks);
  const uint4* a4 = static_cast<const uint4*>(a);
  const uint4* w4 = static_cast<const uint4*>(w);
  uint16_t* c16 = static_cast<uint16_t*>(c);
  const bool dma = dma_ok(Kd);
  const bool xp = dma && xp_ok(Kd);
  if (op == MOE_GEMM_GATE_UP_SWIGLU) {
    if (xp)
      grouped_gemm_dma_kernel<0, false, false, true><<<G, NTHR8, 0, stream>>>(
          a4, offsets, S, w4, N, Kd, c16, nullptr, 1, 0, 1.0f, nullptr, 1.0f);
    else if (dma)
      grouped_gemm_dma_kernel<0, false, false><<<G, NTHR8, 0, stream>>>(
          a4, offsets, S, w4, N, Kd, c16, nullptr, 1, 0, 1.0f, nullptr, 1.0f);
    else
      grouped_gemm_bf16_kernel<0><<<G, NTHR, 0, stream>>>(a4, offsets, S, w4, N, Kd, c16);
  } else {
    if (xp)
      grouped_gemm_dma_kernel<1, false, false, true><<<G, NTHR8, 0, stream>>>(
          a4, offsets, S, w4, N, Kd, c16, nullptr, 1, 0, 1.0f, nullptr, 1.0f);
    else if (dma)
      grouped_gemm_dma_kernel<1, false, false><<<G, NTHR8, 0, stream>>>(
          a4, offsets, S, w4, N, Kd, c16, nullptr, 1, 0, 1.0f, nullptr, 1.0f);
    else
      grouped_gemm_bf16_kernel<1><<<G, NTHR, 0, stream>>>(a4, offsets, S, w4, N, Kd, c16);
  }
  return launch_status();
}

bool gemm_bf16_gather_ok(int T, int H) {
  // Every byte offset into x, plus the out-of-range marker, fits 32 bits.
  return dma_ok(H) && (size_t)T * (size_t)H * 2u < (size_t)kOOB;
}

moe_status_t launch_gemm_bf16_gate_up_gathered(const void* x, int T, int K,
                                               const int32_t* sorted_pairs,
                                               const int32_t* offsets, int S, int max_rows,
                                               const void* w, int H, int I, void* c,
                                               hipStream_t stream, int max_blocks) {
  if (!gemm_bf16_gather_ok(T, H)) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  const int G = gemm_grid(max_rows, S, I, BROWS / 2, max_blocks);
  if (xp_ok(H))
    grouped_gemm_dma_kernel<0, true, false, true><<<G, NTHR8, 0, stream>>>(
        static_cast<const uint4*>(x), offsets, S, static_cast<const uint4*>(w), I, H, c,
        sorted_pairs, K, T, 1.0f, nullptr, 1.0f);
  else
    grouped_gemm_dma_kernel<0, true, false><<<G, NTHR8, 0, stream>>>(
        static_cast<const uint4*>(x), offsets, S, static_cast<const uint4*>(w), I, H, c,
        sorted_pairs, K, T, 1.0f, nullptr, 1.0f);
  return launch_status();
}

// ---------------------------------------------------------------- FP8
bool gemm_fp8_ok(int Kd) { return Kd % (2 * WBK) == 0 && Kd >= 4 * WBK; }

bool gemm_fp8_gather_ok(int T, int H) {
  return gemm_fp8_ok(H) && (size_t)T * (size_t)H < (size_t)kOOB;
}

moe_status_t launch_gemm_fp8(moe_gemm_op_t op, const uint8_t* a, float a_scale,
                             const int32_t* offsets, int S, int max_rows, const uint8_t* w,
                             const float* w_scale, int H, int I, void* c, float out_scale,
                             hipStream_t stream, int max_blocks) {
  const bool gu = op == MOE_GEMM_GATE_UP_SWIGLU;
  const int N = gu ? I : H;
  const int Kd = gu ? H : I;
  if (!gemm_fp8_ok(Kd)) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  const int G = gemm_grid(max_rows, S, N, gu ? BROWS / 2 : BROWS, max_blocks);
  const uint4* a4 = reinterpret_cast<const uint4*>(a);
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  if (gu)
    grouped_gemm_dma_kernel<0, false, true><<<G, NTHR8, 0, stream>>>(
        a4, offsets, S, w4, N, Kd, c, nullptr, 1, 0, a_scale, w_scale, 1.0f / out_scale);
  else
    grouped_gemm_dma_kernel<1, false, true><<<G, NTHR8, 0, stream>>>(
        a4, offsets, S, w4, N, Kd, c, nullptr, 1, 0, a_scale, w_scale, 1.0f);
  return launch_status();
}

moe_status_t launch_gemm_fp8_gate_up_gathered(const uint8_t* xq, int T, int K,
                                              const int32_t* sorted_pairs,
                                              const int32_t* offsets, int S, int max_rows,
                                              const uint8_t* w, const float* w_scale,
                                              float a_scale, int H, int I, void* c,
                                              float out_scale, hipStream_t stream,
                                              int max_blocks) {
  if (!gemm_fp8_gather_ok(T, H)) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  const int G = gemm_grid(max_rows, S, I, BROWS / 2, max_blocks);
  grouped_gemm_dma_kernel<0, true, true><<<G, NTHR8, 0, stream>>>(
      reinterpret_cast<const uint4*>(xq), offsets, S, reinterpret_cast<const uint4*>(w), I, H,
      c, sorted_pairs, K, T, a_scale, w_scale, 1.0f / out_scale);
  return launch_status();
}

}  // namespace moe
