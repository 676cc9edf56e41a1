// Grouped bf16 GEMMs of the expert MLP on gfx950 matrix cores (MFMA).
//
// Source: TensorRT-LLM PR #10985 review of torch_moe.py (gated MLP with an
// activation function over stacked per-expert parameters) and vLLM
// ep_fused_moe_patch.py docstring (per-expert compute that skips experts with
// no tokens). The gate is SwiGLU, silu(z) = z / (1 + exp(-z)).
//
// One persistent launch covers every slot. Rows of slot s are the contiguous
// block a[offsets[s] .. offsets[s+1]) produced by the permutation, so each
// slot is a dense [n_s, Kd] x [Kd, N] product. Work items are
// (row tile, column tile) pairs; the row tiles of all slots are numbered
// through a prefix over ceil(n_s / BM) that every block rebuilds in LDS from
// `offsets`, so slots with no rows produce no items and no host readback of
// the row counts is needed.
//
// Tiles: BM = 128 rows x 256 weight rows x BK = 64, 256 threads (4 waves in a
// 2 x 2 layout). For the gate/up product the 256 weight rows are 128 gate
// rows and the matching 128 up rows, so each block produces a 128 x 128 tile
// of silu(G) * U without ever storing G or U. For the down product they are
// 256 output columns. Both operands are K-contiguous in HBM and in LDS; LDS
// rows are 128 bytes with the 16-byte chunks XOR-swizzled by (row mod 8) to
// spread MFMA fragment reads over the banks. Two LDS stages: the next
// K-slice is fetched into registers while the current one feeds the MFMAs.
//
// MFMA: v_mfma_f32_16x16x32_bf16. A fragment: lane l holds 8 consecutive K
// values of row (l mod 16); B fragment: 8 K values of weight row (l mod 16),
// the same K block for both operands; the accumulator holds rows
// 4*(l/16) + v, v = 0..3, of column (l mod 16).
//
// Item order: with G blocks (one per CU), round r gives block b the item
// r*G + (b mod 8)*(G/8) + b/8. Blocks b, b+8, ... run on the same XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin), so each XCD works
// on a contiguous run of items: the column tiles of a row tile, which share
// the activation rows, and neighbouring row tiles of one slot, which share
// the weight panel, meet in the same L2.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BK = 64;
constexpr int BROWS = 256;  // weight rows per stage
constexpr int NTHR = 256;
constexpr int A_VEC = BM * BK / 8;     // 16-byte vectors per A stage (1024)
constexpr int B_VEC = BROWS * BK / 8;  // 2048
constexpr int STAGE_VEC = A_VEC + B_VEC;

__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// Builds tp[0..S] = prefix over slots of ceil(n_s / BM) in LDS.
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int S, int32_t* tp,
                                  int32_t* scratch) {
  const int tid = threadIdx.x;
  const int per = ceil_div(S, NTHR);
  const int lo = min(tid * per, S);
  const int hi = min(lo + per, S);
  int sum = 0;
  for (int s = lo; s < hi; ++s) sum += ceil_div(offsets[s + 1] - offsets[s], BM);
  scratch[tid] = sum;
  __syncthreads();
  for (int off = 1; off < NTHR; off <<= 1) {
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
  if (tid == NTHR - 1) tp[S] = scratch[NTHR - 1];
  __syncthreads();
}

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
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int kvec = Kd / 8;                       // 16-byte vectors per row
  const size_t w_rows = (OP == 0) ? 2 * (size_t)N : (size_t)N;
  const int BN = (OP == 0) ? 128 : 256;          // output columns per tile
  const int CT = ceil_div(N, BN);
  const int nk = ceil_div(Kd, BK);

  build_tile_prefix(offsets, S, tp, scan_scratch);
  const int total = tp[S] * CT;

  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int slot_in_round = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  for (int item = slot_in_round; item < total; item += G) {
    const int rt = item / CT;
    const int ct = item - rt * CT;
    const int s = find_slot(tp, S, rt);
    const int row0 = offsets[s] + (rt - tp[s]) * BM;
    const int rows = min(BM, offsets[s + 1] - row0);
    const int col0 = ct * BN;
    const uint4* Ab = A + (size_t)row0 * kvec;
    const uint4* Wb = W + (size_t)s * w_rows * kvec;

    // Per-thread global source rows for this item (fixed across K).
    const uint4* a_src[A_VEC / NTHR];
    bool a_ok[A_VEC / NTHR];
#pragma unroll
    for (int i = 0; i < A_VEC / NTHR; ++i) {
      const int r = (i * NTHR + tid) >> 3;
      a_ok[i] = r < rows;
      a_src[i] = Ab + (size_t)r * kvec + (tid & 7);
    }
    const uint4* b_src[B_VEC / NTHR];
    bool b_ok[B_VEC / NTHR];
#pragma unroll
    for (int i = 0; i < B_VEC / NTHR; ++i) {
      const int r = (i * NTHR + tid) >> 3;
      int j, wrow;
      if (OP == 0) {
        j = col0 + (r & 127);
        wrow = (r >> 7) ? N + j : j;
      } else {
        j = col0 + r;
        wrow = j;
      }
      b_ok[i] = j < N;
      b_src[i] = Wb + (size_t)(b_ok[i] ? wrow : 0) * kvec + (tid & 7);
    }

    uint4 ra[A_VEC / NTHR], rb[B_VEC / NTHR];
    auto load_stage = [&](int kt) {
      const int kv = kt * (BK / 8);
      const bool k_ok = kv + (tid & 7) < kvec;
#pragma unroll
      for (int i = 0; i < A_VEC / NTHR; ++i)
        ra[i] = (a_ok[i] && k_ok) ? a_src[i][kv] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < B_VEC / NTHR; ++i)
        rb[i] = (b_ok[i] && k_ok) ? b_src[i][kv] : make_uint4(0, 0, 0, 0);
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

    floatx4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // previous item's readers are done with both buffers
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load_stage(kt + 1);
      const uint4* sa = smem + cur * STAGE_VEC;
      const uint4* sb = sa + A_VEC;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ch = kk * 4 + (lane >> 4);
        bf16x8_t fa[4], fb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 64 + i * 16 + (lane & 15);
          const uint4 v = sa[swz(r, ch)];
          fa[i] = *reinterpret_cast<const bf16x8_t*>(&v);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          int r;
          if (OP == 0)
            r = (j < 4 ? 0 : 128) + wn * 64 + (j & 3) * 16 + (lane & 15);
          else
            r = wn * 128 + j * 16 + (lane & 15);
          const uint4 v = sb[swz(r, ch)];
          fb[j] = *reinterpret_cast<const bf16x8_t*>(&v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store_stage(cur ^ 1);
      __syncthreads();
    }

    // Epilogue: f32 accumulators -> (SwiGLU) -> bf16, rounded once.
    uint16_t* Cb = C + (size_t)row0 * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + v;
        if (r >= rows) continue;
        if (OP == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = col0 + wn * 64 + j * 16 + (lane & 15);
            if (col < N) {
              const float g = acc[i][j][v];
              const float u = acc[i][j + 4][v];
              const float val = g / (1.0f + expf(-g)) * u;
              Cb[(size_t)r * N + col] = (uint16_t)f32_to_bf16(val);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int col = col0 + wn * 128 + j * 16 + (lane & 15);
            if (col < N) Cb[(size_t)r * N + col] = (uint16_t)f32_to_bf16(acc[i][j][v]);
          }
        }
      }
    }
  }
}

}  // namespace

moe_status_t launch_gemm_bf16(moe_gemm_op_t op, const void* a, const int32_t* offsets, int S,
                              int max_rows, const void* w, int H, int I, void* c,
                              hipStream_t stream) {
  if (max_rows == 0) return MOE_OK;
  const int N = (op == MOE_GEMM_GATE_UP_SWIGLU) ? I : H;
  const int Kd = (op == MOE_GEMM_GATE_UP_SWIGLU) ? H : I;
  const int BN = (op == MOE_GEMM_GATE_UP_SWIGLU) ? 128 : 256;
  // Upper bound on items: sum_s ceil(n_s/BM) <= ceil(max_rows/BM) + min(S, max_rows).
  const long long max_items =
      (long long)(ceil_div(max_rows, BM) + (S < max_rows ? S : max_rows)) * ceil_div(N, BN);
  int G = device_cu_count();
  if (max_items < G) G = (int)max_items;
  if (op == MOE_GEMM_GATE_UP_SWIGLU)
    grouped_gemm_bf16_kernel<0><<<G, NTHR, 0, stream>>>(
        static_cast<const uint4*>(a), offsets, S, static_cast<const uint4*>(w), N, Kd,
        static_cast<uint16_t*>(c));
  else
    grouped_gemm_bf16_kernel<1><<<G, NTHR, 0, stream>>>(
        static_cast<const uint4*>(a), offsets, S, static_cast<const uint4*>(w), N, Kd,
        static_cast<uint16_t*>(c));
  return launch_status();
}

}  // namespace moe
