// Internal helpers shared by the HIP kernels of the fused MoE forward pass
// (gfx950, wave64). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
// bfloat16 is kept as raw uint16 bits: the top half of an IEEE binary32.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (lo in bits 0..15) with gfx950's
// v_cvt_pk_bf16_f32: round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

// Wave-wide reductions without LDS traffic: DPP moves inside each 16-lane
// row (swap lane pairs, swap pairs of pairs, mirror the half rows, mirror
// the row), then the row-pair and half-wave swaps (v_permlane16_swap,
// v_permlane32_swap). Every step combines a lane with exactly one partner
// and every lane ends with the full result; for the sum, each partner pair
// adds the same two values, so all lanes hold bit-identical totals.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppQuad1032 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuad2301 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u32<kDppQuad1032>(v));
  v = mx(v, dpp_u32<kDppQuad2301>(v));
  v = mx(v, dpp_u32<kDppRowHalfMirror>(v));
  v = mx(v, dpp_u32<kDppRowMirror>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // {own, partner}
  v = mx(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return mx(b[0], b[1]);
}

// Integer sum over the wave by the same steps (exact, so every lane holds
// the total).
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += (int)dpp_u32<kDppQuad1032>((uint32_t)v);
  v += (int)dpp_u32<kDppQuad2301>((uint32_t)v);
  v += (int)dpp_u32<kDppRowHalfMirror>((uint32_t)v);
  v += (int)dpp_u32<kDppRowMirror>((uint32_t)v);
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)a[0] + (int)a[1];
  const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)b[0] + (int)b[1];
}

__device__ __forceinline__ float wave_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __uint_as_float(dpp_u32<decltype(ctrl)::value>(__float_as_uint(x)));
  };
  v += dpp(v, std::integral_constant<int, kDppQuad1032>{});
  v += dpp(v, std::integral_constant<int, kDppQuad2301>{});
  v += dpp(v, std::integral_constant<int, kDppRowHalfMirror>{});
  v += dpp(v, std::integral_constant<int, kDppRowMirror>{});
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The same reductions over aligned groups of L = 8, 16 or 32 lanes (the
// first steps only; groups never exchange values): every lane of a group
// ends with the group's result, bit-identical across the group.
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(L == 8 || L == 16 || L == 32, "groups of 8, 16 or 32 lanes");
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u32<kDppQuad1032>(v));
  v = mx(v, dpp_u32<kDppQuad2301>(v));
  v = mx(v, dpp_u32<kDppRowHalfMirror>(v));
  if constexpr (L >= 16) v = mx(v, dpp_u32<kDppRowMirror>(v));
  if constexpr (L == 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = mx(a[0], a[1]);
  }
  return v;
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 8 || L == 16 || L == 32, "groups of 8, 16 or 32 lanes");
  auto dpp = [](float x, auto ctrl) {
    return __uint_as_float(dpp_u32<decltype(ctrl)::value>(__float_as_uint(x)));
  };
  v += dpp(v, std::integral_constant<int, kDppQuad1032>{});
  v += dpp(v, std::integral_constant<int, kDppQuad2301>{});
  v += dpp(v, std::integral_constant<int, kDppRowHalfMirror>{});
  if constexpr (L >= 16) v += dpp(v, std::integral_constant<int, kDppRowMirror>{});
  if constexpr (L == 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  return v;
}

template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  const uint32_t hi = group_max_u32<L>((uint32_t)(v >> 32));
  const uint32_t lo = group_max_u32<L>((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// 64-bit maximum as two 32-bit passes: the high words, then the low words of
// the lanes holding that high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- misc
__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Expert-parallel mask / remap and expert -> slot lookup of one pair p =
// t * K + k with expert e and routing weight wv (vLLM ep_fused_moe_patch.py,
// ep_mask_and_remap: local mask for the rank's range [start, start + E_local),
// weight times the mask, local id e - start, non-local ids spread by
// e mod E_local; TensorRT-LLM PR #4495: expert id -> engine-side slot). The
// replica of a local expert is chosen by token index, t mod r. A null table
// is the identity map; an entry outside [0, S) (or an expert without slots)
// gives slot -1.
__device__ __forceinline__ void map_pair(int p, int t, int e, float wv, int start, int E_local,
                                         const int32_t* __restrict__ rep_off,
                                         const int32_t* __restrict__ rep_slots, int S,
                                         int32_t* __restrict__ slot,
                                         float* __restrict__ w_masked,
                                         uint8_t* __restrict__ mask) {
  const bool local = e >= start && e < start + E_local;
  const int lid = local ? e - start : ((e % E_local) + E_local) % E_local;
  int s = lid;
  if (rep_off != nullptr) {
    const int a = rep_off[lid];
    const int b = rep_off[lid + 1];
    const int r = b - a;
    s = -1;
    if (r > 0 && a >= 0 && b <= S) {
      const int v = rep_slots[a + t % r];
      s = (v >= 0 && v < S) ? v : -1;
    }
  }
  slot[p] = s;
  w_masked[p] = wv * (local ? 1.0f : 0.0f);
  mask[p] = local ? 1 : 0;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline moe_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Number of compute units of the current device (queried on every call).
int device_cu_count();

// A slot's weight panel (the 2I x H gate/up rows, the larger of the two
// matrices) must stay below 2^31 bytes: the GEMMs address it through a
// buffer resource with 32-bit offsets and use 2^31 as their out-of-range
// offset.
inline bool weight_panel_ok(int H, int I, int elem_bytes) {
  return 2ull * (unsigned long long)H * (unsigned long long)I * (unsigned)elem_bytes <
         (1ull << 31);
}

// ---------------------------------------------------------------- FP8
// Quantization to OCP E4M3 with one scale per tensor: code = E4M3 value
// nearest to clamp(x * (1 / scale), -448, 448), ties to the even code.
// v_cvt_pk_fp8_f32 rounds to nearest even but turns magnitudes past the
// 448 / 480 midpoint into NaN, so every value is clamped first.
typedef int fp8_i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fp8_clamp448(float v) {
  return fminf(fmaxf(v, -448.0f), 448.0f);
}

// four values -> four codes, first value in the lowest byte
__device__ __forceinline__ uint32_t fp8_q4(float a, float b, float c, float d, float inv) {
  const int lo =
      __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp448(a * inv), fp8_clamp448(b * inv), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp448(c * inv),
                                                   fp8_clamp448(d * inv), lo, true);
}

__device__ __forceinline__ float fp8_ld(const uint16_t* x, int64_t i) {
  return bf16_to_f32(x[i]);
}
__device__ __forceinline__ float fp8_ld(const float* x, int64_t i) { return x[i]; }

// 16 values per thread: 16-byte loads and one 16-byte store; the last
// partial group (n % 16) element by element.
__device__ __forceinline__ void fp8_load16(const uint16_t* x, int64_t i0, float* v) {
  const fp8_i32x4_t* p = reinterpret_cast<const fp8_i32x4_t*>(x + i0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const fp8_i32x4_t w = p[h];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * h + 2 * k] = bf16_to_f32((uint32_t)w[k] & 0xffffu);
      v[8 * h + 2 * k + 1] = bf16_to_f32((uint32_t)w[k] >> 16);
    }
  }
}
__device__ __forceinline__ void fp8_load16(const float* x, int64_t i0, float* v) {
  const float4* p = reinterpret_cast<const float4*>(x + i0);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 w = p[h];
    v[4 * h] = w.x;
    v[4 * h + 1] = w.y;
    v[4 * h + 2] = w.z;
    v[4 * h + 3] = w.w;
  }
}

// Thread g of a quantization of n values: values [16 g, 16 g + 16).
template <typename XT>
__device__ __forceinline__ void quantize16(const XT* __restrict__ x, int64_t n, float inv,
                                           uint8_t* __restrict__ q, int64_t g) {
  const int64_t i0 = g * 16;
  if (i0 >= n) return;
  if (i0 + 16 <= n) {
    float v[16];
    fp8_load16(x, i0, v);
    fp8_i32x4_t out;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = (int)fp8_q4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3], inv);
    *reinterpret_cast<fp8_i32x4_t*>(q + i0) = out;
  } else {
    for (int64_t i = i0; i < n; ++i)
      q[i] = (uint8_t)(fp8_q4(fp8_ld(x, i), 0.0f, 0.0f, 0.0f, inv) & 0xffu);
  }
}

// ---------------------------------------------------------------- launchers
// Host-side launchers; arguments are validated by the C-ABI layer.
// G == 0: plain top-K; else group-limited routing over G groups keeping TG.
moe_status_t launch_route(const float* logits, int T, int E, int K, int renorm, int G, int TG,
                          int32_t* ids, float* w, hipStream_t stream);
// launch_route followed by launch_slot_map, as one kernel where the router
// runs with lane groups (the same bits as the two calls).
moe_status_t launch_route_map(const float* logits, int T, int E, int K, int renorm, int G,
                              int TG, int32_t* ids, float* w, int start, int E_local,
                              const int32_t* rep_off, const int32_t* rep_slots, int S,
                              int32_t* slot, float* w_masked, uint8_t* mask,
                              hipStream_t stream);
moe_status_t launch_slot_map(const int32_t* ids, const float* w, int T, int K, int start,
                             int E_local, const int32_t* rep_off, const int32_t* rep_slots,
                             int S, int32_t* slot, float* w_masked, uint8_t* mask,
                             hipStream_t stream);

// Quantization of a bf16 tensor of n values to E4M3 codes (scale 1 / inv),
// run as extra blocks of the permutation's scatter launch (independent work).
struct FusedQuant {
  const uint16_t* x;
  int64_t n;
  float inv;
  uint8_t* q;
};

struct PermutePlan {
  int P;        // pairs
  int chunk;    // pairs per chunk: whole tokens (a multiple of K)
  int nchunks;  // ceil(P / chunk)
  size_t ws_bytes;
};
PermutePlan permute_plan(int T, int K, int S);
// Entries of the static histogram array behind moe_permute_noalloc (256 KiB
// per device): permute_plan never needs more than 65536 / S chunks of S.
constexpr int kPermuteScratchInts = 65536;
// Device address of that array on the current device, looked up on the
// first call per device (hipGetSymbolAddress) and kept for later calls.
moe_status_t permute_scratch(int32_t** out);
// pair_w non-null: the row of pair p is pair_w[p] * x[p / K] (f32 product,
// rounded once). quant non-null: its quantization runs as extra blocks of the
// ranking launch.
moe_status_t launch_permute(const void* x, int elem_bytes, int T, int H, int K,
                            const int32_t* slot, const uint8_t* mask, int S, int32_t* offsets,
                            int32_t* sorted_pairs, int32_t* pair_row, void* x_perm, void* ws,
                            hipStream_t stream, const float* pair_w = nullptr,
                            const FusedQuant* quant = nullptr);

// max_blocks > 0 caps the persistent GEMM grid (default: one block per
// compute unit); the results do not depend on the grid.
moe_status_t launch_gemm_bf16(moe_gemm_op_t op, const void* a, const int32_t* offsets, int S,
                              int max_rows, const void* w, int H, int I, void* c,
                              hipStream_t stream, int max_blocks = 0);
// Gate/up product with the permutation's gather folded into the operand fetch:
// row r of the permuted order is token sorted_pairs[r] / K of x [T, H]. Only
// for shapes where gemm_bf16_gather_ok(T, H) holds.
bool gemm_bf16_gather_ok(int T, int H);
moe_status_t launch_gemm_bf16_gate_up_gathered(const void* x, int T, int K,
                                               const int32_t* sorted_pairs,
                                               const int32_t* offsets, int S, int max_rows,
                                               const void* w, int H, int I, void* c,
                                               hipStream_t stream, int max_blocks = 0);
moe_status_t launch_gemm_f32(moe_gemm_op_t op, const void* a, const int32_t* offsets, int S,
                             int max_rows, const void* w, int H, int I, void* c,
                             hipStream_t stream);

// FP8 (E4M3) grouped GEMMs: a and w are codes, slot s's products are scaled by
// a_scale * w_scale[s]. Gate/up writes the SwiGLU output as codes quantized
// with out_scale; down writes bf16. Both need the contraction length to be a
// multiple of 128 and at least 256 (gemm_fp8_ok).
bool gemm_fp8_ok(int Kd);
bool gemm_fp8_gather_ok(int T, int H);
moe_status_t launch_gemm_fp8(moe_gemm_op_t op, const uint8_t* a, float a_scale,
                             const int32_t* offsets, int S, int max_rows, const uint8_t* w,
                             const float* w_scale, int H, int I, void* c, float out_scale,
                             hipStream_t stream, int max_blocks = 0);
moe_status_t launch_gemm_fp8_gate_up_gathered(const uint8_t* xq, int T, int K,
                                              const int32_t* sorted_pairs,
                                              const int32_t* offsets, int S, int max_rows,
                                              const uint8_t* w, const float* w_scale,
                                              float a_scale, int H, int I, void* c,
                                              float out_scale, hipStream_t stream,
                                              int max_blocks = 0);
// q[i] = E4M3 code of clamp(x[i] * (1 / scale), -448, 448), rounded to nearest even.
moe_status_t launch_quantize_fp8(const void* x, bool x_bf16, int64_t n, float scale, uint8_t* q,
                                 hipStream_t stream);

// All-to-all dispatch workspace (carved in this order, 256-byte aligned).
struct A2aLayout {
  size_t bits, hist, total;  // per-token rank masks, per-chunk rank counts
};
A2aLayout a2a_layout(int T, int R, int cap);
moe_status_t launch_a2a_dispatch(const void* x, int elem_bytes, int T, int H, int K,
                                 const int32_t* ids, const float* w, int E_global, int R, int cap,
                                 int32_t* offsets, int32_t* token_pos, int32_t* send_token,
                                 void* send_x, int32_t* send_ids, float* send_w, void* ws,
                                 hipStream_t stream);

// w_masked may be null: every pair then has weight 1. shared (non-null,
// [T, H] of shared_dt) is added to the token's sum before the rounding.
moe_status_t launch_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                            const float* w_masked, int T, int K, int H, void* out,
                            moe_dtype_t out_dt, int accumulate, hipStream_t stream,
                            const void* shared = nullptr, moe_dtype_t shared_dt = MOE_DTYPE_BF16);

}  // namespace moe
