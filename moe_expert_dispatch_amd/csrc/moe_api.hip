// C ABI of the fused MoE forward pass: host-side argument validation,
// workspace planning and the fused stage sequence. Every kernel launch is
// asynchronous on the caller's stream; nothing here allocates or waits.
//
// Sources: TensorRT-LLM PR #10985 walkthrough (the fused op takes tokens,
// selected experts and routing weights; MoE mapping configuration with EP
// size / rank and max num tokens sizing the workspace); vLLM
// ep_fused_moe_patch.py _ep_init (E % ep_size asserted, start = rank * E_l).
#include "common.h"

namespace moe {

// Asked of the runtime on every GEMM launch (a host-side attribute read), so
// the library keeps no per-device state for it.
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 1;
  return n;
}

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(moe_dtype_t dt) { return dt == MOE_DTYPE_F32 || dt == MOE_DTYPE_BF16; }
int dtype_bytes(moe_dtype_t dt) {
  return dt == MOE_DTYPE_F32 ? 4 : dt == MOE_DTYPE_FP8_E4M3 ? 1 : 2;
}
bool scale_ok(float s) { return s > 0.0f && s <= 3.4e38f; }  // finite, positive (false for NaN)

// T * K and T * K * max(H, I) must stay addressable with 32-bit row indices.
bool pairs_fit(int T, int K) { return (long long)T * K < (1LL << 31); }

moe_status_t check_route(const float* logits, int T, int E, int K, const int32_t* ids,
                         const float* w) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (!pairs_fit(T, K) || (long long)T * E >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!logits || !ids || !w)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_slot_map(const int32_t* ids, const float* w, int T, int K, int E_global,
                            int ep_size, int ep_rank, const int32_t* rep_off,
                            const int32_t* rep_slots, int S, const int32_t* slot,
                            const float* w_masked, const uint8_t* mask) {
  if (T < 0 || K < 1 || E_global < 1 || ep_size < 1) return MOE_ERR_INVALID_ARG;
  if (E_global % ep_size != 0 || ep_rank < 0 || ep_rank >= ep_size) return MOE_ERR_INVALID_ARG;
  const int E_local = E_global / ep_size;
  if (S < E_local) return MOE_ERR_INVALID_ARG;
  if (!rep_off && S != E_local) return MOE_ERR_INVALID_ARG;
  if (rep_off && !rep_slots) return MOE_ERR_INVALID_ARG;
  if (S > MOE_MAX_SLOTS || K > MOE_MAX_TOPK || E_global > MOE_MAX_EXPERTS)
    return MOE_ERR_UNSUPPORTED;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!ids || !w || !slot || !w_masked || !mask)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_permute(const void* x, moe_dtype_t dt, int T, int H, int K,
                           const int32_t* slot, const uint8_t* mask, int S,
                           const int32_t* offsets, const int32_t* sorted_pairs,
                           const int32_t* pair_row, const void* x_perm, const void* ws,
                           size_t ws_bytes) {
  if (T < 0 || K < 1 || S < 1 || H < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (S > MOE_MAX_SLOTS || K > MOE_MAX_TOPK || H % 8 != 0 || !pairs_fit(T, K))
    return MOE_ERR_UNSUPPORTED;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!slot || !mask || !sorted_pairs || !pair_row)) return MOE_ERR_INVALID_ARG;
  if (x_perm && T > 0 && (!x || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  const size_t need = permute_plan(T, K, S).ws_bytes;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// elem_bytes: operand bytes for the weight-panel limit (0: those of dt).
moe_status_t check_gemm(moe_gemm_op_t op, moe_dtype_t dt, const void* a, const int32_t* offsets,
                        int S, int max_rows, const void* w, int H, int I, const void* c,
                        int elem_bytes = 0) {
  if (op != MOE_GEMM_GATE_UP_SWIGLU && op != MOE_GEMM_DOWN) return MOE_ERR_INVALID_ARG;
  if (S < 1 || max_rows < 0 || H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (S > MOE_MAX_SLOTS || H % 8 != 0 || I % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!weight_panel_ok(H, I, elem_bytes > 0 ? elem_bytes : dtype_bytes(dt)))
    return MOE_ERR_UNSUPPORTED;
  if ((long long)max_rows * (H > I ? H : I) >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && (!a || !w || !c)) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && (!aligned16(a) || !aligned16(w) || !aligned16(c)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// weights_required: moe_combine needs w_masked; moe_combine_shared accepts NULL.
moe_status_t check_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                           const float* w_masked, int T, int K, int H, const void* out,
                           moe_dtype_t out_dt, bool weights_required = true) {
  if (T < 0 || K < 1 || H < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(y_dt) || !dtype_ok(out_dt)) return MOE_ERR_UNSUPPORTED;
  if (K > MOE_MAX_TOPK || H % 8 != 0 || !pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!y || !pair_row || !out)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && weights_required && !w_masked) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(y) || !aligned16(out))) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t launch_gemm(moe_gemm_op_t op, moe_dtype_t dt, const void* a, const int32_t* offsets,
                         int S, int max_rows, const void* w, int H, int I, void* c,
                         hipStream_t stream, int max_blocks = 0) {
  return dt == MOE_DTYPE_BF16
             ? launch_gemm_bf16(op, a, offsets, S, max_rows, w, H, I, c, stream, max_blocks)
             : launch_gemm_f32(op, a, offsets, S, max_rows, w, H, I, c, stream);
}

// Workspace of moe_forward, carved in this order (each 256-byte aligned).
struct ForwardLayout {
  size_t ids, w, slot, w_masked, mask, offsets, sorted_pairs, pair_row, perm_ws, x_perm, act, xq;
  size_t total;
};

ForwardLayout forward_layout(const moe_config_t* c) {
  ForwardLayout L;
  const size_t P = (size_t)c->T_max * c->K;
  const bool fp8 = c->dtype == MOE_DTYPE_FP8_E4M3;
  const size_t eb = dtype_bytes(c->dtype);
  const size_t yb = fp8 ? 2 : eb;  // FP8: the expert outputs are bf16
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.ids = take(P * 4);
  L.w = take(P * 4);
  L.slot = take(P * 4);
  L.w_masked = take(P * 4);
  L.mask = take(P);
  L.offsets = take(((size_t)c->S + 1) * 4);
  L.sorted_pairs = take(P * 4);
  L.pair_row = take(P * 4);
  L.perm_ws = take(permute_plan(c->T_max, c->K, c->S).ws_bytes);
  L.x_perm = take(P * c->H * yb);  // later reused for the down-projection output
  L.act = take(P * c->I * eb);
  L.xq = take(fp8 ? (size_t)c->T_max * c->H : 0);  // FP8: the quantized input
  L.total = off;
  return L;
}

moe_status_t check_a2a_dispatch(const void* x, moe_dtype_t dt, int T, int H, int K,
                                const int32_t* ids, const float* w, int E_global, int ep_size,
                                int cap, const int32_t* offsets, const int32_t* token_pos,
                                const int32_t* send_token, const void* send_x,
                                const int32_t* send_ids, const float* send_w) {
  if (T < 0 || K < 1 || E_global < 1 || ep_size < 1 || cap < T) return MOE_ERR_INVALID_ARG;
  if (E_global % ep_size != 0) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (ep_size > MOE_MAX_A2A_RANKS || K > MOE_MAX_TOPK || E_global > MOE_MAX_EXPERTS)
    return MOE_ERR_UNSUPPORTED;
  if (H < 1 || (H * dtype_bytes(dt)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (!pairs_fit(T, ep_size) || !pairs_fit(cap, ep_size) || !pairs_fit(cap * ep_size, K))
    return MOE_ERR_UNSUPPORTED;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !ids || !w || !token_pos || !aligned16(x))) return MOE_ERR_INVALID_ARG;
  if (cap > 0 && (!send_token || !send_x || !send_ids || !send_w || !aligned16(send_x)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Group-limited routing: 1 <= topk_groups <= num_groups <= 64, E divisible
// by num_groups, and the kept groups hold at least K experts.
moe_status_t check_groups(int E, int K, int num_groups, int topk_groups) {
  if (num_groups < 1 || topk_groups < 1 || topk_groups > num_groups) return MOE_ERR_INVALID_ARG;
  if (E % num_groups != 0 || K > topk_groups * (E / num_groups)) return MOE_ERR_INVALID_ARG;
  if (num_groups > MOE_MAX_EXPERT_GROUPS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T_max < 0 || c->T < 0 || c->T > c->T_max) return MOE_ERR_INVALID_ARG;
  if (c->H < 1 || c->I < 1 || c->E_global < 1 || c->K < 1 || c->K > c->E_global)
    return MOE_ERR_INVALID_ARG;
  if (c->ep_size < 1 || c->E_global % c->ep_size != 0 || c->ep_rank < 0 ||
      c->ep_rank >= c->ep_size)
    return MOE_ERR_INVALID_ARG;
  if (c->S < c->E_global / c->ep_size) return MOE_ERR_INVALID_ARG;
  const bool fp8 = c->dtype == MOE_DTYPE_FP8_E4M3;
  if ((!dtype_ok(c->dtype) && !fp8) || !dtype_ok(c->out_dtype)) return MOE_ERR_UNSUPPORTED;
  if (fp8 && (!scale_ok(c->a1_scale) || !scale_ok(c->a2_scale))) return MOE_ERR_INVALID_ARG;
  if (fp8 && (c->routing_on_input || !gemm_fp8_ok(c->H) || !gemm_fp8_ok(c->I) ||
              !gemm_fp8_gather_ok(c->T_max, c->H)))
    return MOE_ERR_UNSUPPORTED;
  if (c->E_global > MOE_MAX_EXPERTS || c->K > MOE_MAX_TOPK || c->S > MOE_MAX_SLOTS)
    return MOE_ERR_UNSUPPORTED;
  if (c->H % 8 != 0 || c->I % 8 != 0 || !pairs_fit(c->T_max, c->K)) return MOE_ERR_UNSUPPORTED;
  if (!weight_panel_ok(c->H, c->I, dtype_bytes(c->dtype))) return MOE_ERR_UNSUPPORTED;
  if (c->gemm_blocks < 0) return MOE_ERR_INVALID_ARG;
  const long long P = (long long)c->T_max * c->K;
  if (P * (c->H > c->I ? c->H : c->I) >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (c->num_expert_group != 0 || c->topk_group != 0) {
    const moe_status_t sg = check_groups(c->E_global, c->K, c->num_expert_group, c->topk_group);
    if (sg != MOE_OK) return sg;
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_str(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: dtype or shape not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch or runtime error";
    default: break;
  }
  return "unknown moe_status_t";
}

moe_status_t moe_route(const float* logits, int T, int E, int K, int renormalize, int32_t* ids,
                       float* w, hipStream_t stream) {
  const moe_status_t st = check_route(logits, T, E, K, ids, w);
  if (st != MOE_OK) return st;
  return launch_route(logits, T, E, K, renormalize ? 1 : 0, 0, 0, ids, w, stream);
}

moe_status_t moe_route_grouped(const float* logits, int T, int E, int K, int renormalize,
                               int num_groups, int topk_groups, int32_t* ids, float* w,
                               hipStream_t stream) {
  const moe_status_t st = check_route(logits, T, E, K, ids, w);
  if (st != MOE_OK) return st;
  const moe_status_t sg = check_groups(E, K, num_groups, topk_groups);
  if (sg != MOE_OK) return sg;
  return launch_route(logits, T, E, K, renormalize ? 1 : 0, num_groups, topk_groups, ids, w,
                      stream);
}

moe_status_t moe_slot_map(const int32_t* ids, const float* w, int T, int K, int E_global,
                          int ep_size, int ep_rank, const int32_t* rep_off,
                          const int32_t* rep_slots, int S, int32_t* slot, float* w_masked,
                          uint8_t* mask, hipStream_t stream) {
  const moe_status_t st = check_slot_map(ids, w, T, K, E_global, ep_size, ep_rank, rep_off,
                                         rep_slots, S, slot, w_masked, mask);
  if (st != MOE_OK) return st;
  const int E_local = E_global / ep_size;
  return launch_slot_map(ids, w, T, K, ep_rank * E_local, E_local, rep_off, rep_slots, S, slot,
                         w_masked, mask, stream);
}

size_t moe_permute_workspace_size(int T, int K, int S) {
  if (T < 0 || K < 1 || S < 1 || !pairs_fit(T, K)) return 0;
  return permute_plan(T, K, S).ws_bytes;
}

moe_status_t moe_permute(const void* x, moe_dtype_t dt, int T, int H, int K,
                         const int32_t* slot, const uint8_t* mask, int S, int32_t* offsets,
                         int32_t* sorted_pairs, int32_t* pair_row, void* x_perm, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  const moe_status_t st = check_permute(x, dt, T, H, K, slot, mask, S, offsets, sorted_pairs,
                                        pair_row, x_perm, ws, ws_bytes);
  if (st != MOE_OK) return st;
  return launch_permute(x, dtype_bytes(dt), T, H, K, slot, mask, S, offsets, sorted_pairs,
                        pair_row, x_perm, ws, stream);
}

moe_status_t moe_permute_noalloc(const void* x, moe_dtype_t dt, int T, int H, int K,
                                 const int32_t* slot, const uint8_t* mask, int S,
                                 int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_row,
                                 void* x_perm, hipStream_t stream) {
  constexpr size_t kScratchBytes = (size_t)kPermuteScratchInts * sizeof(int32_t);
  if (T < 0 || K < 1 || S < 1 || !pairs_fit(T, K)) return MOE_ERR_INVALID_ARG;
  if (permute_plan(T, K, S).ws_bytes > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  int32_t* hist = nullptr;
  moe_status_t st = permute_scratch(&hist);
  if (st != MOE_OK) return st;
  st = check_permute(x, dt, T, H, K, slot, mask, S, offsets, sorted_pairs, pair_row, x_perm,
                     hist, kScratchBytes);
  if (st != MOE_OK) return st;
  return launch_permute(x, dtype_bytes(dt), T, H, K, slot, mask, S, offsets, sorted_pairs,
                        pair_row, x_perm, hist, stream);
}

moe_status_t moe_permute_scaled(const void* x, moe_dtype_t dt, int T, int H, int K,
                                const int32_t* slot, const uint8_t* mask, int S,
                                const float* pair_w, int32_t* offsets, int32_t* sorted_pairs,
                                int32_t* pair_row, void* x_perm, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  const moe_status_t st = check_permute(x, dt, T, H, K, slot, mask, S, offsets, sorted_pairs,
                                        pair_row, x_perm, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (T > 0 && (!pair_w || !x_perm)) return MOE_ERR_INVALID_ARG;
  return launch_permute(x, dtype_bytes(dt), T, H, K, slot, mask, S, offsets, sorted_pairs,
                        pair_row, x_perm, ws, stream, pair_w);
}

moe_status_t moe_grouped_gemm(moe_gemm_op_t op, moe_dtype_t dt, const void* a,
                              const int32_t* offsets, int S, int max_rows, const void* w, int H,
                              int I, void* c, hipStream_t stream) {
  const moe_status_t st = check_gemm(op, dt, a, offsets, S, max_rows, w, H, I, c);
  if (st != MOE_OK) return st;
  return launch_gemm(op, dt, a, offsets, S, max_rows, w, H, I, c, stream);
}

moe_status_t moe_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                         const float* w_masked, int T, int K, int H, void* out,
                         moe_dtype_t out_dt, int accumulate, hipStream_t stream) {
  const moe_status_t st = check_combine(y, y_dt, pair_row, w_masked, T, K, H, out, out_dt);
  if (st != MOE_OK) return st;
  return launch_combine(y, y_dt, pair_row, w_masked, T, K, H, out, out_dt, accumulate, stream);
}

moe_status_t moe_combine_shared(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                                const float* w_masked, int T, int K, int H, const void* shared,
                                moe_dtype_t shared_dt, void* out, moe_dtype_t out_dt,
                                int accumulate, hipStream_t stream) {
  const moe_status_t st =
      check_combine(y, y_dt, pair_row, w_masked, T, K, H, out, out_dt, false);
  if (st != MOE_OK) return st;
  if (shared && !dtype_ok(shared_dt)) return MOE_ERR_UNSUPPORTED;
  if (shared && T > 0 && !aligned16(shared)) return MOE_ERR_INVALID_ARG;
  return launch_combine(y, y_dt, pair_row, w_masked, T, K, H, out, out_dt, accumulate, stream,
                        shared, shared_dt);
}

size_t moe_forward_workspace_size(const moe_config_t* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return forward_layout(cfg).total;
}

moe_status_t moe_forward(const moe_config_t* cfg, const moe_forward_args_t* args, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!args) return MOE_ERR_INVALID_ARG;
  const int T = cfg->T, K = cfg->K, H = cfg->H, I = cfg->I, S = cfg->S;
  const int E_local = cfg->E_global / cfg->ep_size;
  if (!args->rep_off && S != E_local) return MOE_ERR_INVALID_ARG;
  if (args->rep_off && !args->rep_slots) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!args->x || !args->w_gate_up || !args->w_down || !args->out) return MOE_ERR_INVALID_ARG;
    if (!args->logits && (!args->topk_ids || !args->topk_w)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(args->x) || !aligned16(args->w_gate_up) || !aligned16(args->w_down) ||
        !aligned16(args->out))
      return MOE_ERR_INVALID_ARG;
    if (args->shared_out && !aligned16(args->shared_out)) return MOE_ERR_INVALID_ARG;
    if (cfg->dtype == MOE_DTYPE_FP8_E4M3 && (!args->w_gate_up_scale || !args->w_down_scale))
      return MOE_ERR_INVALID_ARG;
  }
  const ForwardLayout L = forward_layout(cfg);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;

  char* base = static_cast<char*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(base + L.ids);
  float* w = reinterpret_cast<float*>(base + L.w);
  int32_t* slot = reinterpret_cast<int32_t*>(base + L.slot);
  float* w_masked = reinterpret_cast<float*>(base + L.w_masked);
  uint8_t* mask = reinterpret_cast<uint8_t*>(base + L.mask);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* sorted_pairs = reinterpret_cast<int32_t*>(base + L.sorted_pairs);
  int32_t* pair_row = reinterpret_cast<int32_t*>(base + L.pair_row);
  void* perm_ws = base + L.perm_ws;
  void* x_perm = base + L.x_perm;
  void* act = base + L.act;
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + L.xq);
  void* y = x_perm;  // grouped GEMM 1 has consumed x_perm when GEMM 2 writes
  const bool fp8 = cfg->dtype == MOE_DTYPE_FP8_E4M3;
  const int gb = cfg->gemm_blocks;  // persistent GEMM grid cap (0: one block per CU)

  auto mark = [&](int ev) -> moe_status_t {
    if (args->events[ev] && hipEventRecord(args->events[ev], stream) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  };
#define MOE_TRY(expr)                \
  do {                               \
    const moe_status_t s_ = (expr);  \
    if (s_ != MOE_OK) return s_;     \
  } while (0)

  MOE_TRY(mark(MOE_EV_START));
  const int32_t* ids_in = args->topk_ids;
  const float* w_in = args->topk_w;
  if (args->logits) {
    MOE_TRY(launch_route_map(args->logits, T, cfg->E_global, K, cfg->renormalize ? 1 : 0,
                             cfg->num_expert_group, cfg->topk_group, ids, w,
                             cfg->ep_rank * E_local, E_local, args->rep_off, args->rep_slots, S,
                             slot, w_masked, mask, stream));
  } else {
    MOE_TRY(launch_slot_map(ids_in, w_in, T, K, cfg->ep_rank * E_local, E_local, args->rep_off,
                            args->rep_slots, S, slot, w_masked, mask, stream));
  }
  MOE_TRY(mark(MOE_EV_ROUTED));
  // bf16 with a direct-to-LDS shape: the gate/up GEMM fetches token rows of x
  // itself, so the permutation only orders the pairs (no x_perm copy).
  // Input-side routing gathers rows scaled by the pair weight instead.
  const bool on_input = cfg->routing_on_input != 0;
  // FP8: x is quantized once per token and GEMM 1 gathers the code rows.
  const bool fused_gather =
      fp8 || (!on_input && cfg->dtype == MOE_DTYPE_BF16 && gemm_bf16_gather_ok(T, H));
  // FP8: x is quantized by extra blocks of the permutation's scatter launch
  const FusedQuant fq{static_cast<const uint16_t*>(args->x), (int64_t)T * H,
                      1.0f / cfg->a1_scale, xq};
  MOE_TRY(launch_permute(args->x, fp8 ? 2 : dtype_bytes(cfg->dtype), T, H, K, slot, mask, S,
                         offsets, sorted_pairs, pair_row, fused_gather ? nullptr : x_perm,
                         perm_ws, stream, on_input ? w_masked : nullptr,
                         fp8 ? &fq : nullptr));
  MOE_TRY(mark(MOE_EV_PERMUTED));
  if (fp8)
    MOE_TRY(launch_gemm_fp8_gate_up_gathered(
        xq, T, K, sorted_pairs, offsets, S, T * K, static_cast<const uint8_t*>(args->w_gate_up),
        args->w_gate_up_scale, cfg->a1_scale, H, I, act, cfg->a2_scale, stream, gb));
  else if (fused_gather)
    MOE_TRY(launch_gemm_bf16_gate_up_gathered(args->x, T, K, sorted_pairs, offsets, S, T * K,
                                              args->w_gate_up, H, I, act, stream, gb));
  else
    MOE_TRY(launch_gemm(MOE_GEMM_GATE_UP_SWIGLU, cfg->dtype, x_perm, offsets, S, T * K,
                        args->w_gate_up, H, I, act, stream, gb));
  MOE_TRY(mark(MOE_EV_GATE_UP));
  if (fp8)
    MOE_TRY(launch_gemm_fp8(MOE_GEMM_DOWN, static_cast<const uint8_t*>(act), cfg->a2_scale,
                            offsets, S, T * K, static_cast<const uint8_t*>(args->w_down),
                            args->w_down_scale, H, I, y, 1.0f, stream, gb));
  else
    MOE_TRY(launch_gemm(MOE_GEMM_DOWN, cfg->dtype, act, offsets, S, T * K, args->w_down, H, I,
                        y, stream, gb));
  MOE_TRY(mark(MOE_EV_DOWN));
  const moe_dtype_t ydt = fp8 ? MOE_DTYPE_BF16 : cfg->dtype;
  MOE_TRY(launch_combine(y, ydt, pair_row, on_input ? nullptr : w_masked, T, K, H, args->out,
                         cfg->out_dtype, cfg->accumulate, stream, args->shared_out, ydt));
  MOE_TRY(mark(MOE_EV_COMBINED));
#undef MOE_TRY
  return MOE_OK;
}

moe_status_t moe_quantize_fp8(const void* x, moe_dtype_t x_dt, int64_t n, float scale,
                              uint8_t* q, hipStream_t stream) {
  if (n < 0 || !scale_ok(scale)) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_DTYPE_BF16 && x_dt != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!x || !q || !aligned16(x) || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return launch_quantize_fp8(x, x_dt == MOE_DTYPE_BF16, n, scale, q, stream);
}

moe_status_t moe_grouped_gemm_fp8(moe_gemm_op_t op, const uint8_t* a, float a_scale,
                                  const int32_t* offsets, int S, int max_rows, const uint8_t* w,
                                  const float* w_scale, int H, int I, void* c, float c_scale,
                                  hipStream_t stream) {
  // the shape, pointer and alignment rules of moe_grouped_gemm, with the
  // weight-panel limit taken for one-byte codes
  const moe_status_t st =
      check_gemm(op, MOE_DTYPE_BF16, a, offsets, S, max_rows, w, H, I, c, 1);
  if (st != MOE_OK) return st;
  if (!scale_ok(a_scale) || (op == MOE_GEMM_GATE_UP_SWIGLU && !scale_ok(c_scale)))
    return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && !w_scale) return MOE_ERR_INVALID_ARG;
  if (!gemm_fp8_ok(op == MOE_GEMM_GATE_UP_SWIGLU ? H : I)) return MOE_ERR_UNSUPPORTED;
  return launch_gemm_fp8(op, a, a_scale, offsets, S, max_rows, w, w_scale, H, I, c, c_scale,
                         stream);
}

size_t moe_a2a_dispatch_workspace_size(int T, int ep_size, int cap) {
  if (T < 0 || ep_size < 1 || ep_size > MOE_MAX_A2A_RANKS || cap < T ||
      !pairs_fit(T, ep_size) || !pairs_fit(cap, ep_size))
    return 0;
  return a2a_layout(T, ep_size, cap).total;
}

moe_status_t moe_a2a_dispatch(const void* x, moe_dtype_t dt, int T, int H, int K,
                              const int32_t* topk_ids, const float* topk_w, int E_global,
                              int ep_size, int cap, int32_t* offsets, int32_t* token_pos,
                              int32_t* send_token, void* send_x, int32_t* send_ids,
                              float* send_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status_t st =
      check_a2a_dispatch(x, dt, T, H, K, topk_ids, topk_w, E_global, ep_size, cap, offsets,
                         token_pos, send_token, send_x, send_ids, send_w);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < a2a_layout(T, ep_size, cap).total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  return launch_a2a_dispatch(x, dtype_bytes(dt), T, H, K, topk_ids, topk_w, E_global, ep_size,
                             cap, offsets, token_pos, send_token, send_x, send_ids, send_w, ws,
                             stream);
}

moe_status_t moe_a2a_combine(const void* partial, moe_dtype_t partial_dt,
                             const int32_t* token_pos, int T, int ep_size, int H, void* out,
                             moe_dtype_t out_dt, hipStream_t stream) {
  if (T < 0 || ep_size < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(partial_dt) || !dtype_ok(out_dt)) return MOE_ERR_UNSUPPORTED;
  if (ep_size > MOE_MAX_A2A_RANKS || H % 8 != 0 || !pairs_fit(T, ep_size))
    return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!partial || !token_pos || !out)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(partial) || !aligned16(out))) return MOE_ERR_INVALID_ARG;
  return launch_combine(partial, partial_dt, token_pos, nullptr, T, ep_size, H, out, out_dt, 0,
                        stream);
}

}  // extern "C"
