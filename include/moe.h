/*
 * moe.h -- C ABI of the fused Mixture-of-Experts forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The forward pass, per token t with hidden row x[t]:
 *   1. route      softmax over the router logits, top-K experts, optional
 *                 renormalisation of the K selected probabilities;
 *   2. slot map   expert-parallel (EP) mask and local remap for one rank's
 *                 expert range, then expert id -> engine-side expert slot;
 *   3. permute    group the included (token, slot) pairs by slot with a
 *                 counting sort and gather the hidden rows in that order;
 *   4. grouped GEMM 1   per non-empty slot: a = silu(x Wg^T) * (x Wu^T);
 *   5. grouped GEMM 2   per non-empty slot: y = a Wd^T;
 *   6. combine    out[t] = sum over the included pairs of w'[t,k] * y.
 *
 * Sources (web pages the method is taken from):
 *   [SLOTS]  TensorRT-LLM PR #4495 "large-scale EP (part 3: refactor -
 *            FusedMoe for redundant expert)", Description: the model-side
 *            Expert id versus the engine-side Expert Slot the fused op
 *            computes over; weights are loaded per slot.
 *   [A2A]    TensorRT-LLM PR #10985 "MoE all-to-all paradigm": walkthrough
 *            sequence diagram (fused op on tokens + selected experts +
 *            routing weights; all-reduce path), review of torch_moe.py
 *            (_template_moe, is_gated_mlp / act_fn), and the MoE mapping
 *            configuration indices (EP size / rank, max num tokens for the
 *            workspace).
 *   [EPMASK] vLLM ep_fused_moe_patch.py (model-hub mirror): module
 *            docstring "EP expert dispatch"; ep_mask_and_remap; _ep_init
 *            (expert partition start = rank * E / ep_size, divisibility
 *            asserted); FusedMoE constructor arguments (top_k, renormalize).
 *   [AUTOTP] DeepSpeed PR #6964 "AutoTP for MoE models": the routed output
 *            is the weighted sum of the selected experts' outputs, reduced
 *            once per layer.
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers owned by the caller unless stated.
 *     The library never allocates, frees, or synchronises; every call only
 *     enqueues kernels on `stream` and returns.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing.
 *   - Index and weight arrays are row-major: [T, K] means element (t, k) at
 *     t*K + k. A "pair" p = t*K + k is the k-th routing choice of token t.
 *   - Matrices are row-major with the last index contiguous. Weights are
 *     stored [out_features, in_features] so both GEMM operands are
 *     contiguous along the reduction dimension.
 *   - bf16 data is IEEE binary32 truncated to its top 16 bits (bfloat16);
 *     every conversion to bf16 rounds to nearest, ties to even.
 *   - Device pointers passed for 16-byte vector access (x, x_perm, GEMM
 *     operands, y, out) must be 16-byte aligned.
 *   - Calls on one stream run in order; calls that share output or
 *     workspace buffers on different streams race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The *_ENUM_MIN_ / *_ENUM_MAX_ entries of the enums below are not values to
 * pass or expect: they make every int a valid value of the enum type, so an
 * out-of-range argument from a C caller is rejected with a status code
 * instead of being undefined behaviour in the C++ implementation. */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, negative size, K > E, E % ep_size != 0, ... */
  MOE_ERR_UNSUPPORTED = 2, /* dtype or shape outside what the kernels are built for */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  MOE_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
  MOE_STATUS_ENUM_MIN_ = -0x7fffffff - 1, /* see below: not status codes */
  MOE_STATUS_ENUM_MAX_ = 0x7fffffff
} moe_status_t;

typedef enum {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_FP8_E4M3 = 2, /* OCP FP8 E4M3 codes (moe_quantize_fp8, moe_grouped_gemm_fp8) */
  MOE_DTYPE_ENUM_MIN_ = -0x7fffffff - 1,
  MOE_DTYPE_ENUM_MAX_ = 0x7fffffff
} moe_dtype_t;

typedef enum {
  MOE_GEMM_GATE_UP_SWIGLU = 0, /* c[r, j] = silu(a[r] . Wg[s, j]) * (a[r] . Wu[s, j]) */
  MOE_GEMM_DOWN = 1,           /* c[r, j] = a[r] . Wd[s, j] */
  MOE_GEMM_OP_ENUM_MIN_ = -0x7fffffff - 1,
  MOE_GEMM_OP_ENUM_MAX_ = 0x7fffffff
} moe_gemm_op_t;

/* Compiled limits. */
#define MOE_MAX_EXPERTS 1024 /* E_global */
#define MOE_MAX_TOPK 32      /* K */
#define MOE_MAX_SLOTS 1024   /* S */
#define MOE_MAX_A2A_RANKS 32 /* ep_size of the all-to-all dispatch */
#define MOE_MAX_EXPERT_GROUPS 64 /* num_expert_group of group-limited routing */

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(moe_status_t status);

/*
 * moe_route -- router softmax and top-K selection.
 *   Source: [EPMASK] module docstring, section "EP expert dispatch" (every
 *   rank computes the same global top-k expert ids) and the FusedMoE
 *   constructor's top_k / renormalize (default True) arguments.
 *
 * logits [T, E] f32 (input). For each token t:
 *   m = max_e logits[t, e];  p_e = exp(logits[t,e] - m) / sum_j exp(logits[t,j] - m)
 *   ids[t, 0..K-1]: the K experts with the largest logits, ordered by logit
 *     descending and, among equal logits, by expert id ascending (-0.0 and
 *     +0.0 compare equal). Selection compares the f32 logits exactly.
 *   w[t, k] = p_{ids[t,k]}; if renormalize != 0, w[t, k] /= sum_k' w[t, k'].
 * ids [T, K] int32 (output), w [T, K] f32 (output).
 * Softmax is evaluated in f32 with the device expf and IEEE division.
 * Limits: 1 <= K <= E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK, T >= 0.
 * Logits must be finite; non-finite logits give unspecified ids and
 * weights (the call stays memory-safe and ids stay distinct and in range).
 */
moe_status_t moe_route(const float* logits, int T, int E, int K, int renormalize,
                       int32_t* ids, float* w, hipStream_t stream);

/*
 * moe_route_grouped -- group-limited routing.
 *   Source: [EPMASK] FusedMoE constructor arguments use_grouped_topk,
 *   num_expert_group and topk_group (the pages name them; the selection
 *   below is the plainest reading).
 *
 * As moe_route, except that the K experts are chosen among the experts of
 * the topk_groups best groups: the E experts form num_groups consecutive
 * groups of E / num_groups; a group's score is its largest logit (equivalently
 * its largest probability); groups are ranked by score descending, lower
 * group index first on ties. Weights are the probabilities of the full
 * softmax over all E experts (renormalised over the K when renormalize != 0).
 * Limits: 1 <= topk_groups <= num_groups <= MOE_MAX_EXPERT_GROUPS,
 * E % num_groups == 0, K <= topk_groups * (E / num_groups)
 * (MOE_ERR_INVALID_ARG otherwise; more groups: MOE_ERR_UNSUPPORTED).
 */
moe_status_t moe_route_grouped(const float* logits, int T, int E, int K, int renormalize,
                               int num_groups, int topk_groups, int32_t* ids, float* w,
                               hipStream_t stream);

/*
 * moe_slot_map -- expert-parallel mask / remap and expert -> slot lookup.
 *   Source: [EPMASK] ep_mask_and_remap and _ep_init; [SLOTS] Description.
 *
 * For pair (t, k) with e = ids[t, k], E_l = E_global / ep_size and
 * start = ep_rank * E_l:
 *   mask = (start <= e < start + E_l)
 *   w_masked = w[t,k] * (float)mask
 *   lid  = mask ? e - start : e mod E_l        (non-local ids spread by mod)
 *   r    = rep_off[lid + 1] - rep_off[lid]     (number of replicas of lid)
 *   slot = rep_slots[rep_off[lid] + (t mod r)] (replica chosen by token index)
 * rep_off == NULL selects the identity table (slot = lid, S == E_l).
 * rep_off [E_l + 1] int32 non-decreasing with rep_off[0] = 0 and
 * rep_off[E_l] = S; rep_slots [S] int32, a permutation of 0..S-1 (each
 * slot holds exactly one local expert). Both are device arrays.
 * Outputs: slot [T, K] int32, w_masked [T, K] f32, mask [T, K] uint8 (0/1).
 * The slot of a masked pair is still computed (the output is total); later
 * stages skip masked pairs. Ids outside [0, E_global) are treated as
 * non-local (mod taken on the non-negative residue). A table entry out of
 * range yields slot = -1, which later stages skip.
 * Errors: E_global % ep_size != 0 (as asserted by _ep_init), ep_rank not in
 * [0, ep_size), S < E_l, identity table with S != E_l.
 */
moe_status_t moe_slot_map(const int32_t* ids, const float* w, int T, int K, int E_global,
                          int ep_size, int ep_rank, const int32_t* rep_off,
                          const int32_t* rep_slots, int S, int32_t* slot, float* w_masked,
                          uint8_t* mask, hipStream_t stream);

/*
 * moe_permute -- counting-sort of the included pairs by slot and row gather.
 *   Source: [EPMASK] docstring: per-expert compute skipping empty experts,
 *   and the ragged gather that drops non-local pairs before compute.
 *
 * A pair p = t*K + k is included iff mask[p] != 0 and 0 <= slot[p] < S.
 * Outputs (bit-exact, independent of scheduling):
 *   offsets [S + 1]: offsets[s] = number of included pairs with slot < s;
 *     offsets[S] = P_in, the number of included pairs.
 *   sorted_pairs [T*K]: positions [0, P_in) hold the included pairs sorted
 *     by slot, ties in ascending p (stable); positions >= P_in are untouched.
 *   pair_row [T*K]: the row of pair p in the sorted order, or -1 if p is
 *     not included.
 *   x_perm [T*K, H] (capacity; rows [0, P_in) written):
 *     x_perm[pair_row[p]] = x[p / K] bit for bit.
 * x [T, H] of dtype dt (f32 or bf16); H * sizeof(dt) must be a multiple of
 * 16 bytes. ws: 16-byte aligned device workspace of at least
 * moe_permute_workspace_size() bytes (per-chunk slot histograms; contents on
 * entry are ignored).
 * x_perm may be NULL to compute only the index arrays.
 */
size_t moe_permute_workspace_size(int T, int K, int S);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 * Arguments, outputs and errors as moe_permute. The per-chunk histograms
 * live in a static device array of 65536 int32 (256 KiB), one per device,
 * held until the process ends; every (T, K, S) that moe_permute accepts
 * fits it (MOE_ERR_UNSUPPORTED otherwise). Its device address is looked up
 * once per device, on the first call made while that device is current.
 * Nothing in it needs clearing: each call writes every histogram entry it
 * reads. All calls on one device share the array, so calls that may overlap
 * on one device (different streams, or different host threads) race and
 * must be ordered by the caller.
 */
moe_status_t moe_permute_noalloc(const void* x, moe_dtype_t dt, int T, int H, int K,
                                 const int32_t* slot, const uint8_t* mask, int S,
                                 int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_row,
                                 void* x_perm, hipStream_t stream);

/*
 * moe_permute_scaled -- moe_permute whose gathered rows carry the routing
 * weight: x_perm[pair_row[p]] = round(pair_w[p] * x[p / K]) (f32 product,
 * one rounding to dt), for input-side routing.
 *   Source: [A2A] review of torch_moe.py: _template_moe's
 *   apply_routing_on_input, which applies the routing weights to the experts'
 *   input instead of their output (a different result: the MLP is not
 *   linear); the combine then uses weight 1 (moe_combine_shared with
 *   w_masked = NULL).
 * Arguments as moe_permute plus pair_w [T*K] f32 (the masked weights from
 * moe_slot_map); x_perm must not be NULL.
 */
moe_status_t moe_permute_scaled(const void* x, moe_dtype_t dt, int T, int H, int K,
                                const int32_t* slot, const uint8_t* mask, int S,
                                const float* pair_w, int32_t* offsets, int32_t* sorted_pairs,
                                int32_t* pair_row, void* x_perm, void* ws, size_t ws_bytes,
                                hipStream_t stream);
moe_status_t moe_permute(const void* x, moe_dtype_t dt, int T, int H, int K,
                         const int32_t* slot, const uint8_t* mask, int S, int32_t* offsets,
                         int32_t* sorted_pairs, int32_t* pair_row, void* x_perm, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * moe_grouped_gemm -- one launch computes every non-empty slot's product.
 *   Source: [A2A] review of torch_moe.py (gated MLP with an activation
 *   function, stacked per-expert parameters); [EPMASK] docstring
 *   (per-expert loop that skips experts with no tokens). The gate is
 *   SwiGLU: silu(z) = z / (1 + exp(-z)).
 *
 * Rows of slot s are a[offsets[s] .. offsets[s+1]) (offsets from
 * moe_permute, device array [S+1]); slots with no rows do no work.
 * op == MOE_GEMM_GATE_UP_SWIGLU:
 *   a [rows, H], w [S, 2*I, H] (rows 0..I-1 gate, rows I..2I-1 up),
 *   c [rows, I]: c[r, j] = silu(a[r].w[s,j]) * (a[r].w[s,I+j]).
 * op == MOE_GEMM_DOWN:
 *   a [rows, I], w [S, H, I], c [rows, H]: c[r, j] = a[r] . w[s, j].
 * Accumulation is f32; c is rounded once to dt. max_rows is the row
 * capacity of a and c (T*K from moe_permute); offsets[S] <= max_rows is a
 * device-data precondition (rows beyond max_rows are never touched).
 * H % 8 == 0 and I % 8 == 0. dt MOE_DTYPE_BF16 runs on the matrix cores
 * (MFMA); MOE_DTYPE_F32 uses a vector fused-multiply-add path.
 * One slot's gate/up panel, 2 * I * H elements, must be under 2^31 bytes
 * (MOE_ERR_UNSUPPORTED otherwise; the same limit holds for moe_forward and
 * moe_grouped_gemm_fp8 with their element sizes).
 * No workspace argument: the tile table of the grouped launch is rebuilt
 * by every block from `offsets` in its own shared memory.
 */
moe_status_t moe_grouped_gemm(moe_gemm_op_t op, moe_dtype_t dt, const void* a,
                              const int32_t* offsets, int S, int max_rows, const void* w,
                              int H, int I, void* c, hipStream_t stream);

/*
 * FP8 (E4M3) expert MLP.
 *   Source: [A2A] review of torch_moe.py: the FP8 (and NVFP4) MoE ops run
 *   the same routed template (routing, gated MLP per expert, output-side
 *   combine) with quantized expert linears. The pages give no quantization
 *   scheme; the one implemented here:
 *   - codes are OCP FP8 E4M3: s eeee mmm, value (-1)^s 2^(e-7) (1 + m/8) for
 *     e > 0, (-1)^s 2^-6 (m/8) for e = 0; s 1111 111 is NaN; max 448;
 *   - quantize(v, scale) = the E4M3 value nearest to
 *     clamp(fl32(v * fl32(1 / scale)), -448, 448), ties to the even code;
 *   - activations carry one scale per tensor, fixed ahead of time: a1 for
 *     the expert input x, a2 for the SwiGLU output; weights carry one scale
 *     per slot and matrix: w_scale[s] for the stacked gate/up rows, another
 *     array for down;
 *   - a linear layer computes (s_in * s_w) * sum_k dec(q_in[k]) dec(q_w[n,k])
 *     with f32 accumulation of the exact code products.
 */

/*
 * moe_quantize_fp8 -- q[i] = quantize(x[i], scale) for i < n.
 * x of x_dt (MOE_DTYPE_BF16 or MOE_DTYPE_F32) and q (bytes) are device
 * buffers, 16-byte aligned; scale must be finite and > 0. x must hold
 * finite values (a NaN input gives an unspecified code).
 */
moe_status_t moe_quantize_fp8(const void* x, moe_dtype_t x_dt, int64_t n, float scale,
                              uint8_t* q, hipStream_t stream);

/*
 * moe_grouped_gemm_fp8 -- moe_grouped_gemm on E4M3 codes.
 * a: codes [rows, H] (gate/up) or [rows, I] (down), scale a_scale; w: codes
 * laid out as for moe_grouped_gemm, slot s scaled by w_scale[s] (device f32
 * array [S]). op == MOE_GEMM_GATE_UP_SWIGLU: c holds codes [rows, I] of
 * quantize(silu(g) * u, c_scale), the SwiGLU evaluated in f32 on the scaled
 * accumulators g, u. op == MOE_GEMM_DOWN: c is bf16 [rows, H], the scaled
 * accumulator rounded once (c_scale unused). The contraction length (H for
 * gate/up, I for down) must be a multiple of 128 and at least 256
 * (MOE_ERR_UNSUPPORTED otherwise); scales finite and > 0; a, w, c 16-byte
 * aligned.
 */
moe_status_t moe_grouped_gemm_fp8(moe_gemm_op_t op, const uint8_t* a, float a_scale,
                                  const int32_t* offsets, int S, int max_rows, const uint8_t* w,
                                  const float* w_scale, int H, int I, void* c, float c_scale,
                                  hipStream_t stream);

/*
 * moe_combine -- weighted sum back into token order.
 *   Source: [AUTOTP] the routed output is the weighted sum of the selected
 *   experts' outputs, completed before the single reduction of the layer;
 *   [A2A] _template_moe applies the routing weights on the output side.
 *
 * acc[t] = sum over k = 0..K-1 ascending with pair_row[t*K+k] >= 0 of
 *          w_masked[t*K+k] * y[pair_row[t*K+k]]          (f32 accumulation)
 * accumulate == 0: out[t] = round(acc[t]);
 * accumulate != 0: out[t] = round(out[t] + acc[t])  (f32 add, then rounding).
 * Tokens without included pairs give 0 (or leave out unchanged when
 * accumulating). y [rows, H] of y_dt, out [T, H] of out_dt; rows referenced
 * by pair_row must exist in y (device-data precondition).
 */
moe_status_t moe_combine(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                         const float* w_masked, int T, int K, int H, void* out,
                         moe_dtype_t out_dt, int accumulate, hipStream_t stream);

/*
 * moe_combine_shared -- moe_combine with two options.
 *   Source: [EPMASK] ep_reduce_output: out = routed_out + shared_out before
 *   the layer's single reduction; [A2A] apply_routing_on_input (unit weights
 *   on the output side).
 * w_masked == NULL: every included pair has weight 1.
 * shared != NULL ([T, H] of shared_dt): acc[t] += shared[t] (f32) before
 *   the accumulate step and the single rounding.
 */
moe_status_t moe_combine_shared(const void* y, moe_dtype_t y_dt, const int32_t* pair_row,
                                const float* w_masked, int T, int K, int H, const void* shared,
                                moe_dtype_t shared_dt, void* out, moe_dtype_t out_dt,
                                int accumulate, hipStream_t stream);

/*
 * Fused forward: one call enqueues every stage in order on one stream.
 *   Source: [A2A] walkthrough sequence diagram: one fused MoE op is given the
 *   tokens, the selected experts and their routing weights (or computes the
 *   routing itself) and returns the layer's output; its MoE mapping
 *   configuration carries the EP size and rank and a max-num-tokens field
 *   that sizes the op's workspace (T_max here). [EPMASK] docstring and
 *   ep_mask_and_remap (the share's mask and remap); [SLOTS] Description
 *   (compute over engine-side slots); [AUTOTP] (the weighted sum formed
 *   before the layer's single reduction, so shares can be summed).
 */
typedef struct {
  int T_max;        /* largest T the workspace is sized for ([A2A] max num tokens) */
  int T;            /* tokens in this call, 0 <= T <= T_max */
  int H;            /* hidden size */
  int I;            /* expert intermediate size */
  int E_global;     /* routed experts in the whole layer */
  int K;            /* top-k */
  int renormalize;  /* renormalise the K selected weights to sum 1 */
  int ep_size;      /* expert-parallel ranks */
  int ep_rank;      /* this share's rank */
  int S;            /* slots held by this share */
  moe_dtype_t dtype;     /* x, weights and intermediates */
  moe_dtype_t out_dtype; /* out */
  int accumulate;   /* add into out instead of overwriting it */
  int num_expert_group; /* 0: plain top-K; else group-limited routing (moe_route_grouped) */
  int topk_group;       /* groups kept when num_expert_group > 0 */
  int routing_on_input; /* apply the routing weights to the expert input (see moe_permute_scaled) */
  float a1_scale;       /* dtype MOE_DTYPE_FP8_E4M3: scale of the quantized expert input */
  float a2_scale;       /* dtype MOE_DTYPE_FP8_E4M3: scale of the quantized SwiGLU output */
  int gemm_blocks;      /* 0: the grouped GEMMs run one persistent block per compute unit;
                           n > 0: at most n blocks, leaving the other compute units to work
                           queued on other streams (for instance a collective running beside
                           the layer). The output does not depend on it. Negative: error. */
} moe_config_t;

/* Stage boundaries at which moe_forward records the caller's events. */
enum {
  MOE_EV_START = 0,     /* before routing */
  MOE_EV_ROUTED = 1,    /* after route and slot map */
  MOE_EV_PERMUTED = 2,  /* after permute (index arrays and row gather) */
  MOE_EV_GATE_UP = 3,   /* after grouped GEMM 1 */
  MOE_EV_DOWN = 4,      /* after grouped GEMM 2 */
  MOE_EV_COMBINED = 5,  /* after combine */
  MOE_NUM_EVENTS = 6
};

typedef struct {
  const void* x;            /* [T, H] dtype */
  const float* logits;      /* [T, E_global]; NULL to pass ids/weights instead */
  const int32_t* topk_ids;  /* [T, K] used when logits == NULL ([A2A] fused op form) */
  const float* topk_w;      /* [T, K] used when logits == NULL */
  const void* w_gate_up;    /* [S, 2I, H] dtype, per slot */
  const void* w_down;       /* [S, H, I] dtype, per slot */
  const int32_t* rep_off;   /* [E_l + 1] or NULL for the identity table */
  const int32_t* rep_slots; /* [S] */
  void* out;                /* [T, H] out_dtype */
  hipEvent_t events[MOE_NUM_EVENTS]; /* optional; NULL entries are skipped */
  const void* shared_out;   /* [T, H] dtype or NULL: shared-expert output added in the combine */
  const float* w_gate_up_scale; /* dtype MOE_DTYPE_FP8_E4M3: [S] scales of w_gate_up */
  const float* w_down_scale;    /* dtype MOE_DTYPE_FP8_E4M3: [S] scales of w_down */
} moe_forward_args_t;

/*
 * moe_forward_workspace_size -- bytes of device workspace moe_forward needs
 * for cfg->T_max tokens (routing arrays, permutation, permuted rows and the
 * two intermediate activations). Returns 0 for an invalid configuration.
 *   Source: [A2A] MoE mapping configuration: the workspace is sized by the
 *   maximum number of tokens, so one allocation serves every call with
 *   T <= T_max.
 *
 * moe_forward -- route (or take topk_ids / topk_w), slot map, permute,
 * grouped GEMM 1, grouped GEMM 2 and combine, all enqueued on `stream`.
 * Routing from logits is moe_route, or moe_route_grouped when
 * cfg->num_expert_group > 0 (cfg->topk_group groups kept). With
 * cfg->routing_on_input the permutation is moe_permute_scaled and the combine
 * uses unit weights; args->shared_out, if given, is added in the combine.
 * Equivalent to calling the staged entry points in that order. Intermediate
 * activations are stored in cfg->dtype. The workspace layout is internal;
 * its contents on entry are ignored.
 * cfg->dtype == MOE_DTYPE_FP8_E4M3: x (and shared_out) are bf16; w_gate_up
 * and w_down are E4M3 codes with per-slot scales args->w_gate_up_scale and
 * args->w_down_scale; x is quantized with cfg->a1_scale (moe_quantize_fp8),
 * the grouped GEMMs are moe_grouped_gemm_fp8 with the SwiGLU output
 * quantized with cfg->a2_scale, and the expert outputs are bf16. H and I
 * must be multiples of 128 and at least 256; routing_on_input is not
 * supported with FP8 (MOE_ERR_UNSUPPORTED).
 */
size_t moe_forward_workspace_size(const moe_config_t* cfg);
moe_status_t moe_forward(const moe_config_t* cfg, const moe_forward_args_t* args, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * All-to-all dispatch of expert parallelism (send and return side on one
 * device; the transport between ranks is not part of this library).
 *   Source: [A2A] walkthrough sequence diagram: tokens are dispatched to the
 *   ranks responsible for their experts, each rank computes the MoE on its
 *   local experts and the results are gathered back; the mapping
 *   configuration's max-num-tokens field sizes the exchange workspace.
 *   [EPMASK] _ep_init: rank r owns experts [r*E_l, (r+1)*E_l), E_l =
 *   E_global / ep_size.
 *
 * moe_a2a_dispatch packs the send buffers. A token t goes once to every rank
 * that owns at least one of its valid experts (0 <= topk_ids[t*K+k] <
 * E_global); rank r's block is rows [r*cap, (r+1)*cap) of the send arrays,
 * tokens in ascending order. cap >= T is required (a block then never
 * overflows; size it by the largest token count, as the max-num-tokens field
 * does). Outputs (bit-exact):
 *   offsets [ep_size + 1]: offsets[r] = tokens sent to ranks < r (so rank r
 *     receives offsets[r+1] - offsets[r] tokens);
 *   token_pos [T * ep_size]: the send row of token t for rank r, or -1;
 *   send_token [ep_size * cap]: the token in each row, or -1 if unused;
 *   send_x [ep_size * cap, H] (dtype dt): send_x[row] = x[send_token[row]]
 *     bit for bit (unused rows untouched);
 *   send_ids, send_w [ep_size * cap, K]: the token's topk_ids / topk_w, or
 *     -1 / 0 in unused rows, so a receiving moe_forward over the whole block
 *     (topk form, its own ep_rank) excludes the unused rows.
 * x, send_x: H * sizeof(dt) a multiple of 16 bytes, 16-byte aligned.
 * ws: at least moe_a2a_dispatch_workspace_size(T, ep_size, cap) bytes.
 * Limits: 1 <= ep_size <= MOE_MAX_A2A_RANKS, E_global % ep_size == 0,
 * 1 <= K <= MOE_MAX_TOPK.
 *
 * moe_a2a_combine gathers the ranks' partial outputs back into token order:
 *   out[t] = round(sum over r = 0..ep_size-1 ascending with
 *                  token_pos[t*ep_size + r] >= 0 of partial[token_pos[...]])
 * with f32 accumulation and one rounding to out_dt. partial [ep_size*cap, H]
 * of partial_dt (f32 keeps the single rounding); tokens sent nowhere give 0.
 */
size_t moe_a2a_dispatch_workspace_size(int T, int ep_size, int cap);
moe_status_t moe_a2a_dispatch(const void* x, moe_dtype_t dt, int T, int H, int K,
                              const int32_t* topk_ids, const float* topk_w, int E_global,
                              int ep_size, int cap, int32_t* offsets, int32_t* token_pos,
                              int32_t* send_token, void* send_x, int32_t* send_ids,
                              float* send_w, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status_t moe_a2a_combine(const void* partial, moe_dtype_t partial_dt,
                             const int32_t* token_pos, int T, int ep_size, int H, void* out,
                             moe_dtype_t out_dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
