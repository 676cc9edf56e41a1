"""CPU oracle of the FP8 (E4M3) expert MLP path (numpy).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or call this module; the product path never does.
It shares no code with the HIP library.

Page: [A2A] TensorRT-LLM PR #10985 "MoE all-to-all paradigm", review of
torch_moe.py: the FP8 and NVFP4 MoE ops run the same routed template as the
unquantized op (same routing, gated MLP per expert, output-side combine),
with quantized expert linears. The pages give no quantization scheme; the
reading taken here (the plainest one that keeps every other step unchanged):

  - format: OCP FP8 E4M3. Code bits s eeee mmm; e > 0: (-1)^s 2^(e-7) (1 + m/8);
    e = 0: (-1)^s 2^-6 (m/8); s 1111 111 is NaN; no infinities; largest
    finite magnitude 448 (code 0x7e).
  - quantize(v, scale): p = fl32(v * fl32(1/scale)), clamped to [-448, 448],
    rounded to the nearest E4M3 value, ties to the even code.
  - one scale per tensor for activations, fixed ahead of time ("static"):
    a1 for the expert input x, a2 for the SwiGLU output; one scale per slot
    for each weight matrix: s_gu[s] for the stacked gate/up rows, s_d[s] for
    down.
  - linear layer: out[n] = (s_in * s_w) * sum_k dec(q_in[k]) * dec(q_w[n, k]).
  - expert MLP: g, u from the quantized input row with scale a1 * s_gu;
    a = silu(g) * u; the down linear takes quantize(a, a2) with scale
    a2 * s_d; y in the output dtype. The quantization of a is decided in f32
    (the value a rounded to f32, then the f32 product), as the kernel does.
Precision: products and sums in fp64 on exactly decoded values.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .moe_oracle import _f64, _i64, _take_rows, ep_mask_and_remap, ep_partition, route, silu

E4M3_MAX = 448.0


def _decode_fields(codes) -> np.ndarray:
    """fp64 values of E4M3 codes by the bit-field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


# the definition evaluated once for each of the 256 codes
_DECODED = _decode_fields(np.arange(256))


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (uint8 array-like): the bit-field definition,
    looked up per code (large weight tensors decode in one indexing pass)."""
    return _DECODED[np.asarray(codes, dtype=np.uint8)]


# magnitudes of the non-negative finite codes 0x00..0x7e, in code order
# (strictly increasing: the exponent field is above the mantissa field)
_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), magnitudes
    beyond 448 saturated to 448. `v` holds finite numbers; -0.0 maps to 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, _POS.size - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantize_fp8(x, scale: float) -> np.ndarray:
    """quantize(v, scale) of the reading above for every element of x (an
    array or CPU tensor of bf16 / f32 values): f32 product with the f32
    reciprocal of the scale, clamp, round to E4M3."""
    xf = _f64(x).astype(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    p = (xf * inv).astype(np.float32)
    p = np.clip(p, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(p)


def fp8_linear(q_in, s_in: float, q_w, s_w: float) -> np.ndarray:
    """(s_in * s_w) * dec(q_in) @ dec(q_w)^T: q_in [n, K] codes, q_w [N, K] codes."""
    return (float(s_in) * float(s_w)) * (e4m3_decode(q_in) @ e4m3_decode(q_w).T)


def fp8_grouped_gate_up(aq, offsets, wq_gate_up, a_scale: float, w_scale, I: int) -> np.ndarray:
    """Stage form of the FP8 grouped gate/up GEMM: rows [offsets[s], offsets[s+1])
    of the codes aq [rows, H] use slot s's codes wq_gate_up[s] ([2I, H]) and
    scale w_scale[s]; returns the SwiGLU output a = silu(g) * u (fp64), before
    its quantization."""
    aq = np.asarray(aq, dtype=np.uint8)
    off = _i64(offsets)
    ws = _f64(w_scale)
    out = np.zeros((aq.shape[0], I))
    for s in range(off.size - 1):
        lo, hi = off[s], off[s + 1]
        if hi > lo:
            w = np.asarray(wq_gate_up[s], dtype=np.uint8)
            g = fp8_linear(aq[lo:hi], a_scale, w[:I], ws[s])
            u = fp8_linear(aq[lo:hi], a_scale, w[I:], ws[s])
            out[lo:hi] = silu(g) * u
    return out


def fp8_grouped_down(aq, offsets, wq_down, a_scale: float, w_scale) -> np.ndarray:
    """Stage form of the FP8 grouped down GEMM: codes aq [rows, I] of slot s
    times slot s's codes wq_down[s] ([H, I]), scale a_scale * w_scale[s]."""
    aq = np.asarray(aq, dtype=np.uint8)
    off = _i64(offsets)
    ws = _f64(w_scale)
    H = np.asarray(wq_down[0]).shape[0] if off[-1] > 0 else 0
    out = np.zeros((aq.shape[0], H))
    for s in range(off.size - 1):
        lo, hi = off[s], off[s + 1]
        if hi > lo:
            out[lo:hi] = fp8_linear(aq[lo:hi], a_scale, np.asarray(wq_down[s], np.uint8), ws[s])
    return out


def fp8_expert_mlp(xq, a1: float, wq_gate_up, s_gu: float, wq_down, s_d: float, a2: float,
                   return_act: bool = False):
    """One expert's FP8 MLP on quantized input rows xq [n, H] (codes):
    y = a2 s_d * dec(quantize(silu(g) * u, a2)) @ dec(wq_down)^T."""
    wgu = np.asarray(wq_gate_up, dtype=np.uint8)
    I = wgu.shape[0] // 2
    g = fp8_linear(xq, a1, wgu[:I], s_gu)
    u = fp8_linear(xq, a1, wgu[I:], s_gu)
    a = silu(g) * u
    aq = quantize_fp8(a.astype(np.float32), a2)  # the decision in f32
    y = fp8_linear(aq, a2, wq_down, s_d)
    return (y, a, aq) if return_act else y


def fp8_forward(x, logits, wq_gate_up, s_gate_up, wq_down, s_down, a1: float, a2: float,
                K: int, renormalize: bool, ep_size: int = 1, ep_rank: int = 0,
                tokens: Optional[Sequence[int]] = None,
                topk: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                shared=None) -> np.ndarray:
    """Output rows for `tokens` (default: all), fp64 [n, H], of the FP8 MoE layer.

    x [T, H] (bf16 / f32 values) is quantized with a1; wq_gate_up [E, 2I, H]
    and wq_down [E, H, I] are E4M3 codes indexed by global expert id, with
    per-expert scales s_gate_up [E], s_down [E]. Routing, EP masking and the
    combine are those of the unquantized layer."""
    T = (logits.shape[0] if topk is None else np.asarray(topk[0]).shape[0])
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    if topk is None:
        ids, w = route(_f64(logits)[tok], K, renormalize)
    else:
        ids, w = np.asarray(topk[0])[tok], _f64(topk[1])[tok]
    E_global = np.asarray(wq_gate_up).shape[0]
    E_local, start = ep_partition(E_global, ep_size, ep_rank)
    _, w_masked, mask = ep_mask_and_remap(ids, w, start, E_local)
    xq = quantize_fp8(_take_rows(x, tok), a1)
    n, H = xq.shape
    sgu, sd = _f64(s_gate_up), _f64(s_down)
    y = np.zeros((n, K, H))
    for e in range(start, start + E_local):
        sel = np.nonzero((ids == e) & mask)
        if sel[0].size == 0:
            continue
        y[sel] = fp8_expert_mlp(xq[sel[0]], a1, wq_gate_up[e], sgu[e], wq_down[e], sd[e], a2)
    out = np.zeros((n, H))
    for k in range(K):
        m = mask[:, k]
        out[m] += w_masked[m, k, None] * y[m, k]
    if shared is not None:
        out += _f64(_take_rows(shared, tok))
    return out
