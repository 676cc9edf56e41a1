"""Python binding of the MI355X fused MoE forward library (libmoe_hip.so).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), their device pointers and torch's current HIP stream are passed
to the C ABI declared in include/moe.h, and a non-OK status is raised as
RuntimeError. Every computation runs in the library's HIP kernels; torch
provides device memory and the stream. Calls are asynchronous on the current
stream, exactly like the C entry points.

If the library has not been built, every call raises RuntimeError; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "MOE_DTYPE_F32", "MOE_DTYPE_BF16", "GATE_UP_SWIGLU", "DOWN", "NUM_EVENTS",
    "lib", "library_path", "status_str",
    "route", "slot_map", "permute", "permute_noalloc", "permute_workspace_size",
    "grouped_gemm", "combine",
    "forward", "forward_workspace_size", "ForwardConfig",
    "a2a_dispatch", "a2a_dispatch_workspace_size", "a2a_combine",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_HIP_LIBRARY selects another build of the same library (the tests use it
# for a host-sanitized build); it must exist like the default one.
_LIB_FILE = os.environ.get("MOE_HIP_LIBRARY") or os.path.join(_HERE, "libmoe_hip.so")

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DTYPE_FP8_E4M3 = 2
GATE_UP_SWIGLU = 0
DOWN = 1
NUM_EVENTS = 6
MAX_EXPERTS = 1024
MAX_TOPK = 32
MAX_SLOTS = 1024

_DT = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16,
       torch.float8_e4m3fn: MOE_DTYPE_FP8_E4M3}
FP8 = torch.float8_e4m3fn  # ForwardConfig dtype of the FP8 expert path
_CODES = (torch.uint8, torch.float8_e4m3fn)  # tensors holding E4M3 codes
_TORCH_DT = {MOE_DTYPE_F32: torch.float32, MOE_DTYPE_BF16: torch.bfloat16}

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class _Config(ctypes.Structure):
    _fields_ = [("T_max", _i), ("T", _i), ("H", _i), ("I", _i), ("E_global", _i), ("K", _i),
                ("renormalize", _i), ("ep_size", _i), ("ep_rank", _i), ("S", _i),
                ("dtype", _i), ("out_dtype", _i), ("accumulate", _i),
                ("num_expert_group", _i), ("topk_group", _i), ("routing_on_input", _i),
                ("a1_scale", ctypes.c_float), ("a2_scale", ctypes.c_float),
                ("gemm_blocks", _i)]


class _ForwardArgs(ctypes.Structure):
    _fields_ = [("x", _p), ("logits", _p), ("topk_ids", _p), ("topk_w", _p),
                ("w_gate_up", _p), ("w_down", _p), ("rep_off", _p), ("rep_slots", _p),
                ("out", _p), ("events", _p * NUM_EVENTS), ("shared_out", _p),
                ("w_gate_up_scale", _p), ("w_down_scale", _p)]


_SIGS = {
    "moe_status_str": (ctypes.c_char_p, [_i]),
    "moe_route": (_i, [_p, _i, _i, _i, _i, _p, _p, _p]),
    "moe_route_grouped": (_i, [_p, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "moe_slot_map": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p]),
    "moe_permute_workspace_size": (_sz, [_i, _i, _i]),
    "moe_permute": (_i, [_p, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_permute_scaled": (_i, [_p, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p, _p, _sz,
                                _p]),
    "moe_permute_noalloc": (_i, [_p, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p]),
    "moe_grouped_gemm": (_i, [_i, _i, _p, _p, _i, _i, _p, _i, _i, _p, _p]),
    "moe_combine": (_i, [_p, _i, _p, _p, _i, _i, _i, _p, _i, _i, _p]),
    "moe_combine_shared": (_i, [_p, _i, _p, _p, _i, _i, _i, _p, _i, _p, _i, _i, _p]),
    "moe_forward_workspace_size": (_sz, [ctypes.POINTER(_Config)]),
    "moe_forward": (_i, [ctypes.POINTER(_Config), ctypes.POINTER(_ForwardArgs), _p, _sz, _p]),
    "moe_a2a_dispatch_workspace_size": (_sz, [_i, _i, _i]),
    "moe_a2a_dispatch": (_i, [_p, _i, _i, _i, _i, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _p,
                              _p, _sz, _p]),
    "moe_a2a_combine": (_i, [_p, _i, _p, _i, _i, _i, _p, _i, _p]),
    "moe_quantize_fp8": (_i, [_p, _i, ctypes.c_int64, ctypes.c_float, _p, _p]),
    "moe_grouped_gemm_fp8": (_i, [_i, _p, ctypes.c_float, _p, _i, _i, _p, _p, _i, _i, _p,
                                  ctypes.c_float, _p]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


def library_path() -> str:
    return _LIB_FILE


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_FILE):
            raise RuntimeError(
                f"{_LIB_FILE} is missing: build it with `python -m moe_expert_dispatch_amd.build`; "
                "there is no non-HIP fallback")
        so = ctypes.CDLL(_LIB_FILE)
        for name, (res, args) in _SIGS.items():
            fn = getattr(so, name)
            fn.restype = res
            fn.argtypes = args
        _lib = so
    return _lib


def status_str(code: int) -> str:
    return lib().moe_status_str(code).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what}: {status_str(code)}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {ok}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------- stages
def route(logits: torch.Tensor, K: int, renormalize: bool,
          ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
          num_groups: int = 0, topk_groups: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """moe_route (or moe_route_grouped when num_groups > 0):
    logits [T, E] f32 -> (ids [T, K] int32, w [T, K] f32)."""
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    ids = _empty((T, K), torch.int32, logits) if ids is None else _dev(ids, "ids", torch.int32, (T, K))
    w = _empty((T, K), torch.float32, logits) if w is None else _dev(w, "w", torch.float32, (T, K))
    if num_groups:
        _check(lib().moe_route_grouped(_ptr(logits), T, E, K, int(bool(renormalize)), num_groups,
                                       topk_groups, _ptr(ids), _ptr(w), _stream()),
               "moe_route_grouped")
    else:
        _check(lib().moe_route(_ptr(logits), T, E, K, int(bool(renormalize)), _ptr(ids),
                               _ptr(w), _stream()), "moe_route")
    return ids, w


def slot_map(ids: torch.Tensor, w: torch.Tensor, E_global: int, ep_size: int = 1,
             ep_rank: int = 0, rep_off: Optional[torch.Tensor] = None,
             rep_slots: Optional[torch.Tensor] = None, S: Optional[int] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """moe_slot_map -> (slot [T,K] int32, w_masked [T,K] f32, mask [T,K] uint8)."""
    _dev(ids, "ids", torch.int32)
    if ids.dim() != 2:
        raise ValueError("ids must be [T, K]")
    T, K = ids.shape
    _dev(w, "w", torch.float32, (T, K))
    if rep_off is not None:
        _dev(rep_off, "rep_off", torch.int32)
        _dev(rep_slots, "rep_slots", torch.int32)
        S = rep_slots.numel() if S is None else S
    elif S is None:
        S = E_global // max(ep_size, 1)
    slot = _empty((T, K), torch.int32, ids)
    wm = _empty((T, K), torch.float32, ids)
    mask = _empty((T, K), torch.uint8, ids)
    _check(lib().moe_slot_map(_ptr(ids), _ptr(w), T, K, E_global, ep_size, ep_rank,
                              _ptr(rep_off), _ptr(rep_slots), S, _ptr(slot), _ptr(wm),
                              _ptr(mask), _stream()), "moe_slot_map")
    return slot, wm, mask


def permute_workspace_size(T: int, K: int, S: int) -> int:
    return int(lib().moe_permute_workspace_size(T, K, S))


def permute(x: torch.Tensor, slot: torch.Tensor, mask: torch.Tensor, S: int,
            gather: bool = True, ws: Optional[torch.Tensor] = None,
            pair_w: Optional[torch.Tensor] = None):
    """moe_permute -> (offsets [S+1], sorted_pairs [T*K], pair_row [T*K], x_perm [T*K, H] or None).

    Only rows [0, offsets[S]) of x_perm and sorted_pairs are written. With
    pair_w [T, K] f32 (moe_permute_scaled) each row is pair_w[p] * x[p / K]."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(slot, "slot", torch.int32)
    T, K = slot.shape
    _dev(mask, "mask", torch.uint8, (T, K))
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T matching slot")
    H = x.shape[1]
    offsets = _empty((S + 1,), torch.int32, x)
    sorted_pairs = _empty((T * K,), torch.int32, x)
    pair_row = _empty((T * K,), torch.int32, x)
    x_perm = _empty((T * K, H), x.dtype, x) if gather else None
    need = permute_workspace_size(T, K, S)
    if ws is None:
        ws = _empty((max(need, 1),), torch.uint8, x)
    if pair_w is not None:
        _dev(pair_w, "pair_w", torch.float32, (T, K))
        if x_perm is None:
            raise ValueError("pair_w needs the row gather")
        _check(lib().moe_permute_scaled(_ptr(x), _DT[x.dtype], T, H, K, _ptr(slot), _ptr(mask),
                                        S, _ptr(pair_w), _ptr(offsets), _ptr(sorted_pairs),
                                        _ptr(pair_row), _ptr(x_perm), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream()),
               "moe_permute_scaled")
    else:
        _check(lib().moe_permute(_ptr(x), _DT[x.dtype], T, H, K, _ptr(slot), _ptr(mask), S,
                                 _ptr(offsets), _ptr(sorted_pairs), _ptr(pair_row),
                                 _ptr(x_perm), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream()), "moe_permute")
    return offsets, sorted_pairs, pair_row, x_perm


def permute_noalloc(x: torch.Tensor, slot: torch.Tensor, mask: torch.Tensor, S: int,
                    gather: bool = True, out=None):
    """moe_permute_noalloc: moe_permute with the library's static histogram
    memory (no workspace). `out` may pass preallocated (offsets, sorted_pairs,
    pair_row, x_perm) so that the call itself allocates nothing."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(slot, "slot", torch.int32)
    T, K = slot.shape
    _dev(mask, "mask", torch.uint8, (T, K))
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T matching slot")
    H = x.shape[1]
    if out is None:
        out = (_empty((S + 1,), torch.int32, x), _empty((T * K,), torch.int32, x),
               _empty((T * K,), torch.int32, x),
               _empty((T * K, H), x.dtype, x) if gather else None)
    offsets, sorted_pairs, pair_row, x_perm = out
    _dev(offsets, "offsets", torch.int32, (S + 1,))
    _dev(sorted_pairs, "sorted_pairs", torch.int32, (T * K,))
    _dev(pair_row, "pair_row", torch.int32, (T * K,))
    if x_perm is not None:
        _dev(x_perm, "x_perm", x.dtype, (T * K, H))
    _check(lib().moe_permute_noalloc(_ptr(x), _DT[x.dtype], T, H, K, _ptr(slot), _ptr(mask), S,
                                     _ptr(offsets), _ptr(sorted_pairs), _ptr(pair_row),
                                     _ptr(x_perm), _stream()), "moe_permute_noalloc")
    return offsets, sorted_pairs, pair_row, x_perm


def grouped_gemm(op: int, a: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor,
                 c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_grouped_gemm. op GATE_UP_SWIGLU: a [rows, H], w [S, 2I, H] -> c [rows, I];
    op DOWN: a [rows, I], w [S, H, I] -> c [rows, H]."""
    _dev(a, "a", (torch.float32, torch.bfloat16))
    _dev(w, "w", a.dtype)
    _dev(offsets, "offsets", torch.int32)
    if a.dim() != 2 or w.dim() != 3:
        raise ValueError("a must be 2-D and w 3-D")
    S = w.shape[0]
    if offsets.numel() != S + 1:
        raise ValueError("offsets must have S + 1 entries")
    rows = a.shape[0]
    if op == GATE_UP_SWIGLU:
        H = a.shape[1]
        I = w.shape[1] // 2
        if w.shape[2] != H or w.shape[1] != 2 * I:
            raise ValueError("w must be [S, 2I, H]")
        N = I
    elif op == DOWN:
        I = a.shape[1]
        H = w.shape[1]
        if w.shape[2] != I:
            raise ValueError("w must be [S, H, I]")
        N = H
    else:
        raise ValueError("op must be GATE_UP_SWIGLU or DOWN")
    c = _empty((rows, N), a.dtype, a) if c is None else _dev(c, "c", a.dtype, (rows, N))
    _check(lib().moe_grouped_gemm(op, _DT[a.dtype], _ptr(a), _ptr(offsets), S, rows, _ptr(w),
                                  H, I, _ptr(c), _stream()), "moe_grouped_gemm")
    return c


def quantize_fp8(x: torch.Tensor, scale: float, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_quantize_fp8: E4M3 codes (uint8, shape of x) of x (bf16 or f32) / scale."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    q = _empty(tuple(x.shape), torch.uint8, x) if q is None else _dev(q, "q", _CODES, x.shape)
    _check(lib().moe_quantize_fp8(_ptr(x), _DT[x.dtype], x.numel(), float(scale), _ptr(q),
                                  _stream()), "moe_quantize_fp8")
    return q


def grouped_gemm_fp8(op: int, a: torch.Tensor, a_scale: float, offsets: torch.Tensor,
                     w: torch.Tensor, w_scale: torch.Tensor, c_scale: float = 1.0,
                     c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_grouped_gemm_fp8. Codes a [rows, H] / [rows, I] and w (as grouped_gemm),
    f32 w_scale [S]. GATE_UP_SWIGLU -> codes [rows, I] quantized with c_scale;
    DOWN -> bf16 [rows, H]."""
    _dev(a, "a", _CODES)
    _dev(w, "w", _CODES)
    _dev(offsets, "offsets", torch.int32)
    if a.dim() != 2 or w.dim() != 3:
        raise ValueError("a must be 2-D and w 3-D")
    S = w.shape[0]
    _dev(w_scale, "w_scale", torch.float32, (S,))
    if offsets.numel() != S + 1:
        raise ValueError("offsets must have S + 1 entries")
    rows = a.shape[0]
    if op == GATE_UP_SWIGLU:
        H, I = a.shape[1], w.shape[1] // 2
        if w.shape[2] != H or w.shape[1] != 2 * I:
            raise ValueError("w must be [S, 2I, H]")
        shape, cdt = (rows, I), _CODES
    elif op == DOWN:
        I, H = a.shape[1], w.shape[1]
        if w.shape[2] != I:
            raise ValueError("w must be [S, H, I]")
        shape, cdt = (rows, H), torch.bfloat16
    else:
        raise ValueError("op must be GATE_UP_SWIGLU or DOWN")
    if c is None:
        c = _empty(shape, torch.uint8 if op == GATE_UP_SWIGLU else torch.bfloat16, a)
    else:
        _dev(c, "c", cdt, shape)
    _check(lib().moe_grouped_gemm_fp8(op, _ptr(a), float(a_scale), _ptr(offsets), S, rows,
                                      _ptr(w), _ptr(w_scale), H, I, _ptr(c), float(c_scale),
                                      _stream()), "moe_grouped_gemm_fp8")
    return c


def combine(y: torch.Tensor, pair_row: torch.Tensor, w_masked: Optional[torch.Tensor], K: int,
            out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
            accumulate: bool = False, shared: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_combine: out[t] (+)= sum_k w_masked[t,k] * y[pair_row[t,k]].
    w_masked None (unit weights) or shared [T, H] (added before the rounding)
    use moe_combine_shared."""
    _dev(y, "y", (torch.float32, torch.bfloat16))
    _dev(pair_row, "pair_row", torch.int32)
    P = pair_row.numel()
    if w_masked is not None:
        _dev(w_masked, "w_masked", torch.float32)
        if w_masked.numel() != P:
            raise ValueError("pair_row / w_masked must hold T*K entries")
    if P % K != 0:
        raise ValueError("pair_row must hold T*K entries")
    T = P // K
    H = y.shape[1]
    if out is None:
        out = _empty((T, H), out_dtype or y.dtype, y)
        if accumulate:
            out.zero_()
    else:
        _dev(out, "out", (torch.float32, torch.bfloat16), (T, H))
    if w_masked is None or shared is not None:
        sdt = MOE_DTYPE_BF16
        if shared is not None:
            _dev(shared, "shared", (torch.float32, torch.bfloat16), (T, H))
            sdt = _DT[shared.dtype]
        _check(lib().moe_combine_shared(_ptr(y), _DT[y.dtype], _ptr(pair_row), _ptr(w_masked), T,
                                        K, H, _ptr(shared), sdt, _ptr(out), _DT[out.dtype],
                                        int(bool(accumulate)), _stream()), "moe_combine_shared")
    else:
        _check(lib().moe_combine(_ptr(y), _DT[y.dtype], _ptr(pair_row), _ptr(w_masked), T, K,
                                 H, _ptr(out), _DT[out.dtype], int(bool(accumulate)),
                                 _stream()), "moe_combine")
    return out


# ---------------------------------------------------------------- fused
class ForwardConfig:
    """Plain mirror of moe_config_t."""

    def __init__(self, T: int, H: int, I: int, E_global: int, K: int, renormalize: bool,
                 S: int, dtype: torch.dtype, out_dtype: Optional[torch.dtype] = None,
                 ep_size: int = 1, ep_rank: int = 0, accumulate: bool = False,
                 T_max: Optional[int] = None, num_expert_group: int = 0, topk_group: int = 0,
                 routing_on_input: bool = False, a1_scale: float = 1.0, a2_scale: float = 1.0,
                 gemm_blocks: int = 0):
        self.T, self.H, self.I, self.E_global, self.K = T, H, I, E_global, K
        self.renormalize, self.S, self.dtype = bool(renormalize), S, dtype
        # FP8 (dtype FP8): x, shared_out and the default out are bf16
        self.out_dtype = out_dtype or (torch.bfloat16 if dtype == FP8 else dtype)
        self.a1_scale, self.a2_scale = float(a1_scale), float(a2_scale)
        self.ep_size, self.ep_rank, self.accumulate = ep_size, ep_rank, bool(accumulate)
        self.T_max = T if T_max is None else T_max
        self.num_expert_group, self.topk_group = num_expert_group, topk_group
        self.routing_on_input = bool(routing_on_input)
        self.gemm_blocks = int(gemm_blocks)  # 0: one persistent GEMM block per compute unit

    def c_struct(self) -> _Config:
        return _Config(self.T_max, self.T, self.H, self.I, self.E_global, self.K,
                       int(self.renormalize), self.ep_size, self.ep_rank, self.S,
                       _DT[self.dtype], _DT[self.out_dtype], int(self.accumulate),
                       self.num_expert_group, self.topk_group, int(self.routing_on_input),
                       self.a1_scale, self.a2_scale, self.gemm_blocks)


def forward_workspace_size(cfg: ForwardConfig) -> int:
    c = cfg.c_struct()
    n = int(lib().moe_forward_workspace_size(ctypes.byref(c)))
    if n == 0:
        raise RuntimeError("moe_forward_workspace_size: invalid configuration")
    return n


def forward(cfg: ForwardConfig, x: torch.Tensor, w_gate_up: torch.Tensor, w_down: torch.Tensor,
            logits: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
            topk_w: Optional[torch.Tensor] = None, rep_off: Optional[torch.Tensor] = None,
            rep_slots: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            ws: Optional[torch.Tensor] = None, events: Optional[Sequence[int]] = None,
            shared_out: Optional[torch.Tensor] = None,
            w_gate_up_scale: Optional[torch.Tensor] = None,
            w_down_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward. Pass logits [T, E_global] f32, or topk_ids [T, K] int32 and
    topk_w [T, K] f32. Weights are per slot: w_gate_up [S, 2I, H], w_down [S, H, I].
    `events`: up to NUM_EVENTS raw hipEvent_t handles (0 = skip) recorded at the
    stage boundaries. cfg.dtype FP8: x is bf16, the weights are E4M3 codes
    (uint8 or float8_e4m3fn) with f32 per-slot scales w_gate_up_scale,
    w_down_scale [S]."""
    T, H, I, S = cfg.T, cfg.H, cfg.I, cfg.S
    fp8 = cfg.dtype == FP8
    xdt = torch.bfloat16 if fp8 else cfg.dtype
    wdt = _CODES if fp8 else cfg.dtype
    _dev(x, "x", xdt, (T, H))
    _dev(w_gate_up, "w_gate_up", wdt, (S, 2 * I, H))
    _dev(w_down, "w_down", wdt, (S, H, I))
    if fp8:
        _dev(w_gate_up_scale, "w_gate_up_scale", torch.float32, (S,))
        _dev(w_down_scale, "w_down_scale", torch.float32, (S,))
    if logits is not None:
        _dev(logits, "logits", torch.float32, (T, cfg.E_global))
    else:
        _dev(topk_ids, "topk_ids", torch.int32, (T, cfg.K))
        _dev(topk_w, "topk_w", torch.float32, (T, cfg.K))
    if rep_off is not None:
        _dev(rep_off, "rep_off", torch.int32, (cfg.E_global // cfg.ep_size + 1,))
        _dev(rep_slots, "rep_slots", torch.int32, (S,))
    if out is None:
        out = _empty((T, H), cfg.out_dtype, x)
        if cfg.accumulate:
            out.zero_()
    else:
        _dev(out, "out", cfg.out_dtype, (T, H))
    need = forward_workspace_size(cfg)
    if ws is None:
        ws = _empty((need,), torch.uint8, x)
    ev = (_p * NUM_EVENTS)(*([0] * NUM_EVENTS))
    if events is not None:
        for i, e in enumerate(list(events)[:NUM_EVENTS]):
            ev[i] = e or 0
    if shared_out is not None:
        _dev(shared_out, "shared_out", xdt, (T, H))
    args = _ForwardArgs(_ptr(x), _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate_up),
                        _ptr(w_down), _ptr(rep_off), _ptr(rep_slots), _ptr(out), ev,
                        _ptr(shared_out), _ptr(w_gate_up_scale), _ptr(w_down_scale))
    c = cfg.c_struct()
    _check(lib().moe_forward(ctypes.byref(c), ctypes.byref(args), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream()), "moe_forward")
    return out


# ---------------------------------------------------------------- all-to-all
def a2a_dispatch_workspace_size(T: int, ep_size: int, cap: int) -> int:
    return int(lib().moe_a2a_dispatch_workspace_size(T, ep_size, cap))


def a2a_dispatch(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, E_global: int,
                 ep_size: int, cap: Optional[int] = None, ws: Optional[torch.Tensor] = None):
    """moe_a2a_dispatch -> (offsets [ep+1], token_pos [T, ep], send_token [ep*cap],
    send_x [ep*cap, H], send_ids [ep*cap, K], send_w [ep*cap, K]).

    Rank r's block is rows [r*cap, (r+1)*cap); cap defaults to T."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(topk_ids, "topk_ids", torch.int32)
    T, K = topk_ids.shape
    _dev(topk_w, "topk_w", torch.float32, (T, K))
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T matching topk_ids")
    H = x.shape[1]
    cap = T if cap is None else cap
    offsets = _empty((ep_size + 1,), torch.int32, x)
    token_pos = _empty((T, ep_size), torch.int32, x)
    send_token = _empty((ep_size * cap,), torch.int32, x)
    send_x = _empty((ep_size * cap, H), x.dtype, x)
    send_ids = _empty((ep_size * cap, K), torch.int32, x)
    send_w = _empty((ep_size * cap, K), torch.float32, x)
    need = a2a_dispatch_workspace_size(T, ep_size, cap)
    if ws is None:
        ws = _empty((max(need, 1),), torch.uint8, x)
    _check(lib().moe_a2a_dispatch(_ptr(x), _DT[x.dtype], T, H, K, _ptr(topk_ids), _ptr(topk_w),
                                  E_global, ep_size, cap, _ptr(offsets), _ptr(token_pos),
                                  _ptr(send_token), _ptr(send_x), _ptr(send_ids), _ptr(send_w),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "moe_a2a_dispatch")
    return offsets, token_pos, send_token, send_x, send_ids, send_w


def a2a_combine(partial: torch.Tensor, token_pos: torch.Tensor,
                out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """moe_a2a_combine: out[t] = sum over ranks r (ascending) with
    token_pos[t, r] >= 0 of partial[token_pos[t, r]]."""
    _dev(partial, "partial", (torch.float32, torch.bfloat16))
    _dev(token_pos, "token_pos", torch.int32)
    T, ep_size = token_pos.shape
    H = partial.shape[1]
    out = _empty((T, H), out_dtype or partial.dtype, partial)
    _check(lib().moe_a2a_combine(_ptr(partial), _DT[partial.dtype], _ptr(token_pos), T, ep_size,
                                 H, _ptr(out), _DT[out.dtype], _stream()), "moe_a2a_combine")
    return out
