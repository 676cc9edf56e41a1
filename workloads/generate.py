"""Seeded input generation (torch CPU generators, fp32 draws).

Recipe, per workload (all draws fp32 from torch.Generator on the CPU, then
cast to bf16 with round-to-nearest-even where the workload is bf16):
  x              [T, H]  ~ N(0, 1)
  router         "gauss":      W_r [E, H] ~ N(0, 1/sqrt(H)); logits = x W_r^T
                 "gauss_bias": as "gauss" plus a per-expert bias b ~ N(0, bias_std)
                 "zipf":       a seeded permutation pi of the experts gives each
                               expert its popularity rank; p_e ∝ (pi(e)+1)^-s;
                               logits[t, e] = log p_e + g[t, e], g ~ Gumbel(0, 1)
                               i.i.d., so each token's top-K experts are a draw
                               without replacement with probabilities ∝ p.
                 The router product is evaluated in fp64 from the stored
                 (already cast) x and rounded once to fp32: the logits are the
                 method's input, identical for every implementation.
  expert weights per expert e: gate, up [I, H] ~ N(0, 1/sqrt(H)),
                 down [H, I] ~ N(0, 1/sqrt(I)); stored expert-indexed as
                 w_gate_up [E, 2I, H] (gate rows, then up rows) and
                 w_down [E, H, I].
  fp8 workloads: x and the router as above (x in bf16); expert weights are
                 drawn directly as OCP E4M3 codes: sign uniform, magnitude
                 code uniform over 0x28..0x3f (values 0.25 .. 1.875, rms
                 0.97), with one scale per expert and matrix, 1/sqrt(H) for
                 gate/up and 1/sqrt(I) for down (dequantized std about
                 0.97/sqrt(fan-in), close to the bf16 recipe).
Every tensor draws from its own sub-generator whose seed is derived from
(seed, tensor name, expert index) by SHA-256, so experts can be drawn in
parallel and any subset is reproducible on its own.
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import hashlib
import math
import os
from typing import List, Optional, Sequence, Tuple

import torch

from .configs import WorkloadConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}  # fp8: x


def _sub_seed(seed: int, tag: str, idx: int = 0) -> int:
    h = hashlib.sha256(f"{seed}:{tag}:{idx}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, tag: str, idx: int = 0) -> torch.Generator:
    return torch.Generator().manual_seed(_sub_seed(seed, tag, idx))


def bf16_round(t: torch.Tensor) -> torch.Tensor:
    """Round fp32 values to bf16 (nearest, ties to even), returned as fp32."""
    return t.to(torch.bfloat16).to(torch.float32)


@dataclasses.dataclass
class MoEInputs:
    cfg: WorkloadConfig
    x: torch.Tensor                 # [T, H] cfg.dtype
    logits: torch.Tensor            # [T, E] f32
    w_gate_up: torch.Tensor         # [E, 2I, H] cfg.dtype, expert-indexed
    w_down: torch.Tensor            # [E, H, I] cfg.dtype, expert-indexed
    popularity_rank: Optional[torch.Tensor] = None  # [E] int64 (zipf router)
    w_gate_up_scale: Optional[torch.Tensor] = None  # fp8: [E] f32
    w_down_scale: Optional[torch.Tensor] = None     # fp8: [E] f32

    def share_weights(self, ep_rank: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Expert weights held by one EP rank: experts [r*E_l, (r+1)*E_l)."""
        El = self.cfg.E_local
        lo = ep_rank * El
        return self.w_gate_up[lo:lo + El], self.w_down[lo:lo + El]

    def share_scales(self, ep_rank: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """fp8: the per-expert weight scales of one EP rank's experts."""
        El = self.cfg.E_local
        lo = ep_rank * El
        return self.w_gate_up_scale[lo:lo + El], self.w_down_scale[lo:lo + El]

    def replicated_experts(self) -> List[int]:
        """Experts that get a second slot: the n_replicated most popular ones,
        most popular first (zipf workload only)."""
        n = self.cfg.n_replicated
        if n == 0:
            return []
        assert self.popularity_rank is not None
        order = torch.argsort(self.popularity_rank)  # rank 0 first
        return [int(e) for e in order[:n]]


def _codes(shape, g: torch.Generator) -> torch.Tensor:
    """E4M3 codes: random sign bit, magnitude code uniform over 0x28..0x3f."""
    mag = torch.randint(0x28, 0x40, shape, generator=g, dtype=torch.uint8)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.uint8) << 7
    return mag | sign


def _fill_expert(cfg: WorkloadConfig, e: int, wgu: torch.Tensor, wd: torch.Tensor) -> None:
    H, I = cfg.H, cfg.I
    if cfg.dtype == "fp8":
        wgu[e, :I].copy_(_codes((I, H), _gen(cfg.seed, "w_gate", e)))
        wgu[e, I:].copy_(_codes((I, H), _gen(cfg.seed, "w_up", e)))
        wd[e].copy_(_codes((H, I), _gen(cfg.seed, "w_down", e)))
        return
    dt = _TORCH_DT[cfg.dtype]
    g = _gen(cfg.seed, "w_gate", e)
    wgu[e, :I].copy_((torch.randn(I, H, generator=g) * (1.0 / math.sqrt(H))).to(dt))
    g = _gen(cfg.seed, "w_up", e)
    wgu[e, I:].copy_((torch.randn(I, H, generator=g) * (1.0 / math.sqrt(H))).to(dt))
    g = _gen(cfg.seed, "w_down", e)
    wd[e].copy_((torch.randn(H, I, generator=g) * (1.0 / math.sqrt(I))).to(dt))


def make_expert_weights(cfg: WorkloadConfig, experts: Optional[Sequence[int]] = None,
                        threads: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Expert weights [E, 2I, H] and [E, H, I]; only `experts` are drawn if given
    (the others are left zero)."""
    dt = torch.uint8 if cfg.dtype == "fp8" else _TORCH_DT[cfg.dtype]
    wgu = torch.empty(cfg.E, 2 * cfg.I, cfg.H, dtype=dt)
    wd = torch.empty(cfg.E, cfg.H, cfg.I, dtype=dt)
    if experts is not None:
        wgu.zero_()
        wd.zero_()
    todo = list(range(cfg.E)) if experts is None else list(experts)
    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or len(todo) <= 1:
        for e in todo:
            _fill_expert(cfg, e, wgu, wd)
    else:
        with _fut.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda e: _fill_expert(cfg, e, wgu, wd), todo))
    return wgu, wd


def make_router_logits(cfg: WorkloadConfig, x: torch.Tensor):
    """Router logits [T, E] f32 (the method's input) and, for the zipf router,
    the popularity rank of each expert."""
    T, H, E = cfg.T, cfg.H, cfg.E
    if cfg.router in ("gauss", "gauss_bias"):
        wr = torch.randn(E, H, generator=_gen(cfg.seed, "router")) * (1.0 / math.sqrt(H))
        lg = x.to(torch.float64) @ wr.to(torch.float64).T
        if cfg.router == "gauss_bias":
            bias = torch.randn(E, generator=_gen(cfg.seed, "router_bias")) * cfg.bias_std
            lg = lg + bias.to(torch.float64)
        return lg.to(torch.float32).contiguous(), None
    if cfg.router == "zipf":
        rank = torch.randperm(E, generator=_gen(cfg.seed, "popularity"))
        logp = -cfg.zipf_s * torch.log(rank.to(torch.float64) + 1.0)
        logp = logp - torch.logsumexp(logp, 0)
        u = torch.rand(T, E, generator=_gen(cfg.seed, "gumbel"), dtype=torch.float64)
        tiny = torch.finfo(torch.float64).tiny
        u = u.clamp(min=tiny, max=1.0 - 2.0 ** -53)
        gumbel = -torch.log(-torch.log(u))
        return (logp[None, :] + gumbel).to(torch.float32).contiguous(), rank
    raise ValueError(f"unknown router {cfg.router!r}")


def make_inputs(cfg: WorkloadConfig, with_weights: bool = True,
                experts: Optional[Sequence[int]] = None) -> MoEInputs:
    """All inputs of one workload. `experts` restricts which expert weights are
    drawn (the rest stay zero); with_weights=False skips them entirely."""
    dt = _TORCH_DT[cfg.dtype]
    x = torch.randn(cfg.T, cfg.H, generator=_gen(cfg.seed, "x")).to(dt).contiguous()
    logits, rank = make_router_logits(cfg, x)
    if with_weights:
        wgu, wd = make_expert_weights(cfg, experts)
    else:
        wgu = torch.empty(0, dtype=dt)
        wd = torch.empty(0, dtype=dt)
    inp = MoEInputs(cfg, x, logits, wgu, wd, rank)
    if cfg.dtype == "fp8":
        inp.w_gate_up_scale = torch.full((cfg.E,), 1.0 / math.sqrt(cfg.H), dtype=torch.float32)
        inp.w_down_scale = torch.full((cfg.E,), 1.0 / math.sqrt(cfg.I), dtype=torch.float32)
    return inp


def identity_slot_table(E_local: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """rep_off [E_l+1], rep_slots [E_l]: local expert i lives in slot i only."""
    off = torch.arange(E_local + 1, dtype=torch.int32)
    slots = torch.arange(E_local, dtype=torch.int32)
    return off, slots


def build_slot_table(E_local: int, replicated: Sequence[int]):
    """Slot table with one slot per local expert plus a second slot for each
    expert in `replicated`: slots 0..E_l-1 hold experts 0..E_l-1 and slot
    E_l + j holds replicated[j]. Returns (rep_off [E_l+1], rep_slots [S],
    slot_expert [S]) as int32 tensors; rep_slots lists each expert's slots in
    ascending slot order."""
    per_expert: List[List[int]] = [[e] for e in range(E_local)]
    for j, e in enumerate(replicated):
        per_expert[e].append(E_local + j)
    off = [0]
    slots: List[int] = []
    for lst in per_expert:
        slots.extend(lst)
        off.append(len(slots))
    slot_expert = list(range(E_local)) + list(replicated)
    return (torch.tensor(off, dtype=torch.int32), torch.tensor(slots, dtype=torch.int32),
            torch.tensor(slot_expert, dtype=torch.int32))


def slot_weights(w_expert: torch.Tensor, slot_expert: torch.Tensor) -> torch.Tensor:
    """Per-slot weights: slot s holds a copy of expert slot_expert[s]."""
    return w_expert.index_select(0, slot_expert.to(torch.int64)).contiguous()
