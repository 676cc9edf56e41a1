"""Input-side routing and the shared-expert add on the GPU against the oracle.

moe_permute_scaled's rows are compared bit for bit with round(w * x) formed
the same way (f32 product, one rounding), moe_combine_shared with unit
weights against the f32 sum in the same order, and moe_forward with either
option against the oracle's forward(routing_on_input=..., shared=...), which
its pins tie to a dense brute force.
"""
import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe
import oracle
from gpu_common import BF16_TOL, F32_TOL, announce, assert_close, device, np64
from workloads import WorkloadConfig, make_inputs

pytestmark = pytest.mark.gpu

_TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
CASES = {
    "bf16": WorkloadConfig("s1", T=300, H=256, I=192, E=12, K=3, renormalize=True, dtype="bf16",
                           router="gauss_bias", bias_std=0.5, seed=31),
    "bf16_ep2": WorkloadConfig("s2", T=257, H=128, I=128, E=16, K=4, renormalize=False,
                               dtype="bf16", router="gauss", ep_size=2, seed=32),
    "f32": WorkloadConfig("s3", T=100, H=64, I=32, E=4, K=2, renormalize=True, dtype="f32",
                          router="gauss", seed=33),
}


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_permute_scaled_rows(dt):
    dev = device()
    announce(f"permute scaled {dt}")
    T, K, E, H = 200, 3, 8, 136
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(T, H, generator=g) * 3).to(dt)
    ids = torch.stack([torch.randperm(E, generator=g)[:K] for _ in range(T)]).int()
    w = torch.rand(T, K, generator=g)
    slot, wm, mask = moe.slot_map(ids.to(dev), w.to(dev), E)
    off, sp, pr, xp = moe.permute(x.to(dev), slot, mask, E, pair_w=wm)
    torch.cuda.synchronize()
    pr = pr.cpu().numpy().reshape(T, K)
    want = (x.float()[:, None, :] * wm.cpu()[:, :, None]).to(dt)  # f32 product, one rounding
    got = xp.cpu()
    bits = torch.int16 if dt == torch.bfloat16 else torch.int32
    for t in range(T):
        for k in range(K):
            assert torch.equal(got[pr[t, k]].view(bits), want[t, k].view(bits)), (t, k)


def test_combine_shared_unit_weights_exact():
    dev = device()
    announce("combine shared, unit weights")
    T, K, H = 150, 4, 64
    g = torch.Generator().manual_seed(5)
    y = torch.randn(T * K, H, generator=g)
    pr = torch.randperm(T * K, generator=g).int().reshape(T, K)
    pr[torch.rand(T, K, generator=g) < 0.2] = -1
    sh = torch.randn(T, H, generator=g).to(torch.bfloat16)
    got = moe.combine(y.to(dev), pr.to(dev), None, K, out_dtype=torch.float32, shared=sh.to(dev))
    torch.cuda.synchronize()
    yn, prn = y.numpy(), pr.numpy()
    want = np.zeros((T, H), dtype=np.float32)
    for k in range(K):  # ascending k, f32 adds, then the shared row
        has = prn[:, k] >= 0
        want[has] = want[has] + yn[prn[has, k]]
    want = want + sh.float().numpy()
    assert np.array_equal(got.cpu().numpy(), want)


def _forward(inp, dev, ep_rank=0, on_input=False, shared=None, out_dtype=None, accumulate=False,
             out=None):
    cfg = inp.cfg
    El = cfg.E_local
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=El, dtype=_TDT[cfg.dtype],
                           out_dtype=out_dtype, ep_size=cfg.ep_size, ep_rank=ep_rank,
                           accumulate=accumulate, routing_on_input=on_input)
    wgu, wd = inp.share_weights(ep_rank)
    return moe.forward(fc, inp.x.to(dev), wgu.contiguous().to(dev), wd.contiguous().to(dev),
                       logits=inp.logits.to(dev), out=out,
                       shared_out=None if shared is None else shared.to(dev))


@pytest.mark.parametrize("name", ["bf16", "f32"])
@pytest.mark.parametrize("on_input,with_shared", [(True, False), (False, True), (True, True)])
def test_forward_options_match_oracle(name, on_input, with_shared):
    dev = device()
    inp = make_inputs(CASES[name])
    cfg = inp.cfg
    announce(f"forward {name} routing_on_input={on_input} shared={with_shared}")
    sh = None
    if with_shared:
        sh = torch.randn(cfg.T, cfg.H, generator=torch.Generator().manual_seed(7)).to(
            _TDT[cfg.dtype])
    got = _forward(inp, dev, on_input=on_input, shared=sh)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         routing_on_input=on_input, shared=sh)
    assert_close(np64(got), ref, BF16_TOL if cfg.dtype == "bf16" else F32_TOL, name)


def test_input_routing_shares_sum_to_full():
    """Expert-parallel shares with input-side routing and a shared-output
    shard each: the f32 sum over ranks is the full layer with the whole
    shared output (the identity the pages' single reduction relies on)."""
    dev = device()
    inp = make_inputs(CASES["bf16_ep2"])
    cfg = inp.cfg
    announce("input-side routing, 2 shares with shared shards")
    g = torch.Generator().manual_seed(9)
    shards = [torch.randn(cfg.T, cfg.H, generator=g).to(torch.bfloat16) for _ in range(2)]
    acc = torch.zeros(cfg.T, cfg.H, dtype=torch.float32, device=dev)
    for r in range(2):
        _forward(inp, dev, ep_rank=r, on_input=True, shared=shards[r],
                 out_dtype=torch.float32, accumulate=True, out=acc)
    torch.cuda.synchronize()
    total_shared = shards[0].double() + shards[1].double()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         routing_on_input=True, shared=total_shared.numpy())
    assert_close(np64(acc), ref, BF16_TOL, "input-routing shares + shared shards")
