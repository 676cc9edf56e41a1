"""Fused forward (moe_forward) parity against the CPU oracle, on every
workload shape, plus the invariants the pages fix:
  - zero-weight pairs contribute nothing and masked pairs are never computed
    (vLLM ep_fused_moe_patch.py: ep_mask_and_remap, "EP expert dispatch");
  - the identity expert -> slot table equals expert-indexed compute and
    replicated slots with copied weights give the same output whichever
    replica serves a token (TensorRT-LLM PR #4495, Description);
  - the expert-parallel partial outputs sum to the full output (vLLM
    ep_reduce_output; DeepSpeed PR #6964 single reduction per layer).
Full-size workloads compare the tokens of a covering sample -- at least one
sampled row in every 128-row piece of every slot, so every GEMM work item and
every ragged tail is checked against the oracle -- and check every index
array bit for bit through the staged entry points. Medium shapes spanning
several tiles with ragged tails compare every output, also with the GEMM grid
capped at a few blocks so that each block loops over many work items, and a
16384-token shape whose launches give every block several items compares
every output at the full grid.
"""
import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe
import oracle
from gpu_common import (BF16_TOL, F32_TOL, announce, assert_close, covering_tokens, device,
                        np64, rel_fro)
from workloads import (CONFIGS, WorkloadConfig, build_slot_table, identity_slot_table,
                       make_inputs, slot_weights)

pytestmark = pytest.mark.gpu

_TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    return device()


_INPUTS = {}


def inputs(name):
    if name not in _INPUTS:
        _INPUTS.clear()  # keep one large workload resident at a time
        _INPUTS[name] = make_inputs(CONFIGS[name])
    return _INPUTS[name]


def tol_of(cfg):
    return F32_TOL if cfg.dtype == "f32" else BF16_TOL


def share_tensors(inp, dev, ep_rank=0, replicas=False, flip=False):
    """Per-slot weights and slot table of one share, on the device."""
    cfg = inp.cfg
    wgu, wd = inp.share_weights(ep_rank)
    if replicas:
        ro, rs, se = build_slot_table(cfg.E_local, inp.replicated_experts())
        if flip:  # serve each token from the other replica: (t + 1) mod r
            rs = rs.clone()
            for lid in range(cfg.E_local):
                a, b = int(ro[lid]), int(ro[lid + 1])
                rs[a:b] = torch.roll(rs[a:b], -1)
        wgu, wd = slot_weights(wgu, se), slot_weights(wd, se)
        S = int(se.numel())
    else:
        ro, rs = identity_slot_table(cfg.E_local)
        S = cfg.E_local
    return (wgu.contiguous().to(dev), wd.contiguous().to(dev), ro.to(dev), rs.to(dev), S)


def run_forward(inp, dev, ep_rank=0, replicas=False, flip=False, out=None, accumulate=False,
                out_dtype=None, topk=None, shares=None, T_max=None, ws=None):
    cfg = inp.cfg
    wgu, wd, ro, rs, S = shares or share_tensors(inp, dev, ep_rank, replicas, flip)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=S, dtype=_TDT[cfg.dtype],
                           out_dtype=out_dtype, ep_size=cfg.ep_size, ep_rank=ep_rank,
                           accumulate=accumulate, T_max=T_max,
                           num_expert_group=cfg.num_expert_group, topk_group=cfg.topk_group)
    kw = dict(rep_off=ro, rep_slots=rs, out=out, ws=ws)
    if topk is None:
        kw["logits"] = inp.logits.to(dev)
    else:
        kw["topk_ids"], kw["topk_w"] = topk[0].to(dev), topk[1].to(dev)
    return moe.forward(fc, inp.x.to(dev), wgu, wd, **kw)


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    if T <= n:
        return np.arange(T)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))


def oracle_covering(inp, ep_rank=0, replicas=False, seed=0):
    """Covering sample of one share's permutation, as the oracle computes it
    (routing, EP mask, slot table, counting sort)."""
    cfg = inp.cfg
    ids, w = oracle_route(inp)
    if replicas:
        ro, rs, se = build_slot_table(cfg.E_local, inp.replicated_experts())
        ro, rs, S = ro.numpy(), rs.numpy(), int(se.numel())
    else:
        ro = rs = None
        S = cfg.E_local
    slot, _, mask = oracle.slot_map(ids, w, cfg.E, cfg.ep_size, ep_rank, ro, rs)
    off, sp, pr = oracle.permute_indices(slot, mask, S)
    return covering_tokens(off, sp, pr, cfg.K, seed=seed)


def check_staged_indices(inp, dev, ep_rank=0, replicas=False):
    """Route, slot map and permutation of the full workload, bit for bit."""
    cfg = inp.cfg
    wgu, wd, ro, rs, S = share_tensors(inp, dev, ep_rank, replicas) if replicas else \
        (None, None, *identity_slot_table(cfg.E_local), cfg.E_local)
    ro, rs = ro.to(dev), rs.to(dev)
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize,
                       num_groups=cfg.num_expert_group, topk_groups=cfg.topk_group)
    slot, wm, mask = moe.slot_map(ids, w, cfg.E, cfg.ep_size, ep_rank, ro, rs)
    off, sp, pr, xp = moe.permute(inp.x.to(dev), slot, mask, S)
    torch.cuda.synchronize()
    r_ids, _ = oracle_route(inp)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    r_slot, _, r_mask = oracle.slot_map(ids.cpu(), w.cpu().double(), cfg.E, cfg.ep_size, ep_rank,
                                        ro.cpu().numpy(), rs.cpu().numpy())
    assert np.array_equal(slot.cpu().numpy(), r_slot)
    assert np.array_equal(mask.cpu().numpy(), r_mask)
    r_off, r_sp, r_pr = oracle.permute_indices(r_slot, r_mask, S)
    P_in = int(r_off[-1])
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(sp.cpu().numpy()[:P_in], r_sp)
    assert np.array_equal(pr.cpu().numpy(), r_pr)
    rows = np.random.default_rng(1).choice(P_in, size=min(P_in, 256), replace=False)
    got = xp[torch.from_numpy(rows).to(dev)].cpu()
    ref = inp.x[torch.from_numpy(r_sp[rows] // cfg.K).long()]
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)


def oracle_route(inp):
    """The oracle's routing of a workload (group-limited when configured)."""
    cfg = inp.cfg
    if cfg.num_expert_group:
        return oracle.route_grouped(inp.logits.numpy(), cfg.K, cfg.renormalize,
                                    cfg.num_expert_group, cfg.topk_group)
    return oracle.route(inp.logits, cfg.K, cfg.renormalize)


def compare_tokens(got_dev, inp, tokens, ep_rank=0, what=""):
    cfg = inp.cfg
    got = np64(got_dev[torch.from_numpy(tokens).to(got_dev.device)].cpu())
    if cfg.num_expert_group:
        ids, w = oracle_route(inp)
        ref = oracle.forward(inp.x, None, inp.w_gate_up, inp.w_down, cfg.K, False, cfg.ep_size,
                             ep_rank, tokens=tokens, topk=(ids, w))
    else:
        ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                             cfg.renormalize, cfg.ep_size, ep_rank, tokens=tokens)
    assert_close(got, ref, tol_of(cfg), what)
    return got, ref


# ------------------------------------------------------------------ full workloads
def test_forward_tiny_fp32_all_tokens(dev):
    inp = inputs("tiny_fp32")
    announce("forward tiny_fp32 (all tokens)")
    out = run_forward(inp, dev)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, 2, True)
    assert_close(np64(out.cpu()), ref, F32_TOL, "tiny_fp32")
    assert rel_fro(np64(out.cpu()), ref) < 1e-5
    check_staged_indices(inp, dev)


@pytest.mark.parametrize("name", ["qwen2_moe_bf16", "deepseek_v2_bf16",
                                  "deepseek_v2_grouped_bf16"])
def test_forward_full_size_covering(dev, name):
    inp = inputs(name)
    tokens = oracle_covering(inp)
    announce(f"forward {name} full size, {tokens.size} covering tokens")
    out = run_forward(inp, dev)
    torch.cuda.synchronize()
    compare_tokens(out, inp, tokens, what=name)
    announce(f"staged indices {name}")
    check_staged_indices(inp, dev)


def test_forward_ep_shares_sum_to_full(dev):
    inp = inputs("ep_share_256_bf16")
    cfg = inp.cfg
    tokens = sample_tokens(cfg.T, 32, seed=2)
    acc = torch.zeros(cfg.T, cfg.H, dtype=torch.float32, device=dev)
    for r in range(cfg.ep_size):
        cover = oracle_covering(inp, ep_rank=r, seed=r)
        announce(f"forward ep share rank {r}, {cover.size} covering tokens")
        share = run_forward(inp, dev, ep_rank=r)
        torch.cuda.synchronize()
        compare_tokens(share, inp, cover, ep_rank=r, what=f"share {r}")
        run_forward(inp, dev, ep_rank=r, out=acc, accumulate=True, out_dtype=torch.float32)
        if r == 1:
            check_staged_indices(inp, dev, ep_rank=1)
    announce("forward full 256-expert layer (ep_size=1)")
    full_cfg = cfg.replace(ep_size=1)
    full_inp = type(inp)(full_cfg, inp.x, inp.logits, inp.w_gate_up, inp.w_down)
    full = run_forward(full_inp, dev)
    torch.cuda.synchronize()
    assert_close(np64(acc.cpu()), np64(full.cpu()), BF16_TOL, "sum of shares vs full")
    assert rel_fro(np64(acc.cpu()), np64(full.cpu())) < 1e-2
    compare_tokens(full, full_inp, oracle_covering(full_inp, seed=9), what="full layer")
    # oracle identity on the sampled tokens
    parts = sum(oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                               cfg.renormalize, cfg.ep_size, r, tokens=tokens)
                for r in range(cfg.ep_size))
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         tokens=tokens)
    np.testing.assert_allclose(parts, ref, atol=1e-12)


def test_forward_replicated_slots(dev):
    inp = inputs("redundant_slots_zipf")
    tokens = oracle_covering(inp, replicas=True, seed=3)
    announce(f"forward zipf 80 slots (replicas), {tokens.size} covering tokens")
    rep = run_forward(inp, dev, replicas=True)
    torch.cuda.synchronize()
    compare_tokens(rep, inp, tokens, what="replicas")
    announce("staged indices zipf")
    check_staged_indices(inp, dev, replicas=True)
    announce("forward zipf flipped replicas and 64-slot identity table")
    flip = run_forward(inp, dev, replicas=True, flip=True)
    ident = run_forward(inp, dev, replicas=False)
    torch.cuda.synchronize()
    a, b, c = np64(rep.cpu()), np64(flip.cpu()), np64(ident.cpu())
    assert_close(a, c, BF16_TOL, "replicas vs identity table")
    assert_close(b, c, BF16_TOL, "flipped replicas vs identity table")
    print(f"replica runs bit-identical to the identity-table run: "
          f"{np.array_equal(a, c)} / {np.array_equal(b, c)}", flush=True)


# ------------------------------------------------------------------ medium shapes
MEDIUM = {
    "bf16_ragged": WorkloadConfig("m1", T=300, H=256, I=192, E=12, K=3, renormalize=True,
                                  dtype="bf16", router="gauss_bias", bias_std=0.5, seed=1),
    "bf16_odd_dims": WorkloadConfig("m2", T=517, H=136, I=72, E=5, K=2, renormalize=False,
                                    dtype="bf16", router="gauss", seed=2),
    "bf16_ep_rank1": WorkloadConfig("m3", T=400, H=128, I=128, E=16, K=4, renormalize=True,
                                    dtype="bf16", router="gauss", ep_size=2, seed=3),
    "bf16_replicas": WorkloadConfig("m4", T=333, H=128, I=64, E=8, K=2, renormalize=True,
                                    dtype="bf16", router="zipf", n_replicated=3, seed=4),
    "bf16_k_eq_e": WorkloadConfig("m5", T=64, H=64, I=64, E=4, K=4, renormalize=False,
                                  dtype="bf16", router="gauss", seed=5),
    "f32_k1": WorkloadConfig("m6", T=100, H=64, I=32, E=4, K=1, renormalize=True,
                             dtype="f32", router="gauss", seed=6),
    "bf16_big_tiles": WorkloadConfig("m7", T=1500, H=512, I=320, E=3, K=2, renormalize=True,
                                     dtype="bf16", router="gauss_bias", bias_std=1.0, seed=7),
}


@pytest.mark.parametrize("name", list(MEDIUM))
def test_forward_medium_all_tokens(dev, name):
    cfg = MEDIUM[name]
    inp = make_inputs(cfg)
    ep_rank = cfg.ep_size - 1
    announce(f"forward medium {name}")
    out = run_forward(inp, dev, ep_rank=ep_rank, replicas=cfg.n_replicated > 0)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         cfg.ep_size, ep_rank)
    assert_close(np64(out.cpu()), ref, tol_of(cfg), name)
    assert rel_fro(np64(out.cpu()), ref) < (1e-5 if cfg.dtype == "f32" else 1e-2)


# ------------------------------------------------------------------ invariants
def _medium(name="bf16_ragged"):
    return make_inputs(MEDIUM[name])


def test_zero_weight_pairs(dev):
    inp = _medium()
    cfg = inp.cfg
    ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    w = w.astype(np.float32)
    w[::3, 1] = 0.0
    topk = (torch.from_numpy(ids), torch.from_numpy(w))
    announce("forward zero-weight pairs")
    out = run_forward(inp, dev, topk=topk)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         topk=(ids, w))
    assert_close(np64(out.cpu()), ref, BF16_TOL, "zero weights")


def test_masked_pairs_are_skipped(dev):
    """Which non-local expert a masked pair names does not change a bit of the
    share's output."""
    inp = _medium("bf16_ep_rank1")
    cfg = inp.cfg
    ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    w = w.astype(np.float32)
    ids2 = ids.copy()
    nl = ids2 < cfg.E_local  # rank 1 owns [E_local, E)
    ids2[nl] = (ids2[nl] + 3) % cfg.E_local
    announce("forward masked-pair scramble")
    a = run_forward(inp, dev, ep_rank=1, topk=(torch.from_numpy(ids), torch.from_numpy(w)))
    b = run_forward(inp, dev, ep_rank=1, topk=(torch.from_numpy(ids2), torch.from_numpy(w)))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_slots_are_never_read(dev):
    """Slots with no rows do no work: NaN weights there change nothing."""
    cfg = WorkloadConfig("m8", T=24, H=128, I=64, E=64, K=2, renormalize=True, dtype="bf16",
                         router="gauss", seed=8)
    inp = make_inputs(cfg)
    wgu, wd, ro, rs, S = share_tensors(inp, dev)
    ids, _ = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    empty = sorted(set(range(S)) - set(np.unique(ids).tolist()))
    assert len(empty) >= 16
    announce(f"forward NaN weights in {len(empty)} empty slots")
    base = run_forward(inp, dev, shares=(wgu, wd, ro, rs, S))
    wgu2, wd2 = wgu.clone(), wd.clone()
    idx = torch.tensor(empty, device=dev)
    wgu2[idx] = float("nan")
    wd2[idx] = float("nan")
    got = run_forward(inp, dev, shares=(wgu2, wd2, ro, rs, S))
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(base.view(torch.int16), got.view(torch.int16))
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize)
    assert_close(np64(got.cpu()), ref, BF16_TOL, "empty slots")


def test_determinism_and_topk_form(dev):
    inp = _medium("bf16_big_tiles")
    cfg = inp.cfg
    announce("forward determinism")
    a = run_forward(inp, dev)
    b = run_forward(inp, dev)
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    c = run_forward(inp, dev, topk=(ids, w))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_odd_dims"])
def test_forward_matches_staged_calls(dev, name):
    """moe_forward gives the bits of the staged entry points in sequence, both
    where it folds the row gather into the gate/up GEMM (H = 256) and where
    it runs the permutation's gather (H = 136, not a multiple of 32)."""
    inp = _medium(name)
    cfg = inp.cfg
    wgu, wd, ro, rs, S = share_tensors(inp, dev)
    announce("forward vs staged")
    fused = run_forward(inp, dev, shares=(wgu, wd, ro, rs, S))
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    slot, wm, mask = moe.slot_map(ids, w, cfg.E, 1, 0, ro, rs)
    off, sp, pr, xp = moe.permute(inp.x.to(dev), slot, mask, S)
    a = moe.grouped_gemm(moe.GATE_UP_SWIGLU, xp, off, wgu)
    y = moe.grouped_gemm(moe.DOWN, a, off, wd)
    staged = moe.combine(y, pr, wm, cfg.K)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), staged.view(torch.int16))


def test_workspace_reuse_smaller_T(dev):
    cfg = MEDIUM["bf16_ragged"]
    big = make_inputs(cfg)
    small_cfg = cfg.replace(T=97)
    small = make_inputs(small_cfg)
    shares = share_tensors(big, dev)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=cfg.E, dtype=torch.bfloat16)
    ws = torch.empty(moe.forward_workspace_size(fc), dtype=torch.uint8, device=dev)
    announce("forward T < T_max with a shared workspace")
    out_big = run_forward(big, dev, shares=shares, T_max=cfg.T, ws=ws)
    small.w_gate_up, small.w_down = big.w_gate_up, big.w_down
    out_small = run_forward(small, dev, shares=shares, T_max=cfg.T, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(small.x, small.logits, big.w_gate_up, big.w_down, cfg.K, cfg.renormalize)
    assert_close(np64(out_small.cpu()), ref, BF16_TOL, "small T")
    ref_b = oracle.forward(big.x, big.logits, big.w_gate_up, big.w_down, cfg.K, cfg.renormalize)
    assert_close(np64(out_big.cpu()), ref_b, BF16_TOL, "big T")


def test_forward_zero_tokens(dev):
    cfg = MEDIUM["bf16_ragged"].replace(T=0)
    inp = make_inputs(cfg)
    announce("forward T=0")
    out = run_forward(inp, dev, T_max=16)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)


def test_forward_grouped_routing(dev):
    """moe_forward with num_expert_group / topk_group set routes with the
    group-limited selection: compare with the oracle forward fed by
    oracle.route_grouped."""
    cfg = WorkloadConfig("g1", T=300, H=256, I=192, E=16, K=4, renormalize=True, dtype="bf16",
                         router="gauss_bias", bias_std=0.5, seed=21)
    inp = make_inputs(cfg)
    announce("forward grouped routing E=16 G=4 TG=2")
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=True, S=cfg.E, dtype=torch.bfloat16,
                           num_expert_group=4, topk_group=2)
    got = moe.forward(fc, inp.x.to(dev), inp.w_gate_up.to(dev), inp.w_down.to(dev),
                      logits=inp.logits.to(dev))
    torch.cuda.synchronize()
    ids, w = oracle.route_grouped(inp.logits.numpy(), cfg.K, True, 4, 2)
    ref = oracle.forward(inp.x, None, inp.w_gate_up, inp.w_down, cfg.K, False, topk=(ids, w))
    assert_close(np64(got), ref, BF16_TOL, "grouped-routing forward")
    # the grouping must matter for this input, or the test proves nothing
    plain, _ = oracle.route(inp.logits.numpy(), cfg.K, True)
    assert not np.array_equal(plain, ids)


# ------------------------------------------------------------------ full size, options
@pytest.mark.parametrize("name", ["qwen2_moe_shared_bf16", "qwen2_moe_input_routing_bf16"])
def test_forward_full_size_options_covering(dev, name):
    """The 60-expert layer with a shared-expert output added in the combine,
    and with the routing weights applied on the expert input (the scaled rows
    are gathered by the permutation, not folded into the gate/up GEMM)."""
    inp = inputs(name)
    cfg = inp.cfg
    tokens = oracle_covering(inp)
    announce(f"forward {name} full size, {tokens.size} covering tokens")
    shared = None
    if cfg.shared_expert:
        shared = torch.randn(cfg.T, cfg.H, generator=torch.Generator().manual_seed(1)).to(
            torch.bfloat16)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=cfg.E, dtype=torch.bfloat16,
                           routing_on_input=cfg.routing_on_input)
    out = moe.forward(fc, inp.x.to(dev), inp.w_gate_up.to(dev), inp.w_down.to(dev),
                      logits=inp.logits.to(dev),
                      shared_out=None if shared is None else shared.to(dev))
    torch.cuda.synchronize()
    got = np64(out[torch.from_numpy(tokens).to(dev)].cpu())
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         tokens=tokens, routing_on_input=cfg.routing_on_input, shared=shared)
    assert_close(got, ref, BF16_TOL, name)


# ------------------------------------------------------------------ many items per block
MULTI_ITEM = WorkloadConfig("mi", T=16384, H=512, I=512, E=8, K=4, renormalize=True,
                            dtype="bf16", router="gauss_bias", bias_std=0.3, seed=51)


def test_forward_many_items_per_block_all_tokens(dev):
    """16384 tokens, H = I = 512, 8 experts, top-4: the gate/up launch has
    about 1050 work items and the down launch about 525, so on a full grid
    every block computes several items in a row (the next item's first
    K-slices fetched during the previous epilogue, the gathered token rows
    set up before the last slice). Every output is compared with the oracle,
    and the run with the grid capped at 16 blocks is bit-identical."""
    inp = make_inputs(MULTI_ITEM)
    cfg = inp.cfg
    ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    announce(f"forward many items per block, slot rows {counts.tolist()}")
    out = run_forward(inp, dev)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=cfg.E, dtype=torch.bfloat16,
                           gemm_blocks=16)
    capped = moe.forward(fc, inp.x.to(dev), inp.w_gate_up.to(dev), inp.w_down.to(dev),
                         logits=inp.logits.to(dev))
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize)
    assert_close(np64(out.cpu()), ref, BF16_TOL, "many items per block")
    assert rel_fro(np64(out.cpu()), ref) < 1e-2
    assert torch.equal(out.view(torch.int16), capped.view(torch.int16))


@pytest.mark.parametrize("name,blocks", [("bf16_ragged", 3), ("bf16_odd_dims", 2),
                                         ("bf16_ep_rank1", 5), ("bf16_replicas", 4),
                                         ("bf16_k_eq_e", 1), ("bf16_big_tiles", 8)])
def test_forward_medium_capped_grid(dev, name, blocks):
    """The medium shapes with the persistent GEMM grid capped at a few blocks:
    each block then runs many items in a row, mixing full, half-empty and
    two-fragment items and items of different slots. Every output against
    the oracle, and bit-identical to the full-grid run."""
    cfg = MEDIUM[name]
    inp = make_inputs(cfg)
    ep_rank = cfg.ep_size - 1
    announce(f"forward medium {name}, GEMM grid capped at {blocks} blocks")
    shares = share_tensors(inp, dev, ep_rank, replicas=cfg.n_replicated > 0)
    full = run_forward(inp, dev, ep_rank=ep_rank, shares=shares)
    wgu, wd, ro, rs, S = shares
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=S, dtype=_TDT[cfg.dtype],
                           ep_size=cfg.ep_size, ep_rank=ep_rank, gemm_blocks=blocks)
    capped = moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), rep_off=ro,
                         rep_slots=rs)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         cfg.ep_size, ep_rank)
    assert_close(np64(capped.cpu()), ref, tol_of(cfg), name)
    assert torch.equal(full.view(torch.int16), capped.view(torch.int16))


def test_forward_input_routing_capped_grid(dev):
    """Input-side routing runs the gate/up GEMM on the permuted rows (not the
    gathered kernel): with the grid capped, every output against the oracle."""
    cfg = MEDIUM["bf16_big_tiles"]
    inp = make_inputs(cfg)
    announce("forward input-side routing, GEMM grid capped at 4 blocks")
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=cfg.E, dtype=torch.bfloat16,
                           routing_on_input=True, gemm_blocks=4)
    got = moe.forward(fc, inp.x.to(dev), inp.w_gate_up.to(dev), inp.w_down.to(dev),
                      logits=inp.logits.to(dev))
    torch.cuda.synchronize()
    ref = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         routing_on_input=True)
    assert_close(np64(got.cpu()), ref, BF16_TOL, "input routing, capped grid")
