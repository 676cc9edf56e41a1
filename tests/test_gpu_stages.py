"""Stage-by-stage parity of the HIP library against the CPU oracle.

Index work (routing ids, slot map, permutation) must match bit for bit;
floating-point outputs within the stated tolerances. Every call goes through
the C ABI via the Python binding.
"""
import math

import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe
import oracle
from gpu_common import (BF16_TOL, F32_TOL, announce, assert_close, device, f32_bits, np64,
                        rel_fro)
from workloads import CONFIGS, build_slot_table, get_config, identity_slot_table, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


# ------------------------------------------------------------------ route
def _route_case(name):
    g = torch.Generator().manual_seed(1234)
    if name in CONFIGS:
        cfg = CONFIGS[name]
        return make_inputs(cfg, with_weights=False).logits, cfg.K, cfg.renormalize
    if name == "ties":
        return (torch.round(torch.randn(300, 37, generator=g) * 2) / 2), 5, True
    if name == "k_eq_e":
        return torch.randn(50, 16, generator=g), 16, False
    if name == "max_e_k":
        return torch.randn(200, 1024, generator=g) * 3, 32, True
    if name == "e1":
        return torch.randn(33, 1, generator=g), 1, True
    if name == "e65_ragged":
        return torch.randn(129, 65, generator=g), 3, False
    if name == "zeros_equal":
        lg = torch.randn(40, 12, generator=g)
        lg[0] = 0.0
        lg[1] = -0.0
        lg[2, ::2] = -0.0
        lg[2, 1::2] = 0.0
        lg[3] = 5.0
        return lg, 4, True
    if name == "wide_range":
        return torch.randn(100, 64, generator=g) * 40, 8, True
    if name == "t0":
        return torch.zeros(0, 8), 2, True
    # lane-group router forms: 32 lanes per token with K > 16, K = 32 lanes at
    # 256 experts, and a token count that leaves a partial block of 32-lane
    # groups (with tied logits)
    if name == "l32_k24":
        return torch.randn(90, 40, generator=g), 24, True
    if name == "e256_k32":
        return torch.randn(64, 256, generator=g) * 2, 32, False
    if name == "e200_ragged_ties":
        return torch.round(torch.randn(77, 200, generator=g) * 3) / 3, 7, True
    raise KeyError(name)


ROUTE_CASES = list(CONFIGS) + ["ties", "k_eq_e", "max_e_k", "e1", "e65_ragged", "zeros_equal",
                               "wide_range", "t0", "l32_k24", "e256_k32", "e200_ragged_ties"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_parity(dev, name):
    logits, K, renorm = _route_case(name)
    logits = logits.float().contiguous()
    G, TG = (CONFIGS[name].num_expert_group, CONFIGS[name].topk_group) if name in CONFIGS \
        else (0, 0)
    announce(f"route {name} T={logits.shape[0]} E={logits.shape[1]} K={K} renorm={renorm} "
             f"groups={G}/{TG}")
    ids, w = moe.route(logits.to(dev), K, renorm, num_groups=G, topk_groups=TG)
    torch.cuda.synchronize()
    if logits.shape[0] == 0:
        return
    ref_ids, ref_w = (oracle.route_grouped(logits.numpy(), K, renorm, G, TG) if G
                      else oracle.route(logits, K, renorm))
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert_close(np64(w), ref_w, (1e-5, 1e-9), "route weights")


@pytest.mark.parametrize("E", [8, 64, 160, 256, 300])
def test_route_renormalized_weights_exact(dev, E):
    """Renormalisation divides each selected probability by their f32 sum:
    with K = 1 that is p / p, exactly 1.0 under IEEE division; with K = 8
    the weights sum to 1 within the rounding of the K quotients and of the
    sum (at most 2K units of 2^-24). E = 300 takes the wave-per-token
    router, the others the lane-group router."""
    g = torch.Generator().manual_seed(E)
    logits = (torch.randn(257, E, generator=g) * 3).float()
    announce(f"route renormalised weights E={E}")
    ids, w = moe.route(logits.to(dev), 1, True)
    torch.cuda.synchronize()
    assert (w.cpu() == 1.0).all()
    ref_ids, _ = oracle.route(logits, 1, True)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    if E >= 8:
        ids8, w8 = moe.route(logits.to(dev), 8, True)
        torch.cuda.synchronize()
        tot = w8.cpu().double().sum(dim=1).numpy()
        assert np.abs(tot - 1.0).max() <= 2 * 8 * 2.0 ** -24


# ------------------------------------------------------------------ slot map
def _slot_map_check(dev, ids, w, E, ep_size, ep_rank, ro=None, rs=None):
    d = lambda t: None if t is None else t.to(dev)
    slot, wm, mask = moe.slot_map(d(ids), d(w), E, ep_size, ep_rank, d(ro), d(rs))
    torch.cuda.synchronize()
    r_slot, r_wm, r_mask = oracle.slot_map(ids, w.double(), E, ep_size, ep_rank,
                                           None if ro is None else ro.numpy(),
                                           None if rs is None else rs.numpy())
    assert np.array_equal(slot.cpu().numpy(), r_slot)
    assert np.array_equal(mask.cpu().numpy(), r_mask)
    assert np.array_equal(f32_bits(wm.cpu().numpy()), f32_bits(r_wm.astype(np.float32)))


def test_slot_map_ep_shares(dev):
    cfg = CONFIGS["ep_share_256_bf16"]
    inp = make_inputs(cfg, with_weights=False)
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    ids, w = ids.cpu(), w.cpu()
    for r in range(cfg.ep_size):
        announce(f"slot_map ep rank {r}")
        _slot_map_check(dev, ids, w, cfg.E, cfg.ep_size, r)
        ro, rs = identity_slot_table(cfg.E_local)
        _slot_map_check(dev, ids, w, cfg.E, cfg.ep_size, r, ro, rs)


def test_slot_map_replicas(dev):
    cfg = CONFIGS["redundant_slots_zipf"]
    inp = make_inputs(cfg, with_weights=False)
    ro, rs, _ = build_slot_table(cfg.E_local, inp.replicated_experts())
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    announce("slot_map zipf replicas")
    _slot_map_check(dev, ids.cpu(), w.cpu(), cfg.E, 1, 0, ro, rs)


def test_slot_map_out_of_range_and_signs(dev):
    g = torch.Generator().manual_seed(5)
    E, T, K = 24, 257, 5
    ids = torch.randint(-7, E + 9, (T, K), generator=g, dtype=torch.int32)
    w = torch.randn(T, K, generator=g)  # negative weights give -0.0 when masked
    announce("slot_map out-of-range ids")
    for ep_size, r in [(1, 0), (3, 2), (4, 1)]:
        _slot_map_check(dev, ids, w, E, ep_size, r)
    ro, rs, _ = build_slot_table(8, [3, 0, 7])
    _slot_map_check(dev, ids, w, E, 3, 1, ro, rs)


# ------------------------------------------------------------------ permute
def _permute_check(dev, x, slot, mask, S):
    K = slot.shape[1]
    offsets, sp, pr, xp = moe.permute(x.to(dev), slot.to(dev), mask.to(dev), S)
    torch.cuda.synchronize()
    r_off, r_sp, r_pr = oracle.permute_indices(slot, mask, S)
    P_in = int(r_off[-1])
    assert np.array_equal(offsets.cpu().numpy(), r_off)
    assert np.array_equal(sp.cpu().numpy()[:P_in], r_sp)
    assert np.array_equal(pr.cpu().numpy(), r_pr)
    if P_in:
        ref_rows = oracle.permute_rows(x.view(torch.int16 if x.dtype == torch.bfloat16
                                              else torch.int32).numpy(), r_sp, K)
        got = xp[:P_in].cpu()
        got = got.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).numpy()
        assert np.array_equal(got, ref_rows)
    return P_in


def _random_slots(T, K, S, p_mask, seed, lo=0, hi=None):
    g = torch.Generator().manual_seed(seed)
    slot = torch.randint(lo, S if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    mask = (torch.rand(T, K, generator=g) < p_mask).to(torch.uint8)
    return slot, mask


@pytest.mark.parametrize("case", ["zipf_full", "ep_rank1", "s1024_many_chunks", "all_masked",
                                  "one_slot", "invalid_slots", "t0", "s1", "f32_rows",
                                  "ragged_tail"])
def test_permute_parity(dev, case):
    g = torch.Generator().manual_seed(9)
    if case == "zipf_full":
        cfg = CONFIGS["redundant_slots_zipf"]
        inp = make_inputs(cfg, with_weights=False)
        ro, rs, _ = build_slot_table(cfg.E_local, inp.replicated_experts())
        ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
        slot, _, mask = oracle.slot_map(ids, w, cfg.E, 1, 0, ro.numpy(), rs.numpy())
        x, S = inp.x, cfg.S
        slot, mask = torch.from_numpy(slot), torch.from_numpy(mask)
    elif case == "ep_rank1":
        cfg = CONFIGS["ep_share_256_bf16"]
        inp = make_inputs(cfg, with_weights=False)
        ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
        slot, _, mask = oracle.slot_map(ids, w, cfg.E, cfg.ep_size, 1)
        x, S = inp.x, cfg.E_local
        slot, mask = torch.from_numpy(slot), torch.from_numpy(mask)
    elif case == "s1024_many_chunks":
        S = 1024
        slot, mask = _random_slots(20000, 4, S, 0.9, 1)
        x = torch.randn(20000, 64, generator=g).to(torch.bfloat16)
    elif case == "all_masked":
        S = 16
        slot, mask = _random_slots(500, 3, S, 0.0, 2)
        x = torch.randn(500, 32, generator=g).to(torch.bfloat16)
    elif case == "one_slot":
        S = 7
        slot = torch.full((3000, 2), 4, dtype=torch.int32)
        mask = torch.ones(3000, 2, dtype=torch.uint8)
        x = torch.randn(3000, 16, generator=g).to(torch.bfloat16)
    elif case == "invalid_slots":
        S = 10
        slot, mask = _random_slots(777, 3, S, 0.8, 3, lo=-3, hi=14)
        x = torch.randn(777, 24, generator=g).to(torch.bfloat16)
    elif case == "t0":
        S = 5
        slot, mask = _random_slots(0, 2, S, 1.0, 4)
        x = torch.zeros(0, 16, dtype=torch.bfloat16)
    elif case == "s1":
        S = 1
        slot, mask = _random_slots(1000, 8, S, 0.5, 5)
        x = torch.randn(1000, 8, generator=g).to(torch.bfloat16)
    elif case == "f32_rows":
        S = 8
        slot, mask = _random_slots(64, 2, S, 1.0, 6)
        x = torch.randn(64, 128, generator=g)
    elif case == "ragged_tail":
        S = 33
        slot, mask = _random_slots(4099, 3, S, 0.77, 7)
        x = torch.randn(4099, 40, generator=g).to(torch.bfloat16)
    announce(f"permute {case} T={slot.shape[0]} K={slot.shape[1]} S={S}")
    _permute_check(dev, x.contiguous(), slot.contiguous(), mask.contiguous(), S)


# ------------------------------------------------------------------ grouped GEMM
def _offsets(counts):
    return torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)


def _gemm_case(dev, counts, H, I, dtype, seed, sample=None):
    g = torch.Generator().manual_seed(seed)
    S = len(counts)
    rows = int(sum(counts))
    cap = rows + 5  # capacity beyond the used rows must stay untouched
    off = _offsets(counts)
    x = torch.randn(cap, H, generator=g).to(dtype)
    wgu = (torch.randn(S, 2 * I, H, generator=g) / math.sqrt(H)).to(dtype)
    wd = (torch.randn(S, H, I, generator=g) / math.sqrt(I)).to(dtype)
    a_dev = x.to(dev)
    c1 = torch.full((cap, I), 7.0, dtype=dtype, device=dev)
    moe.grouped_gemm(moe.GATE_UP_SWIGLU, a_dev, off.to(dev), wgu.to(dev), c1)
    c2 = torch.full((cap, H), 7.0, dtype=dtype, device=dev)
    moe.grouped_gemm(moe.DOWN, c1, off.to(dev), wd.to(dev), c2)
    torch.cuda.synchronize()
    c1h, c2h = c1.cpu(), c2.cpu()
    assert (c1h[rows:] == 7.0).all() and (c2h[rows:] == 7.0).all()
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    if sample is None:
        ref1 = oracle.grouped_gate_up(x[:rows], off, wgu, I)
        assert_close(np64(c1h[:rows]), ref1, tol, "gate_up")
        ref2 = oracle.grouped_down(c1h[:rows], off, wd)
        assert_close(np64(c2h[:rows]), ref2, tol, "down")
        if rows:
            assert rel_fro(np64(c1h[:rows]), ref1) < 5e-3
            assert rel_fro(np64(c2h[:rows]), ref2) < 5e-3
    else:
        # sampled rows: one random row in every 128-row piece of every slot
        # (every work item and both halves of its row tile) plus each slot's
        # last row; regrouped by slot with their own offsets
        rng = np.random.default_rng(seed)
        o = off.numpy()
        pick = []
        for s_ in range(S):
            lo_s, hi_s = int(o[s_]), int(o[s_ + 1])
            for lo in range(lo_s, hi_s, sample):
                pick.append(int(rng.integers(lo, min(lo + sample, hi_s))))
            if hi_s > lo_s:
                pick.append(hi_s - 1)
        rsel = np.unique(np.asarray(pick, dtype=np.int64))
        slot_of = np.searchsorted(off.numpy(), rsel, side="right") - 1
        sub_off = _offsets(np.bincount(slot_of, minlength=S))
        ref1 = oracle.grouped_gate_up(x[rsel], sub_off, wgu, I)
        assert_close(np64(c1h[rsel]), ref1, tol, "gate_up (sampled)")
        ref2 = oracle.grouped_down(c1h[rsel], sub_off, wd)
        assert_close(np64(c2h[rsel]), ref2, tol, "down (sampled)")


GEMM_CASES = {
    # name: (row counts per slot, H, I, dtype)
    "ragged_slots": ([0, 1, 127, 128, 129, 300, 0, 5], 256, 192, torch.bfloat16),
    "k_not_mult_64": ([70, 0, 200, 3], 72, 136, torch.bfloat16),
    "many_small": ([3, 0, 0, 1, 2, 0, 9, 4] * 8, 128, 64, torch.bfloat16),
    "wide_n": ([257, 31], 512, 384, torch.bfloat16),
    "all_empty": ([0, 0, 0], 64, 64, torch.bfloat16),
    # about 1050 gate/up and 525 down items: several per block on the full
    # grid; last tiles of 37, 100, 128, 129, 200, 255, 64 and 65 rows
    "many_items": ([8229, 0, 8292, 8320, 8321, 8392, 8191, 8256, 8257], 512, 512,
                   torch.bfloat16),
    "f32": ([5, 0, 40, 17, 66], 128, 256, torch.float32),
}


@pytest.mark.parametrize("name", list(GEMM_CASES))
def test_grouped_gemm_parity(dev, name):
    counts, H, I, dt = GEMM_CASES[name]
    announce(f"grouped_gemm {name} rows={sum(counts)} S={len(counts)} H={H} I={I} {dt}")
    _gemm_case(dev, counts, H, I, dt, seed=len(name))


def test_grouped_gemm_zipf_full_size(dev):
    """Row counts of the redundant-slot workload at its full shape (H=4096,
    I=1024, 131072 rows over 80 slots); a row in every 128-row piece of every
    slot, and each slot's last row, against the oracle."""
    cfg = CONFIGS["redundant_slots_zipf"]
    inp = make_inputs(cfg, with_weights=False)
    ro, rs, _ = build_slot_table(cfg.E_local, inp.replicated_experts())
    ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    slot, _, mask = oracle.slot_map(ids, w, cfg.E, 1, 0, ro.numpy(), rs.numpy())
    counts = np.bincount(slot[mask == 1], minlength=cfg.S)
    announce(f"grouped_gemm zipf full size counts max={counts.max()} min={counts.min()}")
    _gemm_case(dev, counts.tolist(), cfg.H, cfg.I, torch.bfloat16, seed=3, sample=128)


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("ydt,odt,accumulate", [
    (torch.bfloat16, torch.bfloat16, False), (torch.bfloat16, torch.float32, False),
    (torch.bfloat16, torch.float32, True), (torch.float32, torch.float32, False),
    (torch.float32, torch.bfloat16, True)])
def test_combine_parity(dev, ydt, odt, accumulate):
    g = torch.Generator().manual_seed(21)
    T, K, H, S = 1031, 6, 136, 12
    slot = torch.randint(0, S, (T, K), generator=g, dtype=torch.int32)
    mask = (torch.rand(T, K, generator=g) < 0.6).to(torch.uint8)
    mask[:5] = 0  # tokens with no included pair
    off, sp, pr = oracle.permute_indices(slot, mask, S)
    P_in = int(off[-1])
    y = torch.randn(P_in, H, generator=g).to(ydt)
    wm = torch.rand(T, K, generator=g) * mask
    prev = torch.randn(T, H, generator=g).to(odt)
    announce(f"combine y={ydt} out={odt} accumulate={accumulate}")
    out = prev.to(dev) if accumulate else None
    got = moe.combine(y.to(dev), torch.from_numpy(pr).to(dev), wm.to(dev), K, out=out,
                      out_dtype=odt, accumulate=accumulate)
    torch.cuda.synchronize()
    ref = oracle.combine_rows(y, pr, wm, K)
    if accumulate:
        ref = ref + np64(prev)
    tol = BF16_TOL if odt == torch.bfloat16 else (1e-5, 1e-6)
    assert_close(np64(got.cpu()), ref, tol, "combine")
    if not accumulate:
        assert (got[:5] == 0).all()


def test_combine_single_pair_is_exact_copy(dev):
    """K = 1 with weight 1.0: combine copies the expert row bit for bit."""
    g = torch.Generator().manual_seed(4)
    T, H = 300, 256
    y = torch.randn(T, H, generator=g).to(torch.bfloat16)
    perm = torch.randperm(T, generator=g).to(torch.int32)
    w = torch.ones(T, 1)
    got = moe.combine(y.to(dev), perm.to(dev), w.to(dev), 1, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu().view(torch.int16), y[perm.long()].view(torch.int16))


# ------------------------------------------------------------------ grouped routing
@pytest.mark.parametrize("E,G,TG,K,ties,T", [
    (160, 8, 3, 6, False, 777),
    (256, 8, 4, 8, True, 512),
    (64, 64, 6, 6, False, 300),
    (16, 1, 1, 4, True, 65),
    (128, 16, 16, 8, False, 200),
    (96, 4, 1, 24, True, 130),
    (32, 4, 2, 3, False, 0),
])
def test_route_grouped_parity(dev, E, G, TG, K, ties, T):
    announce(f"route grouped E={E} G={G} TG={TG} K={K} ties={ties} T={T}")
    g = torch.Generator().manual_seed(E + G + TG)
    logits = torch.randn(T, E, generator=g)
    if ties:
        logits = torch.round(logits * 2) / 2
    logits = logits.float().contiguous()
    for renorm in (False, True):
        ids, w = moe.route(logits.to(dev), K, renorm, num_groups=G, topk_groups=TG)
        torch.cuda.synchronize()
        if T == 0:
            continue
        ref_ids, ref_w = oracle.route_grouped(logits.numpy(), K, renorm, G, TG)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)
        assert_close(np64(w), ref_w, (1e-5, 1e-9), "grouped route weights")
