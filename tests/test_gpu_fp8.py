"""FP8 (E4M3) expert path on the GPU against the FP8 oracle.

- moe_quantize_fp8 is compared bit for bit with the oracle's quantize: both
  take the same decision (the f32 product with the f32 reciprocal scale, then
  the nearest code with ties to even), including midpoints, subnormals and
  saturation.
- The gate/up GEMM writes codes of the SwiGLU output. Floating point decides
  them and the kernel accumulates in f32 in its own order, so each code must
  be the rounding of some value within the f32 error bound of the oracle's
  exact value (K * 2^-24 * sum|products|, carried through silu(g) * u); near
  zero, where codes are 2^-9 apart, that can span several codes. Codes other
  than the exact value's own must be rare.
- The down GEMM and the forward (bf16 outputs) are compared elementwise at
  the bf16 tolerance; the forward also at full size on sampled tokens, with
  replicated slots (bit-identical to the identity table) and EP shares.
  Where a forward compares many outputs, a code that the f32 error bound
  leaves open (see _check_codes) is as correct as the exact value's own, and
  one step of a large code moves its token's outputs by about
  a2 * step * |Wd|: outputs beyond the bf16 tolerance must then be rare and
  within that allowance, and the fused forward bit-identical to the staged
  FP8 calls on the same device.
"""
import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe
import oracle
from gpu_common import BF16_TOL, announce, assert_close, covering_tokens, device, np64, rel_fro
from workloads import (CONFIGS, WorkloadConfig, build_slot_table, identity_slot_table,
                       make_inputs, slot_weights)
from workloads.configs import small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _rand_codes(shape, g, lo=0x20, hi=0x48):
    mag = torch.randint(lo, hi, shape, generator=g, dtype=torch.uint8)
    return mag | (torch.randint(0, 2, shape, generator=g, dtype=torch.uint8) << 7)


# ------------------------------------------------------------------ quantize
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 4096 * 3 + 5])
def test_quantize_bit_exact(dev, dt, n):
    announce(f"quantize fp8 {dt} n={n}")
    g = torch.Generator().manual_seed(n)
    x = torch.randn(n, generator=g) * 10.0 ** torch.randint(-3, 3, (n,), generator=g).float()
    special = torch.tensor([0.0, -0.0, 448.0, 460.0, 464.0, 479.0, 480.0, 1e6, -1e6,
                            2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -9, 1.0625, 1.1875, 248.0])
    m = min(n, special.numel())
    x[:m] = special[:m]
    x = x.to(dt)
    for scale in (1.0, 0.25, 0.0178):
        q = moe.quantize_fp8(x.to(dev), scale)
        torch.cuda.synchronize()
        want = oracle.quantize_fp8(x, scale)
        assert np.array_equal(q.cpu().numpy(), want), (dt, n, scale)


def test_quantize_empty(dev):
    q = moe.quantize_fp8(torch.empty(0, dtype=torch.bfloat16, device=dev), 1.0)
    assert q.numel() == 0


# ------------------------------------------------------------------ GEMM stages
def _stage_inputs(H, I, sizes, seed):
    g = torch.Generator().manual_seed(seed)
    S = len(sizes)
    off = torch.tensor([0] + list(np.cumsum(sizes)), dtype=torch.int32)
    rows = int(off[-1])
    a = _rand_codes((rows, H), g)
    wgu = _rand_codes((S, 2 * I, H), g)
    a2 = _rand_codes((rows, I), g)
    wd = _rand_codes((S, H, I), g)
    # per-slot scales; slot 1 much larger so its SwiGLU outputs saturate
    wsc = (torch.rand(S, generator=g) * 0.5 + 0.75) / np.sqrt(H)
    if S > 1:
        wsc[1] *= 40.0
    wdsc = (torch.rand(S, generator=g) * 0.5 + 0.75) / np.sqrt(I)
    return off, a, wgu, a2, wd, wsc.float(), wdsc.float()


def _swiglu_bound(aq, a_scale, wg, wu, w_scale):
    """Exact SwiGLU values of code rows aq against gate / up code rows wg, wu
    (slot weight scale w_scale) and, per element, a bound on the error of an
    f32 evaluation: the accumulation of K exact code products in any order
    errs by at most K * 2^-24 * sum|products| (times the scale), which
    propagates through silu(g) * u with the derivatives; plus 1e-6 relative
    for the f32 exp and reciprocal."""
    sc = a_scale * w_scale
    g = oracle.fp8_linear(aq, a_scale, wg, w_scale)
    u = oracle.fp8_linear(aq, a_scale, wu, w_scale)
    av = np.abs(oracle.e4m3_decode(aq))
    gam = aq.shape[1] * 2.0 ** -24
    Sg = sc * (av @ np.abs(oracle.e4m3_decode(wg)).T)
    Su = sc * (av @ np.abs(oracle.e4m3_decode(wu)).T)
    sig = 1.0 / (1.0 + np.exp(-g))
    A = g * sig * u
    dsilu = sig * (1.0 + g * (1.0 - sig))
    dA = np.abs(dsilu * u) * gam * Sg + np.abs(g * sig) * gam * Su + 1e-6 * np.abs(A)
    return A, dA


def _gate_up_bounds(a, off, wgu, a_scale, wsc, I):
    """_swiglu_bound over the slots of a grouped gate/up product."""
    a = a.numpy()
    wgu = wgu.numpy()
    off = off.numpy()
    rows = a.shape[0]
    A = np.zeros((rows, I))
    dA = np.zeros((rows, I))
    for s in range(off.size - 1):
        lo, hi = int(off[s]), int(off[s + 1])
        if hi == lo:
            continue
        A[lo:hi], dA[lo:hi] = _swiglu_bound(a[lo:hi], a_scale, wgu[s, :I], wgu[s, I:],
                                            float(wsc[s]))
    return A, dA


def _assert_fp8_forward_close(got, ref, inp, tokens, what):
    """Outputs outside the bf16 tolerance must be rare (at most 1 in 10^4)
    and each within the code-decision allowance of its element
    (_forward_code_allowance, computed for the tokens concerned): a code the
    f32 error bound leaves open moves a few outputs of its token by about
    one large code step, while a wrong row or tile would move most of them."""
    excess = np.abs(got - ref) - (BF16_TOL[1] + BF16_TOL[0] * np.abs(ref))
    bad = excess > 0
    n_bad = int(bad.sum())
    print(f"{what}: {n_bad} of {got.size} outputs outside the bf16 tolerance", flush=True)
    assert n_bad <= max(16, got.size // 10000), f"{what}: {n_bad} outputs out of tolerance"
    if n_bad:
        rows = np.nonzero(bad.any(axis=1))[0]
        allowance = _forward_code_allowance(inp, np.asarray(tokens)[rows])
        over = excess[rows][bad[rows]] - allowance[bad[rows]]
        assert (over <= 0).all(), (
            f"{what}: {int((over > 0).sum())} outputs beyond the code-decision allowance, "
            f"worst by {over.max():.3e}")


def _forward_code_allowance(inp, tokens, ep_rank=0):
    """Per output element of `tokens`, the largest change that SwiGLU codes
    decided on an f32 accumulation (in the kernel's own order) can cause:
    a code may be any rounding of a value within the f32 error bound of the
    exact one (_swiglu_bound), so where that interval spans a rounding
    midpoint the neighbouring code is as correct as the exact value's own.
    Each such code's largest step, times a2 * s_d * |Wd| and the pair's
    routing weight, summed over the token's pairs. Zero almost everywhere."""
    cfg = inp.cfg
    I = cfg.I
    x = inp.x[torch.from_numpy(tokens)]
    ids, w = oracle.route(inp.logits.numpy()[tokens], cfg.K, cfg.renormalize)
    lo_e = ep_rank * cfg.E_local
    xq = oracle.quantize_fp8(x, cfg.a1_scale)
    wgu, wd = inp.w_gate_up.numpy(), inp.w_down.numpy()
    out = np.zeros((tokens.size, cfg.H))
    for e in range(lo_e, lo_e + cfg.E_local):
        rr, kk = np.nonzero(ids == e)
        if rr.size == 0:
            continue
        sg = float(inp.w_gate_up_scale[e])
        A, dA = _swiglu_bound(xq[rr], cfg.a1_scale, wgu[e, :I], wgu[e, I:], sg)
        want = oracle.e4m3_decode(oracle.quantize_fp8(A.astype(np.float32), cfg.a2_scale))
        lo = oracle.e4m3_decode(oracle.quantize_fp8((A - dA).astype(np.float32), cfg.a2_scale))
        hi = oracle.e4m3_decode(oracle.quantize_fp8((A + dA).astype(np.float32), cfg.a2_scale))
        step = np.maximum(hi - want, want - lo) * cfg.a2_scale
        if not step.any():
            continue
        dy = (step @ np.abs(oracle.e4m3_decode(wd[e])).T) * float(inp.w_down_scale[e])
        np.add.at(out, rr, w[rr, kk][:, None] * dy)
    return out


def _check_codes(got, A, dA, c_scale, what):
    """Each code must round (as the kernel does) some value within dA of the
    exact value A; the codes differing from the exact value's own code must be
    few."""
    want = oracle.quantize_fp8(A.astype(np.float32), c_scale)
    lo = oracle.quantize_fp8((A - dA).astype(np.float32), c_scale)
    hi = oracle.quantize_fp8((A + dA).astype(np.float32), c_scale)
    gv = oracle.e4m3_decode(got)
    assert not np.isnan(gv).any(), f"{what}: NaN codes written"
    ok = (gv >= oracle.e4m3_decode(lo)) & (gv <= oracle.e4m3_decode(hi))
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(
            f"{what}: {int((~ok).sum())} codes outside the error bound; first at {tuple(i)}: "
            f"got {gv[tuple(i)]!r}, exact {A[tuple(i)] / c_scale!r} +- {dA[tuple(i)] / c_scale!r}")
    n_diff = int((got != want).sum())
    assert n_diff <= max(8, got.size // 200), f"{what}: {n_diff} codes differ from the exact one"
    return n_diff


@pytest.mark.parametrize("H,I,sizes", [
    (256, 256, [0, 1, 100, 128, 129, 256, 300, 0]),   # empty, tiny, half and ragged tiles
    (512, 384, [513, 7, 0, 256, 1000]),
    (1024, 1408, [700, 1, 300]),                       # I = 11 * 128 (odd slice count)
    # about 1050 items: several per block on the full grid
    (512, 512, [8229, 0, 8292, 8320, 8321, 8392, 8191, 8256, 8257]),
])
def test_gemm_gate_up_codes(dev, H, I, sizes):
    announce(f"fp8 gate/up GEMM H={H} I={I} sizes={sizes}")
    off, a, wgu, _, _, wsc, _ = _stage_inputs(H, I, sizes, seed=H + I)
    a_scale, c_scale = 0.5, 1.0 / 56.0
    got = moe.grouped_gemm_fp8(moe.GATE_UP_SWIGLU, a.to(dev), a_scale, off.to(dev), wgu.to(dev),
                               wsc.to(dev), c_scale)
    torch.cuda.synchronize()
    A, dA = _gate_up_bounds(a, off, wgu, a_scale, wsc.double().numpy(), I)
    # the stage oracle gives the same exact values
    np.testing.assert_allclose(
        A, oracle.fp8_grouped_gate_up(a.numpy(), off.numpy(), wgu.numpy(), a_scale,
                                      wsc.double().numpy(), I), rtol=1e-12, atol=1e-12)
    _check_codes(got.cpu().numpy(), A, dA, c_scale, f"gate/up {H}x{I}")
    if len(sizes) > 1 and sizes[1] > 0:  # the saturated slot
        lo, hi = int(off[1]), int(off[2])
        codes = got.cpu().numpy()[lo:hi]
        assert np.isin(codes, [0x7E, 0xFE]).any(), "expected saturated outputs in slot 1"
        assert not np.isin(codes, [0x7F, 0xFF]).any(), "NaN codes written"


@pytest.mark.parametrize("H,I,sizes", [
    (256, 256, [0, 1, 100, 128, 129, 256, 300, 0]),
    (640, 384, [513, 7, 0, 256, 1000]),
    (512, 512, [8229, 0, 8292, 8320, 8321, 8392, 8191, 8256, 8257]),  # ~525 items
])
def test_gemm_down_bf16(dev, H, I, sizes):
    announce(f"fp8 down GEMM H={H} I={I} sizes={sizes}")
    off, _, _, a2, wd, _, wdsc = _stage_inputs(H, I, sizes, seed=7 * H + I)
    a_scale = 0.25
    got = moe.grouped_gemm_fp8(moe.DOWN, a2.to(dev), a_scale, off.to(dev), wd.to(dev),
                               wdsc.to(dev))
    torch.cuda.synchronize()
    ref = oracle.fp8_grouped_down(a2.numpy(), off.numpy(), wd.numpy(), a_scale,
                                  wdsc.double().numpy())
    assert_close(np64(got.cpu()), ref, BF16_TOL, f"down {H}x{I}")
    assert rel_fro(np64(got.cpu()), ref) < 5e-3


# ------------------------------------------------------------------ forward
def _share(inp, dev, ep_rank=0, replicas=False):
    cfg = inp.cfg
    wgu, wd = inp.share_weights(ep_rank)
    sgu, sd = inp.share_scales(ep_rank)
    if replicas:
        ro, rs, se = build_slot_table(cfg.E_local, inp.replicated_experts())
        wgu, wd = slot_weights(wgu, se), slot_weights(wd, se)
        sgu, sd = slot_weights(sgu, se), slot_weights(sd, se)
        S = int(se.numel())
    else:
        ro, rs = identity_slot_table(cfg.E_local)
        S = cfg.E_local
    return [t.contiguous().to(dev) for t in (wgu, wd, sgu, sd, ro, rs)] + [S]


def _run(inp, dev, ep_rank=0, replicas=False, shared=None):
    cfg = inp.cfg
    wgu, wd, sgu, sd, ro, rs, S = _share(inp, dev, ep_rank, replicas)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=S, dtype=moe.FP8,
                           ep_size=cfg.ep_size, ep_rank=ep_rank, a1_scale=cfg.a1_scale,
                           a2_scale=cfg.a2_scale)
    return moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), rep_off=ro,
                       rep_slots=rs, w_gate_up_scale=sgu, w_down_scale=sd,
                       shared_out=None if shared is None else shared.to(dev))


def _oracle(inp, tokens=None, ep_rank=0, shared=None):
    cfg = inp.cfg
    return oracle.fp8_forward(inp.x, inp.logits, inp.w_gate_up.numpy(), inp.w_gate_up_scale,
                              inp.w_down.numpy(), inp.w_down_scale, cfg.a1_scale, cfg.a2_scale,
                              cfg.K, cfg.renormalize, cfg.ep_size, ep_rank, tokens=tokens,
                              shared=shared)


MEDIUM = {
    "zipf_replicas": small("redundant_slots_zipf_fp8", 700, H=256, I=384),
    "deepseek_ragged": small("deepseek_v2_fp8", 333, H=512, I=256),
}


@pytest.mark.parametrize("name", list(MEDIUM))
def test_forward_medium_all_tokens(dev, name):
    inp = make_inputs(MEDIUM[name])
    replicas = inp.cfg.n_replicated > 0
    announce(f"fp8 forward {name} (all tokens, replicas={replicas})")
    out = _run(inp, dev, replicas=replicas)
    torch.cuda.synchronize()
    ref = _oracle(inp)
    assert_close(np64(out.cpu()), ref, BF16_TOL, name)
    assert rel_fro(np64(out.cpu()), ref) < 1e-2
    if replicas:  # replica slots hold copies: bit-identical to the identity table
        ident = _run(inp, dev, replicas=False)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().view(torch.int16), ident.cpu().view(torch.int16))


def test_forward_ep_shares_and_shared_add(dev):
    cfg = WorkloadConfig("fp8_ep", T=300, H=256, I=256, E=16, K=4, renormalize=True,
                         dtype="fp8", router="gauss", ep_size=2, seed=41)
    inp = make_inputs(cfg)
    announce("fp8 forward EP shares + shared-expert add")
    shared = torch.randn(cfg.T, cfg.H, generator=torch.Generator().manual_seed(2)).to(
        torch.bfloat16)
    parts = []
    for r in range(2):
        out = _run(inp, dev, ep_rank=r, shared=shared if r == 0 else None)
        torch.cuda.synchronize()
        ref = _oracle(inp, ep_rank=r, shared=shared if r == 0 else None)
        assert_close(np64(out.cpu()), ref, BF16_TOL, f"share {r}")
        parts.append(ref)
    full = oracle.fp8_forward(inp.x, inp.logits, inp.w_gate_up.numpy(), inp.w_gate_up_scale,
                              inp.w_down.numpy(), inp.w_down_scale, cfg.a1_scale, cfg.a2_scale,
                              cfg.K, True, shared=shared)
    np.testing.assert_allclose(parts[0] + parts[1], full, rtol=1e-9, atol=1e-9)


def _covering(inp, replicas, seed=0):
    """Covering sample of the layer's permutation as the oracle computes it."""
    cfg = inp.cfg
    ids, w = oracle.route(inp.logits, cfg.K, cfg.renormalize)
    if replicas:
        ro, rs, se = build_slot_table(cfg.E_local, inp.replicated_experts())
        ro, rs, S = ro.numpy(), rs.numpy(), int(se.numel())
    else:
        ro = rs = None
        S = cfg.E_local
    slot, _, mask = oracle.slot_map(ids, w, cfg.E, cfg.ep_size, 0, ro, rs)
    off, sp, pr = oracle.permute_indices(slot, mask, S)
    return covering_tokens(off, sp, pr, cfg.K, seed=seed)


@pytest.mark.parametrize("name,replicas", [("redundant_slots_zipf_fp8", True),
                                           ("deepseek_v2_fp8", False)])
def test_forward_full_size_covering(dev, name, replicas):
    """Full-size FP8 layers on a covering sample: at least one sampled row in
    every 128-row piece of every slot, plus each slot's last row."""
    inp = make_inputs(CONFIGS[name])
    tokens = _covering(inp, replicas, seed=3)
    announce(f"fp8 forward {name} full size, {tokens.size} covering tokens")
    out = _run(inp, dev, replicas=replicas)
    torch.cuda.synchronize()
    got = np64(out[torch.from_numpy(tokens).to(dev)].cpu())
    ref = _oracle(inp, tokens=tokens)
    _assert_fp8_forward_close(got, ref, inp, tokens, name)


def test_forward_many_items_per_block_all_tokens(dev):
    """16384 tokens, H = I = 512, 8 experts, top-4: about 1050 gate/up and 525
    down items, several per block on the full grid. Every output against the
    FP8 oracle; the run with the GEMM grid capped at 16 blocks is
    bit-identical."""
    cfg = WorkloadConfig("fp8_mi", T=16384, H=512, I=512, E=8, K=4, renormalize=True,
                         dtype="fp8", router="gauss_bias", bias_std=0.3, seed=51)
    inp = make_inputs(cfg)
    announce("fp8 forward many items per block (all tokens)")
    out = _run(inp, dev)
    wgu, wd, sgu, sd, ro, rs, S = _share(inp, dev)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=True, S=S, dtype=moe.FP8, a1_scale=cfg.a1_scale,
                           a2_scale=cfg.a2_scale, gemm_blocks=16)
    capped = moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), rep_off=ro,
                         rep_slots=rs, w_gate_up_scale=sgu, w_down_scale=sd)
    # the staged FP8 calls: x quantized, its code rows permuted (bytes, viewed
    # as bf16), the grouped GEMMs on the permuted rows, the combine
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    slot, wm, mask = moe.slot_map(ids, w, cfg.E, 1, 0, ro, rs)
    xq = moe.quantize_fp8(inp.x.to(dev), cfg.a1_scale)
    off, sp, pr, xp = moe.permute(xq.view(torch.bfloat16), slot, mask, S)
    a = moe.grouped_gemm_fp8(moe.GATE_UP_SWIGLU, xp.view(torch.uint8), cfg.a1_scale, off, wgu,
                             sgu, cfg.a2_scale)
    y = moe.grouped_gemm_fp8(moe.DOWN, a, cfg.a2_scale, off, wd, sd)
    staged = moe.combine(y, pr, wm, cfg.K)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), capped.view(torch.int16))
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))
    ref = _oracle(inp)
    _assert_fp8_forward_close(np64(out.cpu()), ref, inp, np.arange(cfg.T),
                              "fp8 many items per block")
    assert rel_fro(np64(out.cpu()), ref) < 1e-2


@pytest.mark.parametrize("name,blocks", [("zipf_replicas", 3), ("deepseek_ragged", 5)])
def test_forward_medium_capped_grid(dev, name, blocks):
    """Medium FP8 shapes with the GEMM grid capped: each block runs many items
    in a row. Every output against the oracle, bit-identical to the full grid."""
    inp = make_inputs(MEDIUM[name])
    cfg = inp.cfg
    replicas = cfg.n_replicated > 0
    announce(f"fp8 forward medium {name}, GEMM grid capped at {blocks} blocks")
    full = _run(inp, dev, replicas=replicas)
    wgu, wd, sgu, sd, ro, rs, S = _share(inp, dev, replicas=replicas)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=S, dtype=moe.FP8,
                           a1_scale=cfg.a1_scale, a2_scale=cfg.a2_scale, gemm_blocks=blocks)
    capped = moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), rep_off=ro,
                         rep_slots=rs, w_gate_up_scale=sgu, w_down_scale=sd)
    torch.cuda.synchronize()
    assert_close(np64(capped.cpu()), _oracle(inp), BF16_TOL, name)
    assert torch.equal(full.view(torch.int16), capped.view(torch.int16))


def test_forward_ep_accumulate_f32(dev):
    """The EP shares accumulated on the device into one f32 output equal the
    full FP8 layer (the partial-sum identity with FP8 experts)."""
    cfg = WorkloadConfig("fp8_ep_acc", T=257, H=256, I=256, E=16, K=3, renormalize=True,
                         dtype="fp8", router="gauss_bias", bias_std=0.5, ep_size=4, seed=43)
    inp = make_inputs(cfg)
    announce("fp8 forward: 4 EP shares accumulated in f32")
    out = torch.zeros(cfg.T, cfg.H, dtype=torch.float32, device=dev)
    for r in range(cfg.ep_size):
        wgu, wd, sgu, sd, ro, rs, S = _share(inp, dev, ep_rank=r)
        fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                               renormalize=True, S=S, dtype=moe.FP8, out_dtype=torch.float32,
                               ep_size=cfg.ep_size, ep_rank=r, accumulate=True,
                               a1_scale=cfg.a1_scale, a2_scale=cfg.a2_scale)
        moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), rep_off=ro,
                    rep_slots=rs, out=out, w_gate_up_scale=sgu, w_down_scale=sd)
    torch.cuda.synchronize()
    full = oracle.fp8_forward(inp.x, inp.logits, inp.w_gate_up.numpy(), inp.w_gate_up_scale,
                              inp.w_down.numpy(), inp.w_down_scale, cfg.a1_scale, cfg.a2_scale,
                              cfg.K, True)
    assert_close(np64(out.cpu()), full, BF16_TOL, "fp8 EP accumulate")


def test_forward_grouped_routing_topk_form(dev):
    """Group-limited routing from logits, and the oracle's routing passed as
    precomputed experts and weights, both match the FP8 oracle."""
    cfg = small("deepseek_v2_fp8", 300, H=256, I=384)
    cfg = cfg.replace(num_expert_group=8, topk_group=3)
    inp = make_inputs(cfg)
    announce("fp8 forward: grouped routing, logits and top-k forms")
    wgu, wd, sgu, sd, ro, rs, S = _share(inp, dev)
    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=True, S=S, dtype=moe.FP8, num_expert_group=8,
                           topk_group=3, a1_scale=cfg.a1_scale, a2_scale=cfg.a2_scale)
    kw = dict(rep_off=ro, rep_slots=rs, w_gate_up_scale=sgu, w_down_scale=sd)
    out = moe.forward(fc, inp.x.to(dev), wgu, wd, logits=inp.logits.to(dev), **kw)
    ids, w = oracle.route_grouped(inp.logits.numpy(), cfg.K, True, 8, 3)
    out2 = moe.forward(fc, inp.x.to(dev), wgu, wd,
                       topk_ids=torch.from_numpy(ids.astype(np.int32)).to(dev),
                       topk_w=torch.from_numpy(w.astype(np.float32)).to(dev), **kw)
    torch.cuda.synchronize()
    ref = oracle.fp8_forward(inp.x, None, inp.w_gate_up.numpy(), inp.w_gate_up_scale,
                             inp.w_down.numpy(), inp.w_down_scale, cfg.a1_scale, cfg.a2_scale,
                             cfg.K, False, topk=(ids, w))
    assert_close(np64(out.cpu()), ref, BF16_TOL, "fp8 grouped routing")
    assert_close(np64(out2.cpu()), ref, BF16_TOL, "fp8 grouped routing, top-k form")
