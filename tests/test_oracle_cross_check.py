"""The blocked oracle forward (each expert's rows evaluated together) against
the literal per-pair form (three matrix-vector products per pair, then the
per-token weighted sum over k ascending), on a fixed sample of tokens of
every workload shape the layer is measured on, at its full size.

Page: DeepSpeed PR #6964 "AutoTP for MoE models", Description -- each
token's routed output is the weighted sum of the outputs of its selected
experts; TensorRT-LLM PR #10985, review of torch_moe.py -- the gated expert
MLP. Only the experts the sampled tokens reach are drawn (the generator
draws each expert from its own seed, so a subset is exact).
"""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
from workloads import CONFIGS, make_inputs
from workloads.generate import make_expert_weights

N_TOKENS = 64


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    if T <= n:
        return np.arange(T)
    return np.sort(rng.choice(T, size=n, replace=False))


def _inputs_for(name, ep_rank, seed):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, with_weights=False)
    tokens = _sample(cfg.T, N_TOKENS, seed)
    ids, _ = oracle.route(inp.logits.numpy()[tokens], cfg.K, cfg.renormalize)
    lo = ep_rank * cfg.E_local
    experts = sorted({int(e) for e in ids.ravel() if lo <= e < lo + cfg.E_local})
    inp.w_gate_up, inp.w_down = make_expert_weights(cfg, experts)
    return cfg, inp, tokens


@pytest.mark.parametrize("name,ep_rank", [
    ("tiny_fp32", 0),
    ("qwen2_moe_bf16", 0),
    ("deepseek_v2_bf16", 0),
    ("ep_share_256_bf16", 1),
    ("redundant_slots_zipf", 0),
])
def test_blocked_forward_equals_per_pair_loop(name, ep_rank):
    cfg, inp, tokens = _inputs_for(name, ep_rank, seed=11)
    blocked = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                             cfg.renormalize, cfg.ep_size, ep_rank, tokens=tokens)
    literal = oracle.forward_per_pair(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                                      cfg.renormalize, cfg.ep_size, ep_rank, tokens=tokens)
    assert np.abs(literal).max() > 0
    # both fp64; only the summation order inside the library products differs
    np.testing.assert_allclose(blocked, literal, rtol=1e-11, atol=1e-12 * np.abs(literal).max())


def test_per_pair_loop_catches_misplaced_rows(monkeypatch):
    """A blocked form that hands an expert's outputs to the wrong pairs (rows
    reversed inside the expert's block) differs from the literal loop."""
    cfg, inp, tokens = _inputs_for("tiny_fp32", 0, seed=11)
    orig = om.swiglu_mlp

    def bad(xrows, wg, wu, wd):
        return orig(xrows, wg, wu, wd)[::-1]
    monkeypatch.setattr(om, "swiglu_mlp", bad)
    blocked = om.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K, cfg.renormalize,
                         tokens=tokens)
    literal = om.forward_per_pair(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                                  cfg.renormalize, tokens=tokens)
    assert np.abs(blocked - literal).max() > 1e-3
