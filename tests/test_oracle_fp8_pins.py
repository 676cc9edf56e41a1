"""Pins of the FP8 (E4M3) oracle against facts fixed outside it: the format's
closed-form values, exhaustive round trips, the tie and saturation rules, a
brute-force nearest-code search, power-of-two scale exactness, agreement with
the (separately pinned) unquantized oracle on dequantized operands, a dense
brute-force MoE on tiny inputs and the EP partial-sum identity."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode, quantize_fp8

ALL = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_closed_forms():
    want = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0x77: 240.0,
            0x78: 256.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
            0x0F: 1.875 * 2.0 ** -6, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in want.items():
        assert e4m3_decode([c])[0] == v, hex(c)
    assert np.signbit(e4m3_decode([0x80])[0]) and e4m3_decode([0x80])[0] == 0.0
    assert np.isnan(e4m3_decode([0x7F, 0xFF])).all()
    assert np.isnan(e4m3_decode(ALL)).sum() == 2


def test_decode_order_and_symmetry():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7e strictly increasing
    assert pos.size == 127 and pos[-1] == oracle.E4M3_MAX
    neg = e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_values_exact_in_bf16():
    v = e4m3_decode(FINITE)
    t = torch.tensor(v, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


def test_encode_round_trip_every_code():
    assert np.array_equal(e4m3_encode(e4m3_decode(FINITE)), FINITE)


def test_encode_ties_to_even_and_neighbours():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(126):
        mid = 0.5 * (pos[c] + pos[c + 1])  # exact in fp64
        even = c if c % 2 == 0 else c + 1
        assert e4m3_encode([mid])[0] == even
        assert e4m3_encode([-mid])[0] == (even | 0x80)
        assert e4m3_encode([np.nextafter(mid, np.inf)])[0] == c + 1
        assert e4m3_encode([np.nextafter(mid, -np.inf)])[0] == c


def test_encode_saturates():
    v = np.array([448.0, 450.0, 464.0, 479.9, 480.0, 1e6, 3.0e38])
    assert np.all(e4m3_encode(v) == 0x7E)
    assert np.all(e4m3_encode(-v) == 0xFE)


def test_encode_brute_force_nearest():
    """Exhaustive nearest-value search over all finite codes (ties: even code)."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-4, 3, 4000),
                        rng.uniform(-500, 500, 1000)]).astype(np.float32).astype(np.float64)
    vals = e4m3_decode(FINITE)
    got = e4m3_encode(v)
    for x, g in zip(v, got):
        a = min(abs(x), 448.0)
        d = np.abs(vals - np.copysign(a, x))
        cand = FINITE[d == d.min()]
        cand = cand[(cand & 0x80) == (0x80 if np.signbit(x) else 0)] if cand.size > 1 else cand
        best = cand[0] if cand.size == 1 else [c for c in cand if c % 2 == 0][0]
        assert g == best, (x, hex(g), hex(best))


def test_decode_and_encode_match_torch_float8():
    """A second, independent implementation of the format: torch's
    float8_e4m3fn (the OCP E4M3 variant without infinities). Decoding every
    code and encoding values of every magnitude inside the finite range,
    midpoints between neighbours included, agree bit for bit. (Beyond 448 the
    two differ by design: torch gives NaN, the reading here saturates.)"""
    tv = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = e4m3_decode(ALL)
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    fin = ~np.isnan(ov)
    assert np.array_equal(tv[fin], ov[fin])
    assert np.array_equal(np.signbit(tv[fin]), np.signbit(ov[fin]))
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = 0.5 * (pos[:-1] + pos[1:])
    rng = np.random.default_rng(12)
    v = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), pos,
                        rng.standard_normal(20000) * 10.0 ** rng.integers(-5, 3, 20000),
                        rng.uniform(-448, 448, 5000), [0.0, -0.0, 2.0 ** -10, -2.0 ** -11]])
    v = v.astype(np.float32)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 448.0]
    tq = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), tq)


def test_quantize_power_of_two_scale_is_exact():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(2000).astype(np.float32)
    for k in (-5, 0, 3):
        s = 2.0 ** k
        assert np.array_equal(quantize_fp8(x * np.float32(s), s), e4m3_encode(x))
    # representable values map to their codes; out-of-range values clamp
    assert np.array_equal(quantize_fp8(e4m3_decode(FINITE).astype(np.float32), 1.0), FINITE)
    assert quantize_fp8(np.array([1000.0], np.float32), 1.0)[0] == 0x7E


def test_quantize_bf16_tensor_input():
    x = torch.randn(64, 32, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    q = quantize_fp8(x, 0.03125)  # 2^-5: exact scaling
    assert np.array_equal(q, e4m3_encode(x.to(torch.float64).numpy() * 32.0))


def _codes(rng, shape, lo=0x20, hi=0x48):
    """Random E4M3 codes with magnitudes in [0x20, 0x48) and random signs."""
    c = rng.integers(lo, hi, size=shape).astype(np.uint8)
    return np.where(rng.random(shape) < 0.5, c | 0x80, c).astype(np.uint8)


def test_linear_brute_force():
    rng = np.random.default_rng(5)
    qa, qw = _codes(rng, (3, 16)), _codes(rng, (5, 16))
    got = oracle.fp8_linear(qa, 0.25, qw, 3.0)
    for i in range(3):
        for n in range(5):
            ref = sum(float(e4m3_decode([qa[i, k]])[0]) * float(e4m3_decode([qw[n, k]])[0])
                      for k in range(16)) * 0.75
            assert got[i, n] == pytest.approx(ref, rel=1e-14, abs=1e-14)


def test_grouped_stages_match_unquantized_oracle_on_dequantized_operands():
    """FP8 stages == the unquantized stage oracle run on dec(q) * scale."""
    rng = np.random.default_rng(6)
    H, I, sizes = 32, 16, [5, 0, 7]
    off = np.concatenate([[0], np.cumsum(sizes)])
    rows = int(off[-1])
    qa = _codes(rng, (rows, H))
    qgu = _codes(rng, (3, 2 * I, H))
    qa2 = _codes(rng, (rows, I))
    qd = _codes(rng, (3, H, I))
    s_a, s_w = 0.125, np.array([0.5, 2.0, 0.0625])
    got = oracle.fp8_grouped_gate_up(qa, off, qgu, s_a, s_w, I)
    ref = oracle.grouped_gate_up(e4m3_decode(qa) * s_a, off,
                                 e4m3_decode(qgu) * s_w[:, None, None], I)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    got = oracle.fp8_grouped_down(qa2, off, qd, s_a, s_w)
    ref = oracle.grouped_down(e4m3_decode(qa2) * s_a, off, e4m3_decode(qd) * s_w[:, None, None])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_expert_mlp_is_the_composition_of_pinned_pieces():
    rng = np.random.default_rng(7)
    H, I = 32, 16
    xq = _codes(rng, (6, H))
    wgu, wd = _codes(rng, (2 * I, H)), _codes(rng, (H, I))
    a1, s_gu, s_d, a2 = 0.25, 0.125, 0.5, 0.75
    y, a, aq = oracle.fp8_expert_mlp(xq, a1, wgu, s_gu, wd, s_d, a2, return_act=True)
    g = (e4m3_decode(xq) * a1) @ (e4m3_decode(wgu[:I]) * s_gu).T
    u = (e4m3_decode(xq) * a1) @ (e4m3_decode(wgu[I:]) * s_gu).T
    np.testing.assert_allclose(a, oracle.silu(g) * u, rtol=1e-12)
    assert np.array_equal(aq, quantize_fp8(a.astype(np.float32), a2))
    np.testing.assert_allclose(y, (e4m3_decode(aq) * a2) @ (e4m3_decode(wd) * s_d).T, rtol=1e-12)
    # the unquantized gated MLP (pinned separately) on the dequantized operands,
    # with the activation quantization removed, differs only by that rounding
    y_unq = oracle.swiglu_mlp(e4m3_decode(xq) * a1, e4m3_decode(wgu[:I]) * s_gu,
                              e4m3_decode(wgu[I:]) * s_gu, e4m3_decode(wd) * s_d)
    np.testing.assert_allclose(y_unq, a @ (e4m3_decode(wd) * s_d).T, rtol=1e-12)


def _tiny_fp8_layer(rng, T=12, H=32, I=16, E=6, K=2):
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    x = x.to(torch.bfloat16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu, wd = _codes(rng, (E, 2 * I, H)), _codes(rng, (E, H, I))
    sgu = rng.uniform(0.01, 0.05, E)
    sd = rng.uniform(0.01, 0.05, E)
    return x, logits, wgu, sgu, wd, sd


def test_forward_dense_brute_force():
    """out[t] = sum over ALL experts e of G[t, e] * MLP8_e(x_t), G the dense routing weights."""
    rng = np.random.default_rng(8)
    T, E, K = 12, 6, 2
    x, logits, wgu, sgu, wd, sd = _tiny_fp8_layer(rng, T=T, E=E, K=K)
    a1, a2 = 0.02, 0.05
    got = oracle.fp8_forward(x, logits, wgu, sgu, wd, sd, a1, a2, K, True)
    ids, w = oracle.route(logits, K, True)
    G = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            G[t, ids[t, k]] += w[t, k]
    xq = quantize_fp8(x, a1)
    ref = np.zeros_like(got)
    for t in range(T):
        for e in range(E):
            if G[t, e] != 0.0:
                ref[t] += G[t, e] * oracle.fp8_expert_mlp(xq[t:t + 1], a1, wgu[e], sgu[e], wd[e],
                                                          sd[e], a2)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_forward_ep_partial_sums():
    rng = np.random.default_rng(9)
    x, logits, wgu, sgu, wd, sd = _tiny_fp8_layer(rng, E=8)
    full = oracle.fp8_forward(x, logits, wgu, sgu, wd, sd, 0.02, 0.05, 2, True)
    parts = sum(oracle.fp8_forward(x, logits, wgu, sgu, wd, sd, 0.02, 0.05, 2, True,
                                   ep_size=4, ep_rank=r) for r in range(4))
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12)


def test_mutation_ties_away_is_caught():
    """Plausible encoder mistakes (ties away from zero; no clamp before rounding)
    fail the tie and saturation checks used above."""
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))

    def away(v):  # nearest, ties away from zero
        a = np.abs(v)
        i = np.clip(np.searchsorted(pos, a), 1, 126)
        return np.where(a - pos[i - 1] < pos[i] - a, i - 1, i).astype(np.uint8)

    mids = 0.5 * (pos[:-1] + pos[1:])
    assert not np.array_equal(away(mids), e4m3_encode(mids))
    # rounding without the clamp: 479 lies nearer 448 than any larger code,
    # but 480 and above have no nearest finite code; the clamp makes them 448
    assert e4m3_encode([479.0, 480.0, 1000.0]).tolist() == [0x7E, 0x7E, 0x7E]
